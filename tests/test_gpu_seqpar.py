"""GPU parity of the sequence-parallel form of the layer shard: LayerNorm on
each rank's sequence shard (tp_layernorm_fwd / tp_layernorm_bwd), the _SP
phases on the all-gathered LayerNorm output and dH, and the partial sums
reduce-scattered.  All t ranks run one after another on the one GPU; a torch
sum over ranks followed by each rank taking its rows stands in for the
reduce-scatter, and writing each rank's shard into one shared buffer for
the all-gather.  Compared with the oracle's unsharded layer (forward and
every gradient; LayerNorm parameter gradients are the sum of the ranks'
shares, i.e. after their all-reduce)."""
import numpy as np
import pytest

import oracle
from tests import gpu_harness as H
from token_transformer_layer_amd import abi, synth
from token_transformer_layer_amd.synth import LayerShape

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
RAGGED_D64 = LayerShape("ragged-d64", 640, 10, 64, 4000, 2, 3, 200, (77, 50, 73), "bf16", seed=2001)


def _run_sp(shape, variant, mode):
    import torch
    from token_transformer_layer_amd.shard import ShardLayer, stream_handle
    cfg = shape.as_dict()
    p = synth.full_params(shape, variant)
    x, dy = synth.activations(shape)
    t, b, h = shape.tp, shape.batch, shape.hidden
    T = shape.seq * b
    layers = [ShardLayer(shape, oracle.shard_params(p, r, cfg)) for r in range(t)]
    L0 = layers[0]
    st = stream_handle()
    xt, dyt = L0.act(x), L0.act(dy)
    ln = {k: L0.upload(p[k]) for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b")}
    b_o, b2 = L0.upload(p["b_o"]), L0.upload(p["b2"])
    u1, u2, h_mid, y, dh, dx = (L0.act() for _ in range(6))
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")  # noqa: E731
    stats = {r: {k: f32(T) for k in ("mu1", "rs1", "mu2", "rs2")} for r in range(t)}
    lng = {r: {k: f32(h) for k in ("g1", "b1", "g2", "b2")} for r in range(t)}
    parts = [L.f32() for L in layers]
    red = L0.f32()
    work = torch.empty(abi.tp_layernorm_work_bytes(L0.cfg, T), dtype=torch.uint8, device="cuda")
    groups = H.groups_of(mode, len(shape.slices))
    bounds = synth.slice_bounds(shape.slices)
    row = lambda buf, r0: buf.data_ptr() + r0 * h * buf.element_size()  # noqa: E731
    srow = lambda buf, r0: buf.data_ptr() + r0 * 4  # noqa: E731
    for L in layers:
        L.new_step()

    def shards(r0, r1):
        return [(int(c[0]), int(c[-1]) + 1) for c in np.array_split(np.arange(r0, r1), t) if len(c)]

    def ln_fwd(r, a, z, src, dst, g, bb, mu, rs):
        abi.tp_layernorm_fwd(L0.cfg, z - a, row(src, a), g.data_ptr(), bb.data_ptr(), row(dst, a),
                             srow(stats[r][mu], a), srow(stats[r][rs], a), st)

    for j0, j1 in groups:
        r0, r1 = bounds[j0] * b, bounds[j1] * b
        sh = shards(r0, r1)
        for r, (a, z) in enumerate(sh):           # LN1 on each shard, gathered into u1
            ln_fwd(r, a, z, xt, u1, ln["ln1_g"], ln["ln1_b"], "mu1", "rs1")
        for L, pt in zip(layers, parts):
            L.fwd(abi.TP_FWD_ATTN_SP, j0, j1, u1, pt)
        red[:] = sum(parts)                        # reduce-scatter: each rank combines its rows
        for r, (a, z) in enumerate(sh):
            abi.tp_residual_combine(L0.cfg, z - a, row(xt, a), srow(red, 0) + a * h * 4, b_o.data_ptr(),
                                    row(h_mid, a), st)
            ln_fwd(r, a, z, h_mid, u2, ln["ln2_g"], ln["ln2_b"], "mu2", "rs2")
        for L, pt in zip(layers, parts):
            L.fwd(abi.TP_FWD_MLP_SP, j0, j1, u2, pt)
        red[:] = sum(parts)
        for r, (a, z) in enumerate(sh):
            abi.tp_residual_combine(L0.cfg, z - a, row(h_mid, a), srow(red, 0) + a * h * 4, b2.data_ptr(),
                                    row(y, a), st)
    for j0, j1 in reversed(groups):
        r0, r1 = bounds[j0] * b, bounds[j1] * b
        sh = shards(r0, r1)
        for L, pt in zip(layers, parts):
            L.bwd(abi.TP_BWD_MLP, j0, j1, dy=dyt, partial_out=pt)
        red[:] = sum(parts)
        for r, (a, z) in enumerate(sh):            # LN2 backward on each shard, dH gathered
            abi.tp_layernorm_bwd(L0.cfg, z - a, srow(red, 0) + a * h * 4, row(dyt, a), row(h_mid, a),
                                 ln["ln2_g"].data_ptr(), srow(stats[r]["mu2"], a), srow(stats[r]["rs2"], a),
                                 row(dh, a), lng[r]["g2"].data_ptr(), lng[r]["b2"].data_ptr(), True,
                                 work.data_ptr(), st)
        for L, pt in zip(layers, parts):
            L.bwd(abi.TP_BWD_ATTN_SP, j0, j1, dy=dyt, partial_out=pt, dh=dh)
        red[:] = sum(parts)
        for r, (a, z) in enumerate(sh):
            abi.tp_layernorm_bwd(L0.cfg, z - a, srow(red, 0) + a * h * 4, row(dh, a), row(xt, a),
                                 ln["ln1_g"].data_ptr(), srow(stats[r]["mu1"], a), srow(stats[r]["rs1"], a),
                                 row(dx, a), lng[r]["g1"].data_ptr(), lng[r]["b1"].data_ptr(), True,
                                 work.data_ptr(), st)
    torch.cuda.synchronize()
    fw = oracle.layer_forward(x, p, cfg)
    gr = oracle.layer_backward(dy, p, cfg, fw)
    tol = TOL[shape.dtype]
    hn = lambda z: z.float().cpu().numpy()  # noqa: E731
    errs = {"y": H.max_rel(hn(y), fw["y"]), "dx": H.max_rel(hn(dx), gr["x"])}
    lnsum = {k: sum(hn(lng[r][k]) for r in range(t)) for k in ("g1", "b1", "g2", "b2")}
    for ours, ref in (("g1", "ln1_g"), ("b1", "ln1_b"), ("g2", "ln2_g"), ("b2", "ln2_b")):
        errs[ref] = H.max_rel(lnsum[ours], gr[ref])
    ht, ft = shape.hidden // t, shape.ffn // t
    g = [{k: hn(v) for k, v in L.g.items()} for L in layers]
    full = {
        "w_q": np.concatenate([gg["w_qkv"][:ht] for gg in g]),
        "w_k": np.concatenate([gg["w_qkv"][ht:2 * ht] for gg in g]),
        "w_v": np.concatenate([gg["w_qkv"][2 * ht:] for gg in g]),
        "b_q": np.concatenate([gg["b_qkv"][:ht] for gg in g]),
        "b_v": np.concatenate([gg["b_qkv"][2 * ht:] for gg in g]),
        "b1": np.concatenate([gg["b1"] for gg in g]),
        "w_o": np.concatenate([gg["w_o"] for gg in g], axis=1),
        "w1": np.concatenate([gg["w1"] for gg in g]),
        "w2": np.concatenate([gg["w2"] for gg in g], axis=1),
        "b_o": g[0]["b_o"], "b2": g[0]["b2"],
    }
    for k, v in full.items():
        errs[k] = H.max_rel(v, gr[k])
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, bad


@pytest.mark.parametrize("mode", ["whole", "per-slice"])
def test_sequence_parallel_fp32(mode):
    _run_sp(synth.CONFIGS["tiny-fp32"], "perturbed", mode)


@pytest.mark.parametrize("mode", ["whole", "per-slice"])
def test_sequence_parallel_bf16(mode):
    _run_sp(RAGGED_D64, "perturbed", mode)
