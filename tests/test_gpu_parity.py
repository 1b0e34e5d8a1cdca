"""GPU parity: the HIP path through the C-ABI against the fp64 CPU oracle.

Tolerances (per tensor, max |gpu - oracle| / max |oracle|): 1e-4 for fp32
storage, 2e-2 for bf16 storage with fp32 accumulation.  Cases span several
GEMM and attention tiles with ragged tails (token rows, widths and slice
lengths that are not tile multiples), head_dim 64 and 128, every call
grouping (one call for all slices, one call per slice, two slices a call),
and the full-size 13B and GPT-3 175B shards in the grouping the benchmark
times.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_harness as H
from token_transformer_layer_amd import synth
from token_transformer_layer_amd.synth import LayerShape

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}

RAGGED_D64 = LayerShape("ragged-d64", 640, 10, 64, 4000, 2, 3, 200, (77, 50, 73), "bf16", seed=2001)
RAGGED_D128 = LayerShape("ragged-d128", 1024, 8, 128, 2816, 2, 2, 300, (100, 150, 50), "bf16", seed=2002)
TINY_RAGGED_F32 = LayerShape("tiny-ragged-f32", 256, 4, 64, 1008, 2, 3, 70, (1, 29, 40), "f32", seed=2003)


def _layer(shape, sp):
    from token_transformer_layer_amd.shard import ShardLayer
    return ShardLayer(shape, sp)


# the last oracle result, reused by the groupings of one case (the oracle's
# result does not depend on the slice boundaries: pinned on the CPU)
_ORACLE_CACHE = {}


def _oracle_step(key, shape, sp, x, h_mid, dy, du2, du1):
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE.clear()
        # one slice: the result does not depend on the partition
        _ORACLE_CACHE[key] = oracle.shard_layer_step(x, h_mid, dy, du2, du1, sp, shape.as_dict(), [0, shape.seq])
    return _ORACLE_CACHE[key]


def _check_shard(shape, variant, mode, rank=0, full=True, split_wgrad=False):
    x, dy = synth.activations(shape)
    if full:
        sp = oracle.shard_params(synth.full_params(shape, variant), rank, shape.as_dict())
    else:
        sp = synth.shard_params_direct(shape, variant, rank)
    h_mid, du2, du1 = H.step_inputs(shape, shape.seed + 1)
    case = "%s variant=%s mode=%s rank=%d split_wgrad=%s" % (shape.name, variant, mode, rank, split_wgrad)
    print("[case] " + case, flush=True)
    layer = _layer(shape, sp)
    got = H.run_shard_step(layer, x, h_mid, dy, du2, du1, H.groups_of(mode, len(shape.slices)), split_wgrad)
    ref = _oracle_step((shape, variant, rank, full), shape, sp, x, h_mid, dy, du2, du1)
    bad = H.compare_step(got, ref, TOL[shape.dtype], meta=H.step_meta(shape), case=case)
    assert not bad, bad
    return got


@pytest.mark.parametrize("mode", ["whole", "per-slice", "pairs"])
def test_tiny_fp32_shard(mode):
    _check_shard(synth.CONFIGS["tiny-fp32"], "perturbed", mode, rank=1)


def test_tiny_fp32_ragged_sharp():
    _check_shard(TINY_RAGGED_F32, "sharp", "per-slice", rank=0)


@pytest.mark.parametrize("mode", ["whole", "per-slice", "pairs"])
@pytest.mark.parametrize("shape", [RAGGED_D64, RAGGED_D128], ids=lambda s: s.name)
def test_bf16_shard_ragged(shape, mode):
    _check_shard(shape, "perturbed", mode, rank=1)


# Slices of 1, 2 and 7 tokens and token-by-token partitions (a partition is
# any l_1..l_M with sum L: "TeraPipe" summary page, section 3) on the bf16
# kernels: single-query attention tiles, the empty prefix of a first slice
# of one token, dK/dV query tiles that start off a 64-row boundary, and
# products of M = batch rows that split their reduction.
SHORT_D128 = LayerShape("short-slices-d128", 1024, 8, 128, 2816, 2, 2, 128, (1, 1, 2, 60, 64), "bf16", seed=2021)
SHORT_D64 = LayerShape("short-slices-d64", 640, 10, 64, 4000, 2, 2, 128, (1, 2, 7, 63, 1, 54), "bf16", seed=2022)
TOKENWISE_D64_B1 = LayerShape("token-by-token-d64-b1", 640, 10, 64, 4000, 2, 1, 8, (1,) * 8, "bf16", seed=2023)
TOKENWISE_D64_B3 = LayerShape("token-by-token-d64-b3", 640, 10, 64, 4000, 2, 3, 8, (1,) * 8, "bf16", seed=2024)
TOKENWISE_D128 = LayerShape("token-by-token-d128", 1024, 8, 128, 2816, 2, 2, 12, (1,) * 12, "bf16", seed=2025)
SHORT = [SHORT_D128, SHORT_D64, TOKENWISE_D64_B1, TOKENWISE_D64_B3, TOKENWISE_D128]


@pytest.mark.parametrize("mode", ["per-slice", "pairs", "whole"])
@pytest.mark.parametrize("shape", SHORT, ids=lambda s: s.name)
def test_bf16_short_slices(shape, mode):
    _check_shard(shape, "perturbed", mode, rank=1)


@pytest.mark.parametrize("shape", SHORT, ids=lambda s: s.name)
def test_bf16_short_slices_split_weight_gradients(shape):
    _check_shard(shape, "perturbed", "per-slice", rank=0, split_wgrad=True)


def test_short_slice_products_run_transposed():
    """Forward and input-gradient products of at most 128 token rows (the
    120- and 128-row slices of this case) take the transposed path, 256
    weight rows a workgroup with split partial sums, and the step still
    matches the oracle."""
    from token_transformer_layer_amd import abi
    abi.tp_trace_enable(True)
    try:
        _check_shard(SHORT_D128, "perturbed", "per-slice", rank=0)
        names = {r[0] for r in abi.tp_trace_read()}
    finally:
        abi.tp_trace_enable(False)
        abi.tp_trace_read(1)
    assert any(n.startswith("gemm_bf16_sk256x128_nt_") for n in names), sorted(names)
    assert any(n.startswith("gemm_bf16_sk256x128_nn_") for n in names), sorted(names)


def test_bf16_short_slices_peaked():
    _check_shard(SHORT_D128, "peaked", "per-slice", rank=0)


@pytest.mark.parametrize("shape", [TINY_RAGGED_F32, RAGGED_D64, RAGGED_D128], ids=lambda s: s.name)
def test_split_weight_gradients(shape):
    """Per-slice data phases, then one weight-gradient call over all slices,
    every gradient overwritten by its first producer."""
    _check_shard(shape, "perturbed", "per-slice", rank=1, split_wgrad=True)


@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5, 6],
                         ids=["t128", "p128", "t256x128", "t256", "t256x192", "t128x192", "t256w8"])
@pytest.mark.parametrize("shape", [RAGGED_D64, RAGGED_D128], ids=lambda s: s.name)
def test_forced_gemm_tiles(shape, tile):
    """Every tile configuration of the bf16 products, forced on every product
    of a ragged shard (rows, widths and reductions that are not multiples of
    any tile), whole-partition and split-weight-gradient schedules."""
    from token_transformer_layer_amd import abi
    abi.tp_gemm_force_tile(tile)
    try:
        _check_shard(shape, "perturbed", "whole", rank=1)
        _check_shard(shape, "perturbed", "per-slice", rank=0, split_wgrad=True)
    finally:
        abi.tp_gemm_force_tile(-1)


WIDE = [
    # hidden widths that give the LayerNorm kernels 2, 4, 5, 7 and 8 vectors
    # of 8 columns per thread (the bf16 backward at 8192 and 10240: 512
    # threads of 2 and 3), with and without the next-row prefetch
    LayerShape("wide-3072-bf16", 3072, 24, 128, 1024, 8, 1, 24, (10, 14), "bf16", seed=2015),
    LayerShape("wide-8192-bf16", 8192, 64, 128, 2048, 16, 1, 24, (10, 14), "bf16", seed=2011),
    LayerShape("wide-10240-bf16", 10240, 80, 128, 2048, 16, 1, 24, (10, 14), "bf16", seed=2016),
    LayerShape("wide-14336-bf16", 14336, 112, 128, 1792, 16, 1, 24, (10, 14), "bf16", seed=2012),
    LayerShape("wide-16384-bf16", 16384, 128, 128, 2048, 16, 1, 24, (10, 14), "bf16", seed=2013),
    LayerShape("wide-12288-f32", 12288, 96, 128, 1536, 16, 1, 16, (7, 9), "f32", seed=2014),
]


@pytest.mark.parametrize("shape", WIDE, ids=lambda s: s.name)
def test_wide_hidden(shape):
    _check_shard(shape, "perturbed", "per-slice", rank=3, full=False)


def test_full_size_split_weight_gradients():
    """The benchmark's per-slice schedule at the GPT-3 175B shard."""
    _check_shard(synth.CONFIGS["gpt3-175b-t8"], "standard", "per-slice", rank=0, full=False, split_wgrad=True)


def test_bf16_peaked_softmax():
    _check_shard(RAGGED_D128, "peaked", "per-slice", rank=0)


@pytest.mark.parametrize("mode,split", [("whole", False), ("per-slice", False), ("per-slice", True)],
                         ids=["whole", "per-slice", "per-slice-split-wgrad"])
def test_medium_bf16_config(mode, split):
    _check_shard(synth.CONFIGS["medium-bf16"], "standard", mode, rank=2, split_wgrad=split)


@pytest.mark.parametrize("name,mode,split", [("gpt13b-t8", "whole", False), ("gpt13b-t8", "per-slice", False),
                                             ("gpt13b-t8", "per-slice", True), ("gpt3-175b-t8", "whole", False)],
                         ids=["gpt13b-t8-whole", "gpt13b-t8-per-slice", "gpt13b-t8-per-slice-split-wgrad",
                              "gpt3-175b-t8-whole"])
def test_full_size_shard(name, mode, split):
    """The full-size shards in the grouping the benchmark times (one call
    per phase over all slices) and, for the 13B shard's non-uniform
    partition, one call per slice; every output against the fp64 oracle."""
    _check_shard(synth.CONFIGS[name], "standard", mode, rank=0, full=False, split_wgrad=split)


def _full_layer_on_gpu(shape, variant, mode):
    """All t ranks of a layer run one after another on the one GPU; a torch
    sum stands in for each all-reduce (the collective is outside this
    library), and tp_residual_combine adds the residual and row-split bias."""
    import torch

    cfg = shape.as_dict()
    p = synth.full_params(shape, variant)
    x, dy = synth.activations(shape)
    t = shape.tp
    layers = [_layer(shape, oracle.shard_params(p, r, cfg)) for r in range(t)]
    L0 = layers[0]
    xt, dyt = L0.act(x), L0.act(dy)
    b_o, b2 = L0.upload(p["b_o"]), L0.upload(p["b2"])
    h_mid, y, dh, dx = L0.act(), L0.act(), L0.act(), L0.act()
    parts = [L.f32() for L in layers]
    red = L0.f32()
    groups = H.groups_of(mode, len(shape.slices))
    b = shape.batch
    bounds = synth.slice_bounds(shape.slices)
    for L in layers:
        L.new_step()
    for j0, j1 in groups:
        r0, r1 = bounds[j0] * b, bounds[j1] * b
        for L, pt in zip(layers, parts):
            L.fwd(0, j0, j1, xt, pt)
        red[:] = sum(parts)
        L0.combine(xt[bounds[j0]:], red[bounds[j0]:], b_o, h_mid[bounds[j0]:], rows=r1 - r0)
        for L, pt in zip(layers, parts):
            L.fwd(1, j0, j1, h_mid, pt)
        red[:] = sum(parts)
        L0.combine(h_mid[bounds[j0]:], red[bounds[j0]:], b2, y[bounds[j0]:], rows=r1 - r0)
    du2, du1 = L0.f32(), L0.f32()
    for j0, j1 in reversed(groups):
        for L, pt in zip(layers, parts):
            L.bwd(0, j0, j1, dy=dyt, partial_out=pt)
        du2[:] = sum(parts)
        for L, pt in zip(layers, parts):
            L.bwd(1, j0, j1, dy=dyt, ln_in=h_mid, reduced=du2, partial_out=pt, dh=dh)
        du1[:] = sum(parts)
        for L in layers:
            L.bwd(2, j0, j1, ln_in=xt, reduced=du1, dh=dh, dx=dx)
    torch.cuda.synchronize()
    fw = oracle.layer_forward(x, p, cfg)
    gr = oracle.layer_backward(dy, p, cfg, fw)
    tol = TOL[shape.dtype]
    h = lambda z: z.float().cpu().numpy()  # noqa: E731
    errs = {"y": H.max_rel(h(y), fw["y"]), "dx": H.max_rel(h(dx), gr["x"])}
    ht, ft = shape.hidden // t, shape.ffn // t
    g = [{k: h(v) for k, v in L.g.items()} for L in layers]
    full = {
        "w_q": np.concatenate([gg["w_qkv"][:ht] for gg in g]),
        "w_k": np.concatenate([gg["w_qkv"][ht:2 * ht] for gg in g]),
        "w_v": np.concatenate([gg["w_qkv"][2 * ht:] for gg in g]),
        "b_q": np.concatenate([gg["b_qkv"][:ht] for gg in g]),
        "b_v": np.concatenate([gg["b_qkv"][2 * ht:] for gg in g]),
        "w_o": np.concatenate([gg["w_o"] for gg in g], axis=1),
        "w1": np.concatenate([gg["w1"] for gg in g]),
        "b1": np.concatenate([gg["b1"] for gg in g]),
        "w2": np.concatenate([gg["w2"] for gg in g], axis=1),
    }
    for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "b_o", "b2"):
        full[k] = g[0][k]
    for k, v in full.items():
        errs["grad_" + k] = H.max_rel(v, gr[k])
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, bad


@pytest.mark.parametrize("mode", ["whole", "per-slice"])
def test_tiny_fp32_full_layer_tp2(mode):
    _full_layer_on_gpu(synth.CONFIGS["tiny-fp32"], "perturbed", mode)


def test_bf16_full_layer_tp2():
    _full_layer_on_gpu(RAGGED_D64, "perturbed", "per-slice")


def test_deterministic_repeat():
    """Two runs of the same step give bit-identical outputs (no atomics)."""
    shape = RAGGED_D128
    x, dy = synth.activations(shape)
    sp = oracle.shard_params(synth.full_params(shape, "perturbed"), 0, shape.as_dict())
    h_mid, du2, du1 = H.step_inputs(shape, 7)
    layer = _layer(shape, sp)
    a = H.run_shard_step(layer, x, h_mid, dy, du2, du1, H.groups_of("per-slice", 3))
    b = H.run_shard_step(layer, x, h_mid, dy, du2, du1, H.groups_of("per-slice", 3))
    for k in ("p_attn", "p_mlp", "p_du2", "p_du1", "dx"):
        assert np.array_equal(a[k], b[k]), k
    for k in a["grads"]:
        assert np.array_equal(a["grads"][k], b["grads"][k]), k


def test_cube_block_small():
    import torch
    c = synth.CubeShape("cube-small", 300, 512, 2056, seed=31)
    x, w1, b1, w2 = synth.cube_inputs(c)
    b1 = synth.round_bf16(np.random.default_rng(3).standard_normal(c.ffn).astype(np.float32) * 0.02)
    from token_transformer_layer_amd import abi
    dev = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)  # noqa: E731
    xt, w1t, b1t, w2t = dev(x), dev(w1), dev(b1), dev(w2)
    hb = torch.empty((c.rows, c.ffn), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((c.rows, c.hidden), dtype=torch.float32, device="cuda")
    abi.tp_cube_ffn_block(c.rows, c.hidden, c.ffn, xt.data_ptr(), w1t.data_ptr(), b1t.data_ptr(), w2t.data_ptr(),
                          hb.data_ptr(), out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = oracle.cube_ffn_block(x, w1, b1, w2)
    assert H.max_rel(out.cpu().numpy(), ref) <= TOL["bf16"]


def test_cube_block_full_size_rows():
    """The full cube block (X 4096 x 6144, W1 6144 -> 24576, W2 24576 ->
    6144) on the GPU; the oracle checks a sample of output rows, each
    computed from its own input row."""
    import torch
    c = synth.CUBE
    x, w1, b1, w2 = synth.cube_inputs(c)
    from token_transformer_layer_amd import abi
    dev = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)  # noqa: E731
    xt, w1t, b1t, w2t = dev(x), dev(w1), dev(b1), dev(w2)
    hb = torch.empty((c.rows, c.ffn), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((c.rows, c.hidden), dtype=torch.float32, device="cuda")
    abi.tp_cube_ffn_block(c.rows, c.hidden, c.ffn, xt.data_ptr(), w1t.data_ptr(), b1t.data_ptr(), w2t.data_ptr(),
                          hb.data_ptr(), out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 1000, 2047, 2048, 3333, 4095])
    ref = oracle.cube_ffn_block(x[rows], w1, b1, w2)
    assert H.max_rel(out.cpu().numpy()[rows], ref) <= TOL["bf16"]
