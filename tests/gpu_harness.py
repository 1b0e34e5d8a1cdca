"""Helpers for the GPU parity tests: run one rank's shard through the C-ABI
over a chosen grouping of token slices and bring the results back to host
arrays, and the error metric the tolerances are stated in."""
import numpy as np

from token_transformer_layer_amd.synth import round_bf16

GRAD_NAMES = ["ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g", "ln2_b", "w1", "b1", "w2", "b2"]


def max_rel(got, ref):
    """max |got - ref| / max |ref| over one tensor (the per-tensor relative
    error the tolerances are stated in)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.abs(ref).max())
    num = float(np.abs(got - ref).max())
    if not np.isfinite(num):
        return float("inf")
    return num / den if den > 0 else num


def step_inputs(shape, seed):
    """Seeded stand-ins for the caller-side tensors of one step on one rank:
    h_mid (the combined residual stream, storage dtype) and the two
    all-reduced gradients (fp32), each N(0, 1)."""
    rng = np.random.default_rng(seed)
    sz = (shape.seq, shape.batch, shape.hidden)
    h_mid = rng.standard_normal(sz).astype(np.float32)
    if shape.dtype == "bf16":
        h_mid = round_bf16(h_mid)
    du2 = rng.standard_normal(sz).astype(np.float32)
    du1 = rng.standard_normal(sz).astype(np.float32)
    return h_mid, du2, du1


def groups_of(mode, nslices):
    """Slice ranges [j0, j1) of the calls: 'whole' = one call over all
    slices; 'per-slice' = one call per slice; 'pairs' = two slices a call."""
    if mode == "whole":
        return [(0, nslices)]
    if mode == "per-slice":
        return [(j, j + 1) for j in range(nslices)]
    if mode == "pairs":
        return [(j, min(j + 2, nslices)) for j in range(0, nslices, 2)]
    raise ValueError(mode)


def run_shard_step(layer, x, h_mid, dy, du2, du1, groups, split_wgrad=False):
    """Forward (groups in order: ATTN then MLP per group) and backward
    (groups in reverse) of one rank, with the caller's reduced tensors given.
    split_wgrad=False: MLP, ATTN, LN1 per group, gradients accumulated into
    zeroed buffers.  split_wgrad=True: MLP_DATA, ATTN_DATA, LN1 per group,
    then one WGRAD call over all slices; every gradient is overwritten by its
    first producer (the buffers start as NaN, so a missed overwrite shows).
    Returns host float64 arrays."""
    import torch

    xt, hm, dyt = layer.act(x), layer.act(h_mid), layer.act(dy)
    du2t = torch.from_numpy(du2).to(layer.device)
    du1t = torch.from_numpy(du1).to(layer.device)
    p_attn, p_mlp, p_du2, p_du1 = layer.f32(), layer.f32(), layer.f32(), layer.f32()
    dh, dx = layer.act(), layer.act()
    layer.new_step(float("nan") if split_wgrad else 0.0)
    for j0, j1 in groups:
        layer.fwd(0, j0, j1, xt, p_attn)
        layer.fwd(1, j0, j1, hm, p_mlp)
    first = True
    for j0, j1 in reversed(groups):
        if split_wgrad:
            layer.bwd(3, j0, j1, dy=dyt, partial_out=p_du2, accumulate=not first)
            layer.bwd(4, j0, j1, dy=dyt, ln_in=hm, reduced=du2t, partial_out=p_du1, dh=dh, accumulate=not first)
            layer.bwd(2, j0, j1, ln_in=xt, reduced=du1t, dh=dh, dx=dx, accumulate=not first)
        else:
            layer.bwd(0, j0, j1, dy=dyt, partial_out=p_du2)
            layer.bwd(1, j0, j1, dy=dyt, ln_in=hm, reduced=du2t, partial_out=p_du1, dh=dh)
            layer.bwd(2, j0, j1, ln_in=xt, reduced=du1t, dh=dh, dx=dx)
        first = False
    if split_wgrad:
        layer.bwd(5, groups[0][0], groups[-1][1], dy=dyt, dh=dh, accumulate=False)
    torch.cuda.synchronize()

    def h(t):
        return t.float().cpu().numpy().astype(np.float64)

    out = dict(p_attn=h(p_attn), p_mlp=h(p_mlp), p_du2=h(p_du2), p_du1=h(p_du1), dh=h(dh), dx=h(dx),
               k=h(layer.k), v=h(layer.v))
    out["grads"] = {n: h(layer.g[n]) for n in GRAD_NAMES}
    return out


def compare_step(got, ref, tol, skip=()):
    """Per-tensor relative errors of a GPU step against the oracle's
    shard_layer_step output; returns {name: err} for errors above tol."""
    bad = {}
    for name in ("p_attn", "p_mlp", "p_du2", "p_du1", "dh", "dx"):
        if name in skip:
            continue
        e = max_rel(got[name], ref[name])
        if not e <= tol:
            bad[name] = e
    for name, kk in (("k", "k"), ("v", "v")):
        e = max_rel(got[name], ref["kv"][kk])
        if not e <= tol:
            bad["cache_" + name] = e
    for name in GRAD_NAMES:
        if name in skip:
            continue
        e = max_rel(got["grads"][name], ref["grads"][name])
        if not e <= tol:
            bad["grad_" + name] = e
    return bad
