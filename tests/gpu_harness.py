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


# Every comparison made through compare_step, for the parity report that
# tests/conftest.py writes when TP_PARITY_REPORT names a file.
REPORT = []


def elem_rel(got, ref, floor=1e-3):
    """max_i |got_i - ref_i| / max(|ref_i|, floor * max|ref|): the
    element-wise relative error, with elements below floor * max|ref|
    measured against that floor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    big = float(np.abs(ref).max())
    if big == 0:
        return float(np.abs(got).max())
    r = np.abs(got - ref) / np.maximum(np.abs(ref), floor * big)
    return float(r.max()) if np.all(np.isfinite(r)) else float("inf")


def _starts(n, step):
    return np.arange(0, n, step)


def block_rel(got, ref, row_starts, col_starts):
    """Largest per-block relative error of a 2-D tensor cut into blocks at
    the given row and column starts: max over blocks of max|got - ref| /
    max|ref| within the block.  A block whose reference is zero up to fp64
    rounding (at most 1e-9 of the tensor's maximum: a gradient that vanishes
    exactly, such as that of the key bias) is measured against the tensor's
    maximum instead."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    if not np.all(np.isfinite(d)):
        return float("inf")
    a = np.abs(ref)
    big = float(a.max())
    if big == 0:
        return float(d.max())

    def bmax(x):
        return np.maximum.reduceat(np.maximum.reduceat(x, row_starts, axis=0), col_starts, axis=1)

    dm, rm = bmax(d), bmax(a)
    rm = np.where(rm <= 1e-9 * big, big, rm)
    return float((dm / rm).max())


# Tolerance of the block checks (a gross-error check beside the per-tensor
# bar).  A block's maximum can be well below its tensor's while the
# rounding noise of bf16 operands is not.  The largest noise is in the
# attention path: bf16 Q and K move a logit s by about sqrt(2) u_r
# sqrt(sum_i (q_i k_i)^2) / sqrt(d) (u_r = 2^-8 / sqrt(3), the RMS relative
# error of rounding to bf16), i.e. by sqrt(2) u_r sigma_s for logits of
# standard deviation sigma_s = 0.02^2 h at these weight scales: 1.5e-2 at
# h = 12288 (sigma_s ~ 4.9), 2.1e-2 at h = 16384, and every attention
# weight, hence dQ, dK, dV and their products, carries that relative noise.
# The largest block errors measured on the bf16 cases are 2.1e-2 at
# h = 12288 and 3.6e-2 at h = 14336; a wrong region has an error of the
# order of its own magnitude, twenty times this bound.
BLOCK_TOL = 5e-2


def _partitions(name, arr, meta):
    """Blockings of one output of a step, as (matrix, row starts, column
    starts, label, is_grid).  Activations [s, b, h] by token slice (rows)
    and 128 columns; the K/V cache [b, n_t, s, d] by (batch row, head, token
    slice); weight gradients by head (the Q/K/V rows, the out-projection
    columns) or 256 rows/columns; vectors by head or 256 entries.  Each
    blocking is checked along rows alone, along columns alone, and on the
    grid of both."""
    bounds, b, d = meta["bounds"], meta["batch"], meta["head_dim"]
    if name in ("p_attn", "p_mlp", "p_du2", "p_du1", "dh", "dx"):
        a2 = arr.reshape(-1, arr.shape[-1])
        rows, cols = np.array(bounds[:-1]) * b, _starts(a2.shape[1], 128)
    elif name in ("k", "v"):
        a2 = arr.reshape(-1, arr.shape[-1])          # [(b nt s), d]
        s = arr.shape[2]
        rows = np.concatenate([i * s + np.array(bounds[:-1]) for i in range(arr.shape[0] * arr.shape[1])])
        cols = np.array([0])
    elif arr.ndim == 2:
        a2 = arr
        rows = _starts(arr.shape[0], d if name == "w_qkv" else 256)
        cols = _starts(arr.shape[1], d if name == "w_o" else 256)
    else:
        a2 = arr.reshape(1, -1)
        rows, cols = np.array([0]), _starts(a2.shape[1], d if name == "b_qkv" else 256)
    zero = np.array([0])
    out = []
    if len(rows) > 1:
        out.append((a2, rows, zero, "rows", False))
    if len(cols) > 1:
        out.append((a2, zero, cols, "cols", False))
    if len(rows) > 1 and len(cols) > 1:
        out.append((a2, rows, cols, "grid", True))
    return out


def compare_step(got, ref, tol, skip=(), meta=None, case=""):
    """Relative errors of a GPU step against the oracle's shard_layer_step
    output.  Every tensor is held to tol per tensor (max|Δ| / max|ref|) and,
    when meta (slice bounds, batch, head_dim) is given, per block as well
    (block_rel: a wrong low-magnitude slice, head or column range cannot
    hide under the tensor's maximum): to BLOCK_TOL along each row and
    column blocking and on the grid of both.  The element-wise relative error
    (elem_rel) is computed and reported beside them.  Returns {name: err}
    for the checks above tol."""
    bad = {}
    rec = {"case": case, "tol": tol, "tensors": {}}
    pairs = []
    for name in ("p_attn", "p_mlp", "p_du2", "p_du1", "dh", "dx"):
        if name not in skip:
            pairs.append((name, name, got[name], ref[name]))
    for kk in ("k", "v"):
        pairs.append(("cache_" + kk, kk, got[kk], ref["kv"][kk]))
    for name in GRAD_NAMES:
        if name not in skip:
            pairs.append(("grad_" + name, name, got["grads"][name], ref["grads"][name]))
    for label, kind, g, r in pairs:
        e = max_rel(g, r)
        m = {"tensor": e, "elem": elem_rel(g, r)}
        if not e <= tol:
            bad[label] = e
        if meta is not None:
            for (g2, rows, cols, kind_b, grid), (r2, _, _, _, _) in zip(_partitions(kind, np.asarray(g), meta),
                                                                        _partitions(kind, np.asarray(r), meta)):
                eb = block_rel(g2, r2, rows, cols)
                m[kind_b] = eb
                if not eb <= BLOCK_TOL:
                    bad[label + "/" + kind_b] = eb
        rec["tensors"][label] = m
    REPORT.append(rec)
    worst = {k: max(v.get(k, 0.0) for v in rec["tensors"].values()) for k in ("tensor", "rows", "cols", "grid", "elem")}
    print("[parity] %s worst per-tensor %.2e, by rows %.2e, by columns %.2e, grid %.2e; element-wise (1e-3 floor) "
          "%.2e" % (case, worst["tensor"], worst["rows"], worst["cols"], worst["grid"], worst["elem"]), flush=True)
    return bad


def step_meta(shape):
    bounds = [0]
    for n in shape.slices:
        bounds.append(bounds[-1] + int(n))
    return {"bounds": bounds, "batch": shape.batch, "head_dim": shape.head_dim}
