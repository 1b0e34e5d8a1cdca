"""fp64 definition of one pre-LayerNorm GPT decoder layer, of one
tensor-parallel device's share of it, and of that share run over token slices.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg.

Sources, cited by page title and section:

[MP]  "Maximizing Parallelism in Distributed Training for Huge Neural
      Networks" (Bian, Xu, Wang, You).  Section 3.1.2 (Matrix-matrix
      Operations) gives the three product forms and their gradients;
      section 3.1.3 (Matrix-vector Operations) gives C = A + b / C = A*b and
      their backward (dA = dC, db = sum of dC over rows); section 3.2
      (Parallel Transformer layers) gives the layer as a Self-Attention block
      and an MLP block of two linear layers each, with LayerNorm applying
      gamma and beta as matrix-vector ops; section 2.3 gives the block
      product C_ij = sum_l A_il B_lj.
[TT11] "Transformer Training 11: model parallelism" (slide deck), tensor
      parallelism slide: FC1 split by columns (GELU stays local), FC2 split by
      rows into a partial sum that one all-reduce adds; attention split the
      same way, one group of heads per device; two all-reduces forward and two
      backward.  Sequence-parallelism slide: LayerNorm is not split by tensor
      parallelism (each device holds it whole).
[TP]  "TeraPipe: Token-Level Pipeline Parallelism for Training Large-Scale
      Language Models" (summary page), section 3 (Method): a layer's output at
      token t needs only earlier positions (self-attention) and the current
      one (feed-forward), so a sequence can run as slices l_1..l_M with
      sum l_j = L; section "Takeaways": unidirectional (causal) models only.

Readings where the pages are silent: LayerNorm
with biased variance and eps = 1e-5; exact erf GELU; attention scale 1/sqrt(d);
the causal mask keeps the diagonal; pre-LN with a residual around each block;
the row-split biases b_o and b2 are left out of the partial sums and added
once after the reduction; no dropout; separate W_q, W_k, W_v, each split by
head group, stacked [Q_r; K_r; V_r] on a device.

Conventions: activations are sequence-major [s, b, h]; linear weights are
stored [out, in] and applied as y = x W^T + b; attention tensors per head are
[b, heads, positions, d].  Everything is float64 numpy.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "normal_cdf", "normal_pdf", "gelu", "gelu_grad",
    "layer_norm", "layer_norm_backward",
    "heads_split", "heads_merge",
    "causal_attention", "causal_attention_backward",
    "attention_block", "merge_partials", "attention_block_backward",
    "layer_forward", "layer_backward",
    "shard_params", "new_kv_cache", "new_kv_grad",
    "shard_attn_forward", "shard_mlp_forward",
    "shard_mlp_backward", "shard_attn_backward", "ln1_backward",
    "residual_combine", "shard_layer_step", "cube_ffn_block",
]


# ----------------------------------------------------------------------------
# Elementwise pieces
# ----------------------------------------------------------------------------

def normal_cdf(z):
    """Standard normal CDF, Phi(z) = (1 + erf(z / sqrt 2)) / 2."""
    return 0.5 * (1.0 + _erf(np.asarray(z, dtype=np.float64) / math.sqrt(2.0)))


def normal_pdf(z):
    """Standard normal density phi(z)."""
    z = np.asarray(z, dtype=np.float64)
    return np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def gelu(z):
    """GELU in its exact form z * Phi(z).  [TT11] tensor-parallel slide names
    GELU without a formula; the erf form is this repository's reading."""
    z = np.asarray(z, dtype=np.float64)
    return z * normal_cdf(z)


def gelu_grad(z):
    """d/dz [z Phi(z)] = Phi(z) + z phi(z)."""
    z = np.asarray(z, dtype=np.float64)
    return normal_cdf(z) + z * normal_pdf(z)


# ----------------------------------------------------------------------------
# LayerNorm ([MP] section 3.2: gamma/beta applied as matrix-vector ops;
# [MP] section 3.1.3 for the backward of C = A*b and C = A + b)
# ----------------------------------------------------------------------------

def layer_norm(x, gamma, beta, eps):
    """u = (x - mean) / sqrt(var + eps) * gamma + beta over the last axis, with
    the biased variance (divide by h).  Returns (u, mean, rstd)."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean) * rstd
    return xhat * gamma + beta, mean[..., 0], rstd[..., 0]


def layer_norm_backward(du, x, gamma, mean, rstd):
    """Vector-Jacobian product of layer_norm.

    With xhat = (x - mean) rstd and g = du * gamma (the C = A*b backward of
    [MP] 3.1.3), dx = rstd (g - mean_h(g) - xhat mean_h(g xhat)).  The
    parameter gradients are the row sums dgamma = sum du*xhat and
    dbeta = sum du ([MP] 3.1.3: db is dC summed over rows).  Returns
    (dx, dgamma, dbeta)."""
    du = np.asarray(du, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1]
    xhat = (x - mean[..., None]) * rstd[..., None]
    g = du * gamma
    dx = rstd[..., None] * (g - g.mean(axis=-1, keepdims=True)
                            - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    dgamma = (du * xhat).reshape(-1, h).sum(axis=0)
    dbeta = du.reshape(-1, h).sum(axis=0)
    return dx, dgamma, dbeta


# ----------------------------------------------------------------------------
# Attention heads and causal attention ([TT11] tensor-parallel slide: heads
# are independent; [TP] section 3: position p attends to positions <= p)
# ----------------------------------------------------------------------------

def heads_split(a, n_heads):
    """[s, b, n*d] -> [b, n, s, d]: head i owns columns [i d, (i+1) d)."""
    s, b, hd = a.shape
    d = hd // n_heads
    return np.ascontiguousarray(a.reshape(s, b, n_heads, d).transpose(1, 2, 0, 3))


def heads_merge(a):
    """[b, n, s, d] -> [s, b, n*d], the inverse of heads_split."""
    b, n, s, d = a.shape
    return np.ascontiguousarray(a.transpose(2, 0, 1, 3).reshape(s, b, n * d))


def causal_attention(q, k, v, q_start=0):
    """Scaled dot-product attention with a causal mask.

    q: [b, n, Lq, d], the queries at positions q_start .. q_start+Lq-1.
    k, v: [b, n, Lk, d], the keys and values at positions 0 .. Lk-1 (the
    prefix cache plus the slice itself when run over token slices).
    Query at position p sees keys j <= p (the diagonal included):
    S_pj = q_p . k_j / sqrt(d); P = softmax_j(S) taken with the row maximum
    subtracted; o_p = sum_j P_pj v_j.  Returns (o, P, lse) with
    lse_p = log sum_{j<=p} exp(S_pj)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    lq, lk = q.shape[-2], k.shape[-2]
    scores = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(d)
    pos_q = q_start + np.arange(lq)
    pos_k = np.arange(lk)
    masked = pos_k[None, :] > pos_q[:, None]
    scores = np.where(masked, -np.inf, scores)
    row_max = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - row_max)
    denom = e.sum(axis=-1, keepdims=True)
    p = e / denom
    lse = (row_max + np.log(denom))[..., 0]
    return p @ v, p, lse


def causal_attention_backward(do, q, k, v, p, o):
    """Vector-Jacobian product of causal_attention for the given P and O.

    The two products S = Q K^T / sqrt(d) and O = P V take the gradients of
    [MP] 3.1.2 (C = AB^T: dA = dC B, dB = dC^T A; C = AB: dA = dC B^T,
    dB = A^T dC); the softmax row backward is dS = P * (dP - rowsum(dP * P)),
    and rowsum(dP * P) = rowsum(dO * O).  Masked entries have P = 0 and so
    take no gradient.  Returns (dq, dk, dv) shaped like q, k, v."""
    do = np.asarray(do, dtype=np.float64)
    d = q.shape[-1]
    dv = np.swapaxes(p, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    row_dot = (do * o).sum(axis=-1, keepdims=True)
    ds = p * (dp - row_dot)
    dq = (ds @ k) / math.sqrt(d)
    dk = (np.swapaxes(ds, -1, -2) @ q) / math.sqrt(d)
    return dq, dk, dv


# ----------------------------------------------------------------------------
# Attention over one block of keys and values, and the merge of two partial
# results ([TT11], the passage after the sequence-parallelism slide on very
# long sequences: the queries stay on their device while the key/value blocks
# of all devices circulate between them).  A device therefore sees the keys
# one block at a time; the exact result over all keys follows from the
# per-block results by the log-sum-exp identity (a reading: the pages do not
# spell out how blocks are combined, and exact attention over the union is
# the plainest one).  The backward of one block takes the merged result.
# ----------------------------------------------------------------------------

def attention_block(q, k, v, q_pos0, k_pos0):
    """Causal attention of queries at positions q_pos0 .. q_pos0+Lq-1 over
    one block of keys at positions k_pos0 .. k_pos0+Lk-1.

    q: [b, n, Lq, d]; k, v: [b, n, Lk, d].  Query at position p sees the
    block's keys at positions j <= p.  Returns (o, lse): o_p = sum_j P_pj v_j
    with P the softmax over the visible keys of the block, lse_p = log sum_j
    exp(q_p . k_j / sqrt(d)) over the same keys; a query that sees none of
    the block's keys gets o = 0 and lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    lq, lk = q.shape[-2], k.shape[-2]
    scores = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(d)
    pos_q = q_pos0 + np.arange(lq)
    pos_k = k_pos0 + np.arange(lk)
    visible = pos_k[None, :] <= pos_q[:, None]
    scores = np.where(visible, scores, -np.inf)
    any_visible = visible.any(axis=-1)
    # (a block of no keys: the maximum over an empty row is -inf, masked out)
    row_max = np.where(any_visible, scores.max(axis=-1, initial=-np.inf), 0.0)[..., None]
    e = np.where(visible, np.exp(scores - row_max), 0.0)
    denom = e.sum(axis=-1, keepdims=True)
    safe = np.where(denom > 0, denom, 1.0)
    o = (e / safe) @ v
    lse = np.where(any_visible, (row_max + np.log(safe))[..., 0], -np.inf)
    return o, lse


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Attention over the union of two disjoint key sets from the results
    over each: with m = max(lse_a, lse_b), w_x = exp(lse_x - m),
    o = (w_a o_a + w_b o_b) / (w_a + w_b) and lse = m + log(w_a + w_b).  A
    side with lse = -inf (no visible key) has weight 0; if both are -inf the
    result is o = 0, lse = -inf."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w_a = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - m_safe))
    w_b = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - m_safe))
    tot = w_a + w_b
    tot_safe = np.where(empty, 1.0, tot)
    o = (w_a[..., None] * o_a + w_b[..., None] * o_b) / tot_safe[..., None]
    lse = np.where(empty, -np.inf, m_safe + np.log(tot_safe))
    return o, lse


def attention_block_backward(do, q, k, v, o, lse, q_pos0, k_pos0):
    """Backward of attention_block for one key block, given the result over
    all blocks: o and lse are the merged output and log-sum-exp of each
    query (over every key it sees, in any block) and do the gradient of o.

    On the block's visible keys the full softmax is P_pj = exp(S_pj - lse_p)
    (S_pj = q_p . k_j / sqrt(d)); with D_p = rowsum(do_p * o_p) the
    gradients of the two products and the softmax (as in
    causal_attention_backward) restricted to the block are dV = P^T do,
    dP = do V^T, dS = P * (dP - D), dq = dS K / sqrt(d) (this block's share
    of the query gradient) and dK = dS^T q / sqrt(d).  Summed over all
    blocks the shares give the full dQ, and each block's dK, dV are the full
    gradients of its keys.  Returns (dq_share, dk, dv)."""
    do, q, k, v, o = (np.asarray(a, dtype=np.float64) for a in (do, q, k, v, o))
    lse = np.asarray(lse, dtype=np.float64)
    d = q.shape[-1]
    lq, lk = q.shape[-2], k.shape[-2]
    scores = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(d)
    pos_q = q_pos0 + np.arange(lq)
    pos_k = k_pos0 + np.arange(lk)
    visible = (pos_k[None, :] <= pos_q[:, None]) & np.isfinite(lse)[..., None]
    lse_safe = np.where(np.isfinite(lse), lse, 0.0)[..., None]
    p = np.where(visible, np.exp(np.where(visible, scores, 0.0) - lse_safe), 0.0)
    dv = np.swapaxes(p, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    row_dot = (do * o).sum(axis=-1, keepdims=True)
    ds = p * (dp - row_dot)
    dq = (ds @ k) / math.sqrt(d)
    dk = (np.swapaxes(ds, -1, -2) @ q) / math.sqrt(d)
    return dq, dk, dv


# ----------------------------------------------------------------------------
# The unsharded layer ([MP] section 3.2; [TT11] tensor-parallel slide)
# ----------------------------------------------------------------------------

def _mm(a, m):
    """a @ m over the last axis of a, as one 2-D product of the flattened
    rows (numpy would otherwise loop over the leading axes)."""
    a = np.asarray(a, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    return (a.reshape(-1, a.shape[-1]) @ m).reshape(a.shape[:-1] + (m.shape[-1],))


def _linear(a, w, b=None):
    """y = a W^T (+ b) with W stored [out, in]."""
    y = _mm(a, np.asarray(w).T)
    return y if b is None else y + b


def layer_forward(x, p, cfg):
    """Forward of the whole (unsharded) pre-LN decoder layer on x [s, b, h]:
    u1 = LN1(x); q, k, v = u1 W^T + b per matrix; o = causal attention per
    head; h_mid = x + concat(o) W_o^T + b_o; u2 = LN2(h_mid);
    z = u2 W1^T + b1; g = GELU(z); y = h_mid + g W2^T + b2.
    Returns a dict with y and every intermediate the backward needs."""
    n, eps = cfg["heads"], cfg["eps"]
    x = np.asarray(x, dtype=np.float64)
    u1, mu1, rstd1 = layer_norm(x, p["ln1_g"], p["ln1_b"], eps)
    q = heads_split(_linear(u1, p["w_q"], p["b_q"]), n)
    k = heads_split(_linear(u1, p["w_k"], p["b_k"]), n)
    v = heads_split(_linear(u1, p["w_v"], p["b_v"]), n)
    o, prob, lse = causal_attention(q, k, v, 0)
    om = heads_merge(o)
    h_mid = x + _linear(om, p["w_o"], p["b_o"])
    u2, mu2, rstd2 = layer_norm(h_mid, p["ln2_g"], p["ln2_b"], eps)
    z = _linear(u2, p["w1"], p["b1"])
    g = gelu(z)
    y = h_mid + _linear(g, p["w2"], p["b2"])
    return dict(y=y, x=x, u1=u1, mu1=mu1, rstd1=rstd1, q=q, k=k, v=v, o=o,
                om=om, prob=prob, lse=lse, h_mid=h_mid, u2=u2, mu2=mu2,
                rstd2=rstd2, z=z, g=g)


def _rows(a):
    return a.reshape(-1, a.shape[-1])


def layer_backward(dy, p, cfg, fw):
    """Vector-Jacobian product of layer_forward for the output gradient dy.

    Each linear layer Y = X W^T + b takes dX = dY W, dW = dY^T X (the C = AB^T
    row of [MP] 3.1.2) and db = sum of dY over tokens ([MP] 3.1.3); the
    residual adds pass the gradient through unchanged.  Returns a dict with
    dx and one entry per parameter of p."""
    n = cfg["heads"]
    dy = np.asarray(dy, dtype=np.float64)
    gr = {}
    # MLP block
    gr["b2"] = _rows(dy).sum(axis=0)
    gr["w2"] = _rows(dy).T @ _rows(fw["g"])
    dg = _mm(dy, p["w2"])
    dz = dg * gelu_grad(fw["z"])
    gr["b1"] = _rows(dz).sum(axis=0)
    gr["w1"] = _rows(dz).T @ _rows(fw["u2"])
    du2 = _mm(dz, p["w1"])
    dln2, gr["ln2_g"], gr["ln2_b"] = layer_norm_backward(
        du2, fw["h_mid"], p["ln2_g"], fw["mu2"], fw["rstd2"])
    dh = dy + dln2
    # attention block
    gr["b_o"] = _rows(dh).sum(axis=0)
    gr["w_o"] = _rows(dh).T @ _rows(fw["om"])
    dom = _mm(dh, p["w_o"])
    dq, dk, dv = causal_attention_backward(
        heads_split(dom, n), fw["q"], fw["k"], fw["v"], fw["prob"], fw["o"])
    du1 = np.zeros_like(fw["u1"])
    for name, dt in (("q", dq), ("k", dk), ("v", dv)):
        dm = heads_merge(dt)
        gr["b_" + name] = _rows(dm).sum(axis=0)
        gr["w_" + name] = _rows(dm).T @ _rows(fw["u1"])
        du1 += _mm(dm, p["w_" + name])
    dln1, gr["ln1_g"], gr["ln1_b"] = layer_norm_backward(
        du1, fw["x"], p["ln1_g"], fw["mu1"], fw["rstd1"])
    gr["x"] = dh + dln1
    return gr


# ----------------------------------------------------------------------------
# One device's share (rank r of t): [TT11] tensor-parallel slide
# ----------------------------------------------------------------------------

def shard_params(p, r, cfg):
    """Rank r's share of the full parameters p.

    Heads H_r = [r n_t, (r+1) n_t) with n_t = n/t, i.e. columns
    C_r = [r h_t, (r+1) h_t) of the attention width: rows C_r of W_q, W_k, W_v
    (and their biases) stacked as W_qkv,r = [W_q[C_r]; W_k[C_r]; W_v[C_r]];
    columns C_r of W_o.  FFN columns F_r = [r f_t, (r+1) f_t): rows F_r of W1
    and b1, columns F_r of W2.  LayerNorm parameters and the row-split biases
    b_o, b2 are replicated."""
    t, h, f = cfg["tp"], cfg["hidden"], cfg["ffn"]
    ht, ft = h // t, f // t
    c = slice(r * ht, (r + 1) * ht)
    fr = slice(r * ft, (r + 1) * ft)
    return dict(
        ln1_g=p["ln1_g"], ln1_b=p["ln1_b"],
        w_qkv=np.concatenate([p["w_q"][c], p["w_k"][c], p["w_v"][c]], axis=0),
        b_qkv=np.concatenate([p["b_q"][c], p["b_k"][c], p["b_v"][c]]),
        w_o=np.ascontiguousarray(p["w_o"][:, c]), b_o=p["b_o"],
        ln2_g=p["ln2_g"], ln2_b=p["ln2_b"],
        w1=p["w1"][fr], b1=p["b1"][fr],
        w2=np.ascontiguousarray(p["w2"][:, fr]), b2=p["b2"],
    )


def _shard_dims(cfg):
    t = cfg["tp"]
    nt = cfg["heads"] // t
    return nt, cfg["hidden"] // t, cfg["ffn"] // t, cfg["head_dim"]


def new_kv_cache(cfg):
    """Empty prefix K/V cache of one device: [b, n_t, s, d] each, no position
    filled yet."""
    nt, _, _, d = _shard_dims(cfg)
    shape = (cfg["batch"], nt, cfg["seq"], d)
    return dict(k=np.zeros(shape), v=np.zeros(shape), filled=0)


def new_kv_grad(cfg):
    """Empty dK/dV accumulators for the backward over token slices, which runs
    the slices in reverse: done_from is the first position already done."""
    nt, _, _, d = _shard_dims(cfg)
    shape = (cfg["batch"], nt, cfg["seq"], d)
    return dict(dk=np.zeros(shape), dv=np.zeros(shape), done_from=cfg["seq"])


def shard_attn_forward(x, sp, cfg, kv, start, stop):
    """Attention block of one device over the token positions [start, stop).

    LN1 (replicated), the column-split QKV product with bias, the slice's
    K and V appended to the prefix cache, causal attention of the slice's
    queries over cache positions [0, stop), and the row-split out-projection
    into a partial sum (no b_o: it is added once after the reduction).
    [TP] section 3: a slice needs only the K/V of earlier positions, so
    kv["filled"] must equal start; it becomes stop.  Returns (partial, saved)
    for the rows [start, stop)."""
    if kv["filled"] != start:
        raise ValueError("slices must run in order: cache holds %d positions, "
                         "slice starts at %d" % (kv["filled"], start))
    nt, ht, _, _ = _shard_dims(cfg)
    xs = np.asarray(x[start:stop], dtype=np.float64)
    u1, mu1, rstd1 = layer_norm(xs, sp["ln1_g"], sp["ln1_b"], cfg["eps"])
    qkv = _linear(u1, sp["w_qkv"], sp["b_qkv"])
    q = heads_split(qkv[..., :ht], nt)
    kv["k"][:, :, start:stop] = heads_split(qkv[..., ht:2 * ht], nt)
    kv["v"][:, :, start:stop] = heads_split(qkv[..., 2 * ht:], nt)
    kv["filled"] = stop
    o, prob, lse = causal_attention(q, kv["k"][:, :, :stop], kv["v"][:, :, :stop], start)
    om = heads_merge(o)
    partial = _linear(om, sp["w_o"])
    saved = dict(start=start, stop=stop, x=xs, u1=u1, mu1=mu1, rstd1=rstd1,
                 q=q, o=o, om=om, prob=prob, lse=lse)
    return partial, saved


def residual_combine(resid, reduced, bias):
    """The caller's step after the all-reduce: resid + sum_r partial_r + bias
    ([TT11] tensor-parallel slide: one all-reduce adds the partial sums)."""
    return np.asarray(resid, dtype=np.float64) + reduced + bias


def shard_mlp_forward(h_mid_rows, sp, cfg):
    """MLP block of one device on some token rows (position-wise, [TP]
    section 3): LN2 (replicated), column-split FC1 with bias and GELU, and
    the row-split FC2 into a partial sum (no b2).  Returns (partial, saved)."""
    hm = np.asarray(h_mid_rows, dtype=np.float64)
    u2, mu2, rstd2 = layer_norm(hm, sp["ln2_g"], sp["ln2_b"], cfg["eps"])
    z = _linear(u2, sp["w1"], sp["b1"])
    g = gelu(z)
    partial = _linear(g, sp["w2"])
    return partial, dict(h_mid=hm, u2=u2, mu2=mu2, rstd2=rstd2, z=z, g=g)


def shard_mlp_backward(dy_rows, sp, saved_mlp):
    """Backward of shard_mlp_forward up to the partial input gradient
    dU2,r = dZ W1,r (one summand of the all-reduce), with the weight gradients
    dW2,r = dY^T G, dW1,r = dZ^T u2 ([MP] 3.1.2), db1,r = sum dZ and the
    replicated db2 = sum dY ([MP] 3.1.3).  Returns (dU2_partial, grads)."""
    dy = np.asarray(dy_rows, dtype=np.float64)
    dg = _mm(dy, sp["w2"])
    dz = dg * gelu_grad(saved_mlp["z"])
    gr = dict(w2=_rows(dy).T @ _rows(saved_mlp["g"]), b2=_rows(dy).sum(axis=0),
              w1=_rows(dz).T @ _rows(saved_mlp["u2"]), b1=_rows(dz).sum(axis=0))
    return _mm(dz, sp["w1"]), gr


def shard_attn_backward(dy_rows, du2_sum_rows, sp, saved_mlp, saved_attn, kv, kvg):
    """Backward of the attention block of one device over the slice the two
    saved dicts describe (positions [start, stop)), given the all-reduced
    MLP input gradient.  Slices go in reverse order: kvg["done_from"] must
    equal stop and becomes start.

    dH = dY + LN2^T(sum_r dU2,r); dO = dH W_o,r; dW_o,r = dH^T O; the
    replicated db_o = sum dH; attention backward of the slice's queries over
    keys [0, stop), whose dK, dV add into the accumulators; keys of this
    slice are then complete (no later query is left), so
    dQKV = [dQ | dK | dV] for the slice's rows gives dU1,r = dQKV W_qkv,r (a
    summand of the second all-reduce), dW_qkv,r = dQKV^T u1 and
    db_qkv,r = sum dQKV.  Returns (dH, dU1_partial, grads)."""
    start, stop = saved_attn["start"], saved_attn["stop"]
    if kvg["done_from"] != stop:
        raise ValueError("backward slices must run in reverse order")
    nt = saved_attn["q"].shape[1]
    dy = np.asarray(dy_rows, dtype=np.float64)
    dln2, dg2, db2 = layer_norm_backward(du2_sum_rows, saved_mlp["h_mid"], sp["ln2_g"],
                                         saved_mlp["mu2"], saved_mlp["rstd2"])
    dh = dy + dln2
    gr = dict(ln2_g=dg2, ln2_b=db2, b_o=_rows(dh).sum(axis=0),
              w_o=_rows(dh).T @ _rows(saved_attn["om"]))
    dom = _mm(dh, sp["w_o"])
    dq, dk, dv = causal_attention_backward(
        heads_split(dom, nt), saved_attn["q"], kv["k"][:, :, :stop],
        kv["v"][:, :, :stop], saved_attn["prob"], saved_attn["o"])
    kvg["dk"][:, :, :stop] += dk
    kvg["dv"][:, :, :stop] += dv
    kvg["done_from"] = start
    dqkv = np.concatenate([heads_merge(dq),
                           heads_merge(kvg["dk"][:, :, start:stop]),
                           heads_merge(kvg["dv"][:, :, start:stop])], axis=-1)
    gr["w_qkv"] = _rows(dqkv).T @ _rows(saved_attn["u1"])
    gr["b_qkv"] = _rows(dqkv).sum(axis=0)
    return dh, _mm(dqkv, sp["w_qkv"]), gr


def ln1_backward(dh_rows, du1_sum_rows, sp, saved_attn):
    """Last backward step of a device: dX = dH + LN1^T(sum_r dU1,r), with the
    replicated dgamma1, dbeta1.  Returns (dx, grads)."""
    dln1, dg1, db1 = layer_norm_backward(du1_sum_rows, saved_attn["x"], sp["ln1_g"],
                                         saved_attn["mu1"], saved_attn["rstd1"])
    return np.asarray(dh_rows, dtype=np.float64) + dln1, dict(ln1_g=dg1, ln1_b=db1)


def shard_layer_step(x, h_mid, dy, du2_sum, du1_sum, sp, cfg, bounds=None):
    """One device's forward and backward over token slices, with the two
    all-reduce inputs supplied by the caller (on one device they stand for
    the sums over all t ranks).

    bounds: slice boundaries [o_0 = 0, o_1, ..., o_M = s]; forward runs the
    slices in order, backward in reverse ([TP] section 3).  h_mid, du2_sum
    and du1_sum are the combined tensors the caller would hand in after each
    all-reduce ([s, b, h] each).  Returns a dict with the four partial sums
    (attn, mlp, du2, du1), dh, dx, the K/V cache and the accumulated
    parameter gradients."""
    s = cfg["seq"]
    if bounds is None:
        bounds = [0, s]
    kv = new_kv_cache(cfg)
    kvg = new_kv_grad(cfg)
    shp = np.asarray(x).shape
    out = {k: np.zeros(shp) for k in ("p_attn", "p_mlp", "p_du2", "p_du1", "dh", "dx")}
    saved = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        pa, sa = shard_attn_forward(x, sp, cfg, kv, a, b)
        pm, sm = shard_mlp_forward(h_mid[a:b], sp, cfg)
        out["p_attn"][a:b], out["p_mlp"][a:b] = pa, pm
        saved.append((sa, sm))
    grads = {}

    def acc(gr):
        for k, v in gr.items():
            grads[k] = grads.get(k, 0.0) + v

    for sa, sm in reversed(saved):
        a, b = sa["start"], sa["stop"]
        pdu2, gr = shard_mlp_backward(dy[a:b], sp, sm)
        acc(gr)
        dh, pdu1, gr = shard_attn_backward(dy[a:b], du2_sum[a:b], sp, sm, sa, kv, kvg)
        acc(gr)
        dx, gr = ln1_backward(dh, du1_sum[a:b], sp, sa)
        acc(gr)
        out["p_du2"][a:b], out["p_du1"][a:b] = pdu2, pdu1
        out["dh"][a:b], out["dx"][a:b] = dh, dx
    out.update(kv=kv, grads=grads)
    return out


# ----------------------------------------------------------------------------
# The cube-partition block ([MP] section 3.1.2: each processor multiplies
# sub-matrices of size (M/p, N/p) and (N/p, K/p); section 2.3: the block sum
# C_ij = sum_l A_il B_lj)
# ----------------------------------------------------------------------------

def cube_ffn_block(x, w1, b1, w2):
    """One device's local FFN chain on its cube block: GELU(X W1^T + b1) W2^T,
    returned as the fp64 partial sum that a reduction over the cube's third
    direction would add (the reduction itself is not taken).  Weights are
    stored [out, in] like the layer's."""
    x = np.asarray(x, dtype=np.float64)
    return gelu(x @ np.asarray(w1, dtype=np.float64).T + b1) @ np.asarray(w2, dtype=np.float64).T
