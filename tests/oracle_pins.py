"""Checks that pin the CPU oracle to something other than itself.

Each function returns an error figure; tests/test_oracle_pins.py asserts it
is small for the oracle as written, and tests/test_oracle_mutants.py plants
plausible mistakes in the oracle (on the CPU) and asserts that at least one
of these figures then becomes large.
"""
import itertools
import math

import numpy as np

from tests import brute

# A layer small enough for pure-Python loops: h = 8, 2 heads of d = 4,
# FFN 32, batch 2, and up to 6 positions.
TINY = dict(hidden=8, heads=2, head_dim=4, ffn=32, tp=1, batch=2, seq=6, eps=1e-5)
PARAM_SHAPES = [("ln1_g", "h"), ("ln1_b", "h"), ("w_q", "hh"), ("b_q", "h"), ("w_k", "hh"),
                ("b_k", "h"), ("w_v", "hh"), ("b_v", "h"), ("w_o", "hh"), ("b_o", "h"),
                ("ln2_g", "h"), ("ln2_b", "h"), ("w1", "fh"), ("b1", "f"), ("w2", "hf"), ("b2", "h")]


def tiny_params(cfg, seed, wstd=0.5):
    """Random parameters with every term switched on (non-zero biases, gamma
    away from 1, beta away from 0) and weights large enough that the softmax
    is far from uniform."""
    rng = np.random.default_rng(seed)
    h, f = cfg["hidden"], cfg["ffn"]
    dims = {"h": (h,), "hh": (h, h), "fh": (f, h), "hf": (h, f), "f": (f,)}
    p = {}
    for name, kind in PARAM_SHAPES:
        if name.endswith("_g"):
            p[name] = 1.0 + 0.3 * rng.standard_normal(dims[kind])
        elif name.startswith("w"):
            p[name] = wstd * rng.standard_normal(dims[kind])
        else:
            p[name] = 0.2 * rng.standard_normal(dims[kind])
    return p


def tiny_inputs(cfg, seed):
    rng = np.random.default_rng(seed + 17)
    shape = (cfg["seq"], cfg["batch"], cfg["hidden"])
    return rng.standard_normal(shape), rng.standard_normal(shape)


def brute_error(orc, seed=0, cfg=TINY):
    """max |oracle y - brute-force y| on a tiny layer."""
    p = tiny_params(cfg, seed)
    x, _ = tiny_inputs(cfg, seed)
    y = orc.layer_forward(x, p, cfg)["y"]
    pl = {k: v.tolist() for k, v in p.items()}
    yb = np.array(brute.layer_forward(x.tolist(), pl, cfg["heads"], cfg["eps"]))
    return float(np.abs(y - yb).max())


def fd_error(orc, seed=1, cfg=None, eps=1e-6):
    """Largest relative gap between the oracle's backward and central
    differences of L = sum(y * dy), over every parameter entry and every
    input entry."""
    cfg = dict(TINY, seq=4) if cfg is None else cfg
    p = tiny_params(cfg, seed)
    x, dy = tiny_inputs(cfg, seed)
    fw = orc.layer_forward(x, p, cfg)
    gr = orc.layer_backward(dy, p, cfg, fw)

    def loss(pp, xx):
        return float((orc.layer_forward(xx, pp, cfg)["y"] * dy).sum())

    worst = 0.0
    targets = [(name, p[name]) for name, _ in PARAM_SHAPES] + [("x", x)]
    for name, arr in targets:
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss(p, x)
            arr[idx] = old - eps
            lm = loss(p, x)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        scale = max(1.0, float(np.abs(num).max()))
        worst = max(worst, float(np.abs(num - gr[name]).max()) / scale)
    return worst


def compositions(n):
    """Every composition of n (ordered partitions into positive parts)."""
    for cuts in itertools.product([0, 1], repeat=n - 1):
        parts, run = [], 1
        for c in cuts:
            if c:
                parts.append(run)
                run = 1
            else:
                run += 1
        parts.append(run)
        yield parts


def bounds_of(parts):
    b = [0]
    for n in parts:
        b.append(b[-1] + n)
    return b


def tp_layer(orc, x, dy, p, cfg, bounds):
    """The whole layer computed the tensor-parallel + token-slice way: t
    shards, each run slice by slice through the shard functions, with the
    all-reduces simulated by sums over ranks.  Returns (y, dx, full grads
    re-assembled from the shards)."""
    t, s = cfg["tp"], cfg["seq"]
    h, f = cfg["hidden"], cfg["ffn"]
    ht, ft = h // t, f // t
    sps = [orc.shard_params(p, r, cfg) for r in range(t)]
    kvs = [orc.new_kv_cache(cfg) for _ in range(t)]
    kvgs = [orc.new_kv_grad(cfg) for _ in range(t)]
    y = np.zeros_like(x)
    dx = np.zeros_like(x)
    saved = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        outs = [orc.shard_attn_forward(x, sps[r], cfg, kvs[r], a, b) for r in range(t)]
        h_mid = orc.residual_combine(x[a:b], sum(o[0] for o in outs), p["b_o"])
        mouts = [orc.shard_mlp_forward(h_mid, sps[r], cfg) for r in range(t)]
        y[a:b] = orc.residual_combine(h_mid, sum(o[0] for o in mouts), p["b2"])
        saved.append(([o[1] for o in outs], [o[1] for o in mouts], a, b))
    grads = [dict() for _ in range(t)]

    def acc(r, gr):
        for k, v in gr.items():
            grads[r][k] = grads[r].get(k, 0.0) + v

    for sa, sm, a, b in reversed(saved):
        res = [orc.shard_mlp_backward(dy[a:b], sps[r], sm[r]) for r in range(t)]
        for r in range(t):
            acc(r, res[r][1])
        du2 = sum(rr[0] for rr in res)
        res = [orc.shard_attn_backward(dy[a:b], du2, sps[r], sm[r], sa[r], kvs[r], kvgs[r])
               for r in range(t)]
        for r in range(t):
            acc(r, res[r][2])
        du1 = sum(rr[1] for rr in res)
        res1 = [orc.ln1_backward(res[r][0], du1, sps[r], sa[r]) for r in range(t)]
        for r in range(t):
            acc(r, res1[r][1])
        dx[a:b] = res1[0][0]
    full = {}
    for name in ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "b_o", "b2"):
        full[name] = grads[0][name]
    full["w_q"] = np.concatenate([g["w_qkv"][:ht] for g in grads])
    full["w_k"] = np.concatenate([g["w_qkv"][ht:2 * ht] for g in grads])
    full["w_v"] = np.concatenate([g["w_qkv"][2 * ht:] for g in grads])
    full["b_q"] = np.concatenate([g["b_qkv"][:ht] for g in grads])
    full["b_k"] = np.concatenate([g["b_qkv"][ht:2 * ht] for g in grads])
    full["b_v"] = np.concatenate([g["b_qkv"][2 * ht:] for g in grads])
    full["w_o"] = np.concatenate([g["w_o"] for g in grads], axis=1)
    full["w1"] = np.concatenate([g["w1"] for g in grads])
    full["b1"] = np.concatenate([g["b1"] for g in grads])
    full["w2"] = np.concatenate([g["w2"] for g in grads], axis=1)
    # replicated parameters must get the same gradient on every rank
    rep_gap = max(float(np.abs(grads[r][k] - grads[0][k]).max())
                  for r in range(t) for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "b_o", "b2"))
    return y, dx, full, rep_gap


def tp_error(orc, t, parts, seed=2, cfg=None):
    """max gap between the tensor-parallel, token-sliced computation and the
    unsharded layer, over y, dx and every parameter gradient."""
    cfg = dict(TINY, tp=t, heads=max(2, t)) if cfg is None else cfg
    cfg = dict(cfg, seq=sum(parts))
    p = tiny_params(cfg, seed)
    x, dy = tiny_inputs(cfg, seed)
    fw = orc.layer_forward(x, p, cfg)
    gr = orc.layer_backward(dy, p, cfg, fw)
    y, dx, full, rep_gap = tp_layer(orc, x, dy, p, cfg, bounds_of(parts))
    err = max(float(np.abs(y - fw["y"]).max()), float(np.abs(dx - gr["x"]).max()), rep_gap)
    for k, v in full.items():
        err = max(err, float(np.abs(v - gr[k]).max()))
    return err


def closed_form_errors(orc):
    """Closed forms and special cases of the layer, returned as a dict of
    error figures (each should be ~0)."""
    cfg = dict(TINY)
    out = {}
    rng = np.random.default_rng(5)
    # attention: the first position sees only itself, so o_0 = v_0
    q, k, v = (rng.standard_normal((2, 3, 5, 4)) for _ in range(3))
    o, prob, lse = orc.causal_attention(q, k, v, 0)
    out["o0_is_v0"] = float(np.abs(o[:, :, 0] - v[:, :, 0]).max())
    # softmax rows sum to 1 and put no weight on later positions
    out["rows_sum_1"] = float(np.abs(prob.sum(-1) - 1).max())
    out["no_future"] = float(np.abs(np.triu(prob, 1)).max())
    # lse is the log of the softmax denominator: P_pj = exp(s_pj - lse_p)
    sc = np.einsum("bnpd,bnjd->bnpj", q, k) / 2.0
    keep = np.tril(np.ones((5, 5), dtype=bool))
    out["lse_relation"] = float(np.abs(np.where(keep, np.exp(sc - lse[..., None]), 0) - prob).max())
    # zero queries and keys: uniform weights, o_p = mean_{j<=p} v_j
    o, _, lse = orc.causal_attention(np.zeros_like(q), np.zeros_like(k), v, 0)
    mean_v = np.cumsum(v, axis=2) / np.arange(1, 6)[None, None, :, None]
    out["uniform_mean"] = float(np.abs(o - mean_v).max())
    out["uniform_lse"] = float(np.abs(lse - np.log(np.arange(1, 6))[None, None, :]).max())
    # a slice that starts at position 2 sees keys 0..2+i
    o2, _, _ = orc.causal_attention(np.zeros((2, 3, 2, 4)), np.zeros((2, 3, 4, 4)), v[:, :, :4], 2)
    out["offset_mean"] = float(np.abs(o2 - mean_v[:, :, 2:4]).max())
    # all weights and biases zero: both blocks add nothing, y = x
    p = tiny_params(cfg, 3)
    for name in p:
        if name.startswith("w") or name.startswith("b"):
            p[name] = np.zeros_like(p[name])
    x, _ = tiny_inputs(cfg, 3)
    out["zero_layer_identity"] = float(np.abs(orc.layer_forward(x, p, cfg)["y"] - x).max())
    # LayerNorm with gamma 1, beta 0: mean 0 and biased variance var/(var+eps)
    xr = rng.standard_normal((7, 16)) * 3 + 1
    u, mean, rstd = orc.layer_norm(xr, np.ones(16), np.zeros(16), 1e-5)
    var = xr.var(axis=-1)
    out["ln_mean"] = float(np.abs(u.mean(-1)).max())
    out["ln_var"] = float(np.abs(u.var(-1) - var / (var + 1e-5)).max())
    out["ln_stats"] = float(max(np.abs(mean - xr.mean(-1)).max(),
                                np.abs(rstd - 1 / np.sqrt(var + 1e-5)).max()))
    # LayerNorm is invariant to shifting and scaling its input row
    u2, _, _ = orc.layer_norm(xr * 2.5 + 4.0, np.ones(16), np.zeros(16), 0.0)
    u3, _, _ = orc.layer_norm(xr, np.ones(16), np.zeros(16), 0.0)
    out["ln_affine_invariance"] = float(np.abs(u2 - u3).max())
    return out


def gelu_table_errors(orc, table):
    """Gap to standard-normal table values: GELU(z) = z Phi(z) and
    GELU'(z) = Phi(z) + z phi(z) at the tabulated points."""
    z = np.array([r["z"] for r in table])
    phi = np.array([r["Phi"] for r in table])
    dens = np.array([r["phi"] for r in table])
    return dict(gelu=float(np.abs(orc.gelu(z) - z * phi).max()),
                gelu_grad=float(np.abs(orc.gelu_grad(z) - (phi + z * dens)).max()))


def cube_error(orc, seed=4):
    """Oracle cube block vs the brute force, and the block identity
    C_ij = sum_l A_il B_lj over a 2-way split of the FFN width."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((3, 6))
    w1 = 0.5 * rng.standard_normal((10, 6))
    b1 = 0.2 * rng.standard_normal(10)
    w2 = 0.5 * rng.standard_normal((6, 10))
    c = orc.cube_ffn_block(x, w1, b1, w2)
    cb = np.array(brute.cube_ffn_block(x.tolist(), w1.tolist(), b1.tolist(), w2.tolist()))
    halves = sum(orc.cube_ffn_block(x, w1[i:i + 5], b1[i:i + 5], w2[:, i:i + 5]) for i in (0, 5))
    return max(float(np.abs(c - cb).max()), float(np.abs(c - halves).max()))


def math_erf_ok():
    return abs(math.erf(1.0) - 0.8427007929497149) < 1e-15


def brute_block_attention(q, k, v, q_pos0, k_pos0):
    """Pure-Python loops: for each query, the softmax over the visible keys
    of the block written out term by term (positions compared directly)."""
    b, n, lq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    lk = len(k[0][0])
    o = [[[[0.0] * d for _ in range(lq)] for _ in range(n)] for _ in range(b)]
    lse = [[[float("-inf")] * lq for _ in range(n)] for _ in range(b)]
    for bi in range(b):
        for h in range(n):
            for i in range(lq):
                s = []
                for j in range(lk):
                    if k_pos0 + j <= q_pos0 + i:
                        dot = sum(q[bi][h][i][x] * k[bi][h][j][x] for x in range(d))
                        s.append((j, dot / math.sqrt(d)))
                if not s:
                    continue
                z = sum(math.exp(val) for _, val in s)
                lse[bi][h][i] = math.log(z)
                for j, val in s:
                    w = math.exp(val) / z
                    for x in range(d):
                        o[bi][h][i][x] += w * v[bi][h][j][x]
    return o, lse


def ring_error(orc, seed=5):
    """Largest deviation of (a) attention_block against the brute force, for
    blocks before, overlapping and after the queries, and (b) the merge of
    per-block results over a partition of the keys against the brute force
    over all keys."""
    rng = np.random.default_rng(seed)
    b, n, d = 2, 2, 4
    q_pos0, lq = 5, 4
    lk_total = q_pos0 + lq + 2  # two keys past the last query
    q = rng.normal(size=(b, n, lq, d))
    k = rng.normal(size=(b, n, lk_total, d))
    v = rng.normal(size=(b, n, lk_total, d))
    err = 0.0
    blocks = [(0, 3), (3, 3), (3, 6), (6, 9), (9, lk_total)]  # (3, 3): a block of no keys
    acc = None
    for k0, k1 in blocks:
        o, lse = orc.attention_block(q, k[:, :, k0:k1], v[:, :, k0:k1], q_pos0, k0)
        bo, bl = brute_block_attention(q.tolist(), k[:, :, k0:k1].tolist(), v[:, :, k0:k1].tolist(), q_pos0, k0)
        bo, bl = np.array(bo), np.array(bl)
        fin = np.isfinite(bl)
        if not np.array_equal(fin, np.isfinite(lse)):
            return float("inf")
        err = max(err, float(np.abs(o - bo).max()), float(np.abs(lse[fin] - bl[fin]).max()) if fin.any() else 0.0)
        acc = (o, lse) if acc is None else orc.merge_partials(acc[0], acc[1], o, lse)
    fo, fl = brute_block_attention(q.tolist(), k.tolist(), v.tolist(), q_pos0, 0)
    err = max(err, float(np.abs(acc[0] - np.array(fo)).max()), float(np.abs(acc[1] - np.array(fl)).max()))
    # merging in the other order gives the same result
    rev = None
    for k0, k1 in reversed(blocks):
        o, lse = orc.attention_block(q, k[:, :, k0:k1], v[:, :, k0:k1], q_pos0, k0)
        rev = (o, lse) if rev is None else orc.merge_partials(rev[0], rev[1], o, lse)
    err = max(err, float(np.abs(rev[0] - acc[0]).max()), float(np.abs(rev[1] - acc[1]).max()))
    return err


def ring_backward_error(orc, seed=7):
    """Largest deviation of attention_block_backward, run block by block with
    the merged forward result (o, lse taken from the brute force over all
    keys), from central finite differences of L = sum(do * o) through the
    pure-Python brute-force forward: the per-block query shares summed over
    the blocks against dL/dq, each block's dk and dv against dL/dk and dL/dv
    of its keys.  Blocks before, across and after the queries."""
    rng = np.random.default_rng(seed)
    b, n, d = 1, 2, 4
    q_pos0, lq = 4, 3
    lk_total = q_pos0 + lq + 1
    q = rng.normal(size=(b, n, lq, d))
    k = rng.normal(size=(b, n, lk_total, d))
    v = rng.normal(size=(b, n, lk_total, d))
    do = rng.normal(size=(b, n, lq, d))

    def loss(qq, kk, vv):
        o, _ = brute_block_attention(qq.tolist(), kk.tolist(), vv.tolist(), q_pos0, 0)
        return float((np.array(o) * do).sum())

    fo, fl = brute_block_attention(q.tolist(), k.tolist(), v.tolist(), q_pos0, 0)
    fo, fl = np.array(fo), np.array(fl)
    blocks = [(0, 3), (3, 6), (6, lk_total)]
    dq = np.zeros_like(q)
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    for k0, k1 in blocks:
        sq, sk, sv = orc.attention_block_backward(do, q, k[:, :, k0:k1], v[:, :, k0:k1], fo, fl, q_pos0, k0)
        dq += sq
        dk[:, :, k0:k1] = sk
        dv[:, :, k0:k1] = sv
    eps = 1e-6
    err = 0.0
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(arr.shape):
            args = {"q": q, "k": k, "v": v}
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args[name] = plus
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = minus
            lm = loss(args["q"], args["k"], args["v"])
            err = max(err, abs((lp - lm) / (2 * eps) - grad[idx]))
    return err
