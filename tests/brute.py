"""Pure-Python brute force of the decoder layer forward, for tiny shapes.

Written from the layer's definition with explicit loops over plain Python
floats and math.erf, independently of oracle/ (no numpy, no shared helper),
so that agreement between the two pins the oracle's forward.  Layout as in
the oracle: x[p][b][i] (position, batch row, feature); weights W[out][in].
"""
import math


def _layer_norm_row(row, gamma, beta, eps):
    h = len(row)
    mean = sum(row) / h
    var = sum((v - mean) * (v - mean) for v in row) / h
    inv = 1.0 / math.sqrt(var + eps)
    return [(row[i] - mean) * inv * gamma[i] + beta[i] for i in range(h)]


def _matvec(w, b, v):
    out = []
    for o in range(len(w)):
        acc = 0.0 if b is None else b[o]
        wr = w[o]
        for i in range(len(v)):
            acc += wr[i] * v[i]
        out.append(acc)
    return out


def _gelu(z):
    return z * 0.5 * (1.0 + math.erf(z / math.sqrt(2.0)))


def layer_forward(x, p, heads, eps):
    """y[p][b][:] for the pre-LN layer: LN1, Q/K/V, causal softmax attention
    per head over positions j <= p with scale 1/sqrt(d), out-projection and
    residual, LN2, FC1 + GELU, FC2 and residual."""
    s, nb, h = len(x), len(x[0]), len(x[0][0])
    d = h // heads
    u1 = [[_layer_norm_row(x[t][b], p["ln1_g"], p["ln1_b"], eps) for b in range(nb)] for t in range(s)]
    q = [[_matvec(p["w_q"], p["b_q"], u1[t][b]) for b in range(nb)] for t in range(s)]
    k = [[_matvec(p["w_k"], p["b_k"], u1[t][b]) for b in range(nb)] for t in range(s)]
    v = [[_matvec(p["w_v"], p["b_v"], u1[t][b]) for b in range(nb)] for t in range(s)]
    y = [[None] * nb for _ in range(s)]
    for t in range(s):
        for b in range(nb):
            att = [0.0] * h
            for hd in range(heads):
                cols = range(hd * d, (hd + 1) * d)
                scores = []
                for j in range(t + 1):
                    dot = 0.0
                    for c in cols:
                        dot += q[t][b][c] * k[j][b][c]
                    scores.append(dot / math.sqrt(d))
                m = max(scores)
                e = [math.exp(sc - m) for sc in scores]
                tot = sum(e)
                for c in cols:
                    acc = 0.0
                    for j in range(t + 1):
                        acc += e[j] / tot * v[j][b][c]
                    att[c] = acc
            proj = _matvec(p["w_o"], p["b_o"], att)
            hmid = [x[t][b][i] + proj[i] for i in range(h)]
            u2 = _layer_norm_row(hmid, p["ln2_g"], p["ln2_b"], eps)
            g = [_gelu(z) for z in _matvec(p["w1"], p["b1"], u2)]
            out = _matvec(p["w2"], p["b2"], g)
            y[t][b] = [hmid[i] + out[i] for i in range(h)]
    return y


def cube_ffn_block(x, w1, b1, w2):
    """GELU(X W1^T + b1) W2^T row by row, weights stored [out, in]."""
    return [_matvec(w2, None, [_gelu(z) for z in _matvec(w1, b1, row)]) for row in x]
