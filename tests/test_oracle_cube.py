"""Pins of the cube-partition oracle (oracle/cube.py): every product form
against explicit index loops, the gradient formulas against finite
differences, and the FFN block assembled from per-device local products with
the reduction taken before bias and GELU against the unsharded block written
out with math.erf, forward and backward; planted mistakes must be caught."""
import inspect
import math

import numpy as np
import pytest

from oracle import cube as C


def loops_product(form, a, b):
    a, b = np.asarray(a), np.asarray(b)
    if form == "ab":
        m, k, n = a.shape[0], a.shape[1], b.shape[1]
        get = lambda i, j, t: a[i, t] * b[t, j]
    elif form == "abt":
        m, k, n = a.shape[0], a.shape[1], b.shape[0]
        get = lambda i, j, t: a[i, t] * b[j, t]
    else:
        m, k, n = a.shape[1], a.shape[0], b.shape[1]
        get = lambda i, j, t: a[t, i] * b[t, j]
    return np.array([[sum(get(i, j, t) for t in range(k)) for j in range(n)] for i in range(m)])


def product_error(orc):
    rng = np.random.default_rng(1)
    err = 0.0
    shapes = {"ab": ((5, 4), (4, 3)), "abt": ((5, 4), (3, 4)), "atb": ((4, 5), (4, 3))}
    for form, (sa, sb) in shapes.items():
        a, b = rng.normal(size=sa), rng.normal(size=sb)
        err = max(err, float(np.abs(orc.cube_matmul(form, a, b) - loops_product(form, a, b)).max()))
    return err


def grad_error(orc):
    rng = np.random.default_rng(2)
    shapes = {"ab": ((3, 4), (4, 2)), "abt": ((3, 4), (2, 4)), "atb": ((4, 3), (4, 2))}
    err = 0.0
    for form, (sa, sb) in shapes.items():
        a, b = rng.normal(size=sa), rng.normal(size=sb)
        w = rng.normal(size=orc.cube_matmul(form, a, b).shape)
        da, db = orc.matmul_grads(form, a, b, w)
        eps = 1e-6
        for x, dx, which in ((a, da, 0), (b, db, 1)):
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = (xp, b) if which == 0 else (a, xp)
                args_m = (xm, b) if which == 0 else (a, xm)
                fd = ((loops_product(form, *args_p) * w).sum() - (loops_product(form, *args_m) * w).sum()) / (2 * eps)
                err = max(err, abs(fd - dx[idx]))
    return err


def _gelu_erf(z):
    return z * 0.5 * (1.0 + math.erf(z / math.sqrt(2.0)))


def ffn_loops(x, w1, b1, w2):
    z = loops_product("abt", x, w1) + b1
    h = np.vectorize(_gelu_erf)(z)
    return loops_product("abt", h, w2)


def ffn_error(orc):
    rng = np.random.default_rng(3)
    rows, hid, f = 3, 4, 6
    x, w1, b1, w2 = (rng.normal(size=s) for s in ((rows, hid), (f, hid), (f,), (hid, f)))
    dout = rng.normal(size=(rows, hid))
    out, g = orc.cube_ffn_devices(x, w1, b1, w2, dout, p=2)
    err = float(np.abs(out - ffn_loops(x, w1, b1, w2)).max())
    for p in (1, 3):
        out_p, g_p = orc.cube_ffn_devices(x, w1, b1, w2, dout, p=p)
        err = max(err, float(np.abs(out_p - out).max()), *(float(np.abs(g_p[k] - g[k]).max()) for k in g))
    eps = 1e-6
    params = dict(x=x, w1=w1, b1=b1, w2=w2)
    for name, val in params.items():
        for idx in np.ndindex(val.shape):
            vp, vm = dict(params), dict(params)
            vp[name], vm[name] = val.copy(), val.copy()
            vp[name][idx] += eps
            vm[name][idx] -= eps
            fd = ((ffn_loops(**vp) * dout).sum() - (ffn_loops(**vm) * dout).sum()) / (2 * eps)
            err = max(err, abs(fd - g[name][idx]) / 10)
    return err


def pin_failures(orc):
    checks = [("products", lambda: product_error(orc) < 1e-12), ("grads", lambda: grad_error(orc) < 1e-7),
              ("ffn", lambda: ffn_error(orc) < 1e-7)]
    for name, ok in checks:
        with np.errstate(all="ignore"):
            try:
                good = bool(ok())
            except Exception:
                good = False
        if not good:
            yield name


def test_products_match_index_loops():
    assert product_error(C) < 1e-12


def test_gradient_formulas_match_finite_differences():
    assert grad_error(C) < 1e-7


def test_cube_ffn_matches_unsharded_block():
    assert ffn_error(C) < 1e-7


def test_gelu_before_reduce_differs():
    """Applying GELU to each device's partial sum (before the reduction)
    gives a different block: the reduction must come first."""
    rng = np.random.default_rng(4)
    x, w1 = rng.normal(size=(3, 4)), rng.normal(size=(6, 4))
    parts = [C.cube_matmul("abt", x[:, c], w1[:, c]) for c in np.array_split(np.arange(4), 2)]
    wrong = sum(C.cube_bias_gelu(p, np.zeros(6))[1] for p in parts)
    right = C.cube_bias_gelu(sum(parts), np.zeros(6))[1]
    assert np.abs(wrong - right).max() > 1e-3


MUTANTS = [
    ("cube_matmul", "return a.T @ b", "return a @ b.T"),
    ("matmul_grads", "return dc @ b, dc.T @ a", "return dc @ b, a.T @ dc"),
    ("matmul_grads", "return b @ dc.T, a @ dc", "return dc @ b.T, a @ dc"),
    ("cube_bias_gelu", "return z, gelu(z)", "return z, gelu(np.asarray(z_sum, dtype=np.float64))"),
    ("cube_gelu_backward", "return dz, dz.sum(axis=0)", "return dz, dz.sum(axis=1)"),
    ("cube_gelu_backward", "dz = np.asarray(dh, dtype=np.float64) * gelu_grad(z)", "dz = np.asarray(dh, dtype=np.float64)"),
    ("cube_ffn_devices", "dx = sum(cube_matmul(\"ab\", dz[:, c], w1[c, :]) for c in fs)",
     "dx = sum(cube_matmul(\"ab\", dz[:, c], w1[c, :]) for c in fs[:1])"),
    ("cube_ffn_devices", "z, h = cube_bias_gelu(z_sum, b1)", "z, h = cube_bias_gelu(z_sum, 0 * b1)"),
]


@pytest.mark.parametrize("fn,old,new", MUTANTS, ids=[f"{m[0]}-{i}" for i, m in enumerate(MUTANTS)])
def test_cube_mutant_is_caught(monkeypatch, fn, old, new):
    src = inspect.getsource(getattr(C, fn))
    assert old in src, "mutation site not found"
    ns = dict(C.__dict__)
    exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), ns)
    monkeypatch.setattr(C, fn, ns[fn])
    assert next(pin_failures(C), None) is not None, "no pin noticed the mutation"


def test_unmutated_cube_oracle_passes_every_pin():
    assert list(pin_failures(C)) == []
