"""fp64 definition of one device's operations in the 3-D (cube) partition of
matrix products and of the FFN block built from them.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg.

Source: "Maximizing Parallelism in Distributed Training for Huge Neural
Networks" (Bian, Xu, Wang, You).  Section 3.1.2 (Matrix-matrix
Operations): the products C = AB, C = AB^T and C = A^T B and their
gradients (C = AB: dA = dC B^T, dB = A^T dC; C = AB^T: dA = dC B,
dB = dC^T A; C = A^T B: dA = B dC^T, dB = A dC); each device multiplies its
gathered sub-blocks and the partial products are reduce-scattered.  Section
2.3: the block product C_ij = sum_l A_il B_lj.  Section 3.1.3 (Matrix-vector
Operations): C = A + b has db = sum of dC over rows.  Section 3.2: the MLP
block is two linear layers with GELU between them.

The FFN block in the 3-D algorithm: a device's local product gives a partial
sum of Z = X W1^T over its share of the reduction, the partial sums are
reduced across the cube, and only then are the bias and GELU applied (a
nonlinearity of a partial sum would be wrong); the second product's partials
are reduced likewise.
"""
import numpy as np

from .layer import gelu, gelu_grad

__all__ = ["cube_matmul", "cube_bias_gelu", "cube_gelu_backward", "matmul_grads", "cube_ffn_devices"]

FORMS = ("ab", "abt", "atb")


def cube_matmul(form, a, b):
    """The local product of one form: AB, AB^T or A^T B (fp64)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if form == "ab":
        return a @ b
    if form == "abt":
        return a @ b.T
    if form == "atb":
        return a.T @ b
    raise ValueError(form)


def matmul_grads(form, a, b, dc):
    """(dA, dB) of each form, as section 3.1.2 writes them."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    dc = np.asarray(dc, dtype=np.float64)
    if form == "ab":
        return dc @ b.T, a.T @ dc
    if form == "abt":
        return dc @ b, dc.T @ a
    if form == "atb":
        return b @ dc.T, a @ dc
    raise ValueError(form)


def cube_bias_gelu(z_sum, bias):
    """Z = (reduced partial sums) + bias, H = GELU(Z)."""
    z = np.asarray(z_sum, dtype=np.float64) + np.asarray(bias, dtype=np.float64)
    return z, gelu(z)


def cube_gelu_backward(dh, z):
    """dZ = dH * GELU'(Z) and the bias gradient db = sum of dZ over rows."""
    dz = np.asarray(dh, dtype=np.float64) * gelu_grad(z)
    return dz, dz.sum(axis=0)


def cube_ffn_devices(x, w1, b1, w2, dout, p):
    """The FFN block out = GELU(x w1^T + b1) w2^T over p devices along each
    reduction (x [rows, hidden], w1 [ffn, hidden], w2 [hidden, ffn]), and its
    backward for the output gradient dout: each device multiplies its
    gathered blocks (the column ranges of the reduction it owns), the
    partial sums are reduced (a sum), and only then are the bias and GELU
    applied.  Returns (out, grads) with grads x, w1, b1, w2 (fp64).  With
    p = 1 this is the unsharded block."""
    x, w1, b1, w2, dout = (np.asarray(t, dtype=np.float64) for t in (x, w1, b1, w2, dout))
    hs = np.array_split(np.arange(x.shape[1]), p)
    fs = np.array_split(np.arange(w1.shape[0]), p)
    z_sum = sum(cube_matmul("abt", x[:, c], w1[:, c]) for c in hs)
    z, h = cube_bias_gelu(z_sum, b1)
    out = sum(cube_matmul("abt", h[:, c], w2[:, c]) for c in fs)
    dh = np.concatenate([cube_matmul("ab", dout, w2[:, c]) for c in fs], axis=1)
    dz, db1 = cube_gelu_backward(dh, z)
    dw2 = np.concatenate([cube_matmul("atb", dout, h[:, c]) for c in fs], axis=1)
    dw1 = np.concatenate([cube_matmul("atb", dz, x[:, c]) for c in hs], axis=1)
    dx = sum(cube_matmul("ab", dz[:, c], w1[c, :]) for c in fs)
    return out, dict(x=dx, w1=dw1, b1=db1, w2=dw2)
