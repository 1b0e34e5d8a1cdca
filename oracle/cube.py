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

__all__ = ["cube_matmul", "cube_bias_gelu", "cube_gelu_backward", "matmul_grads"]

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
