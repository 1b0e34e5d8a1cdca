"""Seeded synthetic inputs for the layer shard, shaped like the GPT-3-family
workloads the pages train (no dataset is involved: every tensor is drawn
from a fixed-seed normal distribution).

This module holds shapes and random draws only: none of the layer's
arithmetic.  Both the GPU path (tests, bench) and the CPU oracle take their
inputs from here, so they see the same values.

Draw order for one configuration: x, then the weights in the order of the
library's weight struct (ln1 gamma, ln1 beta, W_qkv, b_qkv, W_o, b_o, ln2
gamma, ln2 beta, W1, b1, W2, b2), then dY.  Values are drawn in float64 by
numpy's PCG64 generator, cast to float32 and, for bf16 configurations,
rounded to the nearest bf16 value (ties to even), so the float32 arrays
returned here hold exactly the values the device receives.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["LayerShape", "CubeShape", "CONFIGS", "CUBE", "round_bf16",
           "full_params", "shard_params_direct", "activations", "cube_inputs",
           "slice_bounds"]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One decoder layer split t ways, run over a token-slice partition."""
    name: str
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    tp: int
    batch: int
    seq: int
    slices: tuple
    dtype: str  # "f32" or "bf16": storage type; accumulation is always fp32
    eps: float = 1e-5
    seed: int = 0

    def as_dict(self):
        return dict(hidden=self.hidden, heads=self.heads, head_dim=self.head_dim,
                    ffn=self.ffn, tp=self.tp, batch=self.batch, seq=self.seq,
                    eps=self.eps)

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)

    @property
    def tokens(self):
        return self.batch * self.seq


@dataclasses.dataclass(frozen=True)
class CubeShape:
    """One device's block of a 2x2x2 cube partition of a GPT-3 175B FFN."""
    name: str
    rows: int      # X block rows
    hidden: int    # X block columns = W1 block input width
    ffn: int       # W1 block output width
    seed: int = 5


CONFIGS = {
    "tiny-fp32": LayerShape("tiny-fp32", 256, 4, 64, 1024, 2, 2, 128, (32,) * 4, "f32", seed=1001),
    "medium-bf16": LayerShape("medium-bf16", 1024, 16, 64, 4096, 4, 8, 1024, (128,) * 8, "bf16", seed=1002),
    "gpt13b-t8": LayerShape("gpt13b-t8", 5120, 40, 128, 20480, 8, 4, 2048,
                            (512, 384, 320, 288, 256, 160, 128), "bf16", seed=1003),
    "gpt3-175b-t8": LayerShape("gpt3-175b-t8", 12288, 96, 128, 49152, 8, 1, 2048, (128,) * 16, "bf16",
                               seed=1004),
}
CUBE = CubeShape("cube-ffn-block", 4096, 6144, 24576, seed=1005)


def round_bf16(a):
    """Round float32 values to the nearest bf16 value, ties to even, and return
    them as float32 (a pure storage conversion)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def _store(a, dtype):
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else np.ascontiguousarray(a)


def slice_bounds(slices):
    """Slice lengths l_1..l_M -> boundaries [0, o_1, ..., L]."""
    out = [0]
    for n in slices:
        out.append(out[-1] + int(n))
    return out


class _Draw:
    def __init__(self, seed, dtype):
        self.rng = np.random.default_rng(seed)
        self.dtype = dtype

    def normal(self, shape, std):
        return _store(self.rng.standard_normal(shape) * std, self.dtype)

    def const(self, shape, value):
        return _store(np.full(shape, value), self.dtype)

    def bias(self, shape, variant):
        if variant == "standard":
            return self.const(shape, 0.0)
        return self.normal(shape, 0.02)

    def gamma(self, shape, variant):
        if variant == "standard":
            return self.const(shape, 1.0)
        return _store(1.0 + self.rng.standard_normal(shape) * 0.1, self.dtype)

    def beta(self, shape, variant):
        if variant == "standard":
            return self.const(shape, 0.0)
        return self.normal(shape, 0.02)


def _wstd(variant):
    # "sharp" (fp32 storage) and "peaked" (bf16 storage) raise the weight
    # scale so the softmax is far from uniform; with bf16 Q and K the score
    # rounding error grows with the score scale (std ~ w_std^2 h), so the
    # bf16 variant stays at a scale where that error is small.
    return {"sharp": 0.2, "peaked": 0.05}.get(variant, 0.02)


def activations(cfg: LayerShape, seed=None):
    """(x, dy): [s, b, h] each, N(0, 1)."""
    d = _Draw(cfg.seed if seed is None else seed, cfg.dtype)
    x = d.normal((cfg.seq, cfg.batch, cfg.hidden), 1.0)
    dy = d.normal((cfg.seq, cfg.batch, cfg.hidden), 1.0)
    return x, dy


def full_params(cfg: LayerShape, variant="standard", seed=None):
    """Parameters of the whole (unsharded) layer, weights stored [out, in].

    variant "standard": linear weights N(0, 0.02), biases 0, gamma 1, beta 0.
    "perturbed": also biases N(0, 0.02), gamma 1 + N(0, 0.1), beta N(0, 0.02).
    "sharp" / "peaked": as "perturbed" with weights N(0, 0.2) / N(0, 0.05) so
    the softmax is far from uniform."""
    d = _Draw((cfg.seed if seed is None else seed) + 7919, cfg.dtype)
    h, f = cfg.hidden, cfg.ffn
    std = _wstd(variant)
    p = {}
    p["ln1_g"] = d.gamma(h, variant)
    p["ln1_b"] = d.beta(h, variant)
    for m in ("q", "k", "v"):
        p["w_" + m] = d.normal((h, h), std)
        p["b_" + m] = d.bias(h, variant)
    p["w_o"] = d.normal((h, h), std)
    p["b_o"] = d.bias(h, variant)
    p["ln2_g"] = d.gamma(h, variant)
    p["ln2_b"] = d.beta(h, variant)
    p["w1"] = d.normal((f, h), std)
    p["b1"] = d.bias(f, variant)
    p["w2"] = d.normal((h, f), std)
    p["b2"] = d.bias(h, variant)
    return p


def shard_params_direct(cfg: LayerShape, variant="standard", rank=0, seed=None):
    """One device's shard tensors drawn directly (for layers whose full
    weights would not fit a host comfortably), in the library's layout:
    w_qkv [3 h_t, h], b_qkv [3 h_t], w_o [h, h_t], w1 [f_t, h], b1 [f_t],
    w2 [h, f_t]; LayerNorm parameters and b_o, b2 are [h]."""
    d = _Draw((cfg.seed if seed is None else seed) + 104729 * (rank + 1), cfg.dtype)
    h = cfg.hidden
    ht, ft = h // cfg.tp, cfg.ffn // cfg.tp
    std = _wstd(variant)
    p = {}
    p["ln1_g"] = d.gamma(h, variant)
    p["ln1_b"] = d.beta(h, variant)
    p["w_qkv"] = d.normal((3 * ht, h), std)
    p["b_qkv"] = d.bias(3 * ht, variant)
    p["w_o"] = d.normal((h, ht), std)
    p["b_o"] = d.bias(h, variant)
    p["ln2_g"] = d.gamma(h, variant)
    p["ln2_b"] = d.beta(h, variant)
    p["w1"] = d.normal((ft, h), std)
    p["b1"] = d.bias(ft, variant)
    p["w2"] = d.normal((h, ft), std)
    p["b2"] = d.bias(h, variant)
    return p


def cube_inputs(c: CubeShape = CUBE, rows=None):
    """X [rows, hidden] ~ N(0, 1); W1 [ffn, hidden] and W2 [hidden, ffn]
    ~ N(0, 0.02) (stored [out, in]); b1 = 0; all bf16-rounded."""
    d = _Draw(c.seed, "bf16")
    x = d.normal((c.rows if rows is None else rows, c.hidden), 1.0)
    w1 = d.normal((c.ffn, c.hidden), 0.02)
    b1 = d.const(c.ffn, 0.0)
    w2 = d.normal((c.hidden, c.ffn), 0.02)
    return x, w1, b1, w2
