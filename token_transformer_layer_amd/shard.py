"""Device buffers for one rank's layer shard, held as torch tensors, and thin
wrappers that pass their addresses to the C-ABI.

torch provides device memory and the stream only; every step of the layer
runs in libtpshard.so.
"""
import numpy as np
import torch

from . import abi

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def _ptr(t):
    return None if t is None else t.data_ptr()


def stream_handle():
    return torch.cuda.current_stream().cuda_stream


class ShardLayer:
    """One rank's shard of a decoder layer on the current GPU.

    params: dict of host arrays in the library's layout (ln1_g, ln1_b, w_qkv,
    b_qkv, w_o, b_o, ln2_g, ln2_b, w1, b1, w2, b2), already representable in
    the storage dtype."""

    def __init__(self, shape, params, device="cuda"):
        self.shape = shape
        self.dtype = _TORCH_DTYPE[shape.dtype]
        self.device = device
        self.cfg = abi.tp_shard_cfg(shape.hidden, shape.heads, shape.head_dim, shape.ffn, shape.tp, shape.batch,
                                    shape.seq, abi.TP_BF16 if shape.dtype == "bf16" else abi.TP_F32,
                                    shape.eps)
        self.part = abi.make_partition(shape.slices)
        self.bounds = [0]
        for n in shape.slices:
            self.bounds.append(self.bounds[-1] + int(n))
        self.p = {k: self.upload(v) for k, v in params.items()}
        self.w = abi.tp_shard_weights(*[_ptr(self.p[n]) for n in abi.WEIGHT_FIELDS])
        h, s, b = shape.hidden, shape.seq, shape.batch
        nt, d = shape.heads // shape.tp, shape.head_dim
        saved = abi.tp_shard_saved_bytes(self.cfg)
        scratch = abi.tp_shard_scratch_bytes(self.cfg)
        if saved == 0 or scratch == 0:
            raise abi.TPError(abi.TP_ESHAPE, abi.lib().tp_last_error().decode())
        self.saved = torch.empty(saved, dtype=torch.uint8, device=device)
        self.scratch = torch.empty(scratch, dtype=torch.uint8, device=device)
        self.k = torch.zeros((b, nt, s, d), dtype=self.dtype, device=device)
        self.v = torch.zeros((b, nt, s, d), dtype=self.dtype, device=device)
        self.dk = torch.zeros((b, nt, s, d), dtype=torch.float32, device=device)
        self.dv = torch.zeros((b, nt, s, d), dtype=torch.float32, device=device)
        self.kv = abi.tp_kv_cache(_ptr(self.k), _ptr(self.v), 0)
        self.kvg = abi.tp_kv_grad(_ptr(self.dk), _ptr(self.dv), s)
        self.g = {n: torch.zeros(self.p[n].shape if n in self.p else (h,), dtype=torch.float32, device=device)
                  for n in abi.GRAD_FIELDS}
        self.gs = abi.tp_shard_grads(*[_ptr(self.g[n]) for n in abi.GRAD_FIELDS], 1)

    def upload(self, arr):
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(self.device).to(self.dtype)

    def act(self, arr=None):
        """An [s, b, h] activation in the storage dtype (uploaded or empty)."""
        sh = self.shape
        if arr is None:
            return torch.empty((sh.seq, sh.batch, sh.hidden), dtype=self.dtype, device=self.device)
        return self.upload(arr)

    def f32(self):
        sh = self.shape
        return torch.empty((sh.seq, sh.batch, sh.hidden), dtype=torch.float32, device=self.device)

    def new_step(self, fill=0.0):
        """Reset the cache protocol and fill the gradient buffers (zeros for
        steps that accumulate from the first call; any value for steps whose
        first call of each gradient overwrites)."""
        self.kv.filled = 0
        self.kvg.done_from = self.shape.seq
        for t in self.g.values():
            t.fill_(fill)

    # phases -----------------------------------------------------------------
    def fwd(self, phase, j0, j1, inp, partial_out):
        abi.tp_shard_layer_fwd(self.cfg, self.w, self.part, j0, j1, phase, _ptr(inp), _ptr(partial_out),
                               self.kv, _ptr(self.saved), _ptr(self.scratch), stream_handle())

    def bwd(self, phase, j0, j1, dy=None, ln_in=None, reduced=None, partial_out=None, dh=None, dx=None,
            accumulate=True):
        self.gs.accumulate = 1 if accumulate else 0
        abi.tp_shard_layer_bwd(self.cfg, self.w, self.part, j0, j1, phase, _ptr(dy), _ptr(ln_in), _ptr(reduced),
                               _ptr(partial_out), _ptr(dh), _ptr(dx), self.gs, self.kv, self.kvg,
                               _ptr(self.saved), _ptr(self.scratch), stream_handle())

    def combine(self, resid, reduced, bias, out, rows=None):
        sh = self.shape
        rows = sh.seq * sh.batch if rows is None else rows
        abi.tp_residual_combine(self.cfg, rows, _ptr(resid), _ptr(reduced), _ptr(bias), _ptr(out),
                                stream_handle())
