"""ctypes binding of the C-ABI in include/tpshard.h.

Argument marshalling only: the functions below take integers (device
addresses, sizes, a HIP stream handle) and host structs, call the library,
and raise TPError on a non-zero status.  All arithmetic runs in the HIP
kernels of libtpshard.so; loading fails loudly if the library is missing.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpshard.so")

TP_OK, TP_EINVAL, TP_ESHAPE, TP_EALIGN, TP_EORDER, TP_EUNSUPPORTED, TP_EHIP = range(7)
STATUS_NAMES = {0: "TP_OK", 1: "TP_EINVAL", 2: "TP_ESHAPE", 3: "TP_EALIGN", 4: "TP_EORDER",
                5: "TP_EUNSUPPORTED", 6: "TP_EHIP"}
TP_F32, TP_BF16 = 0, 1
TP_FWD_ATTN, TP_FWD_MLP, TP_FWD_ATTN_SP, TP_FWD_MLP_SP = 0, 1, 2, 3
TP_BWD_MLP, TP_BWD_ATTN, TP_BWD_LN1, TP_BWD_MLP_DATA, TP_BWD_ATTN_DATA, TP_BWD_WGRAD = 0, 1, 2, 3, 4, 5
TP_BWD_ATTN_SP, TP_BWD_ATTN_DATA_SP = 6, 7

EXPORTED = ["tp_shard_saved_bytes", "tp_shard_scratch_bytes", "tp_shard_layer_fwd",
            "tp_shard_layer_bwd", "tp_residual_combine", "tp_cube_ffn_block", "tp_attn_block_fwd",
            "tp_attn_merge", "tp_slicing_plan", "tp_plan_latency", "tp_fit_context_model", "tp_slice_cost_table",
            "tp_cube_matmul", "tp_cube_bias_gelu", "tp_cube_work_bytes", "tp_cube_gelu_backward",
            "tp_layernorm_work_bytes", "tp_layernorm_fwd", "tp_layernorm_bwd", "tp_trace_enable", "tp_trace_read",
            "tp_gemm_force_tile", "tp_last_error", "tp_shard_layer_fwd_noalloc", "tp_noalloc_scratch_bytes",
            "tp_attn_block_bwd_work_bytes", "tp_attn_block_bwd"]


class TPError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), msg))
        self.status = status


class tp_shard_cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("tp_size", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("dtype", ctypes.c_int32), ("ln_eps", ctypes.c_float)]


WEIGHT_FIELDS = ["ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "ln2_g", "ln2_b", "w1", "b1", "w2"]
GRAD_FIELDS = ["ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g", "ln2_b", "w1", "b1", "w2", "b2"]


class tp_shard_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class tp_shard_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_FIELDS] + [("accumulate", ctypes.c_int32)]


class tp_partition(ctypes.Structure):
    _fields_ = [("num_slices", ctypes.c_int32), ("len", ctypes.POINTER(ctypes.c_int32))]


class tp_kv_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("filled", ctypes.c_int32)]


class tp_trace_record(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("flops", ctypes.c_double), ("bytes", ctypes.c_double),
                ("ms", ctypes.c_float)]


class tp_attn_block_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "heads", "head_dim", "nq", "nk", "q_pos0", "k_pos0")]


class tp_kv_grad(ctypes.Structure):
    _fields_ = [("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p), ("done_from", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library (loaded once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libtpshard.so is not built (run python -m token_transformer_layer_amd.build); "
                           "there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.tp_shard_saved_bytes.argtypes = [P(tp_shard_cfg)]
    L.tp_shard_saved_bytes.restype = ctypes.c_size_t
    L.tp_shard_scratch_bytes.argtypes = [P(tp_shard_cfg)]
    L.tp_shard_scratch_bytes.restype = ctypes.c_size_t
    L.tp_shard_layer_fwd.argtypes = [P(tp_shard_cfg), P(tp_shard_weights), P(tp_partition), i32, i32, i32,
                                     vp, vp, P(tp_kv_cache), vp, vp, vp]
    L.tp_shard_layer_fwd.restype = ctypes.c_int
    L.tp_shard_layer_fwd_noalloc.argtypes = [P(tp_shard_cfg), P(tp_shard_weights), P(tp_partition), i32, i32,
                                             i32, vp, vp, P(tp_kv_cache), vp, vp]
    L.tp_shard_layer_fwd_noalloc.restype = ctypes.c_int
    L.tp_noalloc_scratch_bytes.argtypes = []
    L.tp_noalloc_scratch_bytes.restype = ctypes.c_size_t
    L.tp_shard_layer_bwd.argtypes = [P(tp_shard_cfg), P(tp_shard_weights), P(tp_partition), i32, i32, i32,
                                     vp, vp, vp, vp, vp, vp, P(tp_shard_grads), P(tp_kv_cache), P(tp_kv_grad),
                                     vp, vp, vp]
    L.tp_shard_layer_bwd.restype = ctypes.c_int
    L.tp_residual_combine.argtypes = [P(tp_shard_cfg), i64, vp, vp, vp, vp, vp]
    L.tp_residual_combine.restype = ctypes.c_int
    L.tp_cube_ffn_block.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.tp_cube_ffn_block.restype = ctypes.c_int
    L.tp_attn_block_fwd.argtypes = [P(tp_attn_block_shape), vp, vp, vp, vp, vp, vp]
    L.tp_attn_block_fwd.restype = ctypes.c_int
    L.tp_attn_merge.argtypes = [P(tp_attn_block_shape), vp, vp, vp, vp, vp, vp, vp]
    L.tp_attn_block_bwd_work_bytes.argtypes = [P(tp_attn_block_shape)]
    L.tp_attn_block_bwd_work_bytes.restype = ctypes.c_size_t
    L.tp_attn_block_bwd.argtypes = [P(tp_attn_block_shape), vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]
    L.tp_attn_block_bwd.restype = ctypes.c_int
    L.tp_attn_merge.restype = ctypes.c_int
    L.tp_layernorm_work_bytes.argtypes = [P(tp_shard_cfg), i64]
    L.tp_layernorm_work_bytes.restype = ctypes.c_size_t
    L.tp_layernorm_fwd.argtypes = [P(tp_shard_cfg), i64, vp, vp, vp, vp, vp, vp, vp]
    L.tp_layernorm_fwd.restype = ctypes.c_int
    L.tp_layernorm_bwd.argtypes = [P(tp_shard_cfg), i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]
    L.tp_layernorm_bwd.restype = ctypes.c_int
    L.tp_cube_matmul.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, vp]
    L.tp_cube_matmul.restype = ctypes.c_int
    L.tp_cube_bias_gelu.argtypes = [i32, i32, vp, vp, vp, vp, vp]
    L.tp_cube_bias_gelu.restype = ctypes.c_int
    L.tp_cube_work_bytes.argtypes = [i32, i32]
    L.tp_cube_work_bytes.restype = ctypes.c_size_t
    L.tp_cube_gelu_backward.argtypes = [i32, i32, vp, vp, vp, vp, i32, vp, vp]
    L.tp_cube_gelu_backward.restype = ctypes.c_int
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    L.tp_slicing_plan.argtypes = [i32, dp, i32, ip, ip, dp]
    L.tp_slicing_plan.restype = ctypes.c_int
    L.tp_plan_latency.argtypes = [i32, dp, i32, i32, ip, dp]
    L.tp_plan_latency.restype = ctypes.c_int
    L.tp_fit_context_model.argtypes = [i32, ip, ip, dp, dp]
    L.tp_fit_context_model.restype = ctypes.c_int
    L.tp_slice_cost_table.argtypes = [i32, i32, dp, dp, dp]
    L.tp_slice_cost_table.restype = ctypes.c_int
    L.tp_trace_enable.argtypes = [i32]
    L.tp_trace_enable.restype = None
    L.tp_trace_read.argtypes = [P(tp_trace_record), i32]
    L.tp_trace_read.restype = i32
    L.tp_gemm_force_tile.argtypes = [i32]
    L.tp_gemm_force_tile.restype = ctypes.c_int
    L.tp_last_error.argtypes = []
    L.tp_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status):
    if status != TP_OK:
        raise TPError(status, lib().tp_last_error().decode())


def tp_gemm_force_tile(tile):
    """-1: the library picks the bf16 product tiles per shape; 0..6 force one."""
    _check(lib().tp_gemm_force_tile(int(tile)))


def make_partition(lengths):
    """Host partition struct; the returned object keeps its array alive."""
    arr = (ctypes.c_int32 * len(lengths))(*[int(n) for n in lengths])
    part = tp_partition(len(lengths), ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
    part._keep = arr
    return part


def tp_shard_saved_bytes(cfg):
    return lib().tp_shard_saved_bytes(ctypes.byref(cfg))


def tp_shard_scratch_bytes(cfg):
    return lib().tp_shard_scratch_bytes(ctypes.byref(cfg))


def tp_shard_layer_fwd(cfg, w, part, slice_begin, slice_end, phase, in_ptr, partial_out, kv, saved, scratch,
                       stream):
    _check(lib().tp_shard_layer_fwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(part), slice_begin,
                                    slice_end, phase, in_ptr, partial_out,
                                    ctypes.byref(kv) if kv is not None else None, saved, scratch, stream))


def tp_shard_layer_fwd_noalloc(cfg, w, part, slice_begin, slice_end, phase, in_ptr, partial_out, kv, saved,
                               stream):
    _check(lib().tp_shard_layer_fwd_noalloc(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(part), slice_begin,
                                            slice_end, phase, in_ptr, partial_out,
                                            ctypes.byref(kv) if kv is not None else None, saved, stream))


def tp_noalloc_scratch_bytes():
    return lib().tp_noalloc_scratch_bytes()


def tp_shard_layer_bwd(cfg, w, part, slice_begin, slice_end, phase, dy, ln_in, reduced_in, partial_out, dh, dx,
                       g, kv, kvg, saved, scratch, stream):
    _check(lib().tp_shard_layer_bwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(part), slice_begin,
                                    slice_end, phase, dy, ln_in, reduced_in, partial_out, dh, dx,
                                    ctypes.byref(g), ctypes.byref(kv) if kv is not None else None,
                                    ctypes.byref(kvg) if kvg is not None else None, saved, scratch, stream))


def tp_residual_combine(cfg, rows, resid, reduced, bias, out, stream):
    _check(lib().tp_residual_combine(ctypes.byref(cfg), rows, resid, reduced, bias, out, stream))


def tp_cube_ffn_block(rows, hidden, ffn, x, w1, b1, w2, hbuf, out, stream):
    _check(lib().tp_cube_ffn_block(rows, hidden, ffn, x, w1, b1, w2, hbuf, out, stream))


def tp_attn_block_fwd(shape, q, k, v, o, lse, stream):
    _check(lib().tp_attn_block_fwd(ctypes.byref(shape), q, k, v, o, lse, stream))


def tp_attn_block_bwd_work_bytes(shape):
    return lib().tp_attn_block_bwd_work_bytes(ctypes.byref(shape))


def tp_attn_block_bwd(shape, q, k, v, o, lse, dout, dq, dk, dv, accumulate, work, stream):
    _check(lib().tp_attn_block_bwd(ctypes.byref(shape), q, k, v, o, lse, dout, dq, dk, dv, 1 if accumulate else 0,
                                   work, stream))


def tp_attn_merge(shape, o_a, lse_a, o_b, lse_b, o, lse, stream):
    _check(lib().tp_attn_merge(ctypes.byref(shape), o_a, lse_a, o_b, lse_b, o, lse, stream))


TP_CUBE_AB, TP_CUBE_ABT, TP_CUBE_ATB = 0, 1, 2


def tp_layernorm_work_bytes(cfg, rows):
    return lib().tp_layernorm_work_bytes(ctypes.byref(cfg), rows)


def tp_layernorm_fwd(cfg, rows, x, gamma, beta, u, mean, rstd, stream):
    _check(lib().tp_layernorm_fwd(ctypes.byref(cfg), rows, x, gamma, beta, u, mean, rstd, stream))


def tp_layernorm_bwd(cfg, rows, du, resid, x, gamma, mean, rstd, dx, dgamma, dbeta, accumulate, work, stream):
    _check(lib().tp_layernorm_bwd(ctypes.byref(cfg), rows, du, resid, x, gamma, mean, rstd, dx, dgamma, dbeta,
                                  1 if accumulate else 0, work, stream))


def tp_cube_matmul(form, M, N, K, a, b, c, accumulate, stream):
    _check(lib().tp_cube_matmul(form, M, N, K, a, b, c, 1 if accumulate else 0, stream))


def tp_cube_bias_gelu(rows, n, z_sum, bias, z, h, stream):
    _check(lib().tp_cube_bias_gelu(rows, n, z_sum, bias, z, h, stream))


def tp_cube_work_bytes(rows, n):
    return lib().tp_cube_work_bytes(rows, n)


def tp_cube_gelu_backward(rows, n, dh, z, dz, dbias, accumulate, work, stream):
    _check(lib().tp_cube_gelu_backward(rows, n, dh, z, dz, dbias, 1 if accumulate else 0, work, stream))


def _dbl(a):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _i32(a):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def tp_slicing_plan(units, cost, stages):
    """cost: (units+1, units+1) host array.  Returns (latency, ends)."""
    import numpy as np
    c, cp = _dbl(cost)
    if c.shape != (units + 1, units + 1):
        raise ValueError("cost must be (units+1, units+1)")
    ends, ep = _i32(np.zeros(units))
    n = ctypes.c_int32()
    lat = ctypes.c_double()
    _check(lib().tp_slicing_plan(units, cp, stages, ctypes.byref(n), ep, ctypes.byref(lat)))
    return lat.value, [int(x) for x in ends[:n.value]]


def tp_plan_latency(units, cost, stages, ends):
    """Latency of the plan with the given slice ends under cost (the same
    pipeline model as tp_slicing_plan)."""
    c, cp = _dbl(cost)
    if c.shape != (units + 1, units + 1):
        raise ValueError("cost must be (units+1, units+1)")
    e, ep = _i32(ends)
    lat = ctypes.c_double()
    _check(lib().tp_plan_latency(units, cp, stages, len(e), ep, ctypes.byref(lat)))
    return lat.value


def tp_fit_context_model(lens, offsets, ctx):
    import numpy as np
    l, lp = _i32(lens)
    o, op = _i32(offsets)
    c, cp = _dbl(ctx)
    coef, fp = _dbl(np.zeros(3))
    _check(lib().tp_fit_context_model(len(l), lp, op, cp, fp))
    return tuple(float(x) for x in coef)


def tp_slice_cost_table(units, granularity, fwd, coef):
    import numpy as np
    f, fp = _dbl(fwd)
    if f.shape != (units + 1,):
        raise ValueError("fwd must have units+1 entries")
    k, kp = _dbl(coef)
    cost, cp = _dbl(np.zeros((units + 1, units + 1)))
    _check(lib().tp_slice_cost_table(units, granularity, fp, kp, cp))
    return cost


def tp_trace_enable(on):
    lib().tp_trace_enable(1 if on else 0)


def tp_trace_read(max_records=100000):
    """[(name, flops, bytes, ms), ...] of the launches recorded since tracing
    was enabled (waits for them to finish)."""
    buf = (tp_trace_record * max_records)()
    n = lib().tp_trace_read(buf, max_records)
    return [(buf[i].name.decode(), buf[i].flops, buf[i].bytes, buf[i].ms) for i in range(min(n, max_records))]
