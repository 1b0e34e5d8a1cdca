"""Host-side checks of the C-ABI that need no GPU: the library loads and
exports every function include/tpshard.h declares, buffer sizing, and every
argument check returns its status before anything is enqueued (the checks
run before any HIP call, so invalid calls are safe without a device)."""
import ctypes
import os
import re

import pytest

from token_transformer_layer_amd import abi, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(abi.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = abi.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def cfg_of(shape):
    return abi.tp_shard_cfg(shape.hidden, shape.heads, shape.head_dim, shape.ffn, shape.tp, shape.batch, shape.seq,
                            abi.TP_BF16 if shape.dtype == "bf16" else abi.TP_F32, shape.eps)


def test_buffer_sizes_cover_the_saved_tensors():
    for shape in synth.CONFIGS.values():
        c = cfg_of(shape)
        es = 2 if shape.dtype == "bf16" else 4
        T, h = shape.batch * shape.seq, shape.hidden
        ht, ft = h // shape.tp, shape.ffn // shape.tp
        need = T * (2 * h + 2 * ht + 2 * ft) * es + T * (4 * 4) + 4 * T * (shape.heads // shape.tp)
        assert abi.tp_shard_saved_bytes(c) >= need
        assert abi.tp_shard_scratch_bytes(c) >= T * (ft + 4 * ht) * es


BAD_CFGS = [
    (dict(hidden=0), abi.TP_ESHAPE),
    (dict(hidden=1000), abi.TP_ESHAPE),            # != heads * head_dim
    (dict(tp=3), abi.TP_ESHAPE),                   # heads not divisible
    (dict(head_dim=32, hidden=128), abi.TP_EUNSUPPORTED),
    (dict(ffn=1028), abi.TP_ESHAPE),               # ffn / t not a multiple of 8
    (dict(eps=0.0), abi.TP_EINVAL),
    (dict(dtype="f16"), abi.TP_EINVAL),
]


@pytest.mark.parametrize("change,status", BAD_CFGS)
def test_bad_config(change, status):
    shape = synth.CONFIGS["tiny-fp32"]
    fields = dict(hidden=shape.hidden, heads=shape.heads, head_dim=shape.head_dim, ffn=shape.ffn, tp=shape.tp,
                  batch=shape.batch, seq=shape.seq, dtype=abi.TP_F32, eps=shape.eps)
    fields.update(change)
    if fields["dtype"] == "f16":
        fields["dtype"] = 7
    c = abi.tp_shard_cfg(fields["hidden"], fields["heads"], fields["head_dim"], fields["ffn"], fields["tp"],
                         fields["batch"], fields["seq"], fields["dtype"], fields["eps"])
    assert abi.tp_shard_saved_bytes(c) == 0
    with pytest.raises(abi.TPError) as ei:
        _fwd(c, abi.make_partition([shape.seq]), 0, 1)
    assert ei.value.status == status


FAKE = 0x10000  # an aligned address that is never dereferenced: every call below fails its checks first


def _weights(addr=FAKE):
    return abi.tp_shard_weights(*[addr] * len(abi.WEIGHT_FIELDS))


def _fwd(c, part, j0, j1, phase=abi.TP_FWD_ATTN, kv=None, in_ptr=FAKE, saved=FAKE, w=None):
    kv = abi.tp_kv_cache(FAKE, FAKE, 0) if kv is None else kv
    abi.tp_shard_layer_fwd(c, _weights() if w is None else w, part, j0, j1, phase, in_ptr, FAKE, kv, saved,
                           FAKE, None)


def _status(fn):
    with pytest.raises(abi.TPError) as ei:
        fn()
    return ei.value.status


def test_partition_checks():
    c = cfg_of(synth.CONFIGS["tiny-fp32"])
    assert _status(lambda: _fwd(c, abi.make_partition([32, 32, 32]), 0, 1)) == abi.TP_ESHAPE  # sum 96 != 128
    assert _status(lambda: _fwd(c, abi.make_partition([64, 0, 64]), 0, 1)) == abi.TP_ESHAPE  # empty slice
    assert _status(lambda: _fwd(c, abi.make_partition([128]), 0, 2)) == abi.TP_EINVAL       # range past the end
    assert _status(lambda: _fwd(c, abi.make_partition([64, 64]), 1, 1)) == abi.TP_EINVAL    # empty range
    assert _status(lambda: _fwd(c, abi.make_partition([64, 64]), -1, 1)) == abi.TP_EINVAL


def test_pointer_checks():
    c = cfg_of(synth.CONFIGS["tiny-fp32"])
    part = abi.make_partition([64, 64])
    assert _status(lambda: _fwd(c, part, 0, 1, in_ptr=None)) == abi.TP_EINVAL
    assert _status(lambda: _fwd(c, part, 0, 1, in_ptr=FAKE + 8)) == abi.TP_EALIGN
    assert _status(lambda: _fwd(c, part, 0, 1, saved=None)) == abi.TP_EINVAL
    assert _status(lambda: _fwd(c, part, 0, 1, w=_weights(FAKE + 2))) == abi.TP_EALIGN
    assert _status(lambda: _fwd(c, part, 0, 1, phase=4)) == abi.TP_EINVAL


def test_forward_slice_order_is_enforced():
    c = cfg_of(synth.CONFIGS["tiny-fp32"])
    part = abi.make_partition([32, 32, 32, 32])
    kv = abi.tp_kv_cache(FAKE, FAKE, 0)
    assert _status(lambda: _fwd(c, part, 1, 2, kv=kv)) == abi.TP_EORDER  # slice 1 before slice 0
    kv.filled = 64
    assert _status(lambda: _fwd(c, part, 0, 1, kv=kv)) == abi.TP_EORDER  # slice 0 again
    assert kv.filled == 64  # a failed call leaves the struct untouched


def test_backward_slice_order_is_enforced():
    c = cfg_of(synth.CONFIGS["tiny-fp32"])
    part = abi.make_partition([32, 32, 32, 32])
    g = abi.tp_shard_grads(*[FAKE] * len(abi.GRAD_FIELDS), 1)
    kv = abi.tp_kv_cache(FAKE, FAKE, 128)
    kvg = abi.tp_kv_grad(FAKE, FAKE, 128)

    def bwd(j0, j1):
        abi.tp_shard_layer_bwd(c, _weights(), part, j0, j1, abi.TP_BWD_ATTN, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               g, kv, kvg, FAKE, FAKE, None)

    assert _status(lambda: bwd(0, 1)) == abi.TP_EORDER  # must start from the last slice
    kvg.done_from = 64
    assert _status(lambda: bwd(3, 4)) == abi.TP_EORDER  # slice 3 is already done
    kv.filled = 32
    kvg.done_from = 128
    assert _status(lambda: bwd(3, 4)) == abi.TP_EORDER  # forward has not reached slice 3
    kv.filled = 128
    g.accumulate = 2
    assert _status(lambda: bwd(3, 4)) == abi.TP_EINVAL  # accumulate must be 0 or 1
    g.accumulate = 1

    def bwd_phase(phase):
        abi.tp_shard_layer_bwd(c, _weights(), part, 3, 4, phase, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               g, kv, kvg, FAKE, FAKE, None)

    assert _status(lambda: bwd_phase(8)) == abi.TP_EINVAL
    assert _status(lambda: bwd_phase(-1)) == abi.TP_EINVAL
    kvg.done_from = 32
    assert _status(lambda: bwd_phase(abi.TP_BWD_ATTN_DATA)) == abi.TP_EORDER


def test_combine_and_cube_checks():
    c = cfg_of(synth.CONFIGS["tiny-fp32"])
    assert _status(lambda: abi.tp_residual_combine(c, -1, FAKE, FAKE, FAKE, FAKE, None)) == abi.TP_ESHAPE
    assert _status(lambda: abi.tp_residual_combine(c, 10, FAKE, None, FAKE, FAKE, None)) == abi.TP_EINVAL
    assert _status(lambda: abi.tp_cube_ffn_block(16, 100, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)) == \
        abi.TP_ESHAPE
    assert _status(lambda: abi.tp_cube_ffn_block(16, 64, 64, FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, None)) == \
        abi.TP_EALIGN


def test_last_error_names_the_problem():
    c = cfg_of(synth.CONFIGS["tiny-fp32"])
    _status(lambda: _fwd(c, abi.make_partition([100]), 0, 1))
    assert b"seq_len" in abi.lib().tp_last_error()


def test_force_tile_range():
    for bad in (-2, 7, 100):
        assert _status(lambda: abi.tp_gemm_force_tile(bad)) == abi.TP_EINVAL
    abi.tp_gemm_force_tile(3)
    abi.tp_gemm_force_tile(-1)


def test_block_attention_checks():
    good = abi.tp_attn_block_shape(1, 2, 128, 10, 10, 0, 0)
    call = lambda s, q=FAKE, o=FAKE: abi.tp_attn_block_fwd(s, q, FAKE, FAKE, o, FAKE, None)
    assert _status(lambda: call(abi.tp_attn_block_shape(1, 2, 96, 10, 10, 0, 0))) == abi.TP_EUNSUPPORTED
    assert _status(lambda: call(abi.tp_attn_block_shape(0, 2, 128, 10, 10, 0, 0))) == abi.TP_ESHAPE
    assert _status(lambda: call(abi.tp_attn_block_shape(1, 2, 128, -1, 10, 0, 0))) == abi.TP_ESHAPE
    assert _status(lambda: call(abi.tp_attn_block_shape(1, 2, 128, 10, 10, -5, 0))) == abi.TP_ESHAPE
    assert _status(lambda: call(good, q=None)) == abi.TP_EINVAL
    assert _status(lambda: call(good, o=FAKE + 4)) == abi.TP_EALIGN
    merge = lambda s, o=FAKE: abi.tp_attn_merge(s, FAKE, FAKE, FAKE, FAKE, o, FAKE, None)
    assert _status(lambda: merge(good, o=None)) == abi.TP_EINVAL
    assert _status(lambda: merge(good, o=FAKE + 8)) == abi.TP_EALIGN
    assert _status(lambda: merge(abi.tp_attn_block_shape(1, 2, 32, 10, 0, 0, 0))) == abi.TP_EUNSUPPORTED
    # buffers sized by a count of 0 are never addressed and may be NULL (no
    # query: nothing to launch)
    empty = abi.tp_attn_block_shape(1, 2, 128, 0, 0, 0, 0)
    abi.tp_attn_block_fwd(empty, None, None, None, None, None, None)
    abi.tp_attn_merge(empty, None, None, None, None, None, None, None)
    no_keys = abi.tp_attn_block_shape(1, 2, 128, 10, 0, 0, 0)
    assert _status(lambda: abi.tp_attn_block_fwd(no_keys, None, None, None, FAKE, FAKE, None)) == abi.TP_EINVAL


def test_cube_op_checks():
    mm = lambda form=0, M=16, N=16, K=16, acc=0, c=FAKE: abi.lib().tp_cube_matmul(form, M, N, K, FAKE, FAKE, c, acc,
                                                                                   None)
    assert mm(form=3) == abi.TP_EINVAL
    assert mm(M=12) == abi.TP_ESHAPE
    assert mm(K=0) == abi.TP_ESHAPE
    assert mm(acc=2) == abi.TP_EINVAL
    assert mm(c=None) == abi.TP_EINVAL
    assert mm(c=FAKE + 4) == abi.TP_EALIGN
    assert abi.lib().tp_cube_bias_gelu(4, 12, FAKE, FAKE, FAKE, FAKE, None) == abi.TP_ESHAPE
    assert abi.lib().tp_cube_gelu_backward(4, 16, FAKE, FAKE, FAKE, FAKE, 0, None, None) == abi.TP_EINVAL
    assert abi.tp_cube_work_bytes(0, 16) == 0 and abi.tp_cube_work_bytes(4096, 24576) > 0


def test_layernorm_checks():
    c = cfg_of(synth.CONFIGS["tiny-fp32"])
    L = abi.lib()
    assert L.tp_layernorm_fwd(c, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == abi.TP_ESHAPE
    assert L.tp_layernorm_fwd(c, 10, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == abi.TP_EINVAL
    assert L.tp_layernorm_fwd(c, 10, FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == abi.TP_EALIGN
    args = [FAKE] * 9
    assert L.tp_layernorm_bwd(c, 10, *args, 2, FAKE, None) == abi.TP_EINVAL
    assert L.tp_layernorm_bwd(c, 10, *args[:8], None, 0, FAKE, None) == abi.TP_EINVAL
    assert abi.tp_layernorm_work_bytes(c, 0) == 0 and abi.tp_layernorm_work_bytes(c, 100) > 0


def test_sequence_parallel_phases_need_their_inputs():
    c = cfg_of(synth.CONFIGS["tiny-fp32"])
    part = abi.make_partition([64, 64])
    g = abi.tp_shard_grads(*[FAKE] * len(abi.GRAD_FIELDS), 1)
    kv = abi.tp_kv_cache(FAKE, FAKE, 128)
    kvg = abi.tp_kv_grad(FAKE, FAKE, 128)
    # the SP attention backward needs dh (given) but not ln_in / reduced_in
    st = abi.lib().tp_shard_layer_bwd(c, _weights(), part, 1, 2, abi.TP_BWD_ATTN_SP, FAKE, None, None, FAKE, None,
                                      FAKE, g, kv, kvg, FAKE, FAKE, None)
    assert st == abi.TP_EINVAL and b"dh" in abi.lib().tp_last_error()
    # the SP forward does not need LayerNorm parameters
    w = abi.tp_shard_weights(*[None if n.startswith("ln") else FAKE for n in abi.WEIGHT_FIELDS])
    assert _status(lambda: _fwd(c, part, 0, 1, phase=abi.TP_FWD_ATTN_SP, w=w, in_ptr=None)) == abi.TP_EINVAL
    assert b"in" in abi.lib().tp_last_error()
