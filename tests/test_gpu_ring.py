"""GPU parity of attention over key/value blocks and of the merge of
partial results, through the C-ABI, against the fp64 oracle.

Tolerances: the block outputs come from bf16 Q/K/V (rounded once on the
host, the same values the oracle gets) with fp32 accumulation and bf16
probabilities, so O and LSE take the bf16 bar of the layer tests (2e-2 of the
tensor's largest magnitude); the merge is fp32 elementwise arithmetic
(1e-5).  Which queries see no key of a block is decided by integer
positions and must match exactly (LSE = -inf and O = 0 there)."""
import numpy as np
import pytest

import oracle
from token_transformer_layer_amd import abi, synth

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-5


def _torch():
    import torch
    return torch


def _dev(a, dtype):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(dtype)


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _shape(b, n, d, nq, nk, qp, kp):
    return abi.tp_attn_block_shape(b, n, d, nq, nk, qp, kp)


def _inputs(b, n, d, nq, nk, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    q = synth.round_bf16(rng.normal(size=(b, n, nq, d)) * scale)
    k = synth.round_bf16(rng.normal(size=(b, n, nk, d)) * scale)
    v = synth.round_bf16(rng.normal(size=(b, n, nk, d)))
    return q, k, v


def _block_gpu(q, k, v, qp, kp):
    torch = _torch()
    b, n, nq, d = q.shape
    nk = k.shape[2]
    o = torch.empty((b, n, nq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((b, n, nq), dtype=torch.float32, device="cuda")
    tq, tk, tv = _dev(q, torch.bfloat16), _dev(k, torch.bfloat16), _dev(v, torch.bfloat16)
    abi.tp_attn_block_fwd(_shape(b, n, d, nq, nk, qp, kp), tq.data_ptr(), tk.data_ptr(), tv.data_ptr(),
                          o.data_ptr(), lse.data_ptr(), _stream())
    torch.cuda.synchronize()
    return o, lse


def _compare(o, lse, ro, rl, tol):
    o = o.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin), "queries with no visible key differ"
    assert np.all(np.isneginf(lse[~fin])) and np.all(o[~fin] == 0)
    if fin.any():
        e_o = np.abs(o - ro).max() / max(np.abs(ro).max(), 1e-30)
        e_l = np.abs(lse[fin] - rl[fin]).max() / max(np.abs(rl[fin]).max(), 1e-30)
        assert e_o <= tol and e_l <= tol, (e_o, e_l)


# (d, nq, nk, q_pos0, k_pos0): blocks before the queries, on the diagonal,
# straddling it, after every query, single rows, ragged tile tails, and
# blocks of no keys or no queries (empty buffers passed as NULL)
BLOCKS = [
    (128, 200, 150, 300, 0),
    (128, 200, 200, 300, 300),
    (128, 130, 260, 64, 0),
    (128, 96, 70, 10, 200),
    (64, 77, 333, 400, 50),
    (64, 257, 257, 0, 0),
    (64, 1, 129, 128, 0),
    (128, 129, 1, 5, 5),
    (64, 50, 0, 100, 0),
    (128, 0, 70, 0, 0),
]


@pytest.mark.parametrize("d,nq,nk,qp,kp", BLOCKS)
def test_block_against_oracle(d, nq, nk, qp, kp):
    print("[case] block d=%d nq=%d nk=%d q_pos0=%d k_pos0=%d" % (d, nq, nk, qp, kp), flush=True)
    q, k, v = _inputs(2, 3, d, nq, nk, seed=nq * 7 + nk)
    o, lse = _block_gpu(q, k, v, qp, kp)
    ro, rl = oracle.attention_block(q, k, v, qp, kp)
    _compare(o, lse, ro, rl, TOL_BF16)


def test_merge_against_oracle():
    torch = _torch()
    rng = np.random.default_rng(7)
    b, n, nq, d = 2, 3, 50, 128
    oa, ob = rng.normal(size=(2, b, n, nq, d))
    la, lb = rng.normal(size=(2, b, n, nq)) * 3
    la[0, 0, :5] = -np.inf
    lb[0, 1, 3:9] = -np.inf
    la[1, 2, 10:12] = -np.inf
    lb[1, 2, 10:12] = -np.inf
    oa[np.isneginf(la)] = 0
    ob[np.isneginf(lb)] = 0
    shape = _shape(b, n, d, nq, 0, 0, 0)
    t = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda() for x in (oa, la, ob, lb)]
    o = torch.empty_like(t[0])
    lse = torch.empty_like(t[1])
    abi.tp_attn_merge(shape, t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), t[3].data_ptr(), o.data_ptr(),
                      lse.data_ptr(), _stream())
    # in place over the first operand gives the same bits
    abi.tp_attn_merge(shape, t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), t[3].data_ptr(), t[0].data_ptr(),
                      t[1].data_ptr(), _stream())
    torch.cuda.synchronize()
    assert torch.equal(o, t[0]) and torch.equal(lse, t[1])
    ro, rl = oracle.merge_partials(oa.astype(np.float32), la.astype(np.float32), ob.astype(np.float32),
                                   lb.astype(np.float32))
    _compare(o, lse, ro, rl, TOL_F32)


@pytest.mark.parametrize("d", [64, 128])
def test_ring_of_blocks_equals_causal_attention(d):
    """Queries of one device against every device's block, merged in ring
    order starting from its own block: causal attention over all keys."""
    torch = _torch()
    devices, per = 4, 96
    b, n = 1, 4
    L = devices * per
    rng = np.random.default_rng(31 + d)
    q_all = synth.round_bf16(rng.normal(size=(b, n, L, d)))
    k_all = synth.round_bf16(rng.normal(size=(b, n, L, d)))
    v_all = synth.round_bf16(rng.normal(size=(b, n, L, d)))
    for me in range(devices):
        print("[case] ring d=%d device %d" % (d, me), flush=True)
        qs = q_all[:, :, me * per:(me + 1) * per]
        acc = None
        for step in range(devices):
            src = (me - step) % devices
            ks, vs = k_all[:, :, src * per:(src + 1) * per], v_all[:, :, src * per:(src + 1) * per]
            o, lse = _block_gpu(qs, ks, vs, me * per, src * per)
            if acc is None:
                acc = (o, lse)
            else:
                abi.tp_attn_merge(_shape(b, n, d, per, per, 0, 0), acc[0].data_ptr(), acc[1].data_ptr(),
                                  o.data_ptr(), lse.data_ptr(), acc[0].data_ptr(), acc[1].data_ptr(), _stream())
        torch.cuda.synchronize()
        ro, _, rl = oracle.causal_attention(qs, k_all, v_all, q_start=me * per)
        _compare(acc[0], acc[1], ro, rl, TOL_BF16)


def test_long_context_blocks_sampled():
    """The benchmark's block shapes (4096 queries against a 4096-key block of
    another device, and against its own diagonal block; 12 heads of 128),
    checked on sampled queries of every head."""
    torch = _torch()
    b, n, d, nq = 1, 12, 128, 4096
    for qp, kp in [(4096, 0), (4096, 4096)]:
        print("[case] long block q_pos0=%d k_pos0=%d" % (qp, kp), flush=True)
        q, k, v = _inputs(b, n, d, nq, nq, seed=qp + kp + 1)
        o, lse = _block_gpu(q, k, v, qp, kp)
        o, lse = o.cpu().numpy(), lse.cpu().numpy()
        rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, nq - 1], np.random.default_rng(3).integers(0, nq, 24)]))
        for r in rows:
            ro, rl = oracle.attention_block(q[:, :, r:r + 1], k, v, qp + r, kp)
            e_o = np.abs(o[:, :, r:r + 1] - ro).max() / np.abs(ro).max()
            e_l = np.abs(lse[:, :, r:r + 1] - rl).max() / np.abs(rl).max()
            assert e_o <= TOL_BF16 and e_l <= TOL_BF16, (r, e_o, e_l)
