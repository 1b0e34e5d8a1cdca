"""GPU parity of the backward of attention over one key block (ring
attention's per-block backward step), through the C-ABI, against the fp64
oracle (oracle.attention_block_backward).

The kernels take bf16 Q, K, V and dO (rounded once on the host, the values
the oracle gets) with fp32 accumulation, bf16 probabilities and bf16 dS, so
the bar is the layer's bf16 one: 2e-2 of each tensor's largest magnitude.
Keys no query sees and queries that see no key (log-sum-exp -inf) must get
exactly zero gradient."""
import numpy as np
import pytest

import oracle
from token_transformer_layer_amd import abi, synth

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _torch():
    import torch
    return torch


def _dev(a, dtype):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(dtype)


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    big = np.abs(ref).max()
    if big == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / big)


def _bwd_gpu(q, k, v, o, lse, do, qp, kp, outs=None, accumulate=False):
    """One tp_attn_block_bwd call; returns the torch tensors dq, dk, dv
    (given ones are stored into or added to)."""
    torch = _torch()
    b, n, nq, d = q.shape
    nk = k.shape[2]
    shape = abi.tp_attn_block_shape(b, n, d, nq, nk, qp, kp)
    if outs is None:
        outs = (torch.empty((b, n, nq, d), dtype=torch.float32, device="cuda"),
                torch.empty((b, n, nk, d), dtype=torch.float32, device="cuda"),
                torch.empty((b, n, nk, d), dtype=torch.float32, device="cuda"))
    t = [_dev(a, torch.bfloat16) for a in (q, k, v, do)]
    to, tl = _dev(o, torch.float32), _dev(lse, torch.float32)
    work = torch.empty(abi.tp_attn_block_bwd_work_bytes(shape), dtype=torch.uint8, device="cuda")
    abi.tp_attn_block_bwd(shape, t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), to.data_ptr(), tl.data_ptr(),
                          t[3].data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), accumulate,
                          work.data_ptr(), _stream())
    torch.cuda.synchronize()
    return outs


def _inputs(b, n, d, nq, nk_total, seed):
    rng = np.random.default_rng(seed)
    q = synth.round_bf16(rng.normal(size=(b, n, nq, d)))
    k = synth.round_bf16(rng.normal(size=(b, n, nk_total, d)))
    v = synth.round_bf16(rng.normal(size=(b, n, nk_total, d)))
    do = synth.round_bf16(rng.normal(size=(b, n, nq, d)))
    return q, k, v, do


# (d, nq, nk, q_pos0, k_pos0, first key position of the merged key set):
# the block is the last nk keys of a key set starting at `first`; blocks
# before, on and across the diagonal, after every query, single rows and
# columns, ragged tile tails, blocks of no queries or no keys (empty buffers
# passed as NULL); first = k_pos0 makes the block the only one, so queries
# before it see no key (log-sum-exp -inf).
CASES = [
    (128, 200, 150, 300, 100, 0),
    (128, 200, 200, 300, 300, 0),
    (128, 130, 260, 64, 0, 0),
    (128, 96, 70, 10, 200, 0),
    (64, 77, 333, 400, 50, 0),
    (64, 257, 257, 0, 0, 0),
    (64, 1, 129, 128, 0, 0),
    (128, 129, 1, 5, 5, 0),
    (128, 90, 50, 0, 20, 20),
    (64, 200, 64, 30, 100, 100),
    (128, 0, 100, 50, 20, 0),
    (64, 80, 0, 100, 30, 0),
]


@pytest.mark.parametrize("d,nq,nk,qp,kp,first", CASES)
def test_block_backward_against_oracle(d, nq, nk, qp, kp, first):
    print("[case] block backward d=%d nq=%d nk=%d q_pos0=%d k_pos0=%d keys from %d" % (d, nq, nk, qp, kp, first),
          flush=True)
    b, n = 2, 3
    q, k_all, v_all, do = _inputs(b, n, d, nq, kp + nk - first, seed=nq * 11 + nk + kp)
    o, lse = oracle.attention_block(q, k_all, v_all, qp, first)   # the merged forward over every key
    kb, vb = k_all[:, :, kp - first:], v_all[:, :, kp - first:]
    dq, dk, dv = _bwd_gpu(q, kb, vb, o, lse, do, qp, kp)
    rq, rk, rv = oracle.attention_block_backward(do, q, kb, vb, o, lse, qp, kp)
    got = [t.cpu().numpy() for t in (dq, dk, dv)]
    # (query, key) pairs of the block that take part: key position <= query
    # position, and the query sees some key (finite log-sum-exp)
    pairs = ((kp + np.arange(nk))[None, :] <= (qp + np.arange(nq))[:, None])[None, None] & \
        np.isfinite(lse)[..., None]
    unseen = {"dq": ~pairs.any(axis=-1), "dk": ~pairs.any(axis=-2), "dv": ~pairs.any(axis=-2)}
    for name, g, r in zip(("dq", "dk", "dv"), got, (rq, rk, rv)):
        assert np.isfinite(g).all(), name
        assert np.all(g[unseen[name]] == 0), name
        assert _rel(g, r) <= TOL, (name, _rel(g, r))


def test_block_backward_accumulates():
    """accumulate = 1 adds each result to what the buffers hold."""
    torch = _torch()
    b, n, d, nq, nk, qp, kp = 1, 2, 128, 100, 90, 60, 20
    q, k, v, do = _inputs(b, n, d, nq, nk, seed=5)
    o, lse = oracle.attention_block(q, k, v, qp, kp)
    first = [t.clone() for t in _bwd_gpu(q, k, v, o, lse, do, qp, kp)]
    outs = tuple(t.clone() for t in first)
    _bwd_gpu(q, k, v, o, lse, do, qp, kp, outs=outs, accumulate=True)
    for a, s in zip(first, outs):
        assert torch.equal(a * 2, s)


@pytest.mark.parametrize("d", [64, 128])
def test_ring_backward_equals_causal_backward(d):
    """Each device's queries against every device's block, in ring order: the
    forward merged on the GPU (block attention and merge), then the per-block
    backward with the merged result, dQ summed over the blocks on the GPU
    (accumulate) and each block's dK, dV kept; against the causal backward of
    the device's queries over all keys."""
    torch = _torch()
    devices, per, b, n = 4, 96, 1, 4
    L = devices * per
    q_all, k_all, v_all, do_all = _inputs(b, n, d, L, L, seed=41 + d)
    for me in range(devices):
        print("[case] ring backward d=%d device %d" % (d, me), flush=True)
        qs, dos = q_all[:, :, me * per:(me + 1) * per], do_all[:, :, me * per:(me + 1) * per]
        order = [(me - step) % devices for step in range(devices)]
        acc = None
        tq = _dev(qs, torch.bfloat16)
        for src in order:
            ks, vs = k_all[:, :, src * per:(src + 1) * per], v_all[:, :, src * per:(src + 1) * per]
            o = torch.empty((b, n, per, d), dtype=torch.float32, device="cuda")
            lse = torch.empty((b, n, per), dtype=torch.float32, device="cuda")
            shape = abi.tp_attn_block_shape(b, n, d, per, per, me * per, src * per)
            tk, tv = _dev(ks, torch.bfloat16), _dev(vs, torch.bfloat16)
            abi.tp_attn_block_fwd(shape, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  _stream())
            if acc is None:
                acc = (o, lse)
            else:
                abi.tp_attn_merge(shape, acc[0].data_ptr(), acc[1].data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  acc[0].data_ptr(), acc[1].data_ptr(), _stream())
        torch.cuda.synchronize()
        mo, ml = acc[0].cpu().numpy(), acc[1].cpu().numpy()
        dq = torch.zeros((b, n, per, d), dtype=torch.float32, device="cuda")
        dk = np.zeros((b, n, L, d))
        dv = np.zeros((b, n, L, d))
        for src in order:
            ks, vs = k_all[:, :, src * per:(src + 1) * per], v_all[:, :, src * per:(src + 1) * per]
            # dK, dV of each block start at zero: the call adds (dQ sums over blocks)
            outs = (dq, torch.zeros((b, n, per, d), dtype=torch.float32, device="cuda"),
                    torch.zeros((b, n, per, d), dtype=torch.float32, device="cuda"))
            _bwd_gpu(qs, ks, vs, mo, ml, dos, me * per, src * per, outs=outs, accumulate=src != order[0])
            dk[:, :, src * per:(src + 1) * per] = outs[1].cpu().numpy()
            dv[:, :, src * per:(src + 1) * per] = outs[2].cpu().numpy()
        ro, rp, rl = oracle.causal_attention(qs, k_all[:, :, :(me + 1) * per], v_all[:, :, :(me + 1) * per],
                                             q_start=me * per)
        rq, rk, rv = oracle.causal_attention_backward(dos, qs, k_all[:, :, :(me + 1) * per],
                                                      v_all[:, :, :(me + 1) * per], rp, ro)
        assert _rel(dq.cpu().numpy(), rq) <= TOL
        assert _rel(dk[:, :, :(me + 1) * per], rk) <= TOL
        assert _rel(dv[:, :, :(me + 1) * per], rv) <= TOL
        assert np.all(dk[:, :, (me + 1) * per:] == 0) and np.all(dv[:, :, (me + 1) * per:] == 0)


def test_long_context_block_backward_sampled():
    """The benchmark's shapes (4096 queries of 12 heads of 128 against an
    earlier 4096-key block, and against their own diagonal block), with the
    block as the only one (its own forward is the merged result): sampled
    query rows of dQ and key rows of dK, dV against the oracle."""
    b, n, d, L = 1, 12, 128, 4096
    rng = np.random.default_rng(17)
    for qp, kp in [(4096, 0), (4096, 4096)]:
        print("[case] long block backward q_pos0=%d k_pos0=%d" % (qp, kp), flush=True)
        q, k, v, do = _inputs(b, n, d, L, L, seed=qp + kp + 3)
        o, lse = oracle.attention_block(q, k, v, qp, kp)
        dq, dk, dv = (t.cpu().numpy() for t in _bwd_gpu(q, k, v, o, lse, do, qp, kp))
        rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, L - 1], rng.integers(0, L, 16)]))
        for r in rows:
            rq, _, _ = oracle.attention_block_backward(do[:, :, r:r + 1], q[:, :, r:r + 1], k, v, o[:, :, r:r + 1],
                                                       lse[:, :, r:r + 1], qp + r, kp)
            assert _rel(dq[:, :, r:r + 1], rq) <= TOL, ("dq", r)
            _, rk, rv = oracle.attention_block_backward(do, q, k[:, :, r:r + 1], v[:, :, r:r + 1], o, lse, qp,
                                                        kp + r)
            assert _rel(dk[:, :, r:r + 1], rk) <= TOL, ("dk", r)
            assert _rel(dv[:, :, r:r + 1], rv) <= TOL, ("dv", r)
