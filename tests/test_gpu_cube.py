"""GPU parity of one device's cube-partition ops through the C-ABI against
the fp64 oracle: the three product forms (fp32 results of bf16 operands:
1e-4 of the largest magnitude), also with every GEMM tile configuration
forced, the elementwise bias/GELU and GELU-backward
steps (bf16 results: 2e-2), the FFN block assembled from two devices'
local products with the reduction before bias and GELU, forward and
backward, and sampled rows of the full-size backward products."""
import numpy as np
import pytest

import oracle
from oracle import cube as OC
from token_transformer_layer_amd import abi, synth

pytestmark = pytest.mark.gpu

FORMS = {abi.TP_CUBE_AB: "ab", abi.TP_CUBE_ABT: "abt", abi.TP_CUBE_ATB: "atb"}


def _t(a, dt):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(dt)


def _st():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _rel(got, ref):
    got = got.float().cpu().numpy() if hasattr(got, "cpu") else got
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def _shapes(form, M, N, K):
    return {"ab": ((M, K), (K, N)), "abt": ((M, K), (N, K)), "atb": ((K, M), (K, N))}[form]


def gpu_matmul(form_id, a, b, M, N, K, c=None, accumulate=False):
    import torch
    ta, tb = _t(a, torch.bfloat16), _t(b, torch.bfloat16)
    if c is None:
        c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    abi.tp_cube_matmul(form_id, M, N, K, ta.data_ptr(), tb.data_ptr(), c.data_ptr(), accumulate, _st())
    # the operands' memory may be reused by later allocations on this stream
    # only after the product has read it: torch's allocator orders reuse on
    # the stream, so dropping them here is safe
    return c


@pytest.mark.parametrize("form_id", list(FORMS))
@pytest.mark.parametrize("M,N,K", [(200, 136, 264), (8, 8, 8), (1032, 520, 2056)])
def test_cube_forms(form_id, M, N, K):
    import torch
    form = FORMS[form_id]
    print("[case] cube form %s M=%d N=%d K=%d" % (form, M, N, K), flush=True)
    rng = np.random.default_rng(M + N + K + form_id)
    sa, sb = _shapes(form, M, N, K)
    a, b = synth.round_bf16(rng.normal(size=sa)), synth.round_bf16(rng.normal(size=sb))
    ref = OC.cube_matmul(form, a, b)
    c = gpu_matmul(form_id, a, b, M, N, K)
    torch.cuda.synchronize()
    assert _rel(c, ref) <= 1e-4
    gpu_matmul(form_id, a, b, M, N, K, c=c, accumulate=True)
    torch.cuda.synchronize()
    assert _rel(c, 2 * ref) <= 1e-4


@pytest.mark.parametrize("tile", range(7))
@pytest.mark.parametrize("form_id", list(FORMS))
@pytest.mark.parametrize("M,N,K", [(264, 392, 328), (520, 200, 1032), (264, 392, 512)])
def test_cube_forms_forced_tiles(tile, form_id, M, N, K):
    """Every GEMM tile configuration (tp_gemm_force_tile) in the three operand
    layouts on ragged shapes: partial edge tiles in M and N, with K not a
    multiple of the 32- or 64-deep K-tiles (every load tested against the end
    of K) or a whole number of them (load offsets fixed per lane)."""
    import torch
    form = FORMS[form_id]
    print("[case] cube form %s tile %d M=%d N=%d K=%d" % (form, tile, M, N, K), flush=True)
    rng = np.random.default_rng(1000 * tile + M + N + K + form_id)
    sa, sb = _shapes(form, M, N, K)
    a, b = synth.round_bf16(rng.normal(size=sa)), synth.round_bf16(rng.normal(size=sb))
    ref = OC.cube_matmul(form, a, b)
    abi.tp_gemm_force_tile(tile)
    try:
        c = gpu_matmul(form_id, a, b, M, N, K)
        torch.cuda.synchronize()
        assert _rel(c, ref) <= 1e-4
        gpu_matmul(form_id, a, b, M, N, K, c=c, accumulate=True)
        torch.cuda.synchronize()
        assert _rel(c, 2 * ref) <= 1e-4
    finally:
        abi.tp_gemm_force_tile(-1)


def test_cube_elementwise_steps():
    import torch
    rng = np.random.default_rng(9)
    rows, n = 300, 520
    zs = rng.normal(size=(rows, n)) * 2
    bias = synth.round_bf16(rng.normal(size=n) * 0.3)
    tz, th = (torch.empty((rows, n), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    # every device tensor stays referenced while the library uses its memory
    tzs, tbias = _t(zs, torch.float32), _t(bias, torch.bfloat16)
    abi.tp_cube_bias_gelu(rows, n, tzs.data_ptr(), tbias.data_ptr(), tz.data_ptr(), th.data_ptr(), _st())
    torch.cuda.synchronize()
    rz, rh = OC.cube_bias_gelu(zs.astype(np.float32), bias)
    assert _rel(tz, rz) <= 2e-2 and _rel(th, rh) <= 2e-2
    dh = rng.normal(size=(rows, n))
    tdz = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
    db = torch.full((n,), 5.0, dtype=torch.float32, device="cuda")
    work = torch.empty(abi.tp_cube_work_bytes(rows, n), dtype=torch.uint8, device="cuda")
    zb = tz.float().cpu().numpy()  # the stored bf16 Z
    tdh = _t(dh, torch.float32)
    for acc in (False, True):
        abi.tp_cube_gelu_backward(rows, n, tdh.data_ptr(), tz.data_ptr(), tdz.data_ptr(), db.data_ptr(), acc,
                                  work.data_ptr(), _st())
    torch.cuda.synchronize()
    rdz, rdb = OC.cube_gelu_backward(dh.astype(np.float32), zb)
    assert _rel(tdz, rdz) <= 2e-2
    assert _rel(db, 2 * rdb) <= 2e-2


def test_cube_ffn_two_devices():
    """FFN block over p = 2 devices along each reduction: local products on
    the GPU, the partial sums reduced (the collective, here a sum), then
    bias and GELU; backward with the same forms."""
    import torch
    rng = np.random.default_rng(12)
    rows, hid, f, p = 136, 256, 512, 2
    x = synth.round_bf16(rng.normal(size=(rows, hid)))
    w1 = synth.round_bf16(rng.normal(size=(f, hid)) * 0.05)
    b1 = synth.round_bf16(rng.normal(size=f) * 0.1)
    w2 = synth.round_bf16(rng.normal(size=(hid, f)) * 0.05)
    dout = synth.round_bf16(rng.normal(size=(rows, hid)))
    hs, fs = np.array_split(np.arange(hid), p), np.array_split(np.arange(f), p)
    # forward: Z partials per device, reduced, bias + GELU
    zsum = sum(gpu_matmul(abi.TP_CUBE_ABT, x[:, c], w1[:, c], rows, f, len(c)) for c in hs)
    tz, th = (torch.empty((rows, f), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    tb1 = _t(b1, torch.bfloat16)
    abi.tp_cube_bias_gelu(rows, f, zsum.data_ptr(), tb1.data_ptr(), tz.data_ptr(), th.data_ptr(), _st())
    hb = th.float().cpu().numpy()
    out = sum(gpu_matmul(abi.TP_CUBE_ABT, hb[:, c], w2[:, c], rows, hid, len(c)) for c in fs)
    # backward
    dh = torch.cat([gpu_matmul(abi.TP_CUBE_AB, dout, w2[:, c], rows, len(c), hid) for c in fs], dim=1).contiguous()
    tdz = torch.empty((rows, f), dtype=torch.bfloat16, device="cuda")
    db1 = torch.empty((f,), dtype=torch.float32, device="cuda")
    work = torch.empty(abi.tp_cube_work_bytes(rows, f), dtype=torch.uint8, device="cuda")
    abi.tp_cube_gelu_backward(rows, f, dh.data_ptr(), tz.data_ptr(), tdz.data_ptr(), db1.data_ptr(), False,
                              work.data_ptr(), _st())
    dzb = tdz.float().cpu().numpy()
    dw2 = torch.cat([gpu_matmul(abi.TP_CUBE_ATB, dout, hb[:, c], hid, len(c), rows) for c in fs], dim=1)
    dw1 = torch.cat([gpu_matmul(abi.TP_CUBE_ATB, dzb, x[:, c], f, len(c), rows) for c in hs], dim=1)
    dx = sum(gpu_matmul(abi.TP_CUBE_AB, dzb[:, c], w1[c, :], rows, hid, len(c)) for c in fs)
    torch.cuda.synchronize()
    # oracle: the unsharded block and its gradients
    r_out, r_g = OC.cube_ffn_devices(x, w1, b1, w2, dout, p=1)
    ref = dict(out=r_out, dw2=r_g["w2"], dw1=r_g["w1"], dx=r_g["x"], db1=r_g["b1"])
    got = dict(out=out, dw2=dw2, dw1=dw1, dx=dx, db1=db1)
    for k in ref:
        assert _rel(got[k], ref[k]) <= 2e-2, k


def test_cube_backward_full_size_sampled():
    """The C5 block's backward products at full size (rows 4096, hidden 6144,
    ffn 24576), checked on sampled output rows."""
    import torch
    c = synth.CUBE
    rng = np.random.default_rng(c.seed + 1)
    dout = synth.round_bf16(rng.normal(size=(c.rows, c.hidden)))
    h = synth.round_bf16(rng.normal(size=(c.rows, c.ffn)))
    w2 = synth.round_bf16(rng.normal(size=(c.hidden, c.ffn)) * 0.02)
    cases = [("dh = dout w2", abi.TP_CUBE_AB, dout, w2, c.rows, c.ffn, c.hidden),
             ("dw2 = dout^T h", abi.TP_CUBE_ATB, dout, h, c.hidden, c.ffn, c.rows)]
    for name, form_id, a, b, M, N, K in cases:
        print("[case] cube full size", name, flush=True)
        got = gpu_matmul(form_id, a, b, M, N, K)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        rows = np.unique(np.concatenate([[0, 1, 127, 128, M - 1], rng.integers(0, M, 12)]))
        form = FORMS[form_id]
        asub = a[rows] if form == "ab" else a[:, rows]
        ref = OC.cube_matmul(form, asub, b)
        assert _rel(got[rows], ref) <= 1e-4, name
