"""GPU parity of the LayerNorm entry points (tp_layernorm_fwd / tp_layernorm_bwd)
against the oracle's layer_norm and layer_norm_backward, over widths and row
counts that take every form of the kernels: rows of at most 2048 columns one
to a wave (fewer rows than a workgroup's four waves, ragged counts, more
workgroups than rows need so that some have no row), wider rows one to a
workgroup, bf16 and fp32 storage.  The parameter gradients are row sums
("Maximizing Parallelism in Distributed Training for Huge Neural Networks",
section 3.1.3), stored and then accumulated."""
import numpy as np
import pytest

import oracle
from tests import gpu_harness as H
from token_transformer_layer_amd import abi
from token_transformer_layer_amd.synth import round_bf16

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
EPS = 1e-5

# (hidden, heads, head_dim, rows, dtype)
CASES = [
    (64, 1, 64, 1, "f32"),
    (64, 1, 64, 3, "bf16"),
    (640, 10, 64, 5, "bf16"),
    (1024, 8, 128, 37, "bf16"),
    (2048, 16, 128, 301, "bf16"),
    (2048, 32, 64, 9, "f32"),
    (2112, 33, 64, 7, "bf16"),
    (12288, 96, 128, 3, "bf16"),
]


def _dev(a, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda").to(torch.bfloat16 if dtype == "bf16" else torch.float32)


@pytest.mark.parametrize("h,heads,hd,rows,dtype", CASES,
                         ids=["%d-%dx%d-%s" % (h, r, hd, dt) for h, _, hd, r, dt in CASES])
def test_layernorm_forward_backward(h, heads, hd, rows, dtype):
    import torch
    from token_transformer_layer_amd.shard import stream_handle
    print("[case] layernorm h=%d rows=%d %s" % (h, rows, dtype), flush=True)
    rng = np.random.default_rng(4000 + h + rows)
    rnd = round_bf16 if dtype == "bf16" else (lambda a: np.asarray(a, dtype=np.float32))
    x = rnd(rng.standard_normal((rows, h)) * 2.0 + 0.5)
    gamma = rnd(1.0 + 0.1 * rng.standard_normal(h))
    beta = rnd(0.1 * rng.standard_normal(h))
    resid = rnd(rng.standard_normal((rows, h)))
    du = rng.standard_normal((rows, h)).astype(np.float32)
    cfg = abi.tp_shard_cfg(h, heads, hd, 8, 1, 1, rows, abi.TP_BF16 if dtype == "bf16" else abi.TP_F32, EPS)
    st = stream_handle()
    xt, gt, bt, rt = _dev(x, dtype), _dev(gamma, dtype), _dev(beta, dtype), _dev(resid, dtype)
    dut = torch.from_numpy(du).cuda()
    u = torch.empty_like(xt)
    dx = torch.empty_like(xt)
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty_like(mean)
    dg = torch.full((h,), float("nan"), dtype=torch.float32, device="cuda")
    db = torch.full_like(dg, float("nan"))
    work = torch.empty(abi.tp_layernorm_work_bytes(cfg, rows), dtype=torch.uint8, device="cuda")

    abi.tp_layernorm_fwd(cfg, rows, xt.data_ptr(), gt.data_ptr(), bt.data_ptr(), u.data_ptr(), mean.data_ptr(),
                         rstd.data_ptr(), st)
    abi.tp_layernorm_bwd(cfg, rows, dut.data_ptr(), rt.data_ptr(), xt.data_ptr(), gt.data_ptr(), mean.data_ptr(),
                         rstd.data_ptr(), dx.data_ptr(), dg.data_ptr(), db.data_ptr(), False, work.data_ptr(), st)
    torch.cuda.synchronize()
    got = dict(u=u.float().cpu().numpy(), mean=mean.cpu().numpy(), rstd=rstd.cpu().numpy(),
               dx=dx.float().cpu().numpy(), dgamma=dg.cpu().numpy(), dbeta=db.cpu().numpy())
    # accumulate = 1 adds this call's shares to the stored ones
    abi.tp_layernorm_bwd(cfg, rows, dut.data_ptr(), rt.data_ptr(), xt.data_ptr(), gt.data_ptr(), mean.data_ptr(),
                         rstd.data_ptr(), dx.data_ptr(), dg.data_ptr(), db.data_ptr(), True, work.data_ptr(), st)
    torch.cuda.synchronize()

    u_ref, m_ref, r_ref = oracle.layer_norm(x, gamma, beta, EPS)
    dx_ref, dg_ref, db_ref = oracle.layer_norm_backward(du, x, gamma, m_ref, r_ref)
    ref = dict(u=u_ref, mean=m_ref, rstd=r_ref, dx=dx_ref + resid, dgamma=dg_ref, dbeta=db_ref)
    tol = TOL[dtype]
    for k in ref:
        # statistics are fp32 in both storage types
        t = 1e-4 if k in ("mean", "rstd") else tol
        e = H.max_rel(got[k], ref[k])
        assert e <= t, (k, e)
    assert H.max_rel(dg.cpu().numpy(), 2 * dg_ref) <= tol
    assert H.max_rel(db.cpu().numpy(), 2 * db_ref) <= tol
