"""Throughput of one rank's share of a tensor-parallel GPT decoder layer, run
over token slices, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

One step = every phase of the layer shard over one batch: forward attention
and MLP blocks, the two residual combines a caller runs after its
all-reduces, and the backward MLP, attention and LN1 phases (the reduced
gradients are this rank's own partials: on one GPU the all-reduce is the
identity).  The headline runs each phase as one library call over all
slices of the partition (position-wise products batch the slices' rows;
attention covers each query against its own prefix).  A second figure runs
one call per slice in slice order (backward in reverse), as a pipeline stage
would receive them.

Inputs are synthetic and seeded (token_transformer_layer_amd.synth): x, dY
~ N(0, 1), linear weights ~ N(0, 0.02), biases 0, gamma 1, beta 0, all bf16.
Each gradient is overwritten by the call that first produces it in a step
(accumulate = 0), so no zeroing pass is needed.  In the per-slice schedule
the backward runs the data phases per slice (reverse order) and every weight
gradient in one call over all slices afterwards.

Prints ONE JSON line.  value = algorithmic fwd+bwd TFLOP/s of the step:
GEMMs 3 x 2 T h (4 h_t + 2 f_t) plus causal attention 3 x 2 b h_t s (s+1)
flops, over the measured time per step (K timed steps after W warm-up steps,
HIP events on the launch stream); an event at the end of each timed step gives
the median and minimum step times beside that average.  Per-kernel durations (the `kernels` table
and the roofline of the dominant kernel) come from a second pass of K steps
with the library's event trace on, whose step time is reported as
`traced_step_ms` (the events between launches cost the step about 6%).
"""
import argparse
import glob
import json
import os
import re
import statistics
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published


def step_flops(shape):
    """Algorithmic flops of one fwd+bwd step of the shard (see module doc)."""
    T, h = shape.batch * shape.seq, shape.hidden
    ht, ft = h // shape.tp, shape.ffn // shape.tp
    gemm = 3 * 2.0 * T * h * (4 * ht + 2 * ft)
    attn = 3 * 2.0 * shape.batch * ht * shape.seq * (shape.seq + 1)
    return gemm, attn


def make_step(layer, bufs, mode):
    from token_transformer_layer_amd import abi
    M = len(layer.shape.slices)
    groups = [(0, M)] if mode == "whole" else [(j, j + 1) for j in range(M)]
    sh = layer.shape
    b = sh.batch
    bounds = layer.bounds
    x, dy, hm, y, dh, dx = bufs["x"], bufs["dy"], bufs["h_mid"], bufs["y"], bufs["dh"], bufs["dx"]
    pa, pm, pu2, pu1 = bufs["p_attn"], bufs["p_mlp"], bufs["p_du2"], bufs["p_du1"]
    b_o, b2 = layer.p["b_o"], layer.p["b2"]

    def step():
        layer.kv.filled = 0
        layer.kvg.done_from = sh.seq
        for j0, j1 in groups:
            o0, o1 = bounds[j0], bounds[j1]
            layer.fwd(abi.TP_FWD_ATTN, j0, j1, x, pa)
            layer.combine(x[o0:], pa[o0:], b_o, hm[o0:], rows=(o1 - o0) * b)
            layer.fwd(abi.TP_FWD_MLP, j0, j1, hm, pm)
            layer.combine(hm[o0:], pm[o0:], b2, y[o0:], rows=(o1 - o0) * b)
        if mode == "whole":
            # one call per phase: every gradient is produced once, so the
            # calls overwrite the gradient buffers (no zeroing needed)
            layer.bwd(abi.TP_BWD_MLP, 0, M, dy=dy, partial_out=pu2, accumulate=False)
            layer.bwd(abi.TP_BWD_ATTN, 0, M, dy=dy, ln_in=hm, reduced=pu2, partial_out=pu1, dh=dh,
                      accumulate=False)
            layer.bwd(abi.TP_BWD_LN1, 0, M, ln_in=x, reduced=pu1, dh=dh, dx=dx, accumulate=False)
            return
        # per slice, in reverse: the data phases only; then every weight
        # gradient in one call over all slices
        first = True
        for j0, j1 in reversed(groups):
            layer.bwd(abi.TP_BWD_MLP_DATA, j0, j1, dy=dy, partial_out=pu2, accumulate=not first)
            layer.bwd(abi.TP_BWD_ATTN_DATA, j0, j1, dy=dy, ln_in=hm, reduced=pu2, partial_out=pu1, dh=dh,
                      accumulate=not first)
            layer.bwd(abi.TP_BWD_LN1, j0, j1, ln_in=x, reduced=pu1, dh=dh, dx=dx, accumulate=not first)
            first = False
        layer.bwd(abi.TP_BWD_WGRAD, 0, M, dy=dy, dh=dh, accumulate=False)
    return step


PEAK_CLOCK_MHZ = 2400.0       # the clock the published peak assumes


class ClockSampler:
    """Samples the graphics clock (MHz) that the amdgpu driver reports as
    current in the device's DPM table (sysfs `pp_dpm_sclk`, the line marked
    `*`) on a host thread, every `period` seconds between start() and stop().
    Only where the node shows exactly one GPU (else the card cannot be matched
    to the device and nothing is sampled)."""

    def __init__(self, period=0.002):
        files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = files[0] if len(files) == 1 else None
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._thread = None

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*mhz", line, re.IGNORECASE)
                    return float(m.group(1)) if m else None
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
            except OSError:
                return
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def start(self):
        if self.path:
            self._stop.clear()
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        if self._thread:
            self._stop.set()
            self._thread.join()
            self._thread = None

    def summary(self, source):
        if not self.samples:
            return None
        return dict(mean=round(statistics.fmean(self.samples), 1), min=min(self.samples), max=max(self.samples),
                    samples=len(self.samples), source=source)


def sustained_clock(torch, step, seconds=1.2, tail=0.6):
    """The graphics clock while `step` repeats back to back for `seconds`,
    sampled over the last `tail` seconds.  The driver's reading is a smoothed
    one that takes about a second to rise from idle (in a 64 ms timed region
    it reads 1.3-1.6 GHz while the step time equals that of runs where it
    reads 1.9 GHz), so it is taken here, after the timed steps, rather than
    during them."""
    clock = ClockSampler(period=0.005)
    if not clock.path:
        return None
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        if not clock._thread and time.perf_counter() - t0 >= seconds - tail:
            clock.start()
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    clock.stop()
    return clock.summary("amdgpu sysfs pp_dpm_sclk while the step repeats for %.1f s, last %.1f s" % (seconds, tail))


def time_steps(torch, step, steps, warmup, trace=False, per_step=None):
    """Average ms per step over `steps` steps after `warmup` untimed ones, the
    host's wall-clock ms per step, and the trace records (if `trace`).  With a
    list as `per_step`, an event marks the end of every step inside the timed
    region and the list receives each step's own duration in ms."""
    from token_transformer_layer_amd import abi
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if trace:
        abi.tp_trace_enable(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps)] if per_step is not None else []
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        step()
        if marks:
            marks[i].record()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if marks:
        per_step[:] = [(ev0 if i == 0 else marks[i - 1]).elapsed_time(m) for i, m in enumerate(marks)]
    recs = []
    if trace:
        recs = abi.tp_trace_read()
        abi.tp_trace_enable(False)
    return ev0.elapsed_time(ev1) / steps, wall / steps * 1e3, recs


def kernel_table(recs, steps):
    """Per kernel name: launches per step, ms per step, average ms per launch,
    algorithmic TFLOP/s and GB/s."""
    agg = {}
    for name, fl, by, ms in recs:
        a = agg.setdefault(name, [0, 0.0, 0.0, 0.0])
        a[0] += 1
        a[1] += fl
        a[2] += by
        a[3] += ms
    out = {}
    for name, (n, fl, by, ms) in sorted(agg.items(), key=lambda kv: -kv[1][3]):
        out[name] = dict(launches_per_step=n / steps, ms_per_step=round(ms / steps, 4),
                         avg_launch_ms=round(ms / n, 5),
                         tflops=round(fl / (ms * 1e-3) / 1e12, 1) if ms > 0 else None,
                         gbs=round(by / (ms * 1e-3) / 1e9, 1) if ms > 0 else None)
    return out


def cpu_baseline(shape, budget_slices):
    """The fp64 oracle on the host cores: one rank's fwd+bwd over the first
    `budget_slices` slices of the sequence (a prefix of the same workload),
    scaled to TFLOP/s by that sample's own algorithmic flops."""
    import oracle
    from tests import gpu_harness as H
    from token_transformer_layer_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    seq = int(sum(shape.slices[:budget_slices]))
    sample = shape.replace(seq=seq, slices=tuple(shape.slices[:budget_slices]))
    x, dy = synth.activations(sample)
    sp = synth.shard_params_direct(shape, "standard", 0)
    h_mid, du2, du1 = H.step_inputs(sample, shape.seed + 1)
    t0 = time.perf_counter()
    oracle.shard_layer_step(x, h_mid, dy, du2, du1, sp, sample.as_dict(), synth.slice_bounds(sample.slices))
    dt = time.perf_counter() - t0
    g, a = step_flops(sample)
    ncpu, model = host_cpu()
    return dict(value=round((g + a) / dt / 1e12, 5), unit="TFLOP/s", cores=threads, kind="oracle",
                sample="%d of %d token slices (positions 0-%d, batch %d) of the same shard, fp64 numpy, %.1f s"
                       % (budget_slices, len(shape.slices), seq - 1, shape.batch, dt),
                seconds=round(dt, 2), host_logical_cpus=ncpu, cpu_model=model,
                threads="%d BLAS threads (numpy's thread pool) on a host with %s logical CPUs" % (threads, ncpu))


def per_slice_figures(torch, layer, bufs, steps, warmup):
    """The pipeline-faithful schedule (one call per slice; backward data
    phases per slice in reverse, then every weight gradient in one call): its
    step time, and the HBM roofline of its 128-row products.  Every slice's
    forward products and backward input-gradient products read the whole
    shard's weights once, so a step streams 2 x slices x (weight bytes) from
    HBM; those products are the launches that split their reduction (the
    `_split` kernels and their reduction kernel), timed in a traced pass."""
    step = make_step(layer, bufs, "per-slice")
    ms, _, _ = time_steps(torch, step, steps, warmup)
    _, _, recs = time_steps(torch, step, steps, 1, trace=True)
    sh = layer.shape
    ht, ft = sh.hidden // sh.tp, sh.ffn // sh.tp
    weight_bytes = 2.0 * (3 * ht * sh.hidden + sh.hidden * ht + 2 * ft * sh.hidden)  # bf16 W_qkv, W_o, W1, W2
    streamed = 2.0 * len(sh.slices) * weight_bytes
    prod_ms = sum(r[3] for r in recs if r[0].endswith("_split") or r[0].startswith("splitk_reduce")) / steps
    g_fl, a_fl = step_flops(sh)
    achieved = streamed / (prod_ms * 1e-3) / 1e9 if prod_ms > 0 else None
    return dict(ms_per_step=round(ms, 4), tflops=round((g_fl + a_fl) / (ms * 1e-3) / 1e12, 1),
                roofline=dict(bound="hbm", unit="GB/s", peak=PEAK_HBM_GBS,
                              achieved=round(achieved, 1) if achieved else None,
                              frac=round(achieved / PEAK_HBM_GBS, 4) if achieved else None,
                              weight_bytes_per_step=streamed, products_ms_per_step=round(prod_ms, 4),
                              what="shard weights streamed by the per-slice 128-row products (forward and "
                                   "input-gradient, each slice reads every weight once) over those products' "
                                   "kernel time, traced pass"))


def config_step(torch, name, steps, warmup):
    """The whole-partition step of another workload's shard (same schedule
    as the headline): ms per step and algorithmic TFLOP/s."""
    from token_transformer_layer_amd import synth
    from token_transformer_layer_amd.shard import ShardLayer
    sh = synth.CONFIGS[name]
    x, dy = synth.activations(sh)
    L = ShardLayer(sh, synth.shard_params_direct(sh, "standard", 0))
    bufs = dict(x=L.act(x), dy=L.act(dy), h_mid=L.act(), y=L.act(), dh=L.act(), dx=L.act(), p_attn=L.f32(),
                p_mlp=L.f32(), p_du2=L.f32(), p_du1=L.f32())
    L.new_step()
    ms, _, _ = time_steps(torch, make_step(L, bufs, "whole"), steps, warmup)
    g_fl, a_fl = step_flops(sh)
    tf = (g_fl + a_fl) / (ms * 1e-3) / 1e12
    out = dict(ms_per_step=round(ms, 4), tflops=round(tf, 1), frac_of_bf16_peak=round(tf / PEAK_BF16_TFLOPS, 4),
               gflop_per_step=round((g_fl + a_fl) / 1e9, 1),
               shape="h %d, %d x %d heads, t %d, batch %d, seq %d, slices %s" % (
                   sh.hidden, sh.heads, sh.head_dim, sh.tp, sh.batch, sh.seq, list(sh.slices)))
    del L, bufs
    torch.cuda.empty_cache()
    return out


def host_cpu():
    """The host's logical CPU count and model name (from /proc/cpuinfo)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def cube_block(torch, steps, warmup):
    """The cube-partition FFN block (X 4096x6144, W1 6144->24576, W2
    24576->6144, bf16): forward TFLOP/s."""
    from token_transformer_layer_amd import abi, synth
    c = synth.CUBE
    dev = torch.device("cuda")
    g = torch.Generator(device="cpu").manual_seed(c.seed)
    x = (torch.randn((c.rows, c.hidden), generator=g)).to(dev, torch.bfloat16)
    w1 = (torch.randn((c.ffn, c.hidden), generator=g) * 0.02).to(dev, torch.bfloat16)
    w2 = (torch.randn((c.hidden, c.ffn), generator=g) * 0.02).to(dev, torch.bfloat16)
    b1 = torch.zeros(c.ffn, dtype=torch.bfloat16, device=dev)
    hb = torch.empty((c.rows, c.ffn), dtype=torch.bfloat16, device=dev)
    out = torch.empty((c.rows, c.hidden), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream().cuda_stream

    def step():
        abi.tp_cube_ffn_block(c.rows, c.hidden, c.ffn, x.data_ptr(), w1.data_ptr(), b1.data_ptr(), w2.data_ptr(),
                              hb.data_ptr(), out.data_ptr(), st)
    ms, _, _ = time_steps(torch, step, steps, warmup)
    fl = 4.0 * c.rows * c.hidden * c.ffn
    return dict(ms=round(ms, 4), tflops=round(fl / (ms * 1e-3) / 1e12, 1))


def clock_probe(torch, seconds=1.6, tail=0.8):
    """Throughput and sustained graphics clock of single kernels repeated back
    to back: the 175B shard's FC1 weight-gradient product (A^T B, 6144 x 12288
    x 2048), its FC2-shaped forward product (A B^T, 2048 x 6144 x 12288) and a
    long-context attention block (12 heads x 128, 4096 queries against an
    earlier 4096-key block).  One JSON line per kernel; the clock is sampled
    over the last `tail` seconds, and so is the time per call."""
    from token_transformer_layer_amd import abi
    st = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device="cpu").manual_seed(1007)

    def run(name, fn, flops):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        clock = ClockSampler(period=0.005)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0, n, timing = time.perf_counter(), 0, False
        while time.perf_counter() - t0 < seconds:
            if not timing and time.perf_counter() - t0 >= seconds - tail:
                torch.cuda.synchronize()
                clock.start()
                e0.record()
                timing, n = True, 0
            for _ in range(4):
                fn()
            n += 4
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        clock.stop()
        ms = e0.elapsed_time(e1) / n
        tf = flops / (ms * 1e-3) / 1e12
        clk = clock.summary("amdgpu sysfs pp_dpm_sclk over the last %.1f s of %.1f s" % (tail, seconds))
        rec = dict(kernel=name, ms=round(ms, 4), tflops=round(tf, 1), frac=round(tf / PEAK_BF16_TFLOPS, 4),
                   gfx_clock_mhz=clk)
        if clk:
            rec["frac_at_measured_clock"] = round(tf / (PEAK_BF16_TFLOPS * clk["mean"] / PEAK_CLOCK_MHZ), 4)
        print(json.dumps(rec), flush=True)

    for name, form, (M, N, K) in [("weight-gradient product 6144x12288x2048 (A^T B)", abi.TP_CUBE_ATB, (6144, 12288, 2048)),
                                  ("forward product 2048x6144x12288 (A B^T)", abi.TP_CUBE_ABT, (2048, 6144, 12288))]:
        ashape = (K, M) if form == abi.TP_CUBE_ATB else (M, K)
        bshape = (K, N) if form == abi.TP_CUBE_ATB else (N, K)
        a = torch.randn(ashape, generator=g).to("cuda", torch.bfloat16)
        b = torch.randn(bshape, generator=g).to("cuda", torch.bfloat16)
        c = torch.empty((M, N), dtype=torch.float32, device="cuda")
        run(name, lambda: abi.tp_cube_matmul(form, M, N, K, a.data_ptr(), b.data_ptr(), c.data_ptr(), 0, st),
            2.0 * M * N * K)
        del a, b, c
    bq, n, d, L = 1, 12, 128, 4096
    q, k, v = [torch.randn((bq, n, L, d), generator=g).to("cuda", torch.bfloat16) for _ in range(3)]
    o = torch.empty((bq, n, L, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((bq, n, L), dtype=torch.float32, device="cuda")
    shape = abi.tp_attn_block_shape(bq, n, d, L, L, L, 0)
    run("attention block 12x128, 4096 queries x 4096 earlier keys",
        lambda: abi.tp_attn_block_fwd(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      st), 4.0 * d * L * L * n * bq)


def sequence_parallel_step(torch, layer, bufs, steps, warmup):
    """One rank's step in the sequence-parallel form: LayerNorm, its backward
    and the residual combines on the rank's 1/t shard of the rows, the
    products and attention over all rows (the all-gathers and
    reduce-scatters between them belong to the caller and are not run on
    one GPU).  Same algorithmic flops as the headline step."""
    from token_transformer_layer_amd import abi
    sh = layer.shape
    b, h = sh.batch, sh.hidden
    T = sh.seq * b
    rows = T // sh.tp
    st = torch.cuda.current_stream().cuda_stream
    M = len(sh.slices)
    x, dy, hm, y, dh, dx = (bufs[k] for k in ("x", "dy", "h_mid", "y", "dh", "dx"))
    pa, pm, pu2, pu1 = (bufs[k] for k in ("p_attn", "p_mlp", "p_du2", "p_du1"))
    u1, u2 = layer.act(), layer.act()
    f32 = lambda n: torch.zeros(n, dtype=torch.float32, device="cuda")  # noqa: E731
    mu1, rs1, mu2, rs2 = f32(rows), f32(rows), f32(rows), f32(rows)
    lg = [f32(h) for _ in range(4)]
    work = torch.empty(abi.tp_layernorm_work_bytes(layer.cfg, rows), dtype=torch.uint8, device="cuda")
    P = layer.p
    cfg = layer.cfg

    def step():
        layer.kv.filled = 0
        layer.kvg.done_from = sh.seq
        abi.tp_layernorm_fwd(cfg, rows, x.data_ptr(), P["ln1_g"].data_ptr(), P["ln1_b"].data_ptr(), u1.data_ptr(),
                             mu1.data_ptr(), rs1.data_ptr(), st)
        layer.fwd(abi.TP_FWD_ATTN_SP, 0, M, u1, pa)
        abi.tp_residual_combine(cfg, rows, x.data_ptr(), pa.data_ptr(), P["b_o"].data_ptr(), hm.data_ptr(), st)
        abi.tp_layernorm_fwd(cfg, rows, hm.data_ptr(), P["ln2_g"].data_ptr(), P["ln2_b"].data_ptr(), u2.data_ptr(),
                             mu2.data_ptr(), rs2.data_ptr(), st)
        layer.fwd(abi.TP_FWD_MLP_SP, 0, M, u2, pm)
        abi.tp_residual_combine(cfg, rows, hm.data_ptr(), pm.data_ptr(), P["b2"].data_ptr(), y.data_ptr(), st)
        layer.bwd(abi.TP_BWD_MLP, 0, M, dy=dy, partial_out=pu2, accumulate=False)
        abi.tp_layernorm_bwd(cfg, rows, pu2.data_ptr(), dy.data_ptr(), hm.data_ptr(), P["ln2_g"].data_ptr(),
                             mu2.data_ptr(), rs2.data_ptr(), dh.data_ptr(), lg[0].data_ptr(), lg[1].data_ptr(), False,
                             work.data_ptr(), st)
        layer.bwd(abi.TP_BWD_ATTN_SP, 0, M, dy=dy, partial_out=pu1, dh=dh, accumulate=False)
        abi.tp_layernorm_bwd(cfg, rows, pu1.data_ptr(), dh.data_ptr(), x.data_ptr(), P["ln1_g"].data_ptr(),
                             mu1.data_ptr(), rs1.data_ptr(), dx.data_ptr(), lg[2].data_ptr(), lg[3].data_ptr(), False,
                             work.data_ptr(), st)
    ms, _, _ = time_steps(torch, step, steps, warmup)
    g_fl, a_fl = step_flops(sh)
    layer.new_step()
    return dict(ms_per_step=round(ms, 4), tflops=round((g_fl + a_fl) / (ms * 1e-3) / 1e12, 1),
                shard_rows=rows, collectives="not run (one GPU)")


def cube_backward(torch, steps, warmup):
    """The cube-partition FFN block's backward at the same shapes (dH = dOut
    W2, dZ = dH GELU'(Z) with the bias gradient, dW2 = dOut^T H,
    dW1 = dZ^T X, dX = dZ W1): TFLOP/s of its four products."""
    from token_transformer_layer_amd import abi, synth
    c = synth.CUBE
    g = torch.Generator(device="cpu").manual_seed(c.seed + 2)
    bf = torch.bfloat16
    x, dout = [torch.randn(s, generator=g).to("cuda", bf) for s in ((c.rows, c.hidden), (c.rows, c.hidden))]
    w1 = (torch.randn((c.ffn, c.hidden), generator=g) * 0.02).to("cuda", bf)
    w2 = (torch.randn((c.hidden, c.ffn), generator=g) * 0.02).to("cuda", bf)
    z, h = [torch.randn((c.rows, c.ffn), generator=g).to("cuda", bf) for _ in range(2)]
    dh = torch.empty((c.rows, c.ffn), dtype=torch.float32, device="cuda")
    dz = torch.empty((c.rows, c.ffn), dtype=bf, device="cuda")
    db1 = torch.empty((c.ffn,), dtype=torch.float32, device="cuda")
    dw1 = torch.empty((c.ffn, c.hidden), dtype=torch.float32, device="cuda")
    dw2 = torch.empty((c.hidden, c.ffn), dtype=torch.float32, device="cuda")
    dx = torch.empty((c.rows, c.hidden), dtype=torch.float32, device="cuda")
    work = torch.empty(abi.tp_cube_work_bytes(c.rows, c.ffn), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def step():
        abi.tp_cube_matmul(abi.TP_CUBE_AB, c.rows, c.ffn, c.hidden, dout.data_ptr(), w2.data_ptr(), dh.data_ptr(),
                           False, st)
        abi.tp_cube_gelu_backward(c.rows, c.ffn, dh.data_ptr(), z.data_ptr(), dz.data_ptr(), db1.data_ptr(), False,
                                  work.data_ptr(), st)
        abi.tp_cube_matmul(abi.TP_CUBE_ATB, c.hidden, c.ffn, c.rows, dout.data_ptr(), h.data_ptr(), dw2.data_ptr(),
                           False, st)
        abi.tp_cube_matmul(abi.TP_CUBE_ATB, c.ffn, c.hidden, c.rows, dz.data_ptr(), x.data_ptr(), dw1.data_ptr(),
                           False, st)
        abi.tp_cube_matmul(abi.TP_CUBE_AB, c.rows, c.hidden, c.ffn, dz.data_ptr(), w1.data_ptr(), dx.data_ptr(),
                           False, st)
    ms, _, _ = time_steps(torch, step, steps, warmup)
    fl = 8.0 * c.rows * c.hidden * c.ffn
    return dict(ms=round(ms, 4), tflops=round(fl / (ms * 1e-3) / 1e12, 1))


def ring_block(torch, steps, warmup):
    """Attention over key/value blocks (long-context shape: 4096 queries of 12
    heads of 128 against a 4096-key block of an earlier device, and against
    their own diagonal block), its per-block backward, and the merge of two
    partial results."""
    from token_transformer_layer_amd import abi, synth
    b, n, d, L = 1, 12, 128, 4096
    g = torch.Generator(device="cpu").manual_seed(1006)
    q, k, v = [torch.randn((b, n, L, d), generator=g).to("cuda", torch.bfloat16) for _ in range(3)]
    o = torch.empty((b, n, L, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((b, n, L), dtype=torch.float32, device="cuda")
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    st = torch.cuda.current_stream().cuda_stream
    out = {}
    for name, qp, kp, pairs in [("off_diagonal", L, 0, float(L) * L), ("diagonal", L, L, L * (L + 1) / 2.0)]:
        shape = abi.tp_attn_block_shape(b, n, d, L, L, qp, kp)

        def step():
            abi.tp_attn_block_fwd(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), st)
        ms, _, _ = time_steps(torch, step, steps, warmup)
        tf = 4.0 * d * pairs * b * n / (ms * 1e-3) / 1e12
        out[name] = dict(ms=round(ms, 4), tflops=round(tf, 1), frac=round(tf / PEAK_BF16_TFLOPS, 4))
    # the per-block backward (dQ share, dK, dV) of the same blocks, each taken
    # as the only block (its own forward is the merged result)
    do = torch.randn((b, n, L, d), generator=g).to("cuda", torch.bfloat16)
    dq = torch.empty((b, n, L, d), dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)
    for name, qp, kp, pairs in [("backward_off_diagonal", L, 0, float(L) * L),
                                ("backward_diagonal", L, L, L * (L + 1) / 2.0)]:
        shape = abi.tp_attn_block_shape(b, n, d, L, L, qp, kp)
        abi.tp_attn_block_fwd(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), st)
        work = torch.empty(abi.tp_attn_block_bwd_work_bytes(shape), dtype=torch.uint8, device="cuda")

        def bstep():
            abi.tp_attn_block_bwd(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), False, work.data_ptr(),
                                  st)
        ms, _, _ = time_steps(torch, bstep, steps, warmup)
        tf = 8.0 * d * pairs * b * n / (ms * 1e-3) / 1e12  # algorithmic: twice the forward's 4 d per pair
        out[name] = dict(ms=round(ms, 4), tflops=round(tf, 1), frac=round(tf / PEAK_BF16_TFLOPS, 4))
    shape = abi.tp_attn_block_shape(b, n, d, L, L, 0, 0)

    def merge():
        abi.tp_attn_merge(shape, o.data_ptr(), lse.data_ptr(), o2.data_ptr(), lse2.data_ptr(), o2.data_ptr(),
                          lse2.data_ptr(), st)
    o2.zero_()
    lse2.fill_(float("-inf"))
    ms, _, _ = time_steps(torch, merge, steps, warmup)
    by = b * n * L * (3 * d * 4 + 12)
    out["merge"] = dict(ms=round(ms, 4), gbs=round(by / (ms * 1e-3) / 1e9, 1),
                        frac=round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
    out["shape"] = "batch 1, 12 heads x 128, 4096 queries, 4096-key blocks, bf16 in, fp32 O"
    return out


def terapipe_plan(layer, bufs, stages):
    """The token-slicing plan of a `stages`-stage pipeline of this layer
    shard, from slice latencies measured here (16-token granularity)."""
    from token_transformer_layer_amd import terapipe
    timer = terapipe.SliceTimer(layer, bufs)
    L = layer.shape.seq
    check = [(32, 256), (128, 640), (512, 896), (96, 1536), (768, 1280), (192, 1152), (48, 1920)]
    check = [(l, o) for l, o in check if l + o <= L]
    # the context overhead steps with the slice length where the attention
    # kernels' work split changes (a 128-token slice carries less than its
    # neighbours), so the fit samples nine lengths by eight offsets; the
    # check points stay out of it
    fit = [(l, o) for l in (16, 32, 64, 128, 256, 384, 512, 768, 1024)
           for o in (128, 384, 512, 768, 1024, 1280, 1536, 1792) if l + o <= L and (l, o) not in check]
    out = terapipe.plan(timer, L, 16, stages, fit, check, reps=11)
    layer.new_step()
    return out


def note(msg):
    """A progress line on stderr (the JSON result stays alone on stdout)."""
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="gpt3-175b-t8")
    ap.add_argument("--cpu-slices", type=int, default=16, help="slices of the oracle's CPU sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the per-slice and cube figures")
    ap.add_argument("--profile-only", action="store_true",
                    help="warm up and run the timed whole-partition steps only (for rocprofv3)")
    ap.add_argument("--schedule", choices=("whole", "per-slice"), default="whole",
                    help="with --profile-only: the call schedule of the profiled steps (one call per phase over all "
                         "slices, or the pipeline-faithful one call per slice)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="with --profile-only: also run one plain streaming kernel over this many MiB "
                         "(read once, written once), the calibration of rocprofv3's HBM byte counters")
    ap.add_argument("--clock-probe", action="store_true",
                    help="only time single kernels repeated back to back with the graphics clock they sustain")
    args = ap.parse_args()
    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU's shard: the library has no multi-GPU path "
                         "(the all-reduce between tensor-parallel ranks is left to the caller); "
                         "run with --gpus 1\n")
        sys.exit(2)

    import torch
    if args.clock_probe:
        torch.cuda.set_device(0)
        clock_probe(torch)
        return
    from token_transformer_layer_amd import synth
    from token_transformer_layer_amd.shard import ShardLayer

    shape = synth.CONFIGS[args.config]
    torch.cuda.set_device(0)
    x, dy = synth.activations(shape)
    sp = synth.shard_params_direct(shape, "standard", 0)
    layer = ShardLayer(shape, sp)
    bufs = dict(x=layer.act(x), dy=layer.act(dy), h_mid=layer.act(), y=layer.act(), dh=layer.act(),
                dx=layer.act(), p_attn=layer.f32(), p_mlp=layer.f32(), p_du2=layer.f32(), p_du1=layer.f32())
    del x, dy, sp
    layer.new_step()
    g_fl, a_fl = step_flops(shape)
    total = g_fl + a_fl

    step = make_step(layer, bufs, args.schedule if args.profile_only else "whole")
    per_step = []
    ms, wall_ms, _ = time_steps(torch, step, args.steps, args.warmup, trace=False, per_step=per_step)
    clk = None if args.profile_only else sustained_clock(torch, step)
    clock_peak = PEAK_BF16_TFLOPS * clk["mean"] / PEAK_CLOCK_MHZ if clk else None
    if args.profile_only:
        if args.copy_mib > 0:
            n = args.copy_mib * (1 << 20) // 4
            src = torch.full((n,), 7, dtype=torch.int32, device="cuda")
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            torch.bitwise_not(src, out=dst)
            torch.cuda.synchronize()
            del src, dst
        print(json.dumps(dict(config=shape.name, ms_per_step=ms)))
        return
    # per-kernel durations: the same K steps again with the library's event
    # trace on the launch stream (the events recorded around every launch
    # add about 6% to a step, so the headline comes from the untraced steps)
    traced_step_ms, _, recs = time_steps(torch, step, args.steps, 1, trace=True)
    kt = kernel_table(recs, args.steps)
    # the dominant kernel: the largest share of the step's time
    dom_name = next(iter(kt))
    dom_recs = [r for r in recs if r[0] == dom_name]
    dom_fl = sum(r[1] for r in dom_recs)
    dom_ms = sum(r[3] for r in dom_recs)
    achieved = dom_fl / (dom_ms * 1e-3) / 1e12
    # measured HBM bytes per launch of the dominant kernel, from the committed
    # counter summary when it was taken on the current sources (else null)
    from token_transformer_layer_amd import profiling
    traffic = profiling.load_traffic(os.path.join(ROOT, "profiles"), dom_name, shape.name)
    roofline = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4), traffic=traffic, kernel=dom_name,
                    launches=len(dom_recs), avg_launch_ms=round(dom_ms / len(dom_recs), 5),
                    algorithmic_bytes_per_launch=round(sum(r[2] for r in dom_recs) / len(dom_recs)),
                    traffic_unit="HBM bytes per launch",
                    frac_at_measured_clock=round(achieved / clock_peak, 4) if clock_peak else None)
    traced_ms = sum(r[3] for r in recs) / args.steps
    gemm_ms = sum(r[3] for r in recs if r[0].startswith("gemm")) / args.steps
    gemm_fl = sum(r[1] for r in recs if r[0].startswith("gemm")) / args.steps

    note("headline step timed: %.4f ms" % ms)
    extra = {}
    if not args.no_extra:
        extra["per_slice_calls"] = per_slice_figures(torch, layer, bufs, max(3, args.steps // 2), 2)
        note("per-slice schedule timed")
        extra["cube_ffn_block"] = cube_block(torch, max(3, args.steps // 2), 2)
        extra["cube_ffn_backward"] = cube_backward(torch, max(3, args.steps // 2), 2)
        note("cube block timed")
        extra["sequence_parallel_step"] = sequence_parallel_step(torch, layer, bufs, max(3, args.steps // 2), 2)
        extra["ring_attention_block"] = ring_block(torch, max(3, args.steps // 2), 2)
        note("sequence-parallel step and ring blocks timed")
        extra["terapipe_slicing"] = terapipe_plan(layer, bufs, stages=8)
        note("slicing plan measured")
        extra["other_workloads"] = {n: config_step(torch, n, max(5, args.steps // 2), 3)
                                    for n in ("gpt13b-t8", "medium-bf16") if n != shape.name}
        note("other workloads timed")

    out = {
        "metric": "shard-layer fwd+bwd TFLOP/s, GPT-3 175B t=8 shard, one MI355X",
        "value": round(total / (ms * 1e-3) / 1e12, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms_median": round(statistics.median(per_step), 4) if per_step else None,
        "step_ms_min": round(min(per_step), 4) if per_step else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": shape.name, "hidden": shape.hidden, "heads": shape.heads,
                   "head_dim": shape.head_dim, "ffn": shape.ffn, "tp": shape.tp, "batch": shape.batch,
                   "seq_len": shape.seq, "slices": list(shape.slices), "calls": "one per phase over all slices",
                   "parallelism": "one tp rank of 8 on 1 GPU"},
        "frac_of_bf16_peak": round(total / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "gfx_clock_mhz": clk,
        "frac_of_clock_peak": round(total / (ms * 1e-3) / 1e12 / clock_peak, 4) if clock_peak else None,
        "gemm": dict(ms_per_step=round(gemm_ms, 4), tflops=round(gemm_fl / (gemm_ms * 1e-3) / 1e12, 1),
                     frac=round(gemm_fl / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)),
        "traced_kernel_ms_per_step": round(traced_ms, 4),
        "traced_step_ms": round(traced_step_ms, 4),
        "wall_ms_per_step": round(wall_ms, 4),
        "roofline": roofline,
        "kernels": kt,
    }
    out.update(extra)
    if not args.no_cpu:
        note("timing the CPU oracle on a sample of the step")
        out["cpu_baseline"] = cpu_baseline(shape, args.cpu_slices)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
