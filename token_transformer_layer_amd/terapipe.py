"""Token-slicing plan from measured slice latencies ("TeraPipe: Token-Level
Pipeline Parallelism for Training Large-Scale Language Models", section 3,
selecting the slicing scheme).

The latency of one slice of l tokens after o tokens of context is measured
on this GPU as one layer shard's forward and backward over that slice (the
library's per-slice calls with the caller's residual combines; gradients
accumulate).  Following the page, it is split into the slice's latency
without context, measured for every slice length on the granularity grid,
and a context overhead predicted by a linear model fitted on a subset of
(length, context) combinations.  The model fills the slice cost table, and
the library's planner picks the slicing that minimises the latency of a
K-stage pipeline (sum of slice latencies plus K - 1 times the largest).
"""
import numpy as np
import torch

from . import abi


class SliceTimer:
    """Times one slice's forward and backward through the C-ABI on a
    ShardLayer (device buffers as in bench.py: x, dy, h_mid, y, dh, dx and
    the four fp32 partials)."""

    def __init__(self, layer, bufs):
        self.layer, self.b = layer, bufs

    def _run(self, o, l):
        layer, b = self.layer, self.b
        sh = layer.shape
        L = sh.seq
        lens = [n for n in (o, l, L - o - l) if n > 0]
        part = abi.make_partition(lens)
        j = 0 if o == 0 else 1
        saved_part = layer.part
        layer.part = part
        try:
            rows = l * sh.batch
            layer.kv.filled = o
            layer.fwd(abi.TP_FWD_ATTN, j, j + 1, b["x"], b["p_attn"])
            layer.combine(b["x"][o:], b["p_attn"][o:], layer.p["b_o"], b["h_mid"][o:], rows=rows)
            layer.fwd(abi.TP_FWD_MLP, j, j + 1, b["h_mid"], b["p_mlp"])
            layer.combine(b["h_mid"][o:], b["p_mlp"][o:], layer.p["b2"], b["y"][o:], rows=rows)
            layer.kvg.done_from = o + l
            layer.bwd(abi.TP_BWD_MLP, j, j + 1, dy=b["dy"], partial_out=b["p_du2"])
            layer.bwd(abi.TP_BWD_ATTN, j, j + 1, dy=b["dy"], ln_in=b["h_mid"], reduced=b["p_du2"],
                      partial_out=b["p_du1"], dh=b["dh"])
            layer.bwd(abi.TP_BWD_LN1, j, j + 1, ln_in=b["x"], reduced=b["p_du1"], dh=b["dh"], dx=b["dx"])
        finally:
            layer.part = saved_part

    def ms(self, l, o, reps=3):
        """Median of `reps` timed runs (after one untimed run)."""
        self._run(o, l)
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            self._run(o, l)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return float(np.median(times))


def plan(timer, seq, granularity, stages, fit_points, check_points, reps=5):
    """Measure, fit, plan.  fit_points / check_points: (length, offset) token
    pairs with offset > 0 used to fit the context model / to measure its
    error.  Every latency figure comes from the library: the model's
    prediction of a slice is its entry of the cost table, and the latencies
    of the plan and of uniform slicings are the library's pipeline latency
    over that table.  Returns a dict with the plan and the model's figures."""
    units = seq // granularity
    fwd = np.zeros(units + 1)
    for k in range(1, units + 1):
        fwd[k] = timer.ms(k * granularity, 0, reps)

    def ctx_of(l, o):
        return timer.ms(l, o, reps) - fwd[l // granularity]
    fl = [l for l, _ in fit_points]
    fo = [o for _, o in fit_points]
    coef = abi.tp_fit_context_model(fl, fo, [ctx_of(l, o) for l, o in fit_points])
    cost = abi.tp_slice_cost_table(units, granularity, fwd, coef)
    rel = []
    for l, o in check_points:
        t = timer.ms(l, o, reps)
        pred = cost[o // granularity, (o + l) // granularity]
        rel.append(abs(pred - t) / t)
    lat, ends = abi.tp_slicing_plan(units, cost, stages)
    lengths = [(b - a) * granularity for a, b in zip([0] + ends[:-1], ends)]
    uni = {n: round(abi.tp_plan_latency(units, cost, stages, [(i + 1) * (units // n) for i in range(n)]), 4)
           for n in (1, 2, 4, 8, 16, 32, 64, 128) if units % n == 0 and n <= units}
    return dict(granularity=granularity, stages=stages, slices=lengths, modeled_latency_ms=round(lat, 4),
                uniform_modeled_latency_ms=uni, context_model=[float("%.6g" % c) for c in coef],
                model_rel_error_max=round(max(rel), 4) if rel else None,
                model_rel_error_mean=round(float(np.mean(rel)), 4) if rel else None,
                fit_points=len(fit_points), check_points=len(check_points), reps=reps,
                fwd_no_context_ms={int(k * granularity): round(float(fwd[k]), 4)
                                   for k in (1, units // 8, units // 2, units) if k >= 1})
