"""fp64 definition of the token-slicing plan of a token-level pipeline and of
its latency model.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg.

Source: "TeraPipe: Token-Level Pipeline Parallelism for Training Large-Scale
Language Models" (summary page), section 3 (Method), "Selecting optimal
slicing scheme": slice lengths l_1..l_M with sum L are chosen by dynamic
programming to minimise the total forward and backward latency; the latency
of a slice is its forward time without extra context plus a context
overhead that a linear model predicts, fitted from a subset of measured
(slice, context) combinations.

Readings where the page is silent:
* pipeline latency: K stages, every stage taking t_i for slice i, slices in
  order; the last slice leaves the last stage at sum_i t_i + (K-1) max_i t_i
  (pipeline_latency; pinned against the stage-by-stage recurrence
  pipeline_latency_sim);
* the search: for each candidate value of the largest slice latency, the
  least sum of slice latencies whose slices all stay within it, by dynamic
  programming over prefixes; the best candidate wins; candidates run in
  increasing order and stop once (K-1) times the candidate alone exceeds the
  best latency found;
* slice lengths are multiples of a granularity g (units of g tokens);
* context model: ctx(l, o) = a_lo * l * o + a_o * o + a_1 for a slice of l
  tokens after o tokens of context, least squares over the samples given;
  as a latency it is taken as max(0, ctx) in the slice costs.
"""
import numpy as np

__all__ = ["pipeline_latency_sim", "pipeline_latency", "slicing_optimal", "fit_context_model", "context_time",
           "slice_cost_table"]


def pipeline_latency_sim(times, stages):
    """Finish time of the last slice in the last stage, stage by stage: stage
    s starts slice i when it has finished slice i-1 and stage s-1 has
    finished slice i; it then takes times[i]."""
    done = [0.0] * len(times)  # finish times in the previous stage
    for _ in range(stages):
        prev = 0.0
        for i, t in enumerate(times):
            start = max(prev, done[i])
            prev = start + float(t)
            done[i] = prev
    return done[-1] if len(times) else 0.0


def pipeline_latency(times, stages):
    """sum_i t_i + (K - 1) max_i t_i."""
    if len(times) == 0:
        return 0.0
    return float(np.sum(times)) + (stages - 1) * float(np.max(times))


def slicing_optimal(units, cost, stages):
    """Optimal plan over `units` granules: cost[a][b] (a < b) is the latency of
    the slice covering granules [a, b).  Returns (latency, ends) with ends
    the cumulative slice boundaries (last = units).

    For each candidate largest latency c (every distinct finite cost value,
    in increasing order): best[b] = min over a < b with cost[a][b] <= c of
    best[a] + cost[a][b] (best[0] = 0); the plan latency is
    best[units] + (K-1) c.  Stops once (K-1) c alone reaches the best plan
    latency found."""
    cost = np.asarray(cost, dtype=np.float64)
    # a +inf cost forbids its slice, so it is never the largest latency of a
    # plan: only finite costs are candidates
    cands = np.unique([cost[a, b] for a in range(units) for b in range(a + 1, units + 1)
                       if np.isfinite(cost[a, b])])
    best_lat, best_ends = np.inf, None
    for c in cands:
        if (stages - 1) * c >= best_lat:
            break
        best = np.full(units + 1, np.inf)
        arg = np.full(units + 1, -1)
        best[0] = 0.0
        for b in range(1, units + 1):
            for a in range(b):
                if cost[a, b] <= c and best[a] + cost[a, b] < best[b]:
                    best[b] = best[a] + cost[a, b]
                    arg[b] = a
        if not np.isfinite(best[units]):
            continue
        lat = best[units] + (stages - 1) * c
        if lat < best_lat:
            ends, b = [], units
            while b > 0:
                ends.append(b)
                b = arg[b]
            best_lat, best_ends = lat, ends[::-1]
    return float(best_lat), best_ends


def fit_context_model(l, o, ctx):
    """Least-squares (a_lo, a_o, a_1) of ctx ~ a_lo * l * o + a_o * o + a_1."""
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    A = np.stack([l * o, o, np.ones_like(l)], axis=1)
    coef, *_ = np.linalg.lstsq(A, np.asarray(ctx, dtype=np.float64), rcond=None)
    return tuple(float(x) for x in coef)


def context_time(model, l, o):
    a_lo, a_o, a_1 = model
    return a_lo * l * o + a_o * o + a_1


def slice_cost_table(units, g, fwd, model):
    """cost[a][b] = fwd[(b-a) g] + max(0, ctx((b-a) g, a g)) (ctx 0 without
    context); fwd maps a slice length in tokens to its measured no-context
    latency.  The context term is a latency, never negative: where the fitted
    line extrapolates below zero it adds nothing."""
    cost = np.full((units + 1, units + 1), np.inf)
    for a in range(units):
        for b in range(a + 1, units + 1):
            l, o = (b - a) * g, a * g
            cost[a, b] = fwd[l] + (max(0.0, context_time(model, l, o)) if o > 0 else 0.0)
    return cost
