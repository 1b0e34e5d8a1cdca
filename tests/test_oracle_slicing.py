"""Pins of the token-slicing oracle (oracle/slicing.py): the latency formula
against the stage-by-stage recurrence, the dynamic program against brute
force over every composition, the least-squares fit against exact recovery
and the normal equations, and planted mistakes that the pins must catch."""
import inspect
import itertools

import numpy as np
import pytest

from oracle import slicing as S


def brute_best(units, cost, stages):
    best = np.inf
    for cut in itertools.product([0, 1], repeat=units - 1):
        ends = [i + 1 for i, c in enumerate(cut) if c] + [units]
        starts = [0] + ends[:-1]
        times = [cost[a][b] for a, b in zip(starts, ends)]
        best = min(best, S.pipeline_latency_sim(times, stages))
    return best


def random_cost(units, rng):
    # slice latency grows with length and offset, with a fixed overhead (as
    # measured kernels behave), plus noise so that ties are rare
    cost = np.full((units + 1, units + 1), np.inf)
    for a in range(units):
        for b in range(a + 1, units + 1):
            cost[a, b] = 1.0 + 0.6 * (b - a) + 0.05 * (b - a) * a + 0.3 * rng.random()
    return cost


def latency_errors(orc):
    rng = np.random.default_rng(1)
    err = 0.0
    for n in [1, 2, 5, 9]:
        for k in [1, 2, 3, 8]:
            t = rng.random(n) * 3
            err = max(err, abs(orc.pipeline_latency(t, k) - orc.pipeline_latency_sim(t, k)))
    return err


def dp_errors(orc):
    rng = np.random.default_rng(2)
    err = 0.0
    for units in [1, 3, 6, 9]:
        for k in [1, 2, 4, 16]:
            cost = random_cost(units, rng)
            lat, ends = orc.slicing_optimal(units, cost, k)
            err = max(err, abs(lat - brute_best(units, cost, k)))
            starts = [0] + ends[:-1]
            if ends[-1] != units or any(b <= a for a, b in zip(starts, ends)):
                return np.inf
            err = max(err, abs(lat - S.pipeline_latency_sim([cost[a][b] for a, b in zip(starts, ends)], k)))
    # a large fixed cost per slice: the optimum is one long slice, whose
    # latency is the largest candidate, so the search must not stop early
    for units in [4, 7]:
        cost = np.full((units + 1, units + 1), np.inf)
        for a in range(units):
            for b in range(a + 1, units + 1):
                cost[a, b] = 10.0 + 0.1 * (b - a) + 0.01 * a
        for k in [2, 3]:
            lat, _ = orc.slicing_optimal(units, cost, k)
            err = max(err, abs(lat - brute_best(units, cost, k)))
    return err


def fit_errors(orc):
    rng = np.random.default_rng(3)
    l = rng.integers(1, 64, 40) * 16.0
    o = rng.integers(0, 128, 40) * 16.0
    true = (2e-9, 3e-7, 4e-4)
    exact = orc.fit_context_model(l, o, S.context_time(true, l, o))
    err = max(abs(a - b) / abs(b) for a, b in zip(exact, true))
    noisy = S.context_time(true, l, o) * (1 + 0.05 * rng.standard_normal(40))
    coef = orc.fit_context_model(l, o, noisy)
    A = np.stack([l * o, o, np.ones_like(l)], axis=1)
    r = noisy - A @ np.array(coef)
    # residual orthogonal to the columns (normal equations), relative to scale
    err = max(err, float(np.abs(A.T @ r).max() / (np.abs(A).max(axis=0) * np.abs(noisy).max() * 40).max()))
    return err


def table_errors(orc):
    fwd = {16 * i: 1.0 + i for i in range(1, 9)}
    model = (1e-3, 2e-2, 0.5)
    cost = orc.slice_cost_table(8, 16, fwd, model)
    err = abs(cost[0, 3] - fwd[48])                                   # no context
    err = max(err, abs(cost[2, 5] - (fwd[48] + 1e-3 * 48 * 32 + 2e-2 * 32 + 0.5)))
    # a fit that extrapolates below zero (short slice, little context) adds
    # nothing: the context term is a latency
    neg = orc.slice_cost_table(8, 16, fwd, (1e-3, 2e-2, -3.0))
    err = max(err, abs(neg[1, 2] - fwd[16]))                          # ctx(16, 16) = 0.256 + 0.32 - 3 < 0
    err = max(err, abs(neg[4, 8] - (fwd[64] + 1e-3 * 64 * 64 + 2e-2 * 64 - 3.0)))  # 4.096 + 1.28 - 3 > 0
    return err


class SimulatedDevice:
    """A stand-in for measured slice latencies whose true values are known:
    a slice of l tokens after o tokens of context takes base(l) +
    ctx(l, o), with base drawn once per length (a noisy, increasing
    function, as measured kernels behave) and ctx = max(0, a l o + b o + c)
    (zero without context).  It is queried like the GPU: the no-context time
    per length, and the context overhead of a few (l, o) samples."""

    def __init__(self, seed, grid, coef):
        rng = np.random.default_rng(seed)
        self.coef = coef
        self.base = {l: 0.02 + 1e-4 * l + 2e-3 * rng.random() for l in grid}

    def latency(self, l, o):
        a, b, c = self.coef
        return self.base[l] + (max(0.0, a * l * o + b * o + c) if o > 0 else 0.0)


def simulated_table_errors(orc):
    """The cost table assembled from a simulated device's no-context times
    and a context model fitted to its samples equals, entry by entry, the
    device's own latency of that slice at that offset; and the plan chosen
    from the table is the best over every composition of the simulated
    latencies."""
    err = 0.0
    rng = np.random.default_rng(11)
    for units, g, coef in [(8, 16, (2e-7, 3e-5, 1e-3)), (6, 32, (3e-7, 2e-5, -2e-3))]:
        grid = [g * k for k in range(1, units + 1)]
        dev = SimulatedDevice(5 + units, grid, coef)
        # samples only where the device's overhead is on its linear part, so
        # the fit recovers it exactly
        samp = [(l, o) for l in grid for o in grid if l + o <= units * g
                and coef[0] * l * o + coef[1] * o + coef[2] > 0]
        samp = [samp[i] for i in rng.permutation(len(samp))[:max(6, len(samp) // 2)]]
        ls, os_ = [p[0] for p in samp], [p[1] for p in samp]
        model = orc.fit_context_model(ls, os_, [dev.latency(l, o) - dev.latency(l, 0) for l, o in samp])
        fwd = {l: dev.latency(l, 0) for l in grid}
        cost = orc.slice_cost_table(units, g, fwd, model)
        for a in range(units):
            for b in range(a + 1, units + 1):
                err = max(err, abs(cost[a, b] - dev.latency((b - a) * g, a * g)) / cost[a, b])
        for k in (1, 3, 8):
            lat, ends = orc.slicing_optimal(units, cost, k)
            starts = [0] + ends[:-1]
            sim = S.pipeline_latency_sim([dev.latency((b - a) * g, a * g) for a, b in zip(starts, ends)], k)
            err = max(err, abs(sim - brute_best(units, cost, k)) / sim)
    return err


def pin_failures(orc):
    checks = [("latency", lambda: latency_errors(orc) < 1e-12), ("dp", lambda: dp_errors(orc) < 1e-12),
              ("fit", lambda: fit_errors(orc) < 1e-9), ("table", lambda: table_errors(orc) < 1e-12),
              ("simulated", lambda: simulated_table_errors(orc) < 1e-9)]
    for name, ok in checks:
        with np.errstate(all="ignore"):
            try:
                good = bool(ok())
            except Exception:
                good = False
        if not good:
            yield name


def test_latency_formula_matches_stage_recurrence():
    assert latency_errors(S) < 1e-12


def test_dynamic_program_matches_brute_force():
    assert dp_errors(S) < 1e-12


def test_context_fit_recovers_and_satisfies_normal_equations():
    assert fit_errors(S) < 1e-9


def test_cost_table_closed_form():
    assert table_errors(S) < 1e-12


def test_cost_table_matches_simulated_device():
    assert simulated_table_errors(S) < 1e-9


def test_single_stage_with_forbidden_slices():
    """One stage and slices forbidden by +inf costs: the plan avoids them and
    the search evaluates no 0 * inf."""
    cost = random_cost(5, np.random.default_rng(4))
    cost[0, 5] = cost[1, 3] = np.inf
    with np.errstate(all="raise"):
        lat, ends = S.slicing_optimal(5, cost, 1)
    assert lat == pytest.approx(brute_best(5, cost, 1))
    starts = [0] + ends[:-1]
    assert all(np.isfinite(cost[a, b]) for a, b in zip(starts, ends))


def test_single_stage_prefers_one_slice_with_overhead():
    # with one stage there is no bubble, so a fixed per-slice overhead makes a
    # single slice optimal
    cost = random_cost(6, np.random.default_rng(9))
    lat, ends = S.slicing_optimal(6, cost, 1)
    assert lat == pytest.approx(min(brute_best(6, cost, 1), cost[0, 6]))


MUTANTS = [
    ("pipeline_latency", "(stages - 1) * float(np.max(times))", "stages * float(np.max(times))"),
    ("slicing_optimal", "if cost[a, b] <= c and", "if cost[a, b] < c and"),
    ("slicing_optimal", "lat = best[units] + (stages - 1) * c", "lat = best[units] + stages * c"),
    ("slicing_optimal", "if (stages - 1) * c >= best_lat:", "if (stages - 1) * c >= best_lat / 2:"),
    ("fit_context_model", "A = np.stack([l * o, o, np.ones_like(l)], axis=1)",
     "A = np.stack([l * o, l, np.ones_like(l)], axis=1)"),
    ("slice_cost_table", "l, o = (b - a) * g, a * g", "l, o = (b - a) * g, b * g"),
    ("slice_cost_table", "max(0.0, context_time(model, l, o))", "context_time(model, l, o)"),
]


@pytest.mark.parametrize("fn,old,new", MUTANTS, ids=[f"{m[0]}-{i}" for i, m in enumerate(MUTANTS)])
def test_slicing_mutant_is_caught(monkeypatch, fn, old, new):
    src = inspect.getsource(getattr(S, fn))
    assert old in src, "mutation site not found"
    ns = dict(S.__dict__)
    exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), ns)
    monkeypatch.setattr(S, fn, ns[fn])
    assert next(pin_failures(S), None) is not None, "no pin noticed the mutation"


def test_unmutated_slicing_oracle_passes_every_pin():
    assert list(pin_failures(S)) == []
