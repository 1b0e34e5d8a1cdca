"""The library's token-slicing planner and latency model (host C++ behind the
C-ABI) against the oracle: equal optimal latency on random and structured
cost tables, a valid plan that attains it, equal fitted coefficients and
equal cost tables; bad arguments rejected."""
import numpy as np
import pytest

from oracle import slicing as S
from tests.test_oracle_slicing import brute_best, random_cost
from token_transformer_layer_amd import abi


def _plan_latency(cost, ends, stages):
    starts = [0] + ends[:-1]
    return S.pipeline_latency([cost[a][b] for a, b in zip(starts, ends)], stages)


@pytest.mark.parametrize("units", [1, 2, 7, 16, 48])
@pytest.mark.parametrize("stages", [1, 2, 8, 96])
def test_plan_matches_oracle(units, stages):
    cost = random_cost(units, np.random.default_rng(units * 100 + stages))
    lat, ends = abi.tp_slicing_plan(units, cost, stages)
    ref, _ = S.slicing_optimal(units, cost, stages)
    assert lat == pytest.approx(ref, rel=1e-12)
    assert ends[-1] == units and all(b > a for a, b in zip([0] + ends[:-1], ends))
    assert _plan_latency(cost, ends, stages) == pytest.approx(lat, rel=1e-12)
    if units <= 7:
        assert lat == pytest.approx(brute_best(units, cost, stages), rel=1e-12)


def test_forbidden_slices_are_avoided():
    units = 6
    cost = random_cost(units, np.random.default_rng(5))
    cost[0, 6] = np.inf
    cost[0, 3] = np.inf
    lat, ends = abi.tp_slicing_plan(units, cost, 1)
    ref, _ = S.slicing_optimal(units, cost, 1)
    assert lat == pytest.approx(ref, rel=1e-12) and ends != [6] and ends[0] != 3


def test_fit_and_cost_table_match_oracle():
    rng = np.random.default_rng(8)
    l = rng.integers(1, 128, 30) * 16
    o = rng.integers(0, 128, 30) * 16
    o[0] = 0
    ctx = S.context_time((3e-9, 2e-7, 5e-4), l, o) * (1 + 0.03 * rng.standard_normal(30))
    coef = abi.tp_fit_context_model(l, o, ctx)
    ref = S.fit_context_model(l, o, ctx)
    for a, b in zip(coef, ref):
        assert a == pytest.approx(b, rel=1e-9, abs=1e-15)
    units, g = 12, 16
    fwd = np.concatenate([[0.0], 0.2 + 0.01 * np.arange(1, units + 1)])
    cost = abi.tp_slice_cost_table(units, g, fwd, coef)
    ref_cost = S.slice_cost_table(units, g, {k * g: fwd[k] for k in range(1, units + 1)}, coef)
    fin = np.isfinite(ref_cost)
    assert np.array_equal(np.isfinite(cost), fin)
    assert np.allclose(cost[fin], ref_cost[fin], rtol=1e-14, atol=0)
    # a model that extrapolates below zero for short slices with little context
    neg = (coef[0], coef[1], -0.05)
    cost = abi.tp_slice_cost_table(units, g, fwd, neg)
    ref_cost = S.slice_cost_table(units, g, {k * g: fwd[k] for k in range(1, units + 1)}, neg)
    assert np.allclose(cost[fin], ref_cost[fin], rtol=1e-14, atol=0)
    assert (cost[fin] >= fwd[1:].min()).all()


def test_bad_arguments():
    cost = np.ones((4, 4))
    for call in [lambda: abi.tp_slicing_plan(3, cost, 0), lambda: abi.tp_slicing_plan(3, -cost, 2),
                 lambda: abi.tp_fit_context_model([16, 32], [0, 16], [1.0, 2.0]),
                 lambda: abi.tp_fit_context_model([16, 32, 48], [0, 0, 0], [1.0, 2.0, 3.0]),
                 lambda: abi.tp_slicing_plan(3, np.full((4, 4), np.inf), 2)]:
        with pytest.raises(abi.TPError) as ei:
            call()
        assert ei.value.status == abi.TP_EINVAL


def test_plan_latency_matches_oracle_pipeline_latency():
    """The library's latency of a given plan against the oracle's pipeline
    latency of the same slices (and the stage-by-stage recurrence)."""
    rng = np.random.default_rng(21)
    for units in (1, 4, 9):
        cost = random_cost(units, rng)
        for stages in (1, 3, 8):
            for _ in range(5):
                cuts = sorted(set(int(x) for x in rng.integers(1, units + 1, rng.integers(1, units + 1)))) or [units]
                ends = [c for c in cuts if c < units] + [units]
                starts = [0] + ends[:-1]
                times = [cost[a, b] for a, b in zip(starts, ends)]
                got = abi.tp_plan_latency(units, cost, stages, ends)
                assert abs(got - S.pipeline_latency(times, stages)) < 1e-12
                assert abs(got - S.pipeline_latency_sim(times, stages)) < 1e-12
        # the optimal plan's own latency
        lat, ends = abi.tp_slicing_plan(units, cost, 3)
        assert abs(abi.tp_plan_latency(units, cost, 3, ends) - lat) < 1e-12


def test_plan_latency_rejects_bad_plans():
    cost = random_cost(4, np.random.default_rng(2))
    for ends in ([2, 1, 4], [1, 2], [0, 4], [2, 5]):
        with pytest.raises(abi.TPError):
            abi.tp_plan_latency(4, cost, 2, ends)
