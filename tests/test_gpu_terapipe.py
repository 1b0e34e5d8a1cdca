"""The token-slicing plan driven by slice latencies measured on the GPU: the
plan covers the sequence in whole granules, the library's planner on the
measured cost table attains the oracle's optimum, and the fitted context
model equals the oracle's least squares on the same measurements."""
import numpy as np
import pytest

from oracle import slicing as S
from tests import gpu_harness as H
from token_transformer_layer_amd import abi, synth
from token_transformer_layer_amd.synth import LayerShape

pytestmark = pytest.mark.gpu

SHAPE = LayerShape("slicing-small", 1024, 16, 64, 4096, 4, 1, 256, (256,), "bf16", seed=2021)


def test_measured_plan():
    import torch
    from token_transformer_layer_amd import terapipe
    from token_transformer_layer_amd.shard import ShardLayer
    print("[case] slicing plan on", SHAPE.name, flush=True)
    x, dy = synth.activations(SHAPE)
    layer = ShardLayer(SHAPE, synth.shard_params_direct(SHAPE, "standard", 0))
    bufs = dict(x=layer.act(x), dy=layer.act(dy), h_mid=layer.act(), y=layer.act(), dh=layer.act(), dx=layer.act(),
                p_attn=layer.f32(), p_mlp=layer.f32(), p_du2=layer.f32(), p_du1=layer.f32())
    layer.new_step()
    timer = terapipe.SliceTimer(layer, bufs)
    g, stages = 32, 4
    fit = [(32, 64), (64, 64), (32, 128), (96, 128), (64, 192)]
    check = [(32, 96), (128, 128)]
    out = terapipe.plan(timer, SHAPE.seq, g, stages, fit, check, reps=2)
    assert sum(out["slices"]) == SHAPE.seq and all(n % g == 0 and n > 0 for n in out["slices"])
    assert np.isfinite(out["model_rel_error_max"])
    # the planner on a measured table: the oracle's optimum
    units = SHAPE.seq // g
    fwd = np.zeros(units + 1)
    for k in range(1, units + 1):
        fwd[k] = timer.ms(k * g, 0, 2)
    ctx = [timer.ms(l, o, 2) - fwd[l // g] for l, o in fit]
    coef = abi.tp_fit_context_model([l for l, _ in fit], [o for _, o in fit], ctx)
    ref = S.fit_context_model([l for l, _ in fit], [o for _, o in fit], ctx)
    assert np.allclose(coef, ref, rtol=1e-9, atol=1e-15)
    cost = abi.tp_slice_cost_table(units, g, fwd, coef)
    lat, ends = abi.tp_slicing_plan(units, cost, stages)
    ref_lat, _ = S.slicing_optimal(units, cost, stages)
    assert lat == pytest.approx(ref_lat, rel=1e-12)
