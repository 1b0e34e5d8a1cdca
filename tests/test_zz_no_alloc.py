"""The allocation-free forward (tp_shard_layer_fwd_noalloc) against the
forward that takes a caller's scratch buffer (tp_shard_layer_fwd): the same
kernels over the same work split, so every output (both partial sums, the
K/V cache and the saved activations) must be bit-identical.  Two calls of the
allocation-free forward run back to back, the second on a smaller input, so
that what the first left in the shared static work space cannot leak into the
second's results."""
import numpy as np
import pytest

import oracle
from tests import gpu_harness as H
from token_transformer_layer_amd import abi, synth
from token_transformer_layer_amd.synth import LayerShape

pytestmark = pytest.mark.gpu

SMALL = LayerShape("short-slices-d64", 640, 10, 64, 4000, 2, 2, 128, (1, 2, 7, 63, 1, 54), "bf16", seed=2022)


def _forward(layer, x, h_mid, groups, noalloc):
    import torch
    from token_transformer_layer_amd.shard import stream_handle

    xt, hm = layer.act(x), layer.act(h_mid)
    p_attn, p_mlp = layer.f32(), layer.f32()
    layer.new_step()
    layer.saved.zero_()
    for j0, j1 in groups:
        for phase, inp, out in ((abi.TP_FWD_ATTN, xt, p_attn), (abi.TP_FWD_MLP, hm, p_mlp)):
            if noalloc:
                abi.tp_shard_layer_fwd_noalloc(layer.cfg, layer.w, layer.part, j0, j1, phase, inp.data_ptr(),
                                               out.data_ptr(), layer.kv, layer.saved.data_ptr(), stream_handle())
            else:
                layer.fwd(phase, j0, j1, inp, out)
    torch.cuda.synchronize()
    return {"p_attn": p_attn.cpu().numpy(), "p_mlp": p_mlp.cpu().numpy(), "k": layer.k.float().cpu().numpy(),
            "v": layer.v.float().cpu().numpy(), "saved": layer.saved.cpu().numpy()}


def _case(shape, full, mode):
    from token_transformer_layer_amd.shard import ShardLayer

    x, _ = synth.activations(shape)
    if full:
        sp = synth.shard_params_direct(shape, "standard", 0)
    else:
        sp = oracle.shard_params(synth.full_params(shape, "perturbed"), 1, shape.as_dict())
    h_mid, _, _ = H.step_inputs(shape, shape.seed + 1)
    return ShardLayer(shape, sp), x, h_mid, H.groups_of(mode, len(shape.slices))


def test_noalloc_forward_matches_scratch_forward():
    cases = [(synth.CONFIGS["gpt3-175b-t8"], True, "whole"), (SMALL, False, "per-slice")]
    layers = [_case(*c) for c in cases]
    ref = [_forward(L, x, hm, grp, noalloc=False) for L, x, hm, grp in layers]
    # the allocation-free calls back to back: the full-size shard, then the
    # smaller one
    got = []
    for (shape, _, mode), (L, x, hm, grp) in zip(cases, layers):
        print("[case] noalloc forward %s mode=%s" % (shape.name, mode), flush=True)
        got.append(_forward(L, x, hm, grp, noalloc=True))
    for (shape, _, _), r, g in zip(cases, ref, got):
        for k in r:
            assert np.isfinite(g[k]).all() if g[k].dtype != np.uint8 else True, (shape.name, k)
            assert np.array_equal(r[k], g[k]), (shape.name, k)


def test_noalloc_scratch_size_and_tracing_refused():
    assert abi.tp_noalloc_scratch_bytes() == 128 << 20
    L, x, hm, grp = _case(SMALL, False, "whole")
    from token_transformer_layer_amd.shard import stream_handle
    xt, out = L.act(x), L.f32()
    L.new_step()
    abi.lib().tp_trace_enable(1)
    try:
        with pytest.raises(abi.TPError) as e:
            abi.tp_shard_layer_fwd_noalloc(L.cfg, L.w, L.part, 0, len(SMALL.slices), abi.TP_FWD_ATTN, xt.data_ptr(),
                                           out.data_ptr(), L.kv, L.saved.data_ptr(), stream_handle())
        assert e.value.status == abi.TP_EUNSUPPORTED
    finally:
        abi.lib().tp_trace_enable(0)
        abi.lib().tp_trace_read(None, 0)
    assert L.kv.filled == 0  # nothing enqueued, the cache protocol untouched
