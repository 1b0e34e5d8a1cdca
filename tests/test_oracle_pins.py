"""CPU pins of the oracle: brute force, finite differences, the
tensor-parallel shard-sum identity, token-slice invariance, closed forms and
normal-table values.  No GPU is involved."""
import json
import os

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_brute_force_forward():
    for seed in range(3):
        assert pins.brute_error(oracle, seed) < 1e-12


def test_finite_differences_backward():
    assert pins.fd_error(oracle) < 1e-6


@pytest.mark.parametrize("t", [1, 2])
def test_shard_sum_whole_sequence(t):
    # one slice covering the sequence: the Megatron split alone
    assert pins.tp_error(oracle, t, [6]) < 1e-12


def test_shard_sum_four_ranks():
    cfg = dict(pins.TINY, hidden=16, heads=4, head_dim=4, ffn=32, tp=4)
    assert pins.tp_error(oracle, 4, [2, 3, 1], cfg=cfg) < 1e-12


def test_every_slice_partition():
    # all 2^(s-1) partitions of s = 6 positions, on two ranks
    worst = max(pins.tp_error(oracle, 2, parts) for parts in pins.compositions(6))
    assert worst < 1e-12


def test_token_by_token_single_rank():
    assert pins.tp_error(oracle, 1, [1] * 6) < 1e-12


def test_closed_forms():
    errs = pins.closed_form_errors(oracle)
    bad = {k: v for k, v in errs.items() if not v < 1e-12}
    assert not bad, bad


def test_gelu_normal_table():
    with open(os.path.join(GOLDEN, "normal_table.json")) as fh:
        table = json.load(fh)["rows"]
    errs = pins.gelu_table_errors(oracle, table)
    assert errs["gelu"] < 1e-14 and errs["gelu_grad"] < 1e-14, errs


def test_cube_block():
    assert pins.cube_error(oracle) < 1e-12


def test_slice_order_is_enforced():
    cfg = dict(pins.TINY, seq=4)
    p = pins.tiny_params(cfg, 0)
    x, _ = pins.tiny_inputs(cfg, 0)
    sp = oracle.shard_params(p, 0, cfg)
    kv = oracle.new_kv_cache(cfg)
    with pytest.raises(ValueError):
        oracle.shard_attn_forward(x, sp, cfg, kv, 2, 4)


def test_shard_layer_step_single_rank():
    """shard_layer_step (one device, reduced inputs handed in) equals the
    unsharded layer at t = 1 once its own partial sums are fed back."""
    cfg = dict(pins.TINY, seq=6)
    p = pins.tiny_params(cfg, 7)
    x, dy = pins.tiny_inputs(cfg, 7)
    fw = oracle.layer_forward(x, p, cfg)
    gr = oracle.layer_backward(dy, p, cfg, fw)
    sp = oracle.shard_params(p, 0, cfg)
    bounds = [0, 2, 3, 6]
    z = np.zeros_like(x)
    r1 = oracle.shard_layer_step(x, fw["h_mid"], dy, z, z, sp, cfg, bounds)
    r2 = oracle.shard_layer_step(x, fw["h_mid"], dy, r1["p_du2"], z, sp, cfg, bounds)
    r3 = oracle.shard_layer_step(x, fw["h_mid"], dy, r1["p_du2"], r2["p_du1"], sp, cfg, bounds)
    assert np.abs(x + r3["p_attn"] + p["b_o"] - fw["h_mid"]).max() < 1e-12
    assert np.abs(fw["h_mid"] + r3["p_mlp"] + p["b2"] - fw["y"]).max() < 1e-12
    assert np.abs(r3["dx"] - gr["x"]).max() < 1e-12
    for k in ("ln1_g", "ln2_g", "b_o", "b2", "w1", "w2"):
        assert np.abs(r3["grads"][k] - gr[k]).max() < 1e-12


def test_attention_block_and_merge_match_brute_force():
    """Blocks before, across and after the queries, and the merge of all
    blocks (in either order) equal to attention over every key, both
    against pure-Python loops."""
    assert pins.ring_error(oracle) < 1e-12


def test_attention_block_special_cases():
    rng = np.random.default_rng(11)
    q = rng.normal(size=(1, 2, 3, 4))
    k = rng.normal(size=(1, 2, 5, 4))
    v = rng.normal(size=(1, 2, 5, 4))
    # every key after every query: nothing visible
    o, lse = oracle.attention_block(q, k, v, q_pos0=10, k_pos0=13)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # merging with an empty result changes nothing
    o2, l2 = oracle.attention_block(q, k, v, q_pos0=10, k_pos0=8)
    mo, ml = oracle.merge_partials(o2, l2, o, lse)
    assert np.array_equal(mo, o2) and np.array_equal(ml, l2)
    mo, ml = oracle.merge_partials(o, lse, o, lse)
    assert np.all(mo == 0) and np.all(np.isneginf(ml))
    # the first query sees exactly one key of a block starting at its position
    o1, l1 = oracle.attention_block(q, k, v, q_pos0=4, k_pos0=4)
    assert np.allclose(o1[..., 0, :], v[..., 0, :], atol=1e-15)
    assert np.allclose(l1[..., 0], (q[..., 0, :] * k[..., 0, :]).sum(-1) / 2.0, atol=1e-15)


def test_attention_block_empty_blocks():
    """A block of no keys leaves every query unseen (o = 0, lse = -inf) and
    merges as the identity; a block of no queries has empty outputs; their
    backward shares are zero or empty."""
    rng = np.random.default_rng(12)
    q = rng.normal(size=(1, 2, 3, 4))
    k = rng.normal(size=(1, 2, 5, 4))
    v = rng.normal(size=(1, 2, 5, 4))
    none_k, none_v = k[:, :, :0], v[:, :, :0]
    o, lse = oracle.attention_block(q, none_k, none_v, q_pos0=7, k_pos0=0)
    assert o.shape == (1, 2, 3, 4) and lse.shape == (1, 2, 3)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o2, l2 = oracle.attention_block(q, k, v, q_pos0=7, k_pos0=2)
    mo, ml = oracle.merge_partials(o2, l2, o, lse)
    assert np.array_equal(mo, o2) and np.array_equal(ml, l2)
    oq, lq = oracle.attention_block(q[:, :, :0], k, v, q_pos0=7, k_pos0=2)
    assert oq.shape == (1, 2, 0, 4) and lq.shape == (1, 2, 0)
    do = rng.normal(size=q.shape)
    dq, dk, dv = oracle.attention_block_backward(do, q, none_k, none_v, o2, l2, 7, 0)
    assert np.all(dq == 0) and dk.shape == (1, 2, 0, 4) and dv.shape == (1, 2, 0, 4)
    dq, dk, dv = oracle.attention_block_backward(do[:, :, :0], q[:, :, :0], k, v, o2[:, :, :0], l2[:, :, :0], 7, 2)
    assert dq.shape == (1, 2, 0, 4) and np.all(dk == 0) and np.all(dv == 0)


def test_attention_block_backward_matches_finite_differences():
    """Per-block backward with the merged forward result, summed over a ring
    of blocks, against finite differences of the brute-force forward."""
    assert pins.ring_backward_error(oracle) < 1e-7


def test_attention_block_backward_single_block_is_causal_backward():
    """One block holding every key from position 0 is plain causal attention:
    its backward equals causal_attention_backward."""
    rng = np.random.default_rng(9)
    q, k, v, do = (rng.normal(size=(2, 3, 5, 8)) for _ in range(4))
    o, p, lse = oracle.causal_attention(q, k, v)
    ref = oracle.causal_attention_backward(do, q, k, v, p, o)
    got = oracle.attention_block_backward(do, q, k, v, o, lse, 0, 0)
    for a, b in zip(got, ref):
        assert np.abs(a - b).max() < 1e-12
