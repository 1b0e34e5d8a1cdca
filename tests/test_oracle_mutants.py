"""Plant plausible mistakes in the oracle (on the CPU, by rewriting one line
of one function) and check that the pins catch every one of them: a pin set
that let a dropped term, a wrong sign, index or transpose through would not
be pinning the oracle to anything."""
import inspect
import json
import os

import numpy as np
import pytest

import oracle.layer as L
from tests import oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MUTANTS = [
    ("causal_attention", "pos_k[None, :] > pos_q[:, None]", "pos_k[None, :] >= pos_q[:, None]"),
    ("causal_attention", "pos_k[None, :] > pos_q[:, None]", "pos_k[None, :] > pos_q[:, None] + 1"),
    ("causal_attention", "/ math.sqrt(d)", "/ d"),
    ("causal_attention", "pos_q = q_start + np.arange(lq)", "pos_q = np.arange(lq)"),
    ("causal_attention", "e = np.exp(scores - row_max)", "e = np.exp(scores)"),
    ("layer_norm", "((x - mean) ** 2).mean(axis=-1, keepdims=True)",
     "((x - mean) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)"),
    ("layer_norm", "return xhat * gamma + beta", "return xhat * gamma"),
    ("layer_norm_backward", "- xhat * (g * xhat).mean(axis=-1, keepdims=True)", ""),
    ("layer_norm_backward", "dgamma = (du * xhat)", "dgamma = (du)"),
    ("causal_attention_backward", "ds = p * (dp - row_dot)", "ds = p * dp"),
    ("causal_attention_backward", "dk = (np.swapaxes(ds, -1, -2) @ q)", "dk = (ds @ q)"),
    ("causal_attention_backward", "dq = (ds @ k) / math.sqrt(d)", "dq = (ds @ k)"),
    ("gelu", "return z * normal_cdf(z)",
     "return 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))"),
    ("gelu_grad", "normal_cdf(z) + z * normal_pdf(z)", "normal_cdf(z)"),
    ("layer_forward", 'h_mid = x + _linear(om, p["w_o"], p["b_o"])', 'h_mid = _linear(om, p["w_o"], p["b_o"])'),
    ("layer_forward", 'k = heads_split(_linear(u1, p["w_k"], p["b_k"]), n)',
     'k = heads_split(_linear(u1, p["w_q"], p["b_k"]), n)'),
    ("layer_backward", 'gr["b1"] = _rows(dz).sum(axis=0)', 'gr["b1"] = _rows(dg).sum(axis=0)'),
    ("layer_backward", 'gr["w_o"] = _rows(dh).T @ _rows(fw["om"])', 'gr["w_o"] = _rows(fw["om"]).T @ _rows(dh)'),
    ("shard_params", 'w_o=np.ascontiguousarray(p["w_o"][:, c])', 'w_o=np.ascontiguousarray(p["w_o"][c, :].T)'),
    ("shard_params", 'w1=p["w1"][fr], b1=p["b1"][fr]', 'w1=p["w1"][fr], b1=p["b1"][c]'),
    ("shard_attn_forward", 'partial = _linear(om, sp["w_o"])', 'partial = _linear(om, sp["w_o"], sp["b_o"])'),
    ("shard_attn_backward", 'kvg["dk"][:, :, :stop] += dk', 'kvg["dk"][:, :, :stop] = dk'),
    ("shard_attn_backward", 'heads_merge(kvg["dv"][:, :, start:stop])', 'heads_merge(kvg["dk"][:, :, start:stop])'),
    ("shard_mlp_backward", 'return _mm(dz, sp["w1"]), gr', 'return _mm(dg, sp["w1"]), gr'),
    ("ln1_backward", 'return np.asarray(dh_rows, dtype=np.float64) + dln1', 'return dln1'),
    ("cube_ffn_block", "return gelu(x @", "return (x @"),
    ("attention_block", "visible = pos_k[None, :] <= pos_q[:, None]", "visible = pos_k[None, :] < pos_q[:, None]"),
    ("attention_block", "pos_k = k_pos0 + np.arange(lk)", "pos_k = np.arange(lk)"),
    ("attention_block", "e = np.where(visible, np.exp(scores - row_max), 0.0)", "e = np.where(visible, np.exp(scores), 0.0)"),
    ("merge_partials", "o = (w_a[..., None] * o_a + w_b[..., None] * o_b) / tot_safe[..., None]",
     "o = (w_a[..., None] * o_a + w_b[..., None] * o_b)"),
    ("merge_partials", "lse = np.where(empty, -np.inf, m_safe + np.log(tot_safe))", "lse = np.where(empty, -np.inf, m_safe)"),
    ("merge_partials", "w_b = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - m_safe))",
     "w_b = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_a - m_safe))"),
    ("attention_block_backward", "ds = p * (dp - row_dot)", "ds = p * dp"),
    ("attention_block_backward", "pos_k = k_pos0 + np.arange(lk)", "pos_k = np.arange(lk)"),
    ("attention_block_backward", "dk = (np.swapaxes(ds, -1, -2) @ q) / math.sqrt(d)",
     "dk = (np.swapaxes(ds, -1, -2) @ q)"),
    ("attention_block_backward", "dv = np.swapaxes(p, -1, -2) @ do", "dv = np.swapaxes(p, -1, -2) @ o"),
    ("attention_block_backward", "np.exp(np.where(visible, scores, 0.0) - lse_safe)",
     "np.exp(np.where(visible, scores, 0.0))"),
]


def _pin_failures(orc):
    """Yield the name of each pin the given oracle fails (lazily)."""
    with open(os.path.join(GOLDEN, "normal_table.json")) as fh:
        table = json.load(fh)["rows"]
    checks = [
        ("brute", lambda: pins.brute_error(orc) < 1e-12),
        ("gelu-table", lambda: max(pins.gelu_table_errors(orc, table).values()) < 1e-14),
        ("closed-forms", lambda: max(pins.closed_form_errors(orc).values()) < 1e-12),
        ("finite-diff", lambda: pins.fd_error(orc) < 1e-6),
        ("tp-2-ranks", lambda: pins.tp_error(orc, 2, [6]) < 1e-12),
        ("slices", lambda: pins.tp_error(orc, 2, [2, 1, 3]) < 1e-12),
        ("cube", lambda: pins.cube_error(orc) < 1e-12),
        ("ring", lambda: pins.ring_error(orc) < 1e-12),
        ("ring-backward", lambda: pins.ring_backward_error(orc) < 1e-7),
    ]
    for name, ok in checks:
        with np.errstate(all="ignore"):
            try:
                good = bool(ok())
            except Exception:  # a mutant may also break shapes outright
                good = False
        if not good:
            yield name


@pytest.mark.parametrize("fn,old,new", MUTANTS, ids=[f"{m[0]}-{i}" for i, m in enumerate(MUTANTS)])
def test_mutant_is_caught(monkeypatch, fn, old, new):
    src = inspect.getsource(getattr(L, fn))
    assert old in src, "mutation site not found"
    ns = dict(L.__dict__)
    exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), ns)
    monkeypatch.setattr(L, fn, ns[fn])
    caught = next(_pin_failures(L), None)
    assert caught is not None, "no pin noticed the mutation"


def test_unmutated_oracle_passes_every_pin():
    assert list(_pin_failures(L)) == []
