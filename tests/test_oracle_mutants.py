"""Planted mistakes in the oracle (on the CPU) must make at least one pin fail.

Each mutant replaces one oracle function with a plausible wrong version (a
dropped term, a wrong sign, a transposed operand, a wrong axis or scale) and
runs the pins that should catch it; the test passes when a pin fails.
"""
import numpy as np
import pytest

import oracle
from oracle import mla_oracle as M
from tests import test_oracle_pins as pins

F64 = np.float64


def _rope_wrong_sign(x, pos, base):
    x = np.asarray(x, F64)
    th = M.rope_frequencies(x.shape[-1], base)
    ang = np.asarray(pos, F64)[..., None] * th
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * np.cos(ang) + x[..., 1::2] * np.sin(ang)
    out[..., 1::2] = -x[..., 0::2] * np.sin(ang) + x[..., 1::2] * np.cos(ang)
    return out


def _rope_halves(x, pos, base):
    """Rotates (x_k, x_k+d/2) pairs instead of interleaved pairs."""
    x = np.asarray(x, F64)
    h = x.shape[-1] // 2
    th = M.rope_frequencies(x.shape[-1], base)
    ang = np.asarray(pos, F64)[..., None] * th
    out = np.empty_like(x)
    out[..., :h] = x[..., :h] * np.cos(ang) - x[..., h:] * np.sin(ang)
    out[..., h:] = x[..., :h] * np.sin(ang) + x[..., h:] * np.cos(ang)
    return out


_orig_order_a = M.attend_order_a
_orig_absorbed = M.absorbed_query


def _order_a_no_rope_term(q_c, q_r, c, k_r, W_UK, W_UV, scale, return_p=False):
    return _orig_order_a(q_c, np.zeros_like(q_r), c, k_r, W_UK, W_UV, scale, return_p)


def _order_a_sqrt_dh(q_c, q_r, c, k_r, W_UK, W_UV, scale, return_p=False):
    return _orig_order_a(q_c, q_r, c, k_r, W_UK, W_UV, 1.0 / np.sqrt(q_c.shape[1]), return_p)


def _absorbed_wrong_block(q_c, q_r, W_UK, scale):
    n_h, d_h = q_c.shape
    W_UK = np.asarray(W_UK, F64)
    # uses head (i+1)'s rows: a wrong head slice
    qt = np.stack([W_UK[((i + 1) % n_h) * d_h:((i + 1) % n_h + 1) * d_h].T @ q_c[i] for i in range(n_h)])
    return np.concatenate([qt, q_r], axis=1) * scale


def _latent_attention_wrong_axis(Qt, rows, d_c):
    rows = np.asarray(rows, F64)
    p = M.softmax(np.asarray(Qt, F64) @ rows.T, axis=0)
    return p @ rows[:, :d_c]


def _integrate_transposed(o, W_O):
    return np.asarray(W_O, F64) @ np.asarray(o, F64).T.reshape(-1)


def _latent_rows_no_rotation(h, W_DKV, W_KR, positions, base):
    h = np.asarray(h, F64)
    return h @ np.asarray(W_DKV, F64).T, h @ np.asarray(W_KR, F64).T


MUTANTS = {
    "rope_wrong_sign": ("rope", _rope_wrong_sign),
    "rope_half_split": ("rope", _rope_halves),
    "order_a_drops_rope_term": ("attend_order_a", _order_a_no_rope_term),
    "order_a_scale_sqrt_dh": ("attend_order_a", _order_a_sqrt_dh),
    "absorb_wrong_head": ("absorbed_query", _absorbed_wrong_block),
    "softmax_wrong_axis": ("latent_attention", _latent_attention_wrong_axis),
    "integrate_transposed_concat": ("integrate", _integrate_transposed),
    "key_rope_not_rotated": ("latent_rows", _latent_rows_no_rotation),
}

PIN_SUITE = [
    lambda: pins.test_rope_matches_complex_rotation(),
    lambda: [pins.test_bruteforce_equals_order_a(si, 17) for si in range(3)],
    lambda: [pins.test_order_a_equals_order_b(si) for si in range(3)],
    lambda: [pins.test_mha_special_case_decode(si) for si in range(3)],
    lambda: pins.test_latent_pipeline_equals_order_b(),
    lambda: pins.test_uniform_attention_closed_form(),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(M, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    caught = 0
    for pin in PIN_SUITE:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught mutant {name}"
