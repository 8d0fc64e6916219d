"""Planted mistakes in the CPU oracle of the context-KV write must each fail at
least one pin of test_oracle_pins.py.

Every mutation below is a plausible slip against the pages' definition (a
dropped rounding, a sign, a pairing, an index, an order, a comparison) and is
planted by monkeypatching the oracle module in this process, on the CPU; the
pins are then run as plain functions. A mutation that a pin does not notice
would mean the oracle is not pinned where that mistake lives.
"""

import os
import sys

import numpy as np
import pytest

from oracle import ctx_kv_oracle as O

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import test_oracle_pins as P  # noqa: E402
from mutation_util import failing_pins  # noqa: E402

ORIG = {name: getattr(O, name) for name in (
    "round_to", "kv_proj_only", "rms_normalize", "apply_k_norm", "neox_rotate", "apply_k_rope",
    "valid_rows", "layer_kv")}


def _failing_pins():
    return failing_pins(P)


# ------------------------------------------------------------------ mutations

def _kv_no_r1(x, qkv_w, qkv_b, q_size, kv_size, dtype):
    xf = O.decode(x, dtype)
    w = O.decode(qkv_w[q_size:q_size + 2 * kv_size], dtype)
    y = xf @ w.T
    if qkv_b is not None:
        y = y + O.decode(qkv_b[q_size:q_size + 2 * kv_size], dtype)[None, :]
    return y[:, :kv_size], y[:, kv_size:]


def _kv_swapped(*args):
    k, v = ORIG["kv_proj_only"](*args)
    return v, k


def _kv_slice_one_row_early(x, qkv_w, qkv_b, q_size, kv_size, dtype):
    return ORIG["kv_proj_only"](x, qkv_w, qkv_b, q_size - 1, kv_size, dtype)


def _kv_bias_after_rounding(x, qkv_w, qkv_b, q_size, kv_size, dtype):
    k, v = ORIG["kv_proj_only"](x, qkv_w, None, q_size, kv_size, dtype)
    if qkv_b is None:
        return k, v
    b = O.decode(qkv_b[q_size:q_size + 2 * kv_size], dtype)
    y = O.round_to(np.concatenate([k, v], axis=1) + b[None, :], dtype)
    return y[:, :kv_size], y[:, kv_size:]


def _norm_sum_not_mean(k_heads, eps):
    ms = np.sum(k_heads * k_heads, axis=-1, keepdims=True)
    return k_heads / np.sqrt(ms + eps)


def _norm_eps_outside_root(k_heads, eps):
    D = k_heads.shape[-1]
    ms = np.sum(k_heads * k_heads, axis=-1, keepdims=True) / D
    return k_heads * (1.0 / np.sqrt(ms) + eps)


def _k_norm_no_r2(k_heads, k_norm_w, eps, dtype):
    return O.rms_normalize(k_heads, eps) * O.decode(k_norm_w, dtype)


def _k_norm_no_weight(k_heads, k_norm_w, eps, dtype):
    return O.round_to(O.rms_normalize(k_heads, eps), dtype)


def _rotate_sign(xn, cos, sin):
    half = xn.shape[-1] // 2
    x1, x2 = xn[..., :half], xn[..., half:]
    return np.concatenate([x1 * cos + x2 * sin, x2 * cos - x1 * sin], axis=-1)


def _rotate_gptj_pairs(xn, cos, sin):
    x1, x2 = xn[..., 0::2], xn[..., 1::2]
    out = np.empty_like(xn)
    out[..., 0::2] = x1 * cos - x2 * sin
    out[..., 1::2] = x2 * cos + x1 * sin
    return out


def _rope_no_r3(positions, xn, table, dtype):
    D = xn.shape[-1]
    rows = np.asarray(table, dtype=np.float32)[np.asarray(positions)].astype(np.float64)
    return O.neox_rotate(xn, rows[:, None, :D // 2], rows[:, None, D // 2:])


def _rope_halves_swapped(positions, xn, table, dtype):
    D = xn.shape[-1]
    rows = np.asarray(table, dtype=np.float32)[np.asarray(positions)].astype(np.float64)
    return O.round_to(O.neox_rotate(xn, rows[:, None, D // 2:], rows[:, None, :D // 2]), dtype)


def _rope_next_position(positions, xn, table, dtype):
    p = (np.asarray(positions) + 1) % len(table)
    return ORIG["apply_k_rope"](p, xn, table, dtype)


def _valid_commit_le(locs, commit_lens=None, row_width=0):
    locs = np.asarray(locs)
    valid = locs >= 0
    if commit_lens is not None:
        t = np.arange(len(locs))
        valid &= (t % row_width) <= np.asarray(commit_lens)[t // row_width]
    return valid


def _valid_loc_positive(locs, commit_lens=None, row_width=0):
    return ORIG["valid_rows"](np.where(np.asarray(locs) == 0, -1, locs), commit_lens, row_width)


def _round_half_up(x, dtype):
    p, emin, _ = O._FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    exp = np.maximum(e.astype(np.int64) - 1, emin)
    quantum = np.ldexp(1.0, (exp - p).astype(np.int32))
    return np.floor(x / quantum + 0.5) * quantum


def _layer_kv_norm_on_v(case, layer, rows=None):
    k, v = ORIG["layer_kv"](case, layer, rows)
    return k, O.apply_k_norm(v, case.k_norm_w[layer], case.eps, case.dtype)


MUTATIONS = {
    "R1 rounding dropped": ("kv_proj_only", _kv_no_r1),
    "K and V swapped": ("kv_proj_only", _kv_swapped),
    "KV slice one row early": ("kv_proj_only", _kv_slice_one_row_early),
    "bias added after rounding": ("kv_proj_only", _kv_bias_after_rounding),
    "mean of squares without 1/D": ("rms_normalize", _norm_sum_not_mean),
    "eps outside the root": ("rms_normalize", _norm_eps_outside_root),
    "R2 rounding dropped": ("apply_k_norm", _k_norm_no_r2),
    "k_norm weight dropped": ("apply_k_norm", _k_norm_no_weight),
    "rotation sign flipped": ("neox_rotate", _rotate_sign),
    "GPT-J pairs instead of neox": ("neox_rotate", _rotate_gptj_pairs),
    "R3 rounding dropped": ("apply_k_rope", _rope_no_r3),
    "cos and sin halves swapped": ("apply_k_rope", _rope_halves_swapped),
    "table row off by one": ("apply_k_rope", _rope_next_position),
    "commit test <= instead of <": ("valid_rows", _valid_commit_le),
    "slot 0 treated as skipped": ("valid_rows", _valid_loc_positive),
    "ties rounded up instead of to even": ("round_to", _round_half_up),
    "norm applied to V": ("layer_kv", _layer_kv_norm_on_v),
}


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_mutation_fails_a_pin(mutation, monkeypatch):
    name, fn = MUTATIONS[mutation]
    monkeypatch.setattr(O, name, fn)
    failed = _failing_pins()
    assert failed, f"no pin notices: {mutation}"
