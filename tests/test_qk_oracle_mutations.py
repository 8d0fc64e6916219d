"""Planted mistakes in the CPU oracle of the in-place QK-norm + rotation must
each fail at least one pin of test_qk_oracle_pins.py (planted by
monkeypatching the oracle module in this process, on the CPU)."""

import os
import sys

import numpy as np
import pytest

from oracle import qk_norm_rope_oracle as Q

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import test_qk_oracle_pins as P  # noqa: E402
from mutation_util import failing_pins  # noqa: E402

ORIG = {name: getattr(Q, name) for name in (
    "widen_weight", "head_columns", "qk_norm_rope_rows", "qk_norm_rope_inplace")}


def _rows_weights_swapped(x_heads, positions, q_w, k_w, weight_dtype, table, nhq, eps, dtype):
    return ORIG["qk_norm_rope_rows"](x_heads, positions, k_w, q_w, weight_dtype, table, nhq, eps,
                                     dtype)


def _columns_without_q_offset(nhq, nhk, D):
    return np.array([h * D for h in range(nhq)] + [j * D for j in range(nhk)], dtype=np.int64)


def _columns_one_head_short(nhq, nhk, D):
    return ORIG["head_columns"](nhq, nhk, D)[:-1]


def _rows(x_heads, positions, q_w, k_w, weight_dtype, table, nhq, eps, dtype, *, r2=True,
          r3=True, weight=True, halves_swapped=False, row_shift=0):
    D = x_heads.shape[-1]
    w = np.concatenate([np.broadcast_to(Q.widen_weight(q_w, weight_dtype), (nhq, D)),
                        np.broadcast_to(Q.widen_weight(k_w, weight_dtype),
                                        (x_heads.shape[1] - nhq, D))], axis=0)
    xn = Q.rms_normalize(x_heads, eps) * (w[None] if weight else 1.0)
    if r2:
        xn = Q.round_to(xn, dtype)
    p = (np.asarray(positions) + row_shift) % len(table)
    rows = np.asarray(table, dtype=np.float32)[p].astype(np.float64)
    c, s = rows[:, None, :D // 2], rows[:, None, D // 2:]
    if halves_swapped:
        c, s = s, c
    o = Q.neox_rotate(xn, c, s)
    return Q.round_to(o, dtype) if r3 else o


def _inplace(qkv, positions, q_w, k_w, weight_dtype, table, nhq, nhk, D, eps, dtype, *,
             upper_inclusive=False, negatives=False, count_kept=False):
    positions = np.asarray(positions, dtype=np.int64)
    P_ = np.asarray(table).shape[0]
    ok = (positions <= P_) if upper_inclusive else (positions < P_)
    if not negatives:
        ok &= positions >= 0
    tok = np.nonzero(ok)[0]
    if len(tok):
        cols = Q.head_columns(nhq, nhk, D)[:, None] + np.arange(D)[None, :]
        x = Q.decode(qkv[tok][:, cols], dtype)
        o = Q.qk_norm_rope_rows(x, np.clip(positions[tok], 0, P_ - 1) if upper_inclusive
                                else positions[tok], q_w, k_w, weight_dtype, table, nhq, eps, dtype)
        block = qkv[tok]
        block[:, cols] = Q.encode(o, dtype)
        qkv[tok] = block
    return int(np.count_nonzero(ok if count_kept else ~ok))


def _fp32_weights_mangled(w, weight_dtype):
    if weight_dtype == "fp32":
        return np.asarray(w, dtype=np.float32).astype(np.float16).astype(np.float64)
    return ORIG["widen_weight"](w, weight_dtype)


MUTATIONS = {
    "query and key weights swapped": ("qk_norm_rope_rows", _rows_weights_swapped),
    "key heads without the q_size offset": ("head_columns", _columns_without_q_offset),
    "last key head left out": ("head_columns", _columns_one_head_short),
    "rounding after the norm dropped": (
        "qk_norm_rope_rows", lambda *a: _rows(*a, r2=False)),
    "rounding after the rotation dropped": (
        "qk_norm_rope_rows", lambda *a: _rows(*a, r3=False)),
    "norm weight dropped": ("qk_norm_rope_rows", lambda *a: _rows(*a, weight=False)),
    "eps dropped": (
        "qk_norm_rope_rows",
        lambda x, p, qw, kw, wd, t, nhq, eps, dt: ORIG["qk_norm_rope_rows"](x, p, qw, kw, wd, t,
                                                                            nhq, 0.0, dt)),
    "table row off by one": ("qk_norm_rope_rows", lambda *a: _rows(*a, row_shift=1)),
    "cos and sin halves swapped": ("qk_norm_rope_rows", lambda *a: _rows(*a, halves_swapped=True)),
    "skipped tokens miscounted": ("qk_norm_rope_inplace", lambda *a: _inplace(*a, count_kept=True)),
    "position P accepted": ("qk_norm_rope_inplace", lambda *a: _inplace(*a, upper_inclusive=True)),
    "negative positions accepted": ("qk_norm_rope_inplace", lambda *a: _inplace(*a, negatives=True)),
    "fp32 weights narrowed": ("widen_weight", _fp32_weights_mangled),
}


def test_unmutated_oracle_passes_every_pin():
    assert failing_pins(P) == []


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_mutation_fails_a_pin(mutation, monkeypatch):
    name, fn = MUTATIONS[mutation]
    monkeypatch.setattr(Q, name, fn)
    assert failing_pins(P), f"no pin notices: {mutation}"
