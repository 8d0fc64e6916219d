"""Planted mistakes in the CPU oracle of the context producer
main_norm(main_proj(.)) must each fail at least one pin of
test_main_proj_oracle_pins.py (planted by monkeypatching the oracle module
in this process, on the CPU)."""

import os
import sys

import numpy as np
import pytest

from oracle import main_proj_oracle as M

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import test_main_proj_oracle_pins as P  # noqa: E402
from mutation_util import failing_pins  # noqa: E402

ORIG = {name: getattr(M, name) for name in ("main_proj", "main_norm")}


def _weight(g, g_dtype, narrow_fp32=False):
    if g_dtype == "fp32":
        g32 = np.asarray(g, dtype=np.float32)
        return (g32.astype(np.float16) if narrow_fp32 else g32).astype(np.float64)
    return M.decode(g, g_dtype)


def _norm(y, g, g_dtype, eps, dtype, *, rounded=True, weight=True, inv_form="mean",
          axis=-1, extra_round=False, narrow_fp32=False):
    gw = _weight(g, g_dtype, narrow_fp32)
    H = y.shape[axis]
    ss = np.sum(y * y, axis=axis, keepdims=True)
    if inv_form == "mean":
        inv = 1.0 / np.sqrt(ss / H + eps)
    elif inv_form == "sum":
        inv = 1.0 / np.sqrt(ss + eps)
    else:
        inv = 1.0 / np.sqrt(ss / H) + eps
    out = y * inv
    if extra_round:
        out = M.round_to(out, dtype)
    if weight:
        out = out * gw[None, :]
    return M.round_to(out, dtype) if rounded else out


def _proj_unrounded(aux, w, dtype):
    return M.decode(aux, dtype) @ M.decode(w, dtype).T


def _proj_rows_reversed(aux, w, dtype):
    return M.round_to(M.decode(aux, dtype) @ M.decode(w, dtype)[::-1].T, dtype)


MUTATIONS = {
    "projection rounding dropped": ("main_proj", _proj_unrounded),
    "norm rounding dropped": ("main_norm", lambda *a: _norm(*a, rounded=False)),
    "weight rows reversed": ("main_proj", _proj_rows_reversed),
    "sum of squares without 1/H": ("main_norm", lambda *a: _norm(*a, inv_form="sum")),
    "eps outside the root": ("main_norm", lambda *a: _norm(*a, inv_form="outside")),
    "norm over tokens": ("main_norm", lambda *a: _norm(*a, axis=0)),
    "norm weight dropped": ("main_norm", lambda *a: _norm(*a, weight=False)),
    "weight after an extra rounding": ("main_norm", lambda *a: _norm(*a, extra_round=True)),
    "fp32 weight narrowed": ("main_norm", lambda *a: _norm(*a, narrow_fp32=True)),
}


def test_unmutated_oracle_passes_every_pin():
    assert failing_pins(P) == []


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_mutation_fails_a_pin(mutation, monkeypatch):
    name, fn = MUTATIONS[mutation]
    monkeypatch.setattr(M, name, fn)
    assert failing_pins(P), f"no pin notices: {mutation}"
