"""Planted mistakes in the CPU oracle of the verify step (accept length and
bonus token) must each fail at least one pin of test_verify_oracle_pins.py
(planted by monkeypatching the oracle module in this process, on the CPU)."""

import os
import sys

import numpy as np
import pytest

from oracle import verify_oracle as V

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import test_verify_oracle_pins as P  # noqa: E402
from mutation_util import failing_pins  # noqa: E402


def _verify(draft, target, *, prefix="cumprod", bonus_shift=0, target_shift=0, id_bits=64,
            bonus_last=False):
    draft = np.asarray(draft, dtype=np.int64)
    target = np.asarray(target, dtype=np.int64)
    B, K = draft.shape
    if target.shape != (B, K + 1):
        raise ValueError("target must be [B, K + 1]")
    if id_bits == 32:
        d, t = draft.astype(np.int32), target.astype(np.int32)
    else:
        d, t = draft, target
    eq = (d == t[:, target_shift:K + target_shift]).astype(np.int64)
    if K == 0:
        accept = np.zeros(B, dtype=np.int64)
    elif prefix == "cumprod":
        accept = np.cumprod(eq, axis=1).sum(axis=1)
    elif prefix == "cumsum":
        accept = np.minimum(np.cumsum(eq, axis=1), 1).sum(axis=1)
    else:
        accept = eq.sum(axis=1)
    col = np.full(B, K) if bonus_last else np.minimum(accept + bonus_shift, K)
    return accept.astype(np.int64), target[np.arange(B), col].astype(np.int64)


MUTATIONS = {
    "cumulative sum instead of product": dict(prefix="cumsum"),
    "every match counted": dict(prefix="all"),
    "bonus one position late": dict(bonus_shift=1),
    "target compared one position late": dict(target_shift=1),
    "ids compared in 32 bits": dict(id_bits=32),
    "last target token as bonus": dict(bonus_last=True),
}


def test_restatement_without_mistakes_equals_the_oracle():
    rng = np.random.default_rng(0)
    d = rng.integers(0, 3, (50, 6))
    t = rng.integers(0, 3, (50, 7))
    a = V.accept_and_bonus(d, t)
    b = _verify(d, t)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_unmutated_oracle_passes_every_pin():
    assert failing_pins(P) == []


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_mutation_fails_a_pin(mutation, monkeypatch):
    knobs = MUTATIONS[mutation]
    monkeypatch.setattr(V, "accept_and_bonus", lambda *a: _verify(*a, **knobs))
    assert failing_pins(P), f"no pin notices: {mutation}"
