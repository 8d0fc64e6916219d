"""Planted mistakes in the CPU oracle of the draft attention must each fail at
least one pin of test_draft_attention_oracle_pins.py (planted by
monkeypatching the oracle module in this process, on the CPU). The oracle is
one function, so each mistake is a switch on a re-statement of it below."""

import os
import sys

import numpy as np
import pytest

from oracle import draft_attention_oracle as A

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import test_draft_attention_oracle_pins as P  # noqa: E402
from mutation_util import failing_pins  # noqa: E402


def _attn(q, k_ext, v_ext, k_pool, v_pool, kv_indptr, kv_indices, block, nhq, nhk, sm_scale,
          dtype, *, own_keys=True, causal=False, head_map="group", scale=True, normalise=True,
          softmax_axis=1, v_from_k=False, rounded=True, keep_bad=False, count_bad=True):
    q = A.decode(q, dtype)
    ke, ve = A.decode(k_ext, dtype), A.decode(v_ext, dtype)
    kp, vp = A.decode(k_pool, dtype), A.decode(v_pool, dtype)
    if v_from_k:
        ve, vp = ke, kp
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    G = nhq // nhk
    out = np.zeros(q.shape, dtype=np.float64)
    skipped = 0
    for b in range(len(kv_indptr) - 1):
        idx = kv_indices[kv_indptr[b]:kv_indptr[b + 1]]
        ok = (idx >= 0) & (idx < kp.shape[0])
        skipped += int(np.count_nonzero(~ok)) if count_bad else 0
        idx = idx % kp.shape[0] if keep_bad else idx[ok]
        rows = slice(b * block, (b + 1) * block)
        K, V = kp[idx], vp[idx]
        if own_keys:
            K = np.concatenate([K, ke[rows]], axis=0)
            V = np.concatenate([V, ve[rows]], axis=0)
        n_prefix = len(idx)
        for h in range(nhq):
            kh = h // G if head_map == "group" else h % nhk
            s = q[rows, h, :] @ K[:, kh, :].T * (sm_scale if scale else 1.0)
            if causal:
                # query i of the block sees the prefix and own keys 0..i
                j = np.arange(s.shape[1])[None, :] - n_prefix
                s = np.where(j <= np.arange(block)[:, None], s, -np.inf)
            s = s - s.max(axis=softmax_axis, keepdims=True)
            p = np.exp(s)
            if normalise:
                p /= p.sum(axis=softmax_axis, keepdims=True)
            out[rows, h, :] = p @ V[:, kh, :]
    return (A.round_to(out, dtype) if rounded else out), skipped


MUTATIONS = {
    "block's own keys dropped": dict(own_keys=False),
    "causal mask inside the block": dict(causal=True),
    "query head h reads KV head h % NHK": dict(head_map="mod"),
    "sm_scale not applied": dict(scale=False),
    "softmax not normalised": dict(normalise=False),
    "softmax over the queries": dict(softmax_axis=0),
    "values taken from the keys": dict(v_from_k=True),
    "rounding dropped": dict(rounded=False),
    "out-of-pool slots kept (wrapped)": dict(keep_bad=True),
    "out-of-pool slots not counted": dict(count_bad=False),
}


def test_restatement_without_mistakes_equals_the_oracle():
    from speculative_decoding_draft_stacked_amd import workloads as W
    c = W.make_attn_case(B=3, block=4, nhq=8, nhk=2, D=64, prefix=[5, 0, 37], slots=64, seed=1)
    args = (c.q, c.k_ext, c.v_ext, c.k_pool, c.v_pool, c.kv_indptr, c.kv_indices, c.block, c.nhq,
            c.nhk, c.sm_scale, c.dtype)
    a, sa = A.draft_attention(*args)
    b, sb = _attn(*args)
    assert sa == sb and np.array_equal(a, b)


def test_unmutated_oracle_passes_every_pin():
    assert failing_pins(P) == []


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_mutation_fails_a_pin(mutation, monkeypatch):
    knobs = MUTATIONS[mutation]
    monkeypatch.setattr(A, "draft_attention", lambda *a: _attn(*a, **knobs))
    assert failing_pins(P), f"no pin notices: {mutation}"
