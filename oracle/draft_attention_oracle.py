"""CPU oracle for the DSpark draft attention over the KV pool (non-causal,
grouped-query, shared prefix plus the block's own keys).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests and the benchmark's CPU-baseline leg use it. It
shares no code with the HIP library.

What it computes (sglang PR #35499 "K3 DSpark draft attention via
verify_shared_kv on ROCm gfx95", implementation breakdown and key source
snippets): every draft request has a block of query tokens; its keys and
values are the request's prefix, gathered from the layer's KV pool through
the request's slot list, followed by the block's own (extend) keys and values;
query head h reads KV head h // (NHQ / NHK); the draft's attention is
bidirectional, so every query of the block sees every key of its request:

    s = (q . k) * sm_scale,   p = softmax(s) over the request's keys,   o = p @ V

in fp64 here, rounded once to the activation dtype.

Readings where the page is silent: the block size is the same for every
request; the prefix comes first and the block's keys last (the order does not
change a bidirectional softmax); ``sm_scale`` is an input; a slot outside the
pool is a precondition violation, skipped (its key does not take part) and
counted.
"""

from __future__ import annotations

import numpy as np

from .ctx_kv_oracle import decode, round_to


def draft_attention(q, k_ext, v_ext, k_pool, v_pool, kv_indptr, kv_indices, block: int,
                    nhq: int, nhk: int, sm_scale: float, dtype: str):
    """q [B*block, NHQ, D], k_ext / v_ext [B*block, NHK, D], pools [slots, NHK, D]
    (dtype patterns); kv_indptr [B+1], kv_indices (int64 slots).
    Returns (out [B*block, NHQ, D] fp64 of dtype numbers, skipped slot count)."""
    q = decode(q, dtype)
    ke, ve = decode(k_ext, dtype), decode(v_ext, dtype)
    kp, vp = decode(k_pool, dtype), decode(v_pool, dtype)
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    B = len(kv_indptr) - 1
    G = nhq // nhk
    out = np.zeros(q.shape, dtype=np.float64)
    skipped = 0
    for b in range(B):
        idx = kv_indices[kv_indptr[b]:kv_indptr[b + 1]]
        ok = (idx >= 0) & (idx < kp.shape[0])
        skipped += int(np.count_nonzero(~ok))
        idx = idx[ok]
        rows = slice(b * block, (b + 1) * block)
        K = np.concatenate([kp[idx], ke[rows]], axis=0)  # [L, NHK, D]
        V = np.concatenate([vp[idx], ve[rows]], axis=0)
        for h in range(nhq):
            kh = h // G
            s = q[rows, h, :] @ K[:, kh, :].T * sm_scale  # [block, L]
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[rows, h, :] = p @ V[:, kh, :]
    return round_to(out, dtype), skipped
