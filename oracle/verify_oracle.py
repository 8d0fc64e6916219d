"""CPU oracle for the verify step's accept length and bonus token.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests and the benchmark's CPU-baseline leg use it. It
shares no code with the HIP library.

What it computes (sglang PR #31847 "[spec decoding] support inkling dspark",
implementation breakdown, step 2: ``compute_dflash_correct_drafts_and_bonus``,
whose CPU branch keeps a cumulative-product form and whose GPU kernel takes the
first mismatching offset). For request b with K drafted tokens ``draft[b, :K]``
and the target model's tokens ``target[b, :K+1]`` at the K + 1 verified
positions:

    accept[b] = number of leading i with draft[b, i] == target[b, i]
              = sum_i prod_{j <= i} [draft[b, j] == target[b, j]]   (cumprod form)
    bonus[b]  = target[b, accept[b]]

i.e. the accepted drafts are the longest matching prefix, and the bonus token
is the target's token at the first position it was not matched (or after the
last draft when all K match).

Reading where the page is silent: the shapes (K drafts against K + 1 target
tokens per request) and int64 token ids; the page names the function and the
first-mismatch rule only.
"""

from __future__ import annotations

import numpy as np


def accept_and_bonus(draft, target):
    """``draft`` [B, K], ``target`` [B, K+1] integer arrays -> (accept [B],
    bonus [B]) as int64, by the cumulative-product form."""
    draft = np.asarray(draft, dtype=np.int64)
    target = np.asarray(target, dtype=np.int64)
    B, K = draft.shape
    if target.shape != (B, K + 1):
        raise ValueError("target must be [B, K + 1]")
    eq = (draft == target[:, :K]).astype(np.int64)
    accept = np.cumprod(eq, axis=1).sum(axis=1) if K else np.zeros(B, dtype=np.int64)
    bonus = target[np.arange(B), accept]
    return accept.astype(np.int64), bonus.astype(np.int64)
