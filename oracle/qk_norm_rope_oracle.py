"""CPU oracle for the in-place table QK-RMSNorm + neox RoPE on a fused QKV tensor.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests and the benchmark's CPU-baseline leg use it. It
shares no code with the HIP library.

What it computes (sglang PR #31847 "[spec decoding] support inkling dspark",
key source snippets: ``table_qk_norm_rope_`` and ``_table_qk_norm_rope_kernel``
in dflash_utils.py). Row t of the fused QKV tensor holds the NHQ query heads,
then the NHK key heads, then the value heads, each head_dim (D) wide, with
q_size = NHQ * D. For every token t and every head h of the NHQ + NHK query and
key heads, the D columns of that head (query head h at h * D, key head j at
q_size + j * D) are replaced, in place, by

    xn = round(x * inv * w)             inv = 1 / sqrt(sum(x^2) / D + eps)
    o  = round(neox_rotate(xn, c, s))   c, s = cos | sin halves of the table
                                        row at positions[t]

with w the query norm weight for query heads and the key norm weight for key
heads, fp32 arithmetic on the page (fp64 here, then one round to the dtype at
each of the two points). Every other column of the row (the value heads and
any padding up to the row stride) keeps its bits.

Reading where the page is silent: a token whose position lies outside the
table, [0, rope_max_pos), is left untouched and counted, as in the stacked
write (the page's kernel does not check the range).

Bit-pattern convention: the tensor is 16-bit patterns (``uint16``) of the dtype
"bf16" or "fp16"; norm weights are patterns of that dtype or fp32 values.
"""

from __future__ import annotations

import numpy as np

from .ctx_kv_oracle import decode, encode, neox_rotate, rms_normalize, round_to


def widen_weight(w, weight_dtype: str) -> np.ndarray:
    """A norm weight as exact fp64 values: fp32 values, or dtype patterns."""
    if weight_dtype == "fp32":
        return np.asarray(w, dtype=np.float32).astype(np.float64)
    return decode(w, weight_dtype)


def head_columns(nhq: int, nhk: int, D: int) -> np.ndarray:
    """First column of each of the NHQ + NHK heads the op rewrites: query head
    h at h * D, key head j at q_size + j * D (``col0`` in the page's kernel)."""
    q_size = nhq * D
    return np.array([h * D for h in range(nhq)] + [q_size + j * D for j in range(nhk)],
                    dtype=np.int64)


def qk_norm_rope_rows(x_heads, positions, q_w, k_w, weight_dtype, table, nhq, eps, dtype):
    """The op on gathered heads: ``x_heads`` [n, NHQ + NHK, D] of fp64 dtype
    values, one row per token. Returns the new head values, fp64 of dtype
    numbers, same shape."""
    D = x_heads.shape[-1]
    w = np.concatenate([np.broadcast_to(widen_weight(q_w, weight_dtype), (nhq, D)),
                        np.broadcast_to(widen_weight(k_w, weight_dtype),
                                        (x_heads.shape[1] - nhq, D))], axis=0)
    xn = round_to(rms_normalize(x_heads, eps) * w[None], dtype)
    rows = np.asarray(table, dtype=np.float32)[np.asarray(positions)].astype(np.float64)
    cos = rows[:, None, : D // 2]
    sin = rows[:, None, D // 2:]
    return round_to(neox_rotate(xn, cos, sin), dtype)


def qk_norm_rope_inplace(qkv, positions, q_w, k_w, weight_dtype, table, nhq, nhk, D, eps,
                         dtype) -> int:
    """Apply the op to ``qkv`` ([T, row_stride] uint16 patterns) in place.
    Returns the number of tokens skipped for a position outside the table."""
    positions = np.asarray(positions, dtype=np.int64)
    P = np.asarray(table).shape[0]
    ok = (positions >= 0) & (positions < P)
    tok = np.nonzero(ok)[0]
    if len(tok):
        cols = head_columns(nhq, nhk, D)[:, None] + np.arange(D)[None, :]  # [NHT, D]
        x = decode(qkv[tok][:, cols], dtype)                                  # [n, NHT, D]
        o = qk_norm_rope_rows(x, positions[tok], q_w, k_w, weight_dtype, table, nhq, eps, dtype)
        block = qkv[tok]
        block[:, cols] = encode(o, dtype)
        qkv[tok] = block
    return int(np.count_nonzero(~ok))
