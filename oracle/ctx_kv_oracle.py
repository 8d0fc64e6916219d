"""CPU oracle for the DSpark cross-layer context-KV write.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests, the package's smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library.

What it computes is the plain per-layer path that the stacked write must
reproduce (sglang PR #31986 "stack every DSpark layer's KV projection into one
GEMM", key source snippets: the per-layer branch of ``write_target_hidden_kv``
and the test helper ``_per_layer_reference``): for every draft layer, on its own,

    k, v = kv_proj_only(ctx_hidden)      # the layer's K/V rows of its QKV projection
    k    = apply_k_norm(k)               # per-head RMSNorm with the layer's k_norm weight
    k    = apply_k_rope(positions, k)    # neox RoPE read from the shared cos/sin table
    write K and V into the layer's pool at the row's slot

and the write's validity rule from sglang PR #31847 "[spec decoding] support
inkling dspark" (key source snippets, ``fused_kv_norm_rope_write`` docstring):
a row whose slot is negative is skipped; with ``commit_lens`` the slots are a
flattened ``[B, W]`` window and only the first ``commit_lens[b]`` columns of
request ``b`` are written.

Arithmetic is fp64 with an explicit round-to-nearest-even into the activation
dtype at three points, the roundings of the eager path:
  R1  the projection output (``F.linear`` returns the activation dtype),
  R2  after the norm (the table kernel in PR #31847 rounds to bf16 after
      ``x * inv * w``, "consistent with the eager path"),
  R3  after the rotation (the rotated halves are stored in the dtype).
The norm is ``ms = sum(x^2)/D``, ``inv = 1/sqrt(ms + eps)``, ``x*inv*w`` and the
rotation is ``o1 = x1*c - x2*s``, ``o2 = x2*c + x1*s`` over the pairs
``(i, i + D/2)`` (PR #31847, ``_table_qk_norm_rope_kernel`` listing).

Bit-pattern convention: activation tensors are 16-bit patterns (``uint16``);
the dtype is "bf16" or "fp16".
"""

from __future__ import annotations

import numpy as np

# IEEE-754 parameters: significand bits after the leading one, minimum normal
# exponent, maximum exponent.
_FORMATS = {
    "bf16": (7, -126, 127),
    "fp16": (10, -14, 15),
}


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit patterns -> exact fp64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    raise ValueError(dtype)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the nearest representable ``dtype`` value, ties to
    even (IEEE-754 roundTiesToEven), and return them as fp64.

    The quantum of a finite x is 2^(E - p) where E is x's binary exponent
    (clamped at the minimum normal exponent, which gives the subnormal spacing)
    and p the stored significand bits. Dividing by a power of two is exact, so
    ``rint`` (ties to even) on x / quantum is the correctly rounded significand.
    Magnitudes past the largest finite value become infinity.
    """
    p, emin, emax = _FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)  # x = m * 2^e with 0.5 <= |m| < 1, so E = e - 1
    exp = np.maximum(e.astype(np.int64) - 1, emin)
    quantum = np.ldexp(1.0, (exp - p).astype(np.int32))
    r = np.rint(x / quantum) * quantum
    max_finite = (2.0 - 2.0 ** (-p)) * 2.0 ** emax
    return np.where(np.abs(r) > max_finite, np.copysign(np.inf, x), r)


def encode(values: np.ndarray, dtype: str) -> np.ndarray:
    """Exactly representable fp64 values -> 16-bit patterns (no rounding here)."""
    values = np.asarray(values, dtype=np.float64)
    if dtype == "bf16":
        return (values.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    if dtype == "fp16":
        return values.astype(np.float16).view(np.uint16)
    raise ValueError(dtype)


def kv_proj_only(x, qkv_w, qkv_b, q_size, kv_size, dtype):
    """The layer's K and V projections: rows [q_size, q_size + kv) and
    [q_size + kv, q_size + 2kv) of its QKV weight (out x in), so
    y = x @ W_kv^T (+ b_kv), rounded to the dtype (R1).

    sglang PR #31986, key source snippets: ``kv_slice = slice(q_size,
    q_size + 2*kv_size)`` with K before V. Bias, when present, is part of the
    linear and added before the rounding."""
    xf = decode(x, dtype)
    w = decode(qkv_w[q_size:q_size + 2 * kv_size], dtype)
    y = xf @ w.T
    if qkv_b is not None:
        y = y + decode(qkv_b[q_size:q_size + 2 * kv_size], dtype)[None, :]
    y = round_to(y, dtype)
    return y[:, :kv_size], y[:, kv_size:]


def rms_normalize(k_heads: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis (head_dim), in fp64,
    before the weight and before rounding (PR #31847, ``_table_qk_norm_rope_kernel``)."""
    D = k_heads.shape[-1]
    ms = np.sum(k_heads * k_heads, axis=-1, keepdims=True) / D
    inv = 1.0 / np.sqrt(ms + eps)
    return k_heads * inv


def apply_k_norm(k_heads: np.ndarray, k_norm_w: np.ndarray, eps: float, dtype: str):
    """Per-head K RMSNorm with the layer's weight, rounded to the dtype (R2).
    ``k_heads`` is [T, NH, D] fp64 (already R1-rounded values)."""
    g = decode(k_norm_w, dtype)
    return round_to(rms_normalize(k_heads, eps) * g, dtype)


def neox_rotate(xn: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Neox rotation of [.., D] by per-row cos/sin [.., D/2]: pairs (i, i + D/2),
    o1 = x1*c - x2*s, o2 = x2*c + x1*s (PR #31847, ``_table_qk_norm_rope_kernel``)."""
    half = xn.shape[-1] // 2
    x1, x2 = xn[..., :half], xn[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def apply_k_rope(positions: np.ndarray, xn: np.ndarray, table: np.ndarray, dtype: str):
    """Rotate normalised K [T, NH, D] with the table row of each token's position
    (row = cos half | sin half, fp32, widened exactly), rounded to the dtype (R3)."""
    D = xn.shape[-1]
    rows = np.asarray(table, dtype=np.float32)[np.asarray(positions)].astype(np.float64)
    cos = rows[:, None, : D // 2]
    sin = rows[:, None, D // 2:]
    return round_to(neox_rotate(xn, cos, sin), dtype)


def valid_rows(locs: np.ndarray, commit_lens=None, row_width: int = 0) -> np.ndarray:
    """Which rows are written (PR #31847, ``fused_kv_norm_rope_write`` docstring):
    ``loc >= 0``, and with commit_lens, column ``t % W`` of request ``t // W`` is
    below ``commit_lens[t // W]``."""
    locs = np.asarray(locs)
    valid = locs >= 0
    if commit_lens is not None:
        t = np.arange(len(locs))
        valid &= (t % row_width) < np.asarray(commit_lens)[t // row_width]
    return valid


def layer_kv(case, layer: int, rows=None):
    """Per-layer K (normed + roped) and raw V for the given rows, as fp64 values
    of dtype numbers, shapes [n_rows, NH, D]."""
    dt = case.dtype
    x = case.x if rows is None else case.x[rows]
    pos = case.positions if rows is None else case.positions[rows]
    bias = None if case.qkv_b is None else case.qkv_b[layer]
    k, v = kv_proj_only(x, case.qkv_w[layer], bias, case.q_size, case.kv, dt)
    k = k.reshape(-1, case.NH, case.D)
    v = v.reshape(-1, case.NH, case.D)
    k = apply_k_norm(k, case.k_norm_w[layer], case.eps, dt)
    k = apply_k_rope(pos, k, case.table, dt)
    return k, v


def ctx_kv_write(case, pools_k, pools_v) -> None:
    """The whole write, layer by layer, into per-layer pools of 16-bit patterns
    [slots, NH, D] (updated in place). Rows that are not valid leave their
    slot untouched."""
    valid = valid_rows(case.locs, case.commit_lens, case.row_width)
    for layer in range(case.L):
        k, v = layer_kv(case, layer)
        kb = encode(k, case.dtype)
        vb = encode(v, case.dtype)
        for t in np.nonzero(valid)[0]:
            pools_k[layer][case.locs[t]] = kb[t]
            pools_v[layer][case.locs[t]] = vb[t]


def rows_kv(case, rows):
    """K and V patterns for selected rows of every layer: [L, n, NH, D] each."""
    rows = np.asarray(rows)
    ks, vs = [], []
    for layer in range(case.L):
        k, v = layer_kv(case, layer, rows)
        ks.append(encode(k, case.dtype))
        vs.append(encode(v, case.dtype))
    return np.stack(ks), np.stack(vs)
