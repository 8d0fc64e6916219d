"""CPU oracle for the DSpark draft's context producer, main_norm(main_proj(.)).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests and the benchmark's CPU-baseline leg use it. It
shares no code with the HIP library.

What it computes (vLLM PR #46995 "[Spec Decode] DSpark", key source snippets:
``DSparkDeepseekV4Model.__init__`` and ``combine_hidden_states``). The target's
auxiliary hidden states of the n chosen layers, concatenated to
``aux [T, n*H]``, are projected by a bias-free linear ``main_proj`` (weight
``[H, n*H]``) to ``[T, H]`` and normalised by an RMSNorm ``main_norm`` over the
H features with weight ``g [H]`` and eps:

    y  = round(aux @ W^T)                        (the linear's output dtype)
    ctx = round(y * inv * g),  inv = 1 / sqrt(sum(y^2) / H + eps)

in fp64 here, with a round-to-nearest-even into the activation dtype at the
two points. The result is the ``ctx_hidden`` the stacked context-KV write
consumes.

Reading where the page is silent: the RMSNorm's internals are not shown. This
oracle takes the form the rest of the pages use for their norms (x * inv * w in
fp32, one rounding), the weight widened exactly to fp32.
"""

from __future__ import annotations

import numpy as np

from .ctx_kv_oracle import decode, round_to


def main_proj(aux, w, dtype: str) -> np.ndarray:
    """round(aux @ W^T): ``aux`` [T, n*H] and ``w`` [H, n*H] dtype patterns ->
    fp64 values of dtype numbers [T, H]."""
    return round_to(decode(aux, dtype) @ decode(w, dtype).T, dtype)


def main_norm(y: np.ndarray, g, g_dtype: str, eps: float, dtype: str) -> np.ndarray:
    """Row RMSNorm of ``y`` [T, H] over H with weight ``g`` (dtype patterns or
    fp32 values when ``g_dtype`` is "fp32"), rounded to the dtype."""
    gw = (np.asarray(g, dtype=np.float32).astype(np.float64) if g_dtype == "fp32"
          else decode(g, g_dtype))
    H = y.shape[-1]
    inv = 1.0 / np.sqrt(np.sum(y * y, axis=-1, keepdims=True) / H + eps)
    return round_to(y * inv * gw[None, :], dtype)


def combine_hidden_states(aux, w, g, g_dtype: str, eps: float, dtype: str) -> np.ndarray:
    """main_norm(main_proj(aux)) as fp64 values of dtype numbers [T, H]."""
    return main_norm(main_proj(aux, w, dtype), g, g_dtype, eps, dtype)
