"""Seeded synthetic inputs for the DSpark cross-layer context-KV write.

This module only draws inputs. It holds none of the write's arithmetic (no
projection, norm, rotation or scatter), so both the CPU oracle and the HIP
path can take their inputs from it without sharing any of the method.

Everything is returned as host numpy arrays. Activation-dtype tensors are
returned as their 16-bit patterns (``uint16``), so the oracle and the GPU see
identical bits.

The shapes follow the draft layers the pages describe: each draft layer has a
fused QKV projection whose rows are ``[Q | K | V]`` (sglang PR #31986,
"_stacked_ctx_kv_params" listing: the KV slice is ``[q_size, q_size+2*kv_size)``),
a per-head K RMSNorm weight of ``head_dim`` entries, and a neox rotary table
``[max_position, head_dim]`` laid out as the cos half followed by the sin half
(sglang PR #31847, "_table_qk_norm_rope_kernel" listing). The KV pool of each
layer is ``[slots, num_kv_heads, head_dim]`` (same PR, "_build_fused_kv_write_bundle").

The rotary table is an input of the write: the path only reads it. It is built
here the way a rotary module precomputes it, with inverse frequencies
``theta ** (-2i/D)`` and angles ``p * f_i`` evaluated in fp64 and stored as fp32.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

BF16 = "bf16"
FP16 = "fp16"
SENTINEL = 0xFFFF  # NaN in both bf16 and fp16; finite inputs never produce it


def _to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (numpy RNE) -> bf16 bit pattern (RNE on the fp32 bits)."""
    u = np.ascontiguousarray(x64, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _to_fp16_bits(x64: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x64, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bits(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Convert drawn fp64 values to the activation dtype's bit patterns."""
    if dtype == BF16:
        return _to_bf16_bits(x64)
    if dtype == FP16:
        return _to_fp16_bits(x64)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclasses.dataclass
class Case:
    """One synthetic instance of the context-KV write (host arrays)."""

    name: str
    dtype: str  # "bf16" | "fp16"
    T: int
    H: int
    L: int
    NH: int
    D: int
    q_size: int
    eps: float
    theta: float
    P: int  # rotary table rows
    slots: int  # pool slots per layer
    x: np.ndarray  # uint16 [T, H]
    qkv_w: List[np.ndarray]  # per layer uint16 [q_size + 2*kv, H]
    qkv_b: Optional[List[np.ndarray]]  # per layer uint16 [q_size + 2*kv] or None
    k_norm_w: List[np.ndarray]  # per layer uint16 [D]
    table: np.ndarray  # float32 [P, D]: cos half | sin half
    positions: np.ndarray  # int64 [T]
    locs: np.ndarray  # int64 [T] (flattened [B, W] window when commit_lens is set)
    commit_lens: Optional[np.ndarray]  # int64 [B] or None
    row_width: int  # W when commit_lens is set, else 0

    @property
    def kv(self) -> int:
        return self.NH * self.D

    @property
    def n_tot(self) -> int:
        return self.L * 2 * self.kv

    @property
    def num_requests(self) -> int:
        return 0 if self.commit_lens is None else len(self.commit_lens)


def rope_table(P: int, D: int, theta: float) -> np.ndarray:
    """Neox rotary table [P, D] fp32: row p = cos(p*f_0..f_{D/2-1}) | sin(...)."""
    half = D // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / D)
    ang = np.arange(P, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def make_case(
    *,
    name: str = "case",
    T: int,
    H: int,
    L: int,
    NH: int,
    D: int,
    dtype: str = BF16,
    bias: bool = False,
    row_width: int = 0,
    commit_range=(1, None),
    theta: float = 1e4,
    P: int = 4096,
    slots: int = 64,
    eps: float = 1e-6,
    seed: int = 0,
    q_size: Optional[int] = None,
    locs_mode: str = "random",
    locs_start: int = 0,
    positions_mode: str = "uniform",
    neg_loc_frac: float = 0.0,
    w_std: float = 0.02,
    x_std: float = 1.0,
) -> Case:
    """Draw one case. Generation order is fixed: X, per-layer Q/K/V rows, bias,
    k_norm, positions, locs, commit_lens (then optional negative-loc holes)."""
    if q_size is None:
        q_size = H
    kv = NH * D
    rng = np.random.Generator(np.random.PCG64(seed))
    x = to_bits(rng.standard_normal((T, H)) * x_std, dtype)
    qkv_w = []
    for _ in range(L):
        q = rng.standard_normal((q_size, H))  # Q rows ~N(0,1): a wrong slice is obvious
        k = rng.standard_normal((kv, H)) * w_std
        v = rng.standard_normal((kv, H)) * w_std
        qkv_w.append(to_bits(np.concatenate([q, k, v], axis=0), dtype))
    qkv_b = None
    if bias:
        qkv_b = [to_bits(rng.standard_normal(q_size + 2 * kv) * 0.01, dtype) for _ in range(L)]
    k_norm_w = [to_bits(1.0 + rng.standard_normal(D) * 0.1, dtype) for _ in range(L)]
    if positions_mode == "uniform":
        positions = rng.integers(0, P, size=T, dtype=np.int64)
    elif positions_mode == "arange":
        positions = np.arange(T, dtype=np.int64)
    else:
        raise ValueError(positions_mode)
    if locs_mode == "random":
        if T > slots:
            raise ValueError("random injective locs need T <= slots")
        locs = rng.permutation(slots)[:T].astype(np.int64)
    elif locs_mode == "contiguous":
        locs = locs_start + np.arange(T, dtype=np.int64)
    else:
        raise ValueError(locs_mode)
    commit_lens = None
    if row_width:
        if T % row_width:
            raise ValueError("T must be a multiple of the window width")
        lo, hi = commit_range
        hi = row_width if hi is None else hi
        commit_lens = rng.integers(lo, hi + 1, size=T // row_width, dtype=np.int64)
    if neg_loc_frac > 0:
        holes = rng.random(T) < neg_loc_frac
        locs = np.where(holes, -1, locs).astype(np.int64)
    return Case(
        name=name, dtype=dtype, T=T, H=H, L=L, NH=NH, D=D, q_size=q_size, eps=eps,
        theta=theta, P=P, slots=slots, x=x, qkv_w=qkv_w, qkv_b=qkv_b, k_norm_w=k_norm_w,
        table=rope_table(P, D, theta), positions=positions, locs=locs,
        commit_lens=commit_lens, row_width=row_width,
    )


# The workloads the context-KV write is measured and checked on: the five
# configurations, and one GPU's share of decode_commit under KV-head sharding.
WORKLOADS = {
    # 2 requests x 8 rows, tiny draft: 2 layers, 2 KV heads of 64.
    "tiny": dict(T=16, H=256, L=2, NH=2, D=64, dtype=BF16, theta=1e4, P=4096, slots=64),
    # Qwen3-8B-like decode commit: 32 requests x 8 columns, commit_lens ~ U{1..8}.
    "decode_commit": dict(T=256, H=4096, L=5, NH=8, D=128, dtype=BF16, row_width=8,
                          theta=1e6, P=32768, slots=65536),
    # One 8k prompt written contiguously from slot 4096 (positions 0..8191).
    "prefill_8k": dict(T=8192, H=4096, L=5, NH=8, D=128, dtype=BF16, theta=1e6, P=32768,
                       slots=16384, locs_mode="contiguous", locs_start=4096,
                       positions_mode="arange"),
    # 16 requests x 128 rows, fp16 with a stacked per-layer KV bias.
    "biased_fp16": dict(T=2048, H=3584, L=5, NH=4, D=128, dtype=FP16, bias=True, theta=1e6,
                        P=32768, slots=32768),
    # Wide hidden, head_dim 64: 64 requests x 8 columns with commit_lens.
    "wide_gqa_d64": dict(T=512, H=7168, L=5, NH=8, D=64, dtype=BF16, row_width=8, theta=5e4,
                         P=32768, slots=131072),
    # One GPU's share of decode_commit when the KV heads are split over 8 (or 4)
    # GPUs: each GPU packs and writes 1 (or 2) KV heads of every layer; nothing
    # is exchanged.
    "decode_commit_kv1": dict(T=256, H=4096, L=5, NH=1, D=128, dtype=BF16, row_width=8,
                              theta=1e6, P=32768, slots=65536),
    "decode_commit_kv2": dict(T=256, H=4096, L=5, NH=2, D=128, dtype=BF16, row_width=8,
                              theta=1e6, P=32768, slots=65536),
}
WORKLOAD_ORDER = ["tiny", "decode_commit", "prefill_8k", "biased_fp16", "wide_gqa_d64",
                  "decode_commit_kv1", "decode_commit_kv2"]


def workload(name: str) -> Case:
    """The named workload with its fixed seed (1000 + its 1-based index)."""
    seed = 1000 + WORKLOAD_ORDER.index(name) + 1
    return make_case(name=name, seed=seed, **WORKLOADS[name])


def hand_case(pos: int) -> Case:
    """The hand-worked case: T=1, H=4, L=1, NH=1, D=4, Q rows 99, W_K=I, W_V=2I,
    no bias, k_norm weight 1, eps 0, theta 1e4, X = [1, 2, 3, 4]."""
    H = D = 4
    w = np.concatenate([np.full((4, 4), 99.0), np.eye(4), 2.0 * np.eye(4)], axis=0)
    return Case(
        name=f"hand_pos{pos}", dtype=BF16, T=1, H=H, L=1, NH=1, D=D, q_size=4, eps=0.0,
        theta=1e4, P=16, slots=4,
        x=to_bits(np.array([[1.0, 2.0, 3.0, 4.0]]), BF16),
        qkv_w=[to_bits(w, BF16)], qkv_b=None, k_norm_w=[to_bits(np.ones(4), BF16)],
        table=rope_table(16, D, 1e4), positions=np.array([pos], dtype=np.int64),
        locs=np.array([2], dtype=np.int64), commit_lens=None, row_width=0,
    )


def sentinel_pools(case: Case) -> tuple:
    """Per-layer K and V pools [slots, NH, D] filled with the 0xFFFF sentinel."""
    shape = (case.slots, case.NH, case.D)
    ks = [np.full(shape, SENTINEL, dtype=np.uint16) for _ in range(case.L)]
    vs = [np.full(shape, SENTINEL, dtype=np.uint16) for _ in range(case.L)]
    return ks, vs


# ---------------------------------------------------------------------------
# Inputs of the in-place table QK-RMSNorm + neox RoPE on a fused QKV tensor
# (sglang PR #31847, key source snippets: ``table_qk_norm_rope_``). A row of the
# tensor is [Q heads | K heads | V heads | padding up to the row stride].


@dataclasses.dataclass
class QkCase:
    """One synthetic instance of the in-place QK norm + rotation (host arrays)."""

    name: str
    dtype: str  # "bf16" | "fp16"
    T: int
    NHQ: int
    NHK: int
    D: int
    row_stride: int  # elements per row, >= (NHQ + 2 NHK) * D
    eps: float
    theta: float
    P: int
    weight_dtype: str  # dtype of the norm weights: the activation dtype or "fp32"
    qkv: np.ndarray  # uint16 [T, row_stride]
    q_w: np.ndarray  # [D] uint16 patterns, or float32 when weight_dtype == "fp32"
    k_w: np.ndarray
    table: np.ndarray  # float32 [P, D]
    positions: np.ndarray  # int64 [T]


def make_qk_case(
    *,
    name: str = "qk_case",
    T: int,
    NHQ: int,
    NHK: int,
    D: int,
    dtype: str = BF16,
    row_pad: int = 0,
    weight_fp32: bool = False,
    theta: float = 1e4,
    P: int = 4096,
    eps: float = 1e-6,
    seed: int = 0,
    positions_mode: str = "uniform",
) -> QkCase:
    """Draw one case. Order: head values, per-head scales, q_w, k_w, positions,
    padding. Head values are N(0, 1) times a per-(token, head) scale e^N(0, 0.5),
    so that head RMS values differ; V and padding columns are drawn too (they
    must come back unchanged)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    width = (NHQ + 2 * NHK) * D
    vals = rng.standard_normal((T, NHQ + 2 * NHK, D))
    scale = np.exp(rng.standard_normal((T, NHQ + 2 * NHK, 1)) * 0.5)
    qkv = np.empty((T, width + row_pad), dtype=np.uint16)
    qkv[:, :width] = to_bits((vals * scale).reshape(T, width), dtype)
    weight_dtype = "fp32" if weight_fp32 else dtype
    def weight():
        w = 1.0 + rng.standard_normal(D) * 0.1
        return w.astype(np.float32) if weight_fp32 else to_bits(w, dtype)
    q_w = weight()
    k_w = weight()
    if positions_mode == "uniform":
        positions = rng.integers(0, P, size=T, dtype=np.int64)
    elif positions_mode == "arange":
        positions = np.arange(T, dtype=np.int64)
    else:
        raise ValueError(positions_mode)
    if row_pad:
        qkv[:, width:] = to_bits(rng.standard_normal((T, row_pad)), dtype)
    return QkCase(name=name, dtype=dtype, T=T, NHQ=NHQ, NHK=NHK, D=D, row_stride=width + row_pad,
                  eps=eps, theta=theta, P=P, weight_dtype=weight_dtype, qkv=qkv, q_w=q_w,
                  k_w=k_w, table=rope_table(P, D, theta), positions=positions)


# Workloads of the QK op: a Qwen3-8B-like draft layer (32 query heads, 8 KV
# heads of 128), on a decode block of 32 requests x 8 tokens and on an 8k
# prompt.
QK_WORKLOADS = {
    "qk_decode": dict(T=256, NHQ=32, NHK=8, D=128, dtype=BF16, theta=1e6, P=32768),
    "qk_prefill_8k": dict(T=8192, NHQ=32, NHK=8, D=128, dtype=BF16, theta=1e6, P=32768,
                          positions_mode="arange"),
}
QK_WORKLOAD_ORDER = ["qk_decode", "qk_prefill_8k"]


def qk_workload(name: str) -> QkCase:
    """The named QK workload with its fixed seed (2000 + its 1-based index)."""
    seed = 2000 + QK_WORKLOAD_ORDER.index(name) + 1
    return make_qk_case(name=name, seed=seed, **QK_WORKLOADS[name])


# ---------------------------------------------------------------------------
# Inputs of the verify step's accept length and bonus token (sglang PR #31847,
# implementation breakdown step 2: ``compute_dflash_correct_drafts_and_bonus``):
# K drafted tokens per request against the target's K + 1 tokens.


@dataclasses.dataclass
class VerifyCase:
    name: str
    B: int
    K: int
    vocab: int
    draft: np.ndarray   # int64 [B, K]
    target: np.ndarray  # int64 [B, K + 1]


def make_verify_case(*, name: str = "verify_case", B: int, K: int, vocab: int = 151936,
                     seed: int = 0, match_len: Optional[np.ndarray] = None) -> VerifyCase:
    """Draw one case. Order: target tokens, matched-prefix lengths (uniform in
    [0, K] unless given), replacement tokens. The draft copies the target's
    first ``match_len[b]`` tokens, then differs at that position (a different
    token id), then holds random tokens that may or may not match again."""
    rng = np.random.Generator(np.random.PCG64(seed))
    target = rng.integers(0, vocab, size=(B, K + 1), dtype=np.int64)
    if match_len is None:
        match_len = rng.integers(0, K + 1, size=B, dtype=np.int64)
    match_len = np.asarray(match_len, dtype=np.int64)
    tail = rng.integers(0, vocab, size=(B, K), dtype=np.int64)
    draft = target[:, :K].copy()
    cols = np.arange(K)[None, :]
    after = cols > match_len[:, None]
    draft = np.where(after, tail, draft)
    at = cols == match_len[:, None]
    shift = 1 + rng.integers(0, vocab - 1, size=(B, K), dtype=np.int64)
    draft = np.where(at, (target[:, :K] + shift) % vocab, draft)  # never equal at the mismatch
    return VerifyCase(name=name, B=B, K=K, vocab=vocab, draft=draft, target=target)


# Verify workloads: a decode step of 32 requests x 7 drafts (blocks of 8), and
# a wide batch of 4096 requests x 15 drafts.
VERIFY_WORKLOADS = {
    "verify_decode": dict(B=32, K=7),
    "verify_wide": dict(B=4096, K=15),
}
VERIFY_WORKLOAD_ORDER = ["verify_decode", "verify_wide"]


def verify_workload(name: str) -> VerifyCase:
    """The named verify workload with its fixed seed (3000 + its 1-based index)."""
    seed = 3000 + VERIFY_WORKLOAD_ORDER.index(name) + 1
    return make_verify_case(name=name, seed=seed, **VERIFY_WORKLOADS[name])


# ---------------------------------------------------------------------------
# Inputs of the context producer ctx_hidden = main_norm(main_proj(aux)) (vLLM
# PR #46995, key source snippets: ``combine_hidden_states``): the target's
# auxiliary hidden states of n layers concatenated to [T, n*H], a bias-free
# [H, n*H] projection and an RMSNorm weight [H].


@dataclasses.dataclass
class ProjCase:
    name: str
    dtype: str
    T: int
    H: int        # output features (the draft's hidden size)
    n_aux: int    # number of target layers concatenated
    eps: float
    g_dtype: str  # norm weight dtype: the activation dtype or "fp32"
    aux: np.ndarray  # uint16 [T, n_aux * H]
    w: np.ndarray    # uint16 [H, n_aux * H]
    g: np.ndarray    # [H] patterns, or float32

    @property
    def K(self) -> int:
        return self.n_aux * self.H


def make_proj_case(*, name: str = "proj_case", T: int, H: int, n_aux: int = 3,
                   dtype: str = BF16, eps: float = 1e-6, g_fp32: bool = False,
                   seed: int = 0, aux_std: float = 1.0) -> ProjCase:
    """Draw one case. Order: aux, weight, norm weight. aux ~ N(0, aux_std) with a
    per-row scale e^N(0, 0.5) (row RMS values differ, which the norm removes);
    weight ~ N(0, 1/sqrt(n*H)) so that projected values are O(1); norm weight
    1 + N(0, 0.1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    K = n_aux * H
    aux = rng.standard_normal((T, K)) * aux_std * np.exp(rng.standard_normal((T, 1)) * 0.5)
    w = rng.standard_normal((H, K)) / np.sqrt(K)
    g = 1.0 + rng.standard_normal(H) * 0.1
    return ProjCase(name=name, dtype=dtype, T=T, H=H, n_aux=n_aux, eps=eps,
                    g_dtype="fp32" if g_fp32 else dtype, aux=to_bits(aux, dtype),
                    w=to_bits(w, dtype),
                    g=g.astype(np.float32) if g_fp32 else to_bits(g, dtype))


# Producer workloads: three target layers of a 4096-wide model (the
# decode_commit / prefill_8k shapes of the write), 256 and 8192 tokens.
PROJ_WORKLOADS = {
    "proj_decode": dict(T=256, H=4096, n_aux=3),
    "proj_prefill_8k": dict(T=8192, H=4096, n_aux=3),
}
PROJ_WORKLOAD_ORDER = ["proj_decode", "proj_prefill_8k"]


def proj_workload(name: str) -> ProjCase:
    """The named producer workload with its fixed seed (4000 + its 1-based index)."""
    seed = 4000 + PROJ_WORKLOAD_ORDER.index(name) + 1
    return make_proj_case(name=name, seed=seed, **PROJ_WORKLOADS[name])


# ---------------------------------------------------------------------------
# Inputs of the draft attention over the KV pool (sglang PR #35499, key source
# snippets: the shared-KV stage-1/stage-2 kernels with KV heads and the causal
# mask off): per request a block of query tokens, the request's prefix in a
# layer's pool [slots, NHK, D] listed by slot, and the block's own K/V.


@dataclasses.dataclass
class AttnCase:
    name: str
    dtype: str
    B: int
    block: int
    nhq: int
    nhk: int
    D: int
    sm_scale: float
    slots: int
    q: np.ndarray           # uint16 [B*block, nhq, D]
    k_ext: np.ndarray       # uint16 [B*block, nhk, D]
    v_ext: np.ndarray
    k_pool: np.ndarray      # uint16 [slots, nhk, D]
    v_pool: np.ndarray
    kv_indptr: np.ndarray   # int64 [B+1]
    kv_indices: np.ndarray  # int64 [kv_indptr[-1]]

    @property
    def max_prefix(self) -> int:
        return int(np.max(np.diff(self.kv_indptr))) if self.B else 0


def make_attn_case(*, name: str = "attn_case", B: int, block: int, nhq: int, nhk: int, D: int,
                   prefix, slots: int, dtype: str = BF16, seed: int = 0,
                   sm_scale: Optional[float] = None, q_std: float = 2.0) -> AttnCase:
    """Draw one case. Order: q, k_ext, v_ext, k_pool, v_pool, slot permutation.
    q ~ N(0, q_std) (peaky softmax rows), keys ~ N(0, 1), values ~ N(0.5, 1) (so
    that outputs are O(1)); requests own disjoint slots, taken in order from
    one seeded permutation of the pool; ``prefix`` is one length or one per
    request."""
    rng = np.random.Generator(np.random.PCG64(seed))
    prefix = np.broadcast_to(np.asarray(prefix, dtype=np.int64), (B,)).copy()
    if prefix.sum() > slots:
        raise ValueError("prefixes need more slots than the pool has")
    T = B * block
    q = to_bits(rng.standard_normal((T, nhq, D)) * q_std, dtype)
    k_ext = to_bits(rng.standard_normal((T, nhk, D)), dtype)
    v_ext = to_bits(rng.standard_normal((T, nhk, D)) + 0.5, dtype)
    k_pool = to_bits(rng.standard_normal((slots, nhk, D)), dtype)
    v_pool = to_bits(rng.standard_normal((slots, nhk, D)) + 0.5, dtype)
    perm = rng.permutation(slots).astype(np.int64)
    kv_indptr = np.concatenate([[0], np.cumsum(prefix)]).astype(np.int64)
    kv_indices = perm[:kv_indptr[-1]].copy()
    return AttnCase(name=name, dtype=dtype, B=B, block=block, nhq=nhq, nhk=nhk, D=D,
                    sm_scale=1.0 / np.sqrt(D) if sm_scale is None else sm_scale, slots=slots,
                    q=q, k_ext=k_ext, v_ext=v_ext, k_pool=k_pool, v_pool=v_pool,
                    kv_indptr=kv_indptr, kv_indices=kv_indices)


# Draft-attention workloads: the write's Qwen3-8B-like layer (32 query heads,
# 8 KV heads of 128) with 32 requests x blocks of 8 over 8k-token prefixes,
# and a head_dim-64 layer (16 query heads, 4 KV heads) over 16k-token prefixes.
ATTN_WORKLOADS = {
    "attn_decode_8k": dict(B=32, block=8, nhq=32, nhk=8, D=128, prefix=8192, slots=32 * 8192),
    "attn_d64_16k": dict(B=8, block=8, nhq=16, nhk=4, D=64, prefix=16384, slots=8 * 16384),
}
ATTN_WORKLOAD_ORDER = ["attn_decode_8k", "attn_d64_16k"]


def attn_workload(name: str) -> AttnCase:
    """The named draft-attention workload with its fixed seed (5000 + index)."""
    seed = 5000 + ATTN_WORKLOAD_ORDER.index(name) + 1
    return make_attn_case(name=name, seed=seed, **ATTN_WORKLOADS[name])


# ---------------------------------------------------------------------------
# One draft step's inputs for the operations chained on one device: the
# producer's auxiliary hidden states of the requests' prefix tokens (whose
# context K/V the stacked write stores), the draft block's fused QKV rows
# (normed and rotated in place, then the block's queries and own keys and
# values), and the attention over one layer's pool. The write's layer that
# the attention reads shares its K norm weight and rotary table with the QK op.


@dataclasses.dataclass
class DraftStepCase:
    name: str
    dtype: str
    B: int
    block: int
    layer: int              # the write's layer whose pool the attention reads
    prefix: np.ndarray      # int64 [B] prefix tokens per request
    proj: ProjCase          # T = prefix.sum() tokens, H features
    write: Case             # x is the producer's output (not drawn: zeros here)
    qk: QkCase              # T = B * block draft tokens
    kv_indptr: np.ndarray   # int64 [B+1]
    kv_indices: np.ndarray  # int64 [prefix.sum()]: the write's slots of each request's prefix
    sm_scale: float


def make_draft_step(*, name: str = "draft_step", B: int, block: int, prefix, H: int,
                    n_aux: int = 3, L: int = 2, NH: int = 2, NHQ: int = 8, D: int = 128,
                    dtype: str = BF16, slots: Optional[int] = None, P: int = 4096,
                    theta: float = 1e4, sm_scale: Optional[float] = None,
                    seed: int = 0) -> DraftStepCase:
    """Draw one draft step from the three generators above (seeds seed,
    seed + 1, seed + 2). Request b's prefix tokens sit at positions
    [0, prefix[b]) and the write's rows are the requests' prefixes in request
    order, stored at the write's random injective slots; the draft block of b
    sits at positions [prefix[b], prefix[b] + block). The last layer of the
    write is the attention's. ``sm_scale`` defaults to 1/sqrt(D); a larger
    one makes each query's output follow its few best-matching keys."""
    prefix = np.broadcast_to(np.asarray(prefix, dtype=np.int64), (B,)).copy()
    T = int(prefix.sum())
    if slots is None:
        slots = T + 16
    if int(prefix.max()) + block > P:
        raise ValueError("the rotary table is shorter than a request's positions")
    proj = make_proj_case(name=name + "_proj", T=T, H=H, n_aux=n_aux, dtype=dtype, seed=seed)
    write = make_case(name=name + "_write", T=T, H=H, L=L, NH=NH, D=D, dtype=dtype, theta=theta,
                      P=P, slots=slots, eps=proj.eps, seed=seed + 1)
    positions = np.concatenate([np.arange(n, dtype=np.int64) for n in prefix])
    write = dataclasses.replace(write, x=np.zeros_like(write.x), positions=positions)
    qk = make_qk_case(name=name + "_qk", T=B * block, NHQ=NHQ, NHK=NH, D=D, dtype=dtype, P=P,
                      theta=theta, eps=proj.eps, seed=seed + 2)
    qk_pos = np.concatenate([n + np.arange(block, dtype=np.int64) for n in prefix])
    layer = L - 1
    qk = dataclasses.replace(qk, k_w=write.k_norm_w[layer].copy(), table=write.table,
                             positions=qk_pos)
    kv_indptr = np.concatenate([[0], np.cumsum(prefix)]).astype(np.int64)
    return DraftStepCase(name=name, dtype=dtype, B=B, block=block, layer=layer, prefix=prefix,
                         proj=proj, write=write, qk=qk, kv_indptr=kv_indptr,
                         kv_indices=write.locs.copy(),
                         sm_scale=1.0 / np.sqrt(D) if sm_scale is None else sm_scale)
