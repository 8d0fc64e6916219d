"""Pins of the draft-attention oracle against a hand-worked block, torch's
scaled_dot_product_attention in float64, closed forms (uniform and one-hot
attention), the grouped-query head mapping, and key-order invariance."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import ctx_kv_oracle as O
from oracle import draft_attention_oracle as A
from speculative_decoding_draft_stacked_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x, dtype="bf16"):
    return W.to_bits(np.asarray(x, dtype=np.float64), dtype)


def test_hand_case():
    g = json.load(open(os.path.join(GOLDEN, "draft_attention_case.json")))
    kp = np.zeros((8, 1, 2)); vp = np.zeros((8, 1, 2))
    kp[5, 0] = g["setup"]["pool"]["slot 5"]["k"]
    vp[5, 0] = g["setup"]["pool"]["slot 5"]["v"]
    q = np.array(g["setup"]["q"], dtype=np.float64)[:, None, :]
    ke = np.array(g["setup"]["k_ext"], dtype=np.float64)[:, None, :]
    ve = np.array(g["setup"]["v_ext"], dtype=np.float64)[:, None, :]
    out, skipped = A.draft_attention(_bits(q), _bits(ke), _bits(ve), _bits(kp), _bits(vp),
                                     [0, 1], [5], 2, 1, 1, math.log(2.0), "bf16")
    assert skipped == 0
    assert out.tolist() == g["expected"]


def test_against_torch_sdpa():
    """Per request: torch SDPA (float64, no mask) over [prefix keys; block keys]
    with KV heads repeated for their query-head groups."""
    c = W.make_attn_case(B=3, block=4, nhq=8, nhk=2, D=64, prefix=[5, 0, 37], slots=64, seed=1)
    out, _ = A.draft_attention(c.q, c.k_ext, c.v_ext, c.k_pool, c.v_pool, c.kv_indptr,
                               c.kv_indices, c.block, c.nhq, c.nhk, c.sm_scale, c.dtype)
    q = O.decode(c.q, "bf16"); ke = O.decode(c.k_ext, "bf16"); ve = O.decode(c.v_ext, "bf16")
    kp = O.decode(c.k_pool, "bf16"); vp = O.decode(c.v_pool, "bf16")
    for b in range(3):
        idx = c.kv_indices[c.kv_indptr[b]:c.kv_indptr[b + 1]]
        r = slice(b * 4, (b + 1) * 4)
        K = torch.from_numpy(np.concatenate([kp[idx], ke[r]])).permute(1, 0, 2)
        V = torch.from_numpy(np.concatenate([vp[idx], ve[r]])).permute(1, 0, 2)
        K = K.repeat_interleave(4, dim=0)
        V = V.repeat_interleave(4, dim=0)
        Q = torch.from_numpy(q[r]).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=c.sm_scale)
        want = O.round_to(ref.permute(1, 0, 2).numpy(), "bf16")
        assert np.array_equal(out[r], want)


def test_uniform_scores_give_the_mean_of_values():
    """A zero query scores every key 0: the output is the mean of the values."""
    c = W.make_attn_case(B=2, block=2, nhq=2, nhk=1, D=64, prefix=[6, 2], slots=16, seed=2)
    q = np.zeros_like(c.q)
    out, _ = A.draft_attention(q, c.k_ext, c.v_ext, c.k_pool, c.v_pool, c.kv_indptr,
                               c.kv_indices, 2, 2, 1, c.sm_scale, "bf16")
    vp = O.decode(c.v_pool, "bf16"); ve = O.decode(c.v_ext, "bf16")
    for b in range(2):
        idx = c.kv_indices[c.kv_indptr[b]:c.kv_indptr[b + 1]]
        mean = np.concatenate([vp[idx, 0], ve[2 * b:2 * b + 2, 0]]).mean(axis=0)
        for r in range(2 * b, 2 * b + 2):
            for h in range(2):
                assert np.array_equal(out[r, h], O.round_to(mean, "bf16"))


def test_one_hot_attention_and_head_groups():
    """A query aligned with a single large key picks that key's value; query
    head h reads KV head h // G (distinct values per KV head)."""
    D, nhq, nhk = 64, 4, 2
    kp = np.zeros((10, nhk, D)); vp = np.zeros((10, nhk, D))
    for kh in range(nhk):
        vp[:, kh, :] = np.arange(10)[:, None] + 100 * kh
    kp[7, :, 0] = 8.0  # slot 7 stands out along feature 0
    q = np.zeros((1, nhq, D)); q[0, :, 0] = 8.0
    ke = np.zeros((1, nhk, D)); ve = np.full((1, nhk, D), -3.0)
    out, _ = A.draft_attention(_bits(q), _bits(ke), _bits(ve), _bits(kp), _bits(vp), [0, 10],
                               np.arange(10), 1, nhq, nhk, 1.0, "bf16")
    for h in range(nhq):
        assert np.all(out[0, h] == 7 + 100 * (h // 2))  # exp(64) dwarfs the rest


def test_key_order_does_not_matter():
    c = W.make_attn_case(B=1, block=3, nhq=4, nhk=4, D=128, prefix=[50], slots=64, seed=3)
    perm = np.random.default_rng(0).permutation(50)
    a, _ = A.draft_attention(c.q, c.k_ext, c.v_ext, c.k_pool, c.v_pool, c.kv_indptr,
                             c.kv_indices, 3, 4, 4, c.sm_scale, "bf16")
    b, _ = A.draft_attention(c.q, c.k_ext, c.v_ext, c.k_pool, c.v_pool, c.kv_indptr,
                             c.kv_indices[perm], 3, 4, 4, c.sm_scale, "bf16")
    assert np.array_equal(a, b)


def test_out_of_pool_slots_are_skipped_and_counted():
    c = W.make_attn_case(B=1, block=2, nhq=2, nhk=1, D=64, prefix=[6], slots=16, seed=4)
    bad = c.kv_indices.copy()
    bad[[1, 4]] = [-1, 16]
    a, skipped = A.draft_attention(c.q, c.k_ext, c.v_ext, c.k_pool, c.v_pool, c.kv_indptr, bad,
                                   2, 2, 1, c.sm_scale, "bf16")
    keep = np.delete(c.kv_indices, [1, 4])
    b, _ = A.draft_attention(c.q, c.k_ext, c.v_ext, c.k_pool, c.v_pool, [0, 4], keep, 2, 2, 1,
                             c.sm_scale, "bf16")
    assert skipped == 2 and np.array_equal(a, b)
