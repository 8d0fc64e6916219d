"""Pins of the context-producer oracle main_norm(main_proj(.)) against a
hand-worked token, exact rational dot products, torch's linear and RMSNorm in
float64, the block structure of the concatenated input, and invariants."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import ctx_kv_oracle as O
from oracle import main_proj_oracle as M
from speculative_decoding_draft_stacked_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("which", ["w_identity_identity", "w_identity_zero"])
def test_hand_case(which):
    g = json.load(open(os.path.join(GOLDEN, "main_proj_case.json")))
    aux = W.to_bits(np.array([g["setup"]["aux"]], dtype=np.float64), "bf16")
    eye = np.eye(4)
    w = np.concatenate([eye, eye if which == "w_identity_identity" else 0 * eye], axis=1)
    out = M.combine_hidden_states(aux, W.to_bits(w, "bf16"), W.to_bits(np.ones(4), "bf16"),
                                  "bf16", 0.0, "bf16")
    assert out[0].tolist() == g["expected"][which]


def test_projection_matches_exact_rationals():
    """Each output of a tiny case equals the exactly computed dot product,
    rounded once: the fp64 sum of products of bf16 numbers over K = 24 terms
    is exact or within one fp64 ulp, far below the bf16 spacing."""
    c = W.make_proj_case(T=3, H=8, n_aux=3, seed=2)
    y = M.main_proj(c.aux, c.w, "bf16")
    a = O.decode(c.aux, "bf16")
    w = O.decode(c.w, "bf16")
    for t in range(3):
        for h in range(8):
            exact = sum(Fraction(float(a[t, k])) * Fraction(float(w[h, k])) for k in range(24))
            assert y[t, h] == O.round_to(np.array([float(exact)]), "bf16")[0]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_against_torch_linear_and_rms_norm(dtype):
    c = W.make_proj_case(T=20, H=256, n_aux=2, dtype=dtype, seed=3)
    x = torch.from_numpy(O.decode(c.aux, dtype))
    w = torch.from_numpy(O.decode(c.w, dtype))
    y = O.round_to(torch.nn.functional.linear(x, w).numpy(), dtype)
    assert np.array_equal(M.main_proj(c.aux, c.w, dtype), y)
    g = torch.from_numpy(O.decode(c.g, dtype))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(y), (256,), eps=c.eps) * g
    want = O.round_to(ref.numpy(), dtype)
    assert np.array_equal(M.main_norm(y, c.g, dtype, c.eps, dtype), want)


def test_concatenated_blocks_add_up():
    """y = sum over the n auxiliary layers of aux_j @ W_j^T (block columns of
    the weight), before the rounding."""
    c = W.make_proj_case(T=6, H=64, n_aux=3, seed=4)
    a = O.decode(c.aux, "bf16")
    w = O.decode(c.w, "bf16")
    blocks = sum(a[:, j * 64:(j + 1) * 64] @ w[:, j * 64:(j + 1) * 64].T for j in range(3))
    assert np.array_equal(M.main_proj(c.aux, c.w, "bf16"), O.round_to(blocks, "bf16"))


def test_doubling_the_input_leaves_the_output_unchanged():
    """2*aux doubles y exactly (bf16 rounding commutes with doubling), and at
    eps = 0 the norm removes the factor: identical output bits."""
    c = W.make_proj_case(T=10, H=128, n_aux=3, seed=5)
    a2 = W.to_bits(O.decode(c.aux, "bf16") * 2.0, "bf16")
    base = M.combine_hidden_states(c.aux, c.w, c.g, "bf16", 0.0, "bf16")
    twice = M.combine_hidden_states(a2, c.w, c.g, "bf16", 0.0, "bf16")
    assert np.array_equal(base, twice)


def test_unit_weight_gives_unit_rms():
    c = W.make_proj_case(T=16, H=512, n_aux=2, seed=6)
    ones = W.to_bits(np.ones(512), "bf16")
    out = M.combine_hidden_states(c.aux, c.w, ones, "bf16", 0.0, "bf16")
    rms = np.sqrt(np.mean(out * out, axis=1))
    assert np.all(np.abs(rms - 1.0) < 2 ** -8)


def test_rows_are_independent():
    c = W.make_proj_case(T=12, H=128, n_aux=2, seed=7)
    perm = np.random.default_rng(0).permutation(12)
    a = M.combine_hidden_states(c.aux, c.w, c.g, "bf16", c.eps, "bf16")
    b = M.combine_hidden_states(c.aux[perm], c.w, c.g, "bf16", c.eps, "bf16")
    assert np.array_equal(a[perm], b)


def test_fp32_norm_weight_equals_patterns_of_the_same_values():
    c = W.make_proj_case(T=5, H=128, n_aux=2, seed=8, dtype="fp16")
    y = M.main_proj(c.aux, c.w, "fp16")
    gf = O.decode(c.g, "fp16").astype(np.float32)
    assert np.array_equal(M.main_norm(y, c.g, "fp16", c.eps, "fp16"),
                          M.main_norm(y, gf, "fp32", c.eps, "fp16"))


def test_fp32_norm_weight_keeps_values_outside_the_fp16_range():
    """fp32 norm weights of 2^-30 times bf16 values (exact in fp32 and bf16,
    below fp16's smallest subnormal) give the same bits as the bf16 patterns
    of those values, and nonzero outputs."""
    c = W.make_proj_case(T=5, H=128, n_aux=2, seed=9)
    y = M.main_proj(c.aux, c.w, "bf16")
    gv = O.decode(c.g, "bf16") * 2.0 ** -30
    a = M.main_norm(y, W.to_bits(gv, "bf16"), "bf16", c.eps, "bf16")
    assert np.array_equal(a, M.main_norm(y, gv.astype(np.float32), "fp32", c.eps, "bf16"))
    assert np.count_nonzero(a) > 0.9 * a.size
