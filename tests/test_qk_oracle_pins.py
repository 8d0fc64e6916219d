"""Pins of the QK-norm + rotation oracle against facts that do not come from
the oracle itself: the hand-worked row in tests/golden/hand_case.json (the same
norm + rotation of one head, worked by hand), exact scaling relations, the
textbook RMSNorm of torch at position 0, complex multiplication for the
rotation, and the column bookkeeping of the fused QKV row.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import ctx_kv_oracle as O
from oracle import qk_norm_rope_oracle as Q
from speculative_decoding_draft_stacked_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand_row(q, k, v, pad, dtype="bf16"):
    vals = np.array(q + k + v + pad, dtype=np.float64)
    return W.to_bits(vals, dtype)[None, :]


def _run(qkv, pos, q_w, k_w, table, nhq, nhk, D, eps=0.0, dtype="bf16", weight_dtype="bf16"):
    out = qkv.copy()
    skipped = Q.qk_norm_rope_inplace(out, pos, q_w, k_w, weight_dtype, table, nhq, nhk, D, eps,
                                     dtype)
    return out, skipped


@pytest.mark.parametrize("pos", [0, 1, 7])
def test_hand_row(pos):
    """Row [Q | K | V | pad] with Q = K = [1, 2, 3, 4]: the key head (weight 1,
    eps 0, theta 1e4) must give the hand-worked K of the golden file; the query
    head has weight 2, and doubling commutes with round-to-nearest-even away
    from overflow and underflow, so it must give exactly twice that. V and the
    padding keep their bits."""
    g = json.load(open(os.path.join(GOLDEN, "hand_case.json")))
    expect_k = np.array(g["expected"][f"pos{pos}"]["k"])
    row = _hand_row([1, 2, 3, 4], [1, 2, 3, 4], [5, 6, 7, 8], [9, 10])
    table = W.rope_table(16, 4, 1e4)
    q_w = W.to_bits(np.full(4, 2.0), "bf16")
    k_w = W.to_bits(np.ones(4), "bf16")
    out, skipped = _run(row, np.array([pos]), q_w, k_w, table, 1, 1, 4)
    vals = O.decode(out[0], "bf16")
    assert skipped == 0
    assert np.array_equal(vals[4:8], expect_k)
    assert np.array_equal(vals[0:4], 2.0 * expect_k)
    assert np.array_equal(out[0, 8:], row[0, 8:])


def test_weights_go_to_their_heads():
    """Identical query and key head values with k_w = 2 q_w: every key output is
    exactly twice the query output of the same values."""
    rng = np.random.default_rng(3)
    D, T = 64, 40
    vals = rng.standard_normal((T, D))
    qkv = W.to_bits(np.concatenate([vals, vals, vals], axis=1), "bf16")
    w = 1.0 + rng.standard_normal(D) * 0.1
    q_w = W.to_bits(w, "bf16")
    k_w = W.to_bits(2.0 * O.decode(q_w, "bf16"), "bf16")
    table = W.rope_table(512, D, 1e4)
    out, _ = _run(qkv, rng.integers(0, 512, T), q_w, k_w, table, 1, 1, D, eps=1e-6)
    qo = O.decode(out[:, :D], "bf16")
    ko = O.decode(out[:, D:2 * D], "bf16")
    assert np.array_equal(ko, 2.0 * qo)
    assert np.array_equal(out[:, 2 * D:], qkv[:, 2 * D:])


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_position_zero_is_torch_rms_norm(dtype):
    """Table row 0 is cos = 1, sin = 0 exactly, so the output is the rounded
    textbook RMSNorm (torch.nn.functional.rms_norm in float64)."""
    c = W.make_qk_case(T=30, NHQ=3, NHK=2, D=128, dtype=dtype, seed=4, P=8)
    pos = np.zeros(c.T, dtype=np.int64)
    out, _ = _run(c.qkv, pos, c.q_w, c.k_w, c.table, 3, 2, 128, eps=c.eps, dtype=dtype,
                  weight_dtype=dtype)
    x = torch.from_numpy(O.decode(c.qkv[:, :5 * 128], dtype).reshape(c.T, 5, 128))
    w = torch.from_numpy(np.stack([O.decode(c.q_w, dtype)] * 3 + [O.decode(c.k_w, dtype)] * 2))
    ref = torch.nn.functional.rms_norm(x, (128,), eps=c.eps) * w[None]
    ref = O.round_to(ref.numpy(), dtype)
    got = O.decode(out[:, :5 * 128], dtype).reshape(c.T, 5, 128)
    assert np.array_equal(got, ref)


def test_rotation_is_complex_multiplication():
    """Output at position p is round((a + i b) * (cos + i sin)) over the pairs
    (i, i + D/2), where a | b is the output at position 0 (the rounded
    normalised head): numpy complex products, independent of the oracle's
    rotation code."""
    c = W.make_qk_case(T=50, NHQ=2, NHK=2, D=64, seed=5, P=4096, theta=1e4)
    zero, _ = _run(c.qkv, np.zeros(c.T, np.int64), c.q_w, c.k_w, c.table, 2, 2, 64, eps=c.eps)
    rot, _ = _run(c.qkv, c.positions, c.q_w, c.k_w, c.table, 2, 2, 64, eps=c.eps)
    xn = O.decode(zero[:, :4 * 64], "bf16").reshape(c.T, 4, 64)
    z = xn[..., :32] + 1j * xn[..., 32:]
    t = c.table[c.positions].astype(np.float64)
    e = t[:, None, :32] + 1j * t[:, None, 32:]
    prod = z * e
    ref = O.round_to(np.concatenate([prod.real, prod.imag], axis=-1), "bf16")
    got = O.decode(rot[:, :4 * 64], "bf16").reshape(c.T, 4, 64)
    assert np.array_equal(got, ref)


def test_power_of_two_scaling_leaves_output_unchanged():
    """With eps = 0 the norm divides by the head's own RMS: scaling one head's
    values by 2^k changes no output bit of any head."""
    c = W.make_qk_case(T=20, NHQ=2, NHK=1, D=128, seed=6)
    base, _ = _run(c.qkv, c.positions, c.q_w, c.k_w, c.table, 2, 1, 128)
    scaled = c.qkv.copy()
    vals = O.decode(scaled[:, 128:256], "bf16") * 8.0
    scaled[:, 128:256] = W.to_bits(vals, "bf16")
    out, _ = _run(scaled, c.positions, c.q_w, c.k_w, c.table, 2, 1, 128)
    assert np.array_equal(out[:, :3 * 128], base[:, :3 * 128])


def test_heads_are_independent():
    """Changing one head (or V) changes no other head's output."""
    c = W.make_qk_case(T=16, NHQ=2, NHK=2, D=64, seed=7)
    base, _ = _run(c.qkv, c.positions, c.q_w, c.k_w, c.table, 2, 2, 64, eps=c.eps)
    mod = c.qkv.copy()
    mod[:, 64:128] = W.to_bits(np.full((16, 64), 3.0), "bf16")   # query head 1
    mod[:, 4 * 64:] = W.to_bits(np.full((16, 2 * 64), 7.0), "bf16")  # V
    out, _ = _run(mod, c.positions, c.q_w, c.k_w, c.table, 2, 2, 64, eps=c.eps)
    keep = np.r_[0:64, 128:256]
    assert np.array_equal(out[:, keep], base[:, keep])
    assert not np.array_equal(out[:, 64:128], base[:, 64:128])


def test_out_of_range_positions_untouched_and_counted():
    c = W.make_qk_case(T=12, NHQ=1, NHK=1, D=64, seed=8, P=100)
    pos = c.positions.copy()
    pos[[2, 5, 9]] = [-1, 100, 10 ** 9]
    out, skipped = _run(c.qkv, pos, c.q_w, c.k_w, c.table, 1, 1, 64, eps=c.eps)
    assert skipped == 3
    assert np.array_equal(out[[2, 5, 9]], c.qkv[[2, 5, 9]])
    others = np.setdiff1d(np.arange(12), [2, 5, 9])
    assert not np.array_equal(out[others, :128], c.qkv[others, :128])


def test_fp32_weights_equal_patterns_of_the_same_values():
    c = W.make_qk_case(T=10, NHQ=2, NHK=1, D=128, seed=9, dtype="fp16")
    a, _ = _run(c.qkv, c.positions, c.q_w, c.k_w, c.table, 2, 1, 128, eps=c.eps, dtype="fp16",
                weight_dtype="fp16")
    qf = O.decode(c.q_w, "fp16").astype(np.float32)
    kf = O.decode(c.k_w, "fp16").astype(np.float32)
    b, _ = _run(c.qkv, c.positions, qf, kf, c.table, 2, 1, 128, eps=c.eps, dtype="fp16",
                weight_dtype="fp32")
    assert np.array_equal(a, b)


def test_fp32_weights_keep_values_outside_the_fp16_range():
    """fp32 weights of 2^-30 times bf16 values (exact in fp32 and bf16, far
    below fp16's smallest subnormal) give the same bits as the bf16 patterns
    of those values: an fp32 weight is used at its own value, not narrowed."""
    c = W.make_qk_case(T=9, NHQ=2, NHK=1, D=64, seed=12)
    qv = O.decode(c.q_w, "bf16") * 2.0 ** -30
    kv = O.decode(c.k_w, "bf16") * 2.0 ** -30
    a, _ = _run(c.qkv, c.positions, W.to_bits(qv, "bf16"), W.to_bits(kv, "bf16"), c.table, 2, 1,
                64, eps=c.eps)
    b, _ = _run(c.qkv, c.positions, qv.astype(np.float32), kv.astype(np.float32), c.table, 2, 1,
                64, eps=c.eps, weight_dtype="fp32")
    assert np.array_equal(a, b)
    assert np.count_nonzero(O.decode(a[:, :192], "bf16")) > 0.9 * a[:, :192].size


def test_key_heads_agree_with_the_write_oracle():
    """Consistency with the stacked write's oracle (same arithmetic, other
    entry point): the key heads equal apply_k_rope(apply_k_norm(...))."""
    c = W.make_qk_case(T=25, NHQ=3, NHK=2, D=128, seed=10)
    out, _ = _run(c.qkv, c.positions, c.q_w, c.k_w, c.table, 3, 2, 128, eps=c.eps)
    k = O.decode(c.qkv[:, 3 * 128:5 * 128], "bf16").reshape(c.T, 2, 128)
    ref = O.apply_k_rope(c.positions, O.apply_k_norm(k, c.k_w, c.eps, "bf16"), c.table, "bf16")
    got = O.decode(out[:, 3 * 128:5 * 128], "bf16").reshape(c.T, 2, 128)
    assert np.array_equal(got, ref)


def test_eps_dominated_heads_follow_torch_rms_norm():
    """Heads of tiny values (mean square far below eps) at position 0: the
    output is the rounded torch RMSNorm, which there is dominated by eps."""
    c = W.make_qk_case(T=8, NHQ=1, NHK=1, D=64, seed=11, P=4, eps=1e-5)
    small = O.decode(c.qkv, "bf16") * 2.0 ** -14
    qkv = W.to_bits(small, "bf16")
    out, _ = _run(qkv, np.zeros(8, np.int64), c.q_w, c.k_w, c.table, 1, 1, 64, eps=c.eps)
    x = torch.from_numpy(O.decode(qkv[:, :128], "bf16").reshape(8, 2, 64))
    w = torch.from_numpy(np.stack([O.decode(c.q_w, "bf16"), O.decode(c.k_w, "bf16")]))
    ref = O.round_to((torch.nn.functional.rms_norm(x, (64,), eps=c.eps) * w[None]).numpy(),
                     "bf16")
    got = O.decode(out[:, :128], "bf16").reshape(8, 2, 64)
    assert np.array_equal(got, ref)
    assert np.abs(got).max() < 0.5  # eps really dominates: unit-RMS heads would reach ~1
