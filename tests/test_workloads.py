"""The seeded input generator: deterministic, with the shapes, distributions
and index structure of the five workloads."""

import numpy as np
import pytest

from speculative_decoding_draft_stacked_amd import workloads as W


def _f(bits, dtype):
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def test_deterministic_per_seed():
    a = W.make_case(T=16, H=64, L=2, NH=2, D=64, row_width=8, seed=3, slots=64)
    b = W.make_case(T=16, H=64, L=2, NH=2, D=64, row_width=8, seed=3, slots=64)
    c = W.make_case(T=16, H=64, L=2, NH=2, D=64, row_width=8, seed=4, slots=64)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.locs, b.locs)
    assert np.array_equal(a.commit_lens, b.commit_lens)
    assert all(np.array_equal(p, q) for p, q in zip(a.qkv_w, b.qkv_w))
    assert not np.array_equal(a.x, c.x)


def test_tiny_workload_shape_and_statistics():
    c = W.workload("tiny")
    assert (c.T, c.H, c.L, c.NH, c.D, c.slots, c.P) == (16, 256, 2, 2, 64, 64, 4096)
    assert c.commit_lens is None and c.qkv_b is None
    assert len(set(c.locs.tolist())) == c.T and c.locs.min() >= 0 and c.locs.max() < c.slots
    assert c.positions.min() >= 0 and c.positions.max() < c.P
    w = _f(c.qkv_w[0], "bf16")
    assert abs(w[c.q_size:].std() - 0.02) < 0.002           # K/V rows ~N(0, 0.02)
    assert abs(w[:c.q_size].std() - 1.0) < 0.05             # Q rows ~N(0, 1)
    g = _f(c.k_norm_w[0], "bf16")
    assert abs(g.mean() - 1.0) < 0.05
    assert not np.array_equal(c.qkv_w[0], c.qkv_w[1])       # distinct per layer


@pytest.mark.parametrize("name", ["decode_commit", "wide_gqa_d64", "decode_commit_kv1",
                                  "decode_commit_kv2"])
def test_commit_workloads_windows(name):
    spec = W.WORKLOADS[name]
    # cheap copy of the index structure without drawing the full weights
    c = W.make_case(name=name, seed=1, **dict(spec, H=8))
    assert c.row_width == 8 and c.T % 8 == 0
    assert c.commit_lens.min() >= 1 and c.commit_lens.max() <= 8
    assert len(set(c.locs.tolist())) == c.T


def test_prefill_indices_contiguous():
    c = W.make_case(name="p", seed=1, **dict(W.WORKLOADS["prefill_8k"], H=8))
    assert np.array_equal(c.positions, np.arange(8192))
    assert np.array_equal(c.locs, 4096 + np.arange(8192))
    assert c.locs.max() < c.slots


def test_rope_table_structure():
    t = W.rope_table(4096, 64, 1e4)
    assert t.dtype == np.float32 and t.shape == (4096, 64)
    assert np.all(t[0, :32] == 1.0) and np.all(t[0, 32:] == 0.0)
    np.testing.assert_allclose(t[:, :32] ** 2 + t[:, 32:] ** 2, 1.0, atol=2e-7)


def test_fp16_workload_has_bias():
    c = W.make_case(name="b", seed=1, **dict(W.WORKLOADS["biased_fp16"], H=8, T=32))
    assert c.dtype == "fp16" and c.qkv_b is not None
    assert c.qkv_b[0].shape == (c.q_size + 2 * c.kv,)


def test_draft_step_inputs_line_up():
    """The chained draft step's inputs: the write's rows are the requests'
    prefixes in order at positions 0..n-1, the attention lists exactly the
    write's slots per request, the draft block follows each prefix, and the
    QK op's key norm weight and table are the attention layer's."""
    s = W.make_draft_step(B=3, block=4, prefix=[5, 0, 9], H=64, L=2, NH=1, NHQ=2, D=64,
                          seed=3)
    assert s.write.T == s.proj.T == 14 and s.qk.T == 12
    assert s.write.positions.tolist() == list(range(5)) + list(range(9))
    assert s.kv_indptr.tolist() == [0, 5, 5, 14]
    assert np.array_equal(s.kv_indices, s.write.locs)
    assert len(set(s.write.locs.tolist())) == 14 and s.write.locs.max() < s.write.slots
    assert s.qk.positions.tolist() == [5, 6, 7, 8, 0, 1, 2, 3, 9, 10, 11, 12]
    assert np.array_equal(s.qk.k_w, s.write.k_norm_w[s.layer]) and s.layer == 1
    assert s.qk.table is s.write.table and s.qk.eps == s.write.eps == s.proj.eps
    assert not s.write.x.any()  # the producer's output, not drawn
