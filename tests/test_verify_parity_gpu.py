"""Parity of the HIP verify accept length + bonus token (through the C ABI)
with the CPU oracle: integer results, compared exactly."""

import numpy as np
import pytest
import torch

import speculative_decoding_draft_stacked_amd as dk
from speculative_decoding_draft_stacked_amd import workloads as W
from oracle import verify_oracle as V

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    dk.lib()


def _run(draft, target, label, pad=0):
    """Run on the device (rows optionally padded to exercise strides) and
    compare with the oracle exactly."""
    B, K = draft.shape
    say(f"[verify] {label}: B={B} K={K} pad={pad}")
    dd = torch.zeros(B, K + pad, dtype=torch.int64)
    dd[:, :K] = torch.from_numpy(draft)
    tt = torch.zeros(B, K + 1 + pad, dtype=torch.int64)
    tt[:, :K + 1] = torch.from_numpy(target)
    dd, tt = dd.cuda()[:, :K], tt.cuda()[:, :K + 1]
    acc = torch.full((B,), -7, dtype=torch.int64, device="cuda")
    bon = torch.full((B,), -7, dtype=torch.int64, device="cuda")
    dk.verify_accept(dd, tt, acc, bon)
    torch.cuda.synchronize()
    ea, eb = V.accept_and_bonus(draft, target)
    assert np.array_equal(acc.cpu().numpy(), ea), label
    assert np.array_equal(bon.cpu().numpy(), eb), label
    return acc, bon


CASES = {
    # K, vocab, B: every lane-group width (1..64 lanes) and the chunked path
    "k7_decode_blocks": (7, 151936, 1000),
    "k1": (1, 3, 257),
    "k3_tiny_vocab": (3, 2, 513),
    "k15": (15, 4, 999),
    "k31": (31, 2, 300),
    "k32": (32, 2, 300),
    "k64": (64, 2, 130),
    "k65_chunked": (65, 2, 70),
    "k200_chunked": (200, 2, 33),
}


@pytest.mark.parametrize("name", list(CASES))
def test_cases(name):
    K, vocab, B = CASES[name]
    rng = np.random.default_rng(K * 7 + B)
    c = W.make_verify_case(B=B, K=K, vocab=max(vocab, 2), seed=K + B)
    # also fully random rows (later re-matches) on small vocabularies
    draft = c.draft.copy()
    target = c.target.copy()
    half = B // 2
    draft[half:] = rng.integers(0, vocab, size=(B - half, K))
    target[half:] = rng.integers(0, vocab, size=(B - half, K + 1))
    _run(draft, target, name)
    _run(draft, target, name + " padded rows", pad=5)


@pytest.mark.parametrize("name", W.VERIFY_WORKLOAD_ORDER)
def test_workloads(name):
    c = W.verify_workload(name)
    _run(c.draft, c.target, name)


def test_no_drafts_and_no_requests():
    target = np.array([[5], [6], [7]], dtype=np.int64)
    _run(np.zeros((3, 0), dtype=np.int64), target, "K=0")
    acc = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    empty_d = torch.zeros(0, 4, dtype=torch.int64, device="cuda")
    empty_t = torch.zeros(0, 5, dtype=torch.int64, device="cuda")
    dk.verify_accept(empty_d, empty_t, acc, acc)
    torch.cuda.synchronize()
    assert acc.item() == -7


def test_large_ids():
    d = np.array([[1 << 40, 5], [1 << 33, 5], [(1 << 62) + 3, 7]], dtype=np.int64)
    t = np.array([[(1 << 40) + (1 << 33), 5, 9], [0, 5, 9], [(1 << 62) + 3, 7, 1 << 61]],
                 dtype=np.int64)
    _run(d, t, "64-bit ids")


def test_graph_replays_match_eager():
    c = W.make_verify_case(B=200, K=7, vocab=5, seed=77)
    acc_ref, bon_ref = _run(c.draft, c.target, "eager reference")
    dd = torch.from_numpy(c.draft).cuda()
    tt = torch.from_numpy(c.target).cuda()
    acc = torch.empty(200, dtype=torch.int64, device="cuda")
    bon = torch.empty(200, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            dk.verify_accept(dd, tt, acc, bon, stream=side)
    for rep in range(4):
        acc.fill_(-1)
        bon.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(acc, acc_ref) and torch.equal(bon, bon_ref), rep


@pytest.mark.parametrize("i", range(24))
def test_random_shapes(i):
    """Seeded sweep: request count 1..3000, draft length 0..260, vocabulary 2
    to 2^40 (64-bit ids), matched-prefix lengths from the generator, row
    padding; compared exactly."""
    rng = np.random.default_rng(7900 + i)
    B = int(rng.integers(1, 3001))
    K = int(rng.choice([int(rng.integers(0, 9)), int(rng.integers(9, 66)),
                        int(rng.integers(66, 261))]))
    vocab = int(rng.choice([2, 7, 151936, 1 << 40]))
    if K == 0:
        draft = np.zeros((B, 0), dtype=np.int64)
        target = rng.integers(0, vocab, size=(B, 1), dtype=np.int64)
    else:
        c = W.make_verify_case(B=B, K=K, vocab=vocab, seed=7900 + i)
        draft, target = c.draft, c.target
    _run(draft, target, f"verify_sweep{i}", pad=int(rng.choice([0, 3])))

