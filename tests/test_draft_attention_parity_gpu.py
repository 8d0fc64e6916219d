"""Parity of the HIP draft attention (through the C ABI) with the CPU oracle.

Tolerance: |gpu - oracle| <= atol + rtol*|oracle| elementwise with (rtol,
atol) = (2e-2, 2e-2) for bf16 and (5e-3, 5e-3) for fp16. The kernel rounds the
probabilities to the dtype for the value product (flash-attention style);
that error is well inside these bounds for O(1) outputs.
"""

import numpy as np
import pytest
import torch

import speculative_decoding_draft_stacked_amd as dk
from speculative_decoding_draft_stacked_amd import workloads as W
from oracle import ctx_kv_oracle as O
from oracle import draft_attention_oracle as A

from gpu_util import TOL, say

pytestmark = pytest.mark.gpu
_T = {"bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    dk.lib()


def _dev16(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(_T[dtype]).cuda()


class DevAttn:
    def __init__(self, c, max_prefix=None, indices=None):
        self.c = c
        self.q = _dev16(c.q, c.dtype)
        self.ke, self.ve = _dev16(c.k_ext, c.dtype), _dev16(c.v_ext, c.dtype)
        self.kp, self.vp = _dev16(c.k_pool, c.dtype), _dev16(c.v_pool, c.dtype)
        self.indptr = torch.from_numpy(c.kv_indptr).cuda()
        idx = c.kv_indices if indices is None else indices
        self.indices = torch.from_numpy(idx if len(idx) else np.zeros(1, np.int64)).cuda()
        self.out = torch.full(c.q.shape, -7, dtype=torch.int16, device="cuda").view(_T[c.dtype])
        self.max_prefix = c.max_prefix if max_prefix is None else max_prefix
        n = dk.draft_attention_workspace_bytes(c.B, c.block, c.nhq, c.nhk, c.D, self.max_prefix)
        self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
        self.err = torch.zeros(1, dtype=torch.int64, device="cuda")

    def run(self, stream=None):
        assert dk.draft_attention(self.q, self.ke, self.ve, self.kp, self.vp, self.indptr,
                                  self.indices, self.out, self.c.block, self.c.sm_scale,
                                  self.max_prefix, self.ws, self.err, stream=stream)

    def host(self):
        torch.cuda.synchronize()
        return self.out.view(torch.int16).cpu().numpy().view(np.uint16)


def _compare(c, got, want, rows, label):
    g = O.decode(got[rows], c.dtype)
    w = want[rows]
    assert np.all(np.isfinite(g)), label
    rtol, atol = TOL[c.dtype]
    err = np.abs(g - w)
    bad = err > atol + rtol * np.abs(w)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {int(bad.sum())} out of tolerance; first at row "
                             f"{rows[i[0]]} head {i[1]} d {i[2]}: gpu {g[tuple(i)]} oracle {w[tuple(i)]}")
    exact = float(np.mean(W.to_bits(w, c.dtype) == got[rows]))
    say(f"  ok: {len(rows)} rows, exact_frac {exact:.3f}, max_abs {float(err.max()):.3g}")


def _run(c, label, requests=None, done=None, **kw):
    say(f"[attn] {label}: B={c.B} block={c.block} heads {c.nhq}/{c.nhk} D={c.D} {c.dtype} "
        f"prefix max {c.max_prefix}")
    if done is None:
        d = DevAttn(c, **kw)
        d.run()
        got = d.host()
    else:  # the device run of an earlier call
        d, got = done
    reqs = np.arange(c.B) if requests is None else np.asarray(requests)
    # oracle on the chosen requests only
    want = np.zeros(c.q.shape)
    for b in reqs:
        r = slice(b * c.block, (b + 1) * c.block)
        ip = c.kv_indptr
        idx = d.indices.cpu().numpy()[ip[b]:ip[b + 1]] if ip[b + 1] > ip[b] else np.zeros(0, np.int64)
        o, _ = A.draft_attention(c.q[r], c.k_ext[r], c.v_ext[r], c.k_pool, c.v_pool,
                                 [0, len(idx)], idx, c.block, c.nhq, c.nhk, c.sm_scale, c.dtype)
        want[r] = o
    rows = np.concatenate([np.arange(b * c.block, (b + 1) * c.block) for b in reqs])
    _compare(c, got, want, rows, label)
    return d, got


SMALL = {
    # prefixes of 0, 1, 31, 32, 33 and 300 keys (split edges); G=4, 32 rows
    "prefix_edges": dict(B=6, block=8, nhq=8, nhk=2, D=128, prefix=[0, 1, 31, 32, 33, 300],
                         slots=512),
    # D=64, a partial 16-row tile
    "d64_partial_tile": dict(B=3, block=4, nhq=16, nhk=4, D=64, prefix=[100, 7, 64], slots=256),
    # G=8: two 32-row tiles per (request, KV head)
    "two_row_tiles": dict(B=2, block=8, nhq=16, nhk=2, D=128, prefix=[70, 129], slots=256),
    # a block of 40 own keys (two 32-key steps in the block's split), no grouping
    "long_block": dict(B=2, block=40, nhq=2, nhk=2, D=64, prefix=[50, 0], slots=128),
    "fp16": dict(B=3, block=8, nhq=8, nhk=2, D=128, prefix=[260, 5, 90], slots=512,
                 dtype="fp16"),
    # many splits: a long prefix over few requests
    "long_prefix": dict(B=1, block=8, nhq=4, nhk=1, D=128, prefix=[5000], slots=6000),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_cases(name):
    c = W.make_attn_case(name=name, seed=sum(map(ord, name)), **SMALL[name])
    d, _ = _run(c, name)
    assert int(d.err.item()) == 0


_WORKLOAD_RUNS = {}


def _workload_run(name):
    """One device run per workload, shared by the tests that check its requests."""
    if name not in _WORKLOAD_RUNS:
        _WORKLOAD_RUNS.clear()
        c = W.attn_workload(name)
        say(f"[attn] {name}: device run")
        d = DevAttn(c)
        d.run()
        _WORKLOAD_RUNS[name] = (c, d, d.host())
    return _WORKLOAD_RUNS[name]


@pytest.mark.parametrize("name,first", [("attn_decode_8k", b) for b in range(0, 32, 8)]
                         + [("attn_d64_16k", 0)])
def test_workloads(name, first):
    """Every request of the workload at its full size, element by element
    (attn_decode_8k's 32 requests in four tests of eight, so that each test's
    oracle time stays well inside the per-test limit)."""
    c, d, got = _workload_run(name)
    reqs = np.arange(first, min(first + 8, c.B)) if name == "attn_decode_8k" else None
    _run(c, f"{name} requests {first}..", reqs, done=(d, got))
    assert int(d.err.item()) == 0


def test_bad_slots_and_short_max_prefix_are_counted():
    c = W.make_attn_case(B=2, block=4, nhq=4, nhk=1, D=64, prefix=[40, 10], slots=64, seed=71)
    bad = c.kv_indices.copy()
    bad[[3, 45]] = [-1, 64]  # one bad slot in each request
    d, got = _run(c, "bad slots", indices=bad)
    assert int(d.err.item()) == 2
    # a max_prefix bound of 8 below both prefixes: each request counted once,
    # and only its first 8 prefix keys attended
    d2 = DevAttn(c, max_prefix=8)
    d2.run()
    got2 = d2.host()
    assert int(d2.err.item()) == 2
    short = W.AttnCase(**{**c.__dict__, "kv_indptr": np.array([0, 8, 16]),
                          "kv_indices": np.concatenate([c.kv_indices[:8], c.kv_indices[40:48]])})
    want = np.zeros(c.q.shape)
    want[:], _ = A.draft_attention(short.q, short.k_ext, short.v_ext, short.k_pool, short.v_pool,
                                   short.kv_indptr, short.kv_indices, c.block, c.nhq, c.nhk,
                                   c.sm_scale, c.dtype)
    _compare(c, got2, want, np.arange(c.B * c.block), "prefixes cut at max_prefix")


def test_graph_replays_match_eager():
    c = W.make_attn_case(B=4, block=8, nhq=8, nhk=2, D=128, prefix=[100, 300, 0, 33], slots=512,
                         seed=72)
    d, ref = _run(c, "eager reference")
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            d.run(stream=side)
    for rep in range(4):
        d.out.view(torch.int16).fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(d.host(), ref), rep


def _draw_attn(i):
    rng = np.random.default_rng(9500 + i)
    nhk = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 13))
    prefix = [int(x) for x in rng.integers(0, 3000, size=B)]
    if rng.random() < 0.3:
        prefix[int(rng.integers(0, B))] = 0
    return dict(name=f"attn_sweep{i}", B=B, block=int(rng.integers(1, 49)), nhq=nhk * G, nhk=nhk,
                D=int(rng.choice([64, 128])), prefix=prefix,
                slots=sum(prefix) + int(rng.integers(1, 100)),
                dtype="fp16" if rng.random() < 0.3 else "bf16", seed=9500 + i)


@pytest.mark.parametrize("i", range(32))
def test_random_shapes(i):
    """Seeded sweep: request count, block length (1..48 own keys), grouping
    (1..8 query heads per KV head, so 1..12 row tiles), head_dim, prefix
    lengths 0..2999 and dtype drawn per case; every request checked."""
    kw = _draw_attn(i)
    c = W.make_attn_case(**kw)
    d, _ = _run(c, kw["name"])
    assert int(d.err.item()) == 0
