"""Parity of the HIP in-place table QK-RMSNorm + neox RoPE (through the C ABI)
with the CPU oracle.

Tolerance: |gpu - oracle| <= atol + rtol*|oracle| elementwise on the query
and key heads with (rtol, atol) = (2e-2, 2e-2) for bf16 and (5e-3, 5e-3) for
fp16, the tolerances the stacked write is held to. Every other column of a
row (value heads, padding) and every row whose position is outside the table
must keep its bits exactly.
"""

import dataclasses
import zlib

import numpy as np
import pytest
import torch

import speculative_decoding_draft_stacked_amd as dk
from speculative_decoding_draft_stacked_amd import workloads as W
from oracle import ctx_kv_oracle as O
from oracle import qk_norm_rope_oracle as Q

from gpu_util import TOL, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    dk.lib()  # raises if the HIP library is not built


_TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _dev16(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(_TORCH[dtype]).cuda()


class DevQk:
    """A QK case on the device (torch plumbing only)."""

    def __init__(self, c):
        self.c = c
        self.qkv = _dev16(c.qkv, c.dtype)
        if c.weight_dtype == "fp32":
            self.qw = torch.from_numpy(c.q_w).cuda()
            self.kw = torch.from_numpy(c.k_w).cuda()
        else:
            self.qw = _dev16(c.q_w, c.dtype)
            self.kw = _dev16(c.k_w, c.dtype)
        self.table = torch.from_numpy(c.table).cuda()
        self.pos = torch.from_numpy(c.positions).cuda()
        self.err = torch.zeros(1, dtype=torch.int64, device="cuda")

    def run(self, stream=None):
        return dk.table_qk_norm_rope(self.qkv, self.pos, self.qw, self.kw, self.table,
                                     self.c.NHQ, self.c.NHK, self.c.D, self.c.eps,
                                     range_errors=self.err, stream=stream)

    def host(self):
        torch.cuda.synchronize()
        return self.qkv.view(torch.int16).cpu().numpy().view(np.uint16)


def _expected(c, rows=None):
    rows = np.arange(c.T) if rows is None else np.asarray(rows)
    out = c.qkv[rows].copy()
    skipped = Q.qk_norm_rope_inplace(out, c.positions[rows], c.q_w, c.k_w, c.weight_dtype,
                                     c.table, c.NHQ, c.NHK, c.D, c.eps, c.dtype)
    return rows, out, skipped


def _compare(c, got, rows, want, label):
    width = (c.NHQ + c.NHK) * c.D
    # columns the op must not touch: bit-exact
    assert np.array_equal(got[rows][:, width:], want[:, width:]), f"{label}: V/padding changed"
    g = O.decode(got[rows][:, :width], c.dtype)
    w = O.decode(want[:, :width], c.dtype)
    assert np.all(np.isfinite(g)), label
    rtol, atol = TOL[c.dtype]
    err = np.abs(g - w)
    bad = err > atol + rtol * np.abs(w)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {int(bad.sum())} out of tolerance; first at row "
                             f"{rows[i[0]]} col {i[1]}: gpu {g[tuple(i)]} oracle {w[tuple(i)]}")
    exact = float(np.mean(got[rows][:, :width] == want[:, :width]))
    say(f"  ok: rows {len(rows)} exact_frac {exact:.4f} max_abs {float(err.max()):.3g}")
    return exact


def _run(c, label, rows=None):
    say(f"[qk] {label}: T={c.T} NHQ={c.NHQ} NHK={c.NHK} D={c.D} {c.dtype} "
        f"w={c.weight_dtype} stride={c.row_stride}")
    d = DevQk(c)
    assert d.run()
    got = d.host()
    rows, want, skipped = _expected(c, rows)
    exact = _compare(c, got, rows, want, label)
    if len(rows) == c.T:
        assert int(d.err.item()) == skipped
    return d, got, exact


SMALL = {
    # 128-wide heads, padded rows, ragged head count per workgroup
    "bf16_d128_pad": dict(T=37, NHQ=4, NHK=2, D=128, row_pad=8),
    "bf16_d64_single_token": dict(T=1, NHQ=3, NHK=1, D=64),
    "fp16_d128_fp32_weights": dict(T=100, NHQ=2, NHK=2, D=128, dtype="fp16", weight_fp32=True),
    # D=64 takes 4 lanes per head, 64 heads per workgroup: 513 tokens x 8 heads
    # leave the last workgroup partial
    "fp16_d64_odd_heads": dict(T=513, NHQ=5, NHK=3, D=64, dtype="fp16", row_pad=16),
    "bf16_d64_fp32_weights_theta1e6": dict(T=1000, NHQ=6, NHK=2, D=64, weight_fp32=True,
                                           theta=1e6, P=32768),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_cases(name):
    c = W.make_qk_case(name=name, seed=zlib.crc32(name.encode()) % 10000, **SMALL[name])
    _run(c, name)


@pytest.mark.parametrize("name", ["qk_decode", "qk_prefill_8k"])
def test_workloads(name):
    """Every token of the workload at its full size, element by element."""
    c = W.qk_workload(name)
    _, _, exact = _run(c, name)
    assert exact > 0.9  # diagnostic only; the bar is the tolerance


def test_out_of_range_positions_untouched_and_counted():
    c = W.make_qk_case(T=64, NHQ=2, NHK=1, D=128, seed=51, P=200)
    c.positions[[0, 17, 63]] = [-5, 200, 1 << 40]
    d, got, _ = _run(c, "out-of-range positions")
    assert int(d.err.item()) == 3
    assert np.array_equal(got[[0, 17, 63]], c.qkv[[0, 17, 63]])


def test_empty_call_is_a_no_op():
    c = W.make_qk_case(T=4, NHQ=1, NHK=1, D=64, seed=52)
    d = DevQk(c)
    empty = d.qkv[:0]
    assert dk.table_qk_norm_rope(empty, d.pos[:0], d.qw, d.kw, d.table, 1, 1, 64, c.eps)
    assert np.array_equal(d.host(), c.qkv)


def test_unsupported_head_dim_falls_back_untouched():
    c = W.make_qk_case(T=4, NHQ=1, NHK=1, D=64, seed=53)
    d = DevQk(c)
    # head_dim 32 over the same buffer: not supported, nothing may change
    assert not dk.table_qk_norm_rope(d.qkv, d.pos, d.qw[:32], d.kw[:32],
                                     d.table[:, :32].contiguous(), 2, 2, 32, c.eps)
    assert np.array_equal(d.host(), c.qkv)


def test_graph_replays_match_eager():
    """Captured in a HIP graph, every replay (on a fresh copy of the input,
    with eager work and syncs in between) gives the eager result."""
    c = W.make_qk_case(T=96, NHQ=4, NHK=2, D=128, seed=54, row_pad=8)
    d, ref, _ = _run(c, "eager reference")
    orig = _dev16(c.qkv, c.dtype)
    d.qkv.copy_(orig)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            assert d.run(stream=side)
    for rep in range(4):
        d.qkv.copy_(orig)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(d.host(), ref), rep


# ------------------------------------------------------ seeded shape sweep

N_SWEEP = 24


def _draw(i):
    """Head counts, head width, dtype, norm-weight dtype, row padding, table
    size and base, position pattern (uniform, consecutive, some outside the
    table) and token count from one seed; sizes keep the oracle to a fraction
    of a second."""
    rng = np.random.default_rng(7300 + i)
    D = int(rng.choice([64, 128]))
    return dict(name=f"qk_sweep{i}", T=int(rng.integers(1, 1500)), NHQ=int(rng.integers(1, 17)),
                NHK=int(rng.integers(1, 5)), D=D,
                dtype="fp16" if rng.random() < 0.4 else "bf16",
                row_pad=int(rng.choice([0, 0, 8, 40])), weight_fp32=bool(rng.random() < 0.3),
                theta=float(rng.choice([1e4, 5e4, 1e6])), P=int(rng.choice([64, 4096, 32768])),
                eps=float(rng.choice([1e-6, 1e-5])), seed=7300 + i,
                positions_mode=str(rng.choice(["uniform", "arange", "some_out"])))


@pytest.mark.parametrize("i", range(N_SWEEP))
def test_random_shape(i):
    kw = _draw(i)
    mode = kw.pop("positions_mode")
    if mode == "arange":
        kw["P"] = max(kw["P"], kw["T"])  # consecutive positions stay inside the table
    c = W.make_qk_case(positions_mode="uniform" if mode == "some_out" else mode, **kw)
    if mode == "some_out":  # a tenth of the tokens outside the table: untouched, counted
        rng = np.random.default_rng(7300 + i)
        pos = c.positions.copy()
        out = rng.random(c.T) < 0.1
        pos[out] = rng.choice(np.array([-1, c.P, 1 << 40], dtype=np.int64), int(out.sum()))
        c = dataclasses.replace(c, positions=pos)
    _run(c, kw["name"])

