"""Parity of the HIP context producer main_norm(main_proj(aux)) (through the C
ABI) with the CPU oracle.

Tolerance: |gpu - oracle| <= atol + rtol*|oracle| elementwise with (rtol,
atol) = (2e-2, 2e-2) for bf16 and (5e-3, 5e-3) for fp16, as for the write.
"""

import zlib

import numpy as np
import pytest
import torch

import speculative_decoding_draft_stacked_amd as dk
from speculative_decoding_draft_stacked_amd import workloads as W
from oracle import ctx_kv_oracle as O
from oracle import main_proj_oracle as M

from gpu_util import TOL, say

pytestmark = pytest.mark.gpu
_T = {"bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    dk.lib()


def _dev16(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(_T[dtype]).cuda()


class DevProj:
    def __init__(self, c, aux_pad=0, ctx_pad=0):
        self.c = c
        aux = np.zeros((c.T, c.K + aux_pad), dtype=np.uint16)
        aux[:, :c.K] = c.aux
        self.aux = _dev16(aux, c.dtype)[:, :c.K]
        self.w = _dev16(c.w, c.dtype)
        self.g = torch.from_numpy(c.g).cuda() if c.g_dtype == "fp32" else _dev16(c.g, c.dtype)
        self.ctx_full = torch.full((c.T, c.H + ctx_pad), -7, dtype=torch.int16,
                                   device="cuda").view(_T[c.dtype])
        self.ctx = self.ctx_full[:, :c.H]
        self.pack = dk.pack_main_proj(self.w, self.g, c.eps)
        assert self.pack is not None
        nbytes = self.pack.workspace_bytes(c.T)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")

    def run(self, stream=None):
        dk.main_proj_norm(self.pack, self.aux, self.ctx, self.ws, stream=stream)

    def host(self):
        torch.cuda.synchronize()
        return self.ctx_full.view(torch.int16).cpu().numpy().view(np.uint16)


def _check(c, got, rows, label):
    want = M.combine_hidden_states(c.aux[rows], c.w, c.g, c.g_dtype, c.eps, c.dtype)
    g = O.decode(got[rows][:, :c.H], c.dtype)
    assert np.all(np.isfinite(g)), label
    rtol, atol = TOL[c.dtype]
    err = np.abs(g - want)
    bad = err > atol + rtol * np.abs(want)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {int(bad.sum())} out of tolerance; first at token "
                             f"{rows[i[0]]} feature {i[1]}: gpu {g[tuple(i)]} oracle {want[tuple(i)]}")
    exact = float(np.mean(W.to_bits(want, c.dtype) == got[rows][:, :c.H]))
    say(f"  ok: {len(rows)} tokens, exact_frac {exact:.4f}, max_abs {float(err.max()):.3g}")
    return exact


def _run(c, label, rows=None, aux_pad=0, ctx_pad=0):
    say(f"[proj] {label}: T={c.T} H={c.H} n={c.n_aux} {c.dtype} g={c.g_dtype} "
        f"pads={aux_pad},{ctx_pad}")
    d = DevProj(c, aux_pad, ctx_pad)
    d.run()
    got = d.host()
    if ctx_pad:
        assert np.all(got[:, c.H:].view(np.int16) == -7), "padding of ctx rows was written"
    rows = np.arange(c.T) if rows is None else np.asarray(rows)
    exact = _check(c, got, rows, label)
    return d, got, exact


SMALL = {
    # one token, one 128-feature group, one auxiliary layer
    "t1_h128": dict(T=1, H=128, n_aux=1),
    # ragged token count, three auxiliary layers (K = 768), streaming kernel
    "t37_h256": dict(T=37, H=256, n_aux=3),
    "fp16_fp32_weight": dict(T=300, H=384, n_aux=2, dtype="fp16", g_fp32=True),
    # large T: tiled kernel, 8 groups, ragged token tail
    "tiled_t5000_h1024": dict(T=5000, H=1024, n_aux=1),
    # tiled kernel with an odd number of 128-row tiles (the last 256-row
    # workgroup tile is half past the weight)
    "tiled_odd_groups": dict(T=5000, H=1152, n_aux=1),
    # K split over workgroups (on 256 compute units): 12 weight tiles x 2 token
    # tiles x 9 K parts of 8 chunks, ragged token tail
    "split_odd_parts": dict(T=200, H=1536, n_aux=3),
    # hidden size not a multiple of 512: no K split (streaming kernel, 7 tiles)
    "nosplit_h896": dict(T=200, H=896, n_aux=3),
    # the largest hidden size of the K-split norm (a row of 8192 in registers,
    # 4 waves x 4 passes of 512): 64 tiles x 1 token tile x 4 K parts
    "split_max_h8192": dict(T=64, H=8192, n_aux=1),
    # 32 tiles x 2 token tiles (the second of 72 tokens) x 4 K parts of 16
    # chunks
    "split_t200_h4096": dict(T=200, H=4096, n_aux=1),
    # fp16 with an fp32 norm weight, a second token tile of 2 tokens, 4 K parts
    # of 32 chunks
    "split_fp16_t130": dict(T=130, H=4096, n_aux=2, dtype="fp16", g_fp32=True),
    # K split, fp16 with an fp32 norm weight: 4 tiles x 1 token tile x 4 parts
    "split_fp16": dict(T=128, H=512, n_aux=4, dtype="fp16", g_fp32=True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_cases(name):
    c = W.make_proj_case(name=name, seed=zlib.crc32(name.encode()) % 10000, **SMALL[name])
    _run(c, name)


def test_padded_strides():
    c = W.make_proj_case(T=70, H=256, n_aux=2, seed=61)
    _run(c, "padded aux and ctx rows", aux_pad=24, ctx_pad=40)


@pytest.mark.parametrize("name", ["proj_decode", "proj_prefill_8k"])
def test_workloads(name):
    """Every token of the workload at its full size, element by element."""
    c = W.proj_workload(name)
    _, _, exact = _run(c, name)
    assert exact > 0.9  # diagnostic only; the bar is the tolerance


def test_repeatable_and_workspace_checked():
    c = W.make_proj_case(T=64, H=512, n_aux=2, seed=62)
    d, first, _ = _run(c, "first call")
    d.run()
    assert np.array_equal(d.host(), first)  # deterministic group-sum order
    small = torch.empty(d.pack.workspace_bytes(c.T) - 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):  # DSPARK_E_INVALID: workspace too small
        dk.main_proj_norm(d.pack, d.aux, d.ctx, small)
    empty = d.aux[:0]
    dk.main_proj_norm(d.pack, empty, d.ctx[:0], d.ws)  # no tokens: nothing enqueued
    assert np.array_equal(d.host(), first)


def test_graph_replays_match_eager():
    c = W.make_proj_case(T=96, H=256, n_aux=3, seed=63)
    d, ref, _ = _run(c, "eager reference")
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            d.run(stream=side)
    for rep in range(4):
        d.ctx_full.view(torch.int16).fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(d.host(), ref), rep


# ------------------------------------------------------ seeded shape sweep

N_SWEEP = 24


def _draw(i):
    """Token count, hidden size (a multiple of 128: the 128-feature norm
    groups), auxiliary layer count, dtype and norm-weight dtype from one seed,
    across the streaming, K-split and tiled plans; the oracle's work stays
    under ~2e9 multiply-adds."""
    rng = np.random.default_rng(7600 + i)
    H = int(rng.integers(1, 25)) * 128
    n_aux = int(rng.integers(1, 5))
    T = int(rng.integers(1, 400)) if rng.random() < 0.6 else int(rng.integers(400, 6000))
    while T > 1 and T * H * H * n_aux > 2e9:
        T = T * 2 // 3
    return dict(name=f"proj_sweep{i}", T=T, H=H, n_aux=n_aux,
                dtype="fp16" if rng.random() < 0.4 else "bf16", g_fp32=bool(rng.random() < 0.3),
                eps=float(rng.choice([1e-6, 1e-5])), seed=7600 + i)


@pytest.mark.parametrize("i", range(N_SWEEP))
def test_random_shape(i):
    kw = _draw(i)
    c = W.make_proj_case(**kw)
    d, _, _ = _run(c, kw["name"])
    say(f"  workspace {d.pack.workspace_bytes(c.T)} bytes")

