"""Seeded sweep of random shapes through the HIP context-KV write (C ABI)
against the CPU oracle, to the same bar as the named cases: the written
(layer, slot) set bit-exact, values within (2e-2, 2e-2) for bf16 and
(5e-3, 5e-3) for fp16.

Each case draws T, H, L, KV heads, head_dim, dtype, bias, and the slot map
(plain slots with holes, or commit windows with lengths 0..W+2) from one
seed, so the sweep crosses both kernels, their tile and token-split choices,
K tails, commit-window compaction and its limit. A second sweep draws shapes
with few weight tiles, H >= 1024 and T <= 1024, which take the K-split form
(K parts over workgroups, parts added in a second launch). A third draws
shapes for the LDS-tiled kernel: T large enough for its plan, D = 64 tiles
holding four heads that may span two layers, odd weight-tile counts whose
last workgroup tile lies half past the stacked weight, bias, commit windows
and negative slots. A fourth draws commit windows for the adaptive K-split
plan, in both of its modes. Sizes keep the fp64 oracle to about a second per
case.
"""

import numpy as np
import pytest
import torch

import speculative_decoding_draft_stacked_amd as dk
from speculative_decoding_draft_stacked_amd import workloads as W

from gpu_util import DeviceCase, check_slot_sets, compare_rows, say

pytestmark = pytest.mark.gpu

N_CASES = 120


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    dk.lib()  # raises if the HIP library is not built


def _draw(i):
    rng = np.random.default_rng(9000 + i)
    D = int(rng.choice([64, 128]))
    NH = int(rng.integers(1, 5))
    L = int(rng.integers(1, 7))
    H = int(rng.integers(1, 129)) * 8
    n_tot = L * 2 * NH * D
    dtype = "fp16" if rng.random() < 0.3 else "bf16"
    bias = bool(rng.random() < 0.3)
    # T: mostly decode-sized, some large enough for the tiled kernel
    T = int(rng.integers(1, 300)) if rng.random() < 0.5 else int(rng.integers(1000, 9000))
    # keep T * n_tot * H (the oracle's work) near or under 4e9
    while T > 1 and T * n_tot * H > 4e9:
        T = T * 2 // 3
    kw = dict(name=f"sweep{i}", T=T, H=H, L=L, NH=NH, D=D, dtype=dtype, bias=bias,
              seed=9000 + i, theta=float(rng.choice([1e4, 5e4, 1e6])), P=4096)
    if rng.random() < 0.5:
        Wd = int(rng.integers(1, 17))
        T = max(Wd, T // Wd * Wd)
        kw.update(T=T, row_width=Wd, commit_range=(0, Wd + 2))
    kw["neg_loc_frac"] = float(rng.choice([0.0, 0.0, 0.1]))
    kw["slots"] = T + int(rng.integers(0, 64))
    return kw


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    kw = _draw(i)
    case = W.make_case(**kw)
    say(f"[sweep {i}] T={case.T} H={case.H} L={case.L} NH={case.NH} D={case.D} {case.dtype} "
        f"bias={case.qkv_b is not None} W={case.row_width}")
    dc = DeviceCase(case)
    pack = dc.pack()
    assert dc.write(pack)
    torch.cuda.synchronize()
    check_slot_sets(dc)
    st = compare_rows(dc, None, f"sweep{i}")  # every stored row
    assert dc.range_errors() == 0
    say(f"  ok: {st}")
    pack.free()


# ------------------------------------------------ shapes for the K-split form

N_KSPLIT_CASES = 64


def _draw_ksplit(i):
    """Few 128-row weight tiles (1 to 6), H >= 1024 and T <= 1024: most such
    shapes split K over workgroups and add the parts in a second launch."""
    rng = np.random.default_rng(9500 + i)
    D = int(rng.choice([64, 128]))
    NH = int(rng.integers(1, 3))
    L = int(rng.integers(1, 4))
    H = int(rng.integers(128, 513)) * 8
    n_tot = L * 2 * NH * D
    dtype = "fp16" if rng.random() < 0.3 else "bf16"
    bias = bool(rng.random() < 0.3)
    T = int(rng.integers(1, 1025))
    while T > 1 and T * n_tot * H > 4e9:
        T = T * 2 // 3
    kw = dict(name=f"ksweep{i}", T=T, H=H, L=L, NH=NH, D=D, dtype=dtype, bias=bias,
              seed=9500 + i, theta=float(rng.choice([1e4, 5e4, 1e6])), P=4096)
    if rng.random() < 0.6:
        Wd = int(rng.integers(1, 17))
        T = max(Wd, T // Wd * Wd)
        kw.update(T=T, row_width=Wd, commit_range=(0, Wd + 2))
    kw["neg_loc_frac"] = float(rng.choice([0.0, 0.0, 0.1]))
    kw["slots"] = T + int(rng.integers(0, 64))
    return kw


@pytest.mark.parametrize("i", range(N_KSPLIT_CASES))
def test_random_shape_k_split(i):
    kw = _draw_ksplit(i)
    case = W.make_case(**kw)
    say(f"[ksweep {i}] T={case.T} H={case.H} L={case.L} NH={case.NH} D={case.D} {case.dtype} "
        f"bias={case.qkv_b is not None} W={case.row_width}")
    dc = DeviceCase(case)
    pack = dc.pack()
    assert dc.write(pack)
    torch.cuda.synchronize()
    check_slot_sets(dc)
    st = compare_rows(dc, None, f"ksweep{i}")
    assert dc.range_errors() == 0
    say(f"  ok: {st}")
    pack.free()


# ------------------------------------ shapes for the adaptive K-split plan

N_ADAPTIVE_CASES = 30
# (layers, KV heads, head_dim) giving 20, 32, 40, 64 and 80 weight tiles of
# 128 rows, i.e. 6, 4, 3, 2 and 1 token splits of 128 slots for two K parts
# on 256 compute units, with the window sizes each plan covers
_ADAPTIVE_SHAPES = [((5, 2, 128), 6), ((4, 4, 128), 4), ((5, 8, 64), 3), ((8, 4, 128), 2),
                    ((5, 8, 128), 1)]


def _draw_adaptive(i):
    """Commit windows too large for one round of K-split workgroups with one
    128-slot token split per 128 rows, but whose 3/4 fits one round: the
    adaptive plan. The committed fraction is drawn so that some windows fit
    the K-split splits and others need K whole."""
    rng = np.random.default_rng(9800 + i)
    (L, NH, D), splits = _ADAPTIVE_SHAPES[i % len(_ADAPTIVE_SHAPES)]
    lo, hi = splits * 128 + 1, min(1024, splits * 128 * 4 // 3)
    Wd = int(rng.choice([4, 8, 16]))
    T = int(rng.integers(lo, hi + 1)) // Wd * Wd
    T = max(T, (lo + Wd - 1) // Wd * Wd)
    H = int(rng.choice([1024, 1096, 1536]))
    frac = float(rng.choice([0.4, 0.6, 1.0]))
    kw = dict(name=f"asweep{i}", T=T, H=H, L=L, NH=NH, D=D,
              dtype="fp16" if rng.random() < 0.4 else "bf16", bias=bool(rng.random() < 0.4),
              seed=9800 + i, theta=float(rng.choice([1e4, 1e6])), P=4096, row_width=Wd,
              commit_range=(max(0, int(frac * Wd) - 2), int(frac * Wd) + 2),
              neg_loc_frac=float(rng.choice([0.0, 0.05])), slots=T + 37)
    return kw, splits


@pytest.mark.parametrize("i", range(N_ADAPTIVE_CASES))
def test_random_shape_adaptive(i):
    kw, splits = _draw_adaptive(i)
    case = W.make_case(**kw)
    say(f"[asweep {i}] T={case.T} H={case.H} L={case.L} NH={case.NH} D={case.D} {case.dtype} "
        f"bias={case.qkv_b is not None} W={case.row_width}")
    dc = DeviceCase(case)
    pack = dc.pack()
    plan = pack.plan(case.T, True)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert plan["adaptive"] and plan["token_splits"] == splits, plan
    assert dc.write(pack)
    torch.cuda.synchronize()
    check_slot_sets(dc)
    st = compare_rows(dc, None, f"asweep{i}")
    assert dc.range_errors() == 0
    say(f"  ok: {st}")
    pack.free()


# ------------------------------------------------ shapes for the tiled kernel

N_TILED_CASES = 30


def _draw_tiled(i):
    """Few heads and a narrow hidden size so that a T past the tiled kernel's
    threshold keeps the oracle cheap."""
    rng = np.random.default_rng(9700 + i)
    D = int(rng.choice([64, 128]))
    NH = int(rng.integers(1, 4))
    L = int(rng.integers(1, 5))
    H = int(rng.integers(8, 41)) * 8
    dtype = "fp16" if rng.random() < 0.4 else "bf16"
    bias = bool(rng.random() < 0.5)
    kw = dict(name=f"tsweep{i}", H=H, L=L, NH=NH, D=D, dtype=dtype, bias=bias,
              seed=9700 + i, theta=float(rng.choice([1e4, 5e4, 1e6])), P=4096,
              neg_loc_frac=float(rng.choice([0.0, 0.05])))
    if rng.random() < 0.4:
        Wd = int(rng.integers(2, 17))
        kw.update(row_width=Wd, commit_range=(0, Wd + 2))
    return kw, int(rng.integers(1, 3000))


@pytest.mark.parametrize("i", range(N_TILED_CASES))
def test_random_shape_tiled(i):
    kw, extra = _draw_tiled(i)
    # the smallest T the device's plan gives to the tiled kernel, plus a
    # ragged amount
    probe = W.make_case(T=64, slots=64, **{k: v for k, v in kw.items()
                                          if k not in ("row_width", "commit_range")})
    pdc = DeviceCase(probe)
    ppack = pdc.pack()
    T = 64
    while ppack.plan(T, False)["kernel"] != "tiled":
        T *= 2
    lo = T // 2
    while lo + 1 < T:  # bisect the threshold
        mid = (lo + T) // 2
        if ppack.plan(mid, False)["kernel"] == "tiled":
            T = mid
        else:
            lo = mid
    ppack.free()
    del pdc
    T += extra
    if "row_width" in kw:
        T = T // kw["row_width"] * kw["row_width"]
    case = W.make_case(T=T, slots=T + 37, **kw)
    say(f"[tsweep {i}] T={case.T} H={case.H} L={case.L} NH={case.NH} D={case.D} {case.dtype} "
        f"bias={case.qkv_b is not None} W={case.row_width}")
    dc = DeviceCase(case)
    pack = dc.pack()
    plan = pack.plan(case.T, case.commit_lens is not None)
    assert plan["kernel"] == "tiled", plan
    assert dc.write(pack)
    torch.cuda.synchronize()
    check_slot_sets(dc)
    st = compare_rows(dc, None, f"tsweep{i}")
    assert dc.range_errors() == 0
    say(f"  ok: {plan['token_tile']}-token tiles, {st}")
    pack.free()
