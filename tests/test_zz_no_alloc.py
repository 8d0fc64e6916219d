"""dspark_ctx_kv_write_static (the write with the library's static device
scratch instead of a caller workspace) against dspark_ctx_kv_write, through
the C ABI: bit-identical pools on two calls in a row, the second smaller,
both in the K-split form that uses the scratch, the adaptive plan in both of
its modes, plus a write that needs no scratch at all."""

import dataclasses

import numpy as np
import pytest
import torch

import speculative_decoding_draft_stacked_amd as dk
from speculative_decoding_draft_stacked_amd import workloads as W

from gpu_util import DeviceCase, check_slot_sets, compare_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    dk.lib()


def _static_write(dc, pack):
    c = dc.case
    return dk.ctx_kv_write_static(pack, dc.x, dc.positions, dc.locs, dc.pool_descs(),
                                  commit_lens=dc.commit,
                                  locs_row_width=c.row_width if dc.commit is not None else None,
                                  range_errors=dc.err)


def _same_as_workspace_entry(case, pack, label):
    """The static entry's pools equal the workspace entry's, bit for bit, and
    match the oracle within the tolerance."""
    say(f"[case] {label}: T={case.T} plan {pack.plan(case.T, case.commit_lens is not None)}")
    ref = DeviceCase(case)
    assert ref.write(pack)
    got = DeviceCase(case)
    assert _static_write(got, pack)
    torch.cuda.synchronize()
    check_slot_sets(got)
    compare_rows(got, None, label)
    rk, rv = ref.pools_host()
    gk, gv = got.pools_host()
    for layer in range(case.L):
        assert np.array_equal(rk[layer], gk[layer]) and np.array_equal(rv[layer], gv[layer]), layer
    assert got.range_errors() == 0 and ref.range_errors() == 0


def test_static_scratch_two_calls_second_smaller():
    # one GPU's share of a decode commit (one KV head of 5 layers): few weight
    # tiles, so the write splits K and the part sums live in the scratch
    big = W.make_case(name="static1", seed=81, T=256, H=4096, L=5, NH=1, D=128, row_width=8,
                      slots=2048, theta=1e6, P=32768)
    ref = DeviceCase(big)
    pack = ref.pack()
    assert pack.plan(big.T, True)["kernel"] == "stream_ksplit"
    _same_as_workspace_entry(big, pack, "first call")
    small = dataclasses.replace(big, name="static2", T=64, x=big.x[:64],
                                positions=big.positions[:64], locs=big.locs[:64],
                                commit_lens=big.commit_lens[:8])
    assert pack.plan(small.T, True)["kernel"] == "stream_ksplit"
    _same_as_workspace_entry(small, pack, "second, smaller call")
    pack.free()


def test_static_entry_adaptive_plan_both_modes():
    # a 512-row window over 40 weight tiles: the adaptive plan's part sums in
    # the scratch (about half of the window committed), then the same pack
    # with every row committed (K whole, the scratch holds only the row map)
    case = W.make_case(name="static5", seed=84, T=512, H=1024, L=5, NH=4, D=128, row_width=8,
                       commit_range=(1, 9), slots=700)
    dc = DeviceCase(case)
    pack = dc.pack()
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert pack.plan(case.T, True)["adaptive"]
    _same_as_workspace_entry(case, pack, "adaptive, K split")
    full = dataclasses.replace(case, name="static6", commit_lens=np.full(64, 8, dtype=np.int64))
    _same_as_workspace_entry(full, pack, "adaptive, K whole")
    pack.free()


def test_static_entry_without_k_split():
    case = W.make_case(name="static3", seed=82, T=300, H=256, L=2, NH=2, D=64, slots=512)
    dc = DeviceCase(case)
    pack = dc.pack()
    assert pack.workspace_bytes(case.T, False) == 0
    _same_as_workspace_entry(case, pack, "no scratch needed")
    pack.free()


def test_static_entry_rejects_flags_and_accepts_empty():
    case = W.make_case(name="static4", seed=83, T=8, H=64, L=1, NH=1, D=64, slots=16)
    dc = DeviceCase(case)
    pack = dc.pack()
    arr = (dk.PoolDesc * 1)(*dc.pool_descs())
    lib = dk.lib()
    assert lib.dspark_ctx_kv_write_static(pack.as_parameter, dc.x.data_ptr(), case.T, case.H,
                                          dc.positions.data_ptr(), dc.locs.data_ptr(), None, 0,
                                          0, arr, 1, None, dk.WRITE_VALIDATE, None,
                                          None) == dk.E_INVALID
    assert lib.dspark_ctx_kv_write_static(pack.as_parameter, None, 0, case.H, None, None, None,
                                          0, 0, arr, 1, None, 0, None, None) == dk.OK
    torch.cuda.synchronize()
    assert len(dc.touched_slots(0, "k")) == 0
    pack.free()
