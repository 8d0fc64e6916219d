"""Parity of the HIP context-KV write (through the C ABI) with the CPU oracle.

Tolerance: |gpu - oracle| <= atol + rtol*|oracle| elementwise with
(rtol, atol) = (2e-2, 2e-2) for bf16 and (5e-3, 5e-3) for fp16, the parity
tolerances of sglang PR #31986's stacked-vs-per-layer test. Which slots are
written is compared bit-exactly against sentinel-filled pools.
"""

import dataclasses
import zlib

import numpy as np
import pytest
import torch

import speculative_decoding_draft_stacked_amd as dk
from speculative_decoding_draft_stacked_amd import workloads as W
from oracle import ctx_kv_oracle as O

from gpu_util import DeviceCase, check_slot_sets, compare_rows, device_to_host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    dk.lib()  # raises if the HIP library is not built


def _run(case, label, rows=None, **kw):
    say(f"[case] {label}: T={case.T} H={case.H} L={case.L} NH={case.NH} D={case.D} "
        f"{case.dtype} bias={case.qkv_b is not None} W={case.row_width}")
    dc = DeviceCase(case, **kw)
    pack = dc.pack()
    assert dc.write(pack)
    torch.cuda.synchronize()
    check_slot_sets(dc)
    st = compare_rows(dc, rows, label)
    assert dc.range_errors() == 0
    say(f"  ok: {st}")
    return dc, pack, st


# ------------------------------------------------------------ small multi-tile cases

SMALL = {
    # ragged token tail (130 = 128 + 2), two 128-heads per layer
    "bf16_d128_ragged_T": dict(T=130, H=320, L=2, NH=2, D=128, slots=400),
    # odd head count: 128-row tiles straddle the K/V boundary; K tail H % 64 = 8;
    # commit window of 7 with lengths 0..9 and 10% negative slots
    "bf16_d64_commit_holes": dict(T=77, H=200, L=3, NH=3, D=64, row_width=7,
                                  commit_range=(0, 9), neg_loc_frac=0.1, slots=300),
    # fp16 with stacked bias, window 10 with lengths 0..12
    "fp16_d128_bias_commit": dict(T=300, H=136, L=4, NH=1, D=128, dtype="fp16", bias=True,
                                  row_width=10, commit_range=(0, 12), slots=512),
    "fp16_d64_bias_small": dict(T=33, H=64, L=1, NH=2, D=64, dtype="fp16", bias=True, slots=40),
    "single_row": dict(T=1, H=64, L=2, NH=1, D=128, slots=4),
    "T32": dict(T=32, H=128, L=2, NH=2, D=64, slots=64),
    "T513_theta1e6": dict(T=513, H=64, L=1, NH=1, D=128, slots=1024, theta=1e6, P=32768),
    "T1000_multi_layer": dict(T=1000, H=128, L=5, NH=2, D=64, slots=2048, row_width=8),
    # wider hidden with a K tail H % 64 = 40, 9 weight tiles, commit window 7
    # with holes
    "wide_h_odd_tiles_ktail": dict(T=77, H=1000, L=3, NH=3, D=64, row_width=7,
                                   commit_range=(0, 9), neg_loc_frac=0.1, slots=300),
    # 33 K chunks with a tail of 8, 8 weight tiles
    "wide_h_eight_tiles": dict(T=200, H=2056, L=2, NH=2, D=128, slots=256),
    # fp16 + bias over 12 K chunks, ragged token tail
    "wide_h_fp16_bias": dict(T=300, H=768, L=1, NH=2, D=64, dtype="fp16", bias=True,
                             slots=512),
    # one row against a 4096-wide hidden
    "single_row_wide_h": dict(T=1, H=4096, L=2, NH=1, D=128, slots=8),
    # Large-T path. The token tile (256, 192 or 128) is picked from the grid it
    # gives on the device (256 compute units on MI355X); the comments name the
    # tile each case gets there.
    # 128-token tiles: an odd number of 128-row weight tiles (the last 256-row
    # workgroup tile is half past the stacked weight), K tail H % 64 = 8
    "tiled_odd_row_tiles": dict(T=11000, H=72, L=3, NH=1, D=64, slots=12000),
    # 128-token tiles: ragged token tail, K tail, commit window 10 with holes
    "tiled_commit_holes": dict(T=8300, H=136, L=2, NH=1, D=128, row_width=10,
                               commit_range=(0, 12), neg_loc_frac=0.05, slots=9000),
    # 192-token tiles (a ragged tail of 32 tokens), odd weight-tile count
    "tiled_t192_ragged": dict(T=20000, H=72, L=3, NH=1, D=64, slots=20500),
    # 256-token tiles (tail of 178), K tail 8, commit window 10 with holes
    "tiled_t256_commit": dict(T=25010, H=136, L=2, NH=1, D=128, row_width=10,
                              commit_range=(0, 12), neg_loc_frac=0.05, slots=25100),
    # 128-token tiles, fp16 + stacked bias, an odd number of 128-row weight
    # tiles (the last workgroup tile's bias rows past the stacked weight read
    # as zero), four 64-wide heads per workgroup tile spanning two layers
    "tiled_d64_bias_odd_tiles": dict(T=11000, H=200, L=3, NH=1, D=64, dtype="fp16",
                                     bias=True, slots=11500),
    # the narrowest hidden size: one K chunk of which 56 of 64 columns are tail
    "hidden_8_stream": dict(T=40, H=8, L=2, NH=1, D=128, slots=64),
    "hidden_8_tiled": dict(T=20000, H=8, L=2, NH=1, D=64, dtype="fp16", bias=True,
                           slots=20100),
    # one request, one column: commit window of width 1 (lengths 0..3)
    "window_width_1": dict(T=1, H=64, L=2, NH=2, D=64, row_width=1, commit_range=(0, 3),
                           slots=8),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_cases(name):
    case = W.make_case(name=name, seed=zlib.crc32(name.encode()) % 10000, **SMALL[name])
    _run(case, name)


def test_k_norm_weight_fp32_and_padded_pool_rows():
    case = W.make_case(T=50, H=96, L=2, NH=2, D=64, slots=80, seed=21)
    _run(case, "fp32 k_norm, pool stride0 = NH*D + 16", k_norm_fp32=True, pool_row_pad=16)


# ------------------------------------------------------------ K split over workgroups

K_SPLIT = {
    # few weight tiles for the device: K is split over workgroups as well, the
    # parts are added in order by a second launch before the epilogue
    "no_commit_4_splits_4_parts": dict(T=200, H=2048, L=2, NH=1, D=128, slots=512),
    "fp16_d64_bias_commit_2_parts": dict(T=96, H=1024, L=1, NH=2, D=64, dtype="fp16", bias=True,
                                         row_width=6, commit_range=(0, 7), neg_loc_frac=0.1,
                                         slots=256),
    "window_1024_8_splits_8_parts": dict(T=1024, H=4096, L=1, NH=1, D=128, row_width=8, slots=2048),
    "fp16_d128_bias_4_splits_2_parts": dict(T=128, H=1024, L=1, NH=1, D=128, dtype="fp16",
                                            bias=True, slots=300),
}


@pytest.mark.parametrize("name", sorted(K_SPLIT))
def test_k_split_form(name):
    case = W.make_case(name=name, seed=40 + sorted(K_SPLIT).index(name), **K_SPLIT[name])
    _run(case, name)


def test_k_split_second_call_same_pack_and_workspace():
    """The K-part workspace belongs to the caller: a second, smaller call
    through the same pack and workspace (the first 64 rows of the batch, fresh
    pools) writes what the oracle gives for those rows."""
    c1 = W.make_case(name="ks1", seed=45, T=200, H=2048, L=2, NH=1, D=128, row_width=8,
                     slots=512)
    dc1 = DeviceCase(c1)
    pack = dc1.pack()
    assert pack.plan(200, True)["kernel"] == "stream_ksplit"
    ws = dc1.workspace(pack)
    assert ws is not None and ws.numel() == pack.workspace_bytes(200, True)
    say("[case] first call: T=200")
    assert dc1.write(pack, workspace=ws)
    torch.cuda.synchronize()
    check_slot_sets(dc1)
    compare_rows(dc1, None, "first call")
    c2 = dataclasses.replace(c1, name="ks2", T=64, x=c1.x[:64], positions=c1.positions[:64],
                             locs=c1.locs[:64], commit_lens=c1.commit_lens[:8])
    dc2 = DeviceCase(c2)
    say("[case] second call through the first pack and workspace: T=64")
    assert dc2.write(pack, workspace=ws)
    torch.cuda.synchronize()
    check_slot_sets(dc2)
    compare_rows(dc2, None, "second call")
    assert dc1.range_errors() == 0 and dc2.range_errors() == 0


# ------------------------------------------------------------ the workloads

@pytest.mark.parametrize("name", ["tiny", "decode_commit", "wide_gqa_d64", "biased_fp16",
                                  "prefill_8k", "decode_commit_kv1", "decode_commit_kv2"])
def test_workload(name):
    """Every stored row of every workload at its full size, element by element."""
    case = W.workload(name)
    dc, pack, st = _run(case, name)
    say(f"  plan: {pack.plan(case.T, case.commit_lens is not None)}")
    # diagnostic only; the bar is the tolerance above
    assert st["exact_frac"] > 0.9


# ------------------------------------------------------------ structure and invariants

def _unblock(blk, rows, H):
    """Inverse of the blocked weight layout documented at dspark_pack_buffers:
    block (rt, c) = 1024 pieces of 8; piece q = (g*4 + s)*64 + l is row
    128 rt + 32 g + l % 32, columns 64 c + 32 (l // 32) + 8 s + [0, 8)."""
    nk = -(-H // 64)
    pieces = blk.reshape(rows // 128, nk, 4, 4, 2, 32, 8)  # rt, c, g, s, half, l%32, e
    # -> rt, g, l%32, c, half, s, e  = row-major [rows, nk*64]
    plain = pieces.transpose(0, 2, 5, 1, 4, 3, 6).reshape(rows, nk * 64)
    assert not plain[:, H:].any()  # padding columns are zero
    return plain[:, :H]


def test_pack_contents():
    """W_stacked is the layers' KV slices in layer order (K rows then V rows),
    the bias is stacked the same way, k_norm is widened to fp32 exactly."""
    case = W.make_case(T=8, H=72, L=3, NH=1, D=128, dtype="fp16", bias=True, seed=22, slots=16)
    dc = DeviceCase(case)
    pack = dc.pack()
    info = pack.info()
    assert info == dict(num_layers=3, hidden=72, kv_size=128, head_dim=128, act_dtype=dk.FP16,
                        has_bias=True)
    w_ptr, b_ptr, k_ptr = pack.buffers()
    n_tot = case.L * 2 * case.kv
    nk = -(-case.H // 64)
    blk = device_to_host(w_ptr, n_tot * nk * 64 * 2).view(np.uint16)
    w = _unblock(blk, n_tot, case.H)
    b = device_to_host(b_ptr, n_tot * 2).view(np.uint16)
    kn = device_to_host(k_ptr, case.L * case.D * 4).view(np.float32).reshape(case.L, case.D)
    sl = slice(case.q_size, case.q_size + 2 * case.kv)
    assert np.array_equal(w, np.concatenate([wl[sl] for wl in case.qkv_w]))
    assert np.array_equal(b, np.concatenate([bl[sl] for bl in case.qkv_b]))
    want_k = np.stack([O.decode(g, "fp16") for g in case.k_norm_w]).astype(np.float32)
    assert np.array_equal(kn, want_k)


def test_stacked_equals_single_layer_packs():
    """An L-layer pack writes what L one-layer packs write, bit for bit."""
    case = W.make_case(T=70, H=128, L=3, NH=2, D=64, row_width=7, slots=128, seed=23)
    dc, pack, _ = _run(case, "3-layer pack")
    k_all, v_all = dc.pools_host()
    for l in range(case.L):
        one = W.make_case(T=70, H=128, L=1, NH=2, D=64, row_width=7, slots=128, seed=23)
        one.qkv_w, one.k_norm_w = [case.qkv_w[l]], [case.k_norm_w[l]]
        one.x, one.positions, one.locs, one.commit_lens = case.x, case.positions, case.locs, case.commit_lens
        d1 = DeviceCase(one)
        p1 = d1.pack()
        assert d1.write(p1)
        k1, v1 = d1.pools_host()
        assert np.array_equal(k1[0], k_all[l]) and np.array_equal(v1[0], v_all[l])


def test_power_of_two_scaling_on_device():
    """No bias: X -> 2X gives exactly 2V; with eps = 0, K is bit-identical."""
    case = W.make_case(T=40, H=128, L=2, NH=1, D=128, eps=0.0, slots=64, seed=24)
    dc, pack, _ = _run(case, "scale x1")
    k1, v1 = dc.pools_host()
    case.x = O.encode(O.decode(case.x, "bf16") * 2.0, "bf16")
    dc2 = DeviceCase(case)
    assert dc2.write(dc2.pack())
    k2, v2 = dc2.pools_host()
    for l in range(case.L):
        assert np.array_equal(k1[l], k2[l])
        sl = case.locs
        np.testing.assert_array_equal(O.decode(v2[l][sl], "bf16"), 2.0 * O.decode(v1[l][sl], "bf16"))


def test_repeatable():
    case = W.make_case(T=100, H=256, L=2, NH=2, D=128, slots=128, seed=25)
    dc, pack, _ = _run(case, "repeat")
    k1, v1 = dc.pools_host()
    dc.reset_pools()
    assert dc.write(pack)
    k2, v2 = dc.pools_host()
    assert all(np.array_equal(a, b) for a, b in zip(k1 + v1, k2 + v2))


# ------------------------------------------------------------ edge cases

def test_commit_len_edges():
    """commit_len 0 writes nothing, W writes the whole row, W+3 the whole row too."""
    case = W.make_case(T=24, H=64, L=2, NH=1, D=64, row_width=8, slots=64, seed=26)
    case.commit_lens = np.array([0, 8, 11], dtype=np.int64)
    dc, _, _ = _run(case, "commit 0 / W / W+3")
    assert len(dc.touched_slots(0, "k")) == 16


@pytest.mark.parametrize("committed", [276, 384, 385, 512])
def test_adaptive_k_split(committed):
    """A 512-row commit window over 40 weight tiles (the wide_gqa_d64 shape):
    on 256 compute units the plan has three token splits of 128 slots and two
    K parts (one round). 276 and 384 written rows fit the three splits (K
    split, part sums and the reduce launch); 385 and 512 do not, and the same
    workgroups keep K whole as six token splits (no part sums; the reduce
    launch finds no rows)."""
    W_, B = 8, 64
    case = W.make_case(T=512, H=1024, L=5, NH=4, D=128, row_width=W_, slots=600, seed=41)
    lens = np.full(B, committed // B, dtype=np.int64)
    lens[: committed % B] += 1
    case.commit_lens = lens
    dc, pack, _ = _run(case, f"{committed} of 512 rows committed")
    plan = pack.plan(case.T, True)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert plan["kernel"] == "stream_ksplit" and plan["k_parts"] == 2, plan
        assert plan["token_splits"] == 3 and plan["adaptive"], plan
    assert len(dc.touched_slots(4, "v")) == committed
    # the same shape with a row count of the other mode
    case.commit_lens = np.full(B, 8 if committed <= 384 else 4, dtype=np.int64)
    dc2, _, _ = _run(case, "other mode, same shape")


ADAPTIVE = {
    # 40 weight tiles each: the adaptive plan on 256 compute units
    "fp16_bias_d64": dict(T=512, H=1024, L=5, NH=8, D=64, dtype="fp16", bias=True),
    "bf16_bias_ktail": dict(T=512, H=1096, L=5, NH=4, D=128, bias=True),
    "fp16_ten_layers": dict(T=512, H=1024, L=10, NH=2, D=128, dtype="fp16"),
    "bf16_T400": dict(T=400, H=1024, L=5, NH=8, D=64),
}


@pytest.mark.parametrize("mode", ["k_split", "k_whole"])
@pytest.mark.parametrize("name", list(ADAPTIVE))
def test_adaptive_k_split_variants(name, mode):
    """The adaptive plan's kernel instances (dtype, bias, head size, a K tail,
    a window that is not a multiple of the split size), each with about half
    of the window committed (K split) and with all of it (K whole)."""
    kw = ADAPTIVE[name]
    case = W.make_case(row_width=8, slots=kw["T"] + 100, commit_range=(1, 9),
                       seed=zlib.crc32(name.encode()) % 10000, **kw)
    if mode == "k_whole":
        case.commit_lens = np.full(kw["T"] // 8, 8, dtype=np.int64)
    dc, pack, _ = _run(case, f"{name} {mode}")
    plan = pack.plan(case.T, True)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert plan["adaptive"] and plan["token_splits"] == 3, plan
    written = int(O.valid_rows(case.locs, case.commit_lens, case.row_width).sum())
    assert (written > 3 * 128) == (mode == "k_whole"), written


def test_commit_rows_spread_over_token_splits():
    """Small-T commit windows: only written rows are projected, numbered in row
    order and dealt to the token splits in turn. Eight splits with three rows
    (five splits get none), no rows at all, a 1000-row window list (32
    splits, two passes of the row scan) with holes and negative slots, and a
    1600-row one, past the scan's limit (contiguous splits, the window applied
    at the store)."""
    case = W.make_case(T=256, H=128, L=2, NH=1, D=64, row_width=8, slots=300, seed=31)
    case.commit_lens = np.zeros(32, dtype=np.int64)
    case.commit_lens[5] = 3
    dc, _, _ = _run(case, "three rows over eight splits")
    assert len(dc.touched_slots(0, "k")) == 3
    case.commit_lens[5] = 0
    dc, _, _ = _run(case, "no committed rows")
    assert len(dc.touched_slots(1, "v")) == 0
    mid = W.make_case(T=1000, H=192, L=1, NH=1, D=64, row_width=8, commit_range=(0, 9),
                      neg_loc_frac=0.1, slots=1200, seed=33)
    _run(mid, "1000 rows, 32 splits")
    big = W.make_case(T=1600, H=192, L=1, NH=1, D=64, row_width=8, commit_range=(0, 9),
                      neg_loc_frac=0.1, slots=2000, seed=32)
    _run(big, "1600 rows, 50 splits")


@pytest.mark.parametrize("T,row_width", [(70, 7), (3000, None)])
def test_max_layers(T, row_width):
    """DSPARK_MAX_LAYERS layers in one pack: every layer's pool descriptor
    travels in the kernel arguments (streaming path with a commit window, and
    the tiled path)."""
    kw = dict(row_width=row_width, commit_range=(0, 8)) if row_width else {}
    case = W.make_case(T=T, H=128, L=dk.MAX_LAYERS, NH=1, D=64, slots=T + 50, seed=34 + T, **kw)
    _run(case, f"{dk.MAX_LAYERS} layers, T={T}")


def test_all_rows_skipped_and_empty():
    case = W.make_case(T=16, H=64, L=1, NH=1, D=64, slots=32, seed=27)
    case.locs[:] = -1
    dc = DeviceCase(case)
    pack = dc.pack()
    assert dc.write(pack)
    assert len(dc.touched_slots(0, "k")) == 0 and len(dc.touched_slots(0, "v")) == 0
    # T == 0: OK and nothing enqueued
    empty = torch.empty((0, case.H), dtype=torch.bfloat16, device="cuda")
    e64 = torch.empty((0,), dtype=torch.int64, device="cuda")
    assert dk.ctx_kv_write(pack, empty, e64, e64, dc.pool_descs(), range_errors=dc.err)
    assert dc.range_errors() == 0


@pytest.mark.parametrize("T,H,L,NH,slots", [(20, 64, 2, 1, 32), (20, 1024, 2, 1, 32),
                                              (6000, 64, 3, 2, 6050)],
                         ids=["plain", "k_split", "tiled"])
def test_out_of_range_rows_are_skipped_and_counted(T, H, L, NH, slots):
    # H = 1024: two weight tiles and 16 chunks of 64, so K is split over
    # workgroups and the count comes from the reduce launch; T = 6000 over six
    # weight tiles takes the tiled kernel
    case = W.make_case(T=T, H=H, L=L, NH=NH, D=64, slots=slots, P=64, seed=28)
    case.positions[3] = 64       # == P
    case.positions[5] = -2
    case.locs[7] = slots         # == slots
    dc = DeviceCase(case)
    pack = dc.pack()
    want_kernel = {20: "stream_ksplit" if H == 1024 else "stream", 6000: "tiled"}[T]
    assert pack.plan(T, False)["kernel"] == want_kernel
    assert dc.write(pack)
    torch.cuda.synchronize()
    assert dc.range_errors() == 3 * case.L
    assert dc.range_errors() == 0  # read-and-clear
    skipped = {3, 5, 7}
    want = np.sort([case.locs[t] for t in range(case.T) if t not in skipped])
    assert np.array_equal(np.sort(dc.touched_slots(0, "k")), want)
    ok_rows = [t for t in range(case.T) if t not in skipped]
    compare_rows(dc, ok_rows, "out-of-range rows")


def test_pool_layout_fallback_and_invalid_pairing():
    case = W.make_case(T=8, H=64, L=2, NH=2, D=64, row_width=4, slots=16, seed=29)
    dc = DeviceCase(case)
    pack = dc.pack()
    pools = dc.pool_descs()
    bad = list(pools)
    bad[1] = dk.PoolDesc(**{f: getattr(pools[1], f) for f, _ in dk.PoolDesc._fields_})
    bad[1].k_stride1 = 2 * case.D
    assert dk.ctx_kv_write(pack, dc.x, dc.positions, dc.locs, bad, commit_lens=dc.commit,
                           locs_row_width=4) is False
    wrong_dtype = list(pools)
    wrong_dtype[0] = dk.PoolDesc(**{f: getattr(pools[0], f) for f, _ in dk.PoolDesc._fields_})
    wrong_dtype[0].dtype = dk.FP16
    assert dk.ctx_kv_write(pack, dc.x, dc.positions, dc.locs, wrong_dtype, commit_lens=dc.commit,
                           locs_row_width=4) is False
    torch.cuda.synchronize()
    assert len(dc.touched_slots(0, "k")) == 0  # nothing written on fallback
    raw = lambda **kw: dk.ctx_kv_write_raw(
        pack, dc.x.data_ptr(), kw.get("T", 8), case.H, dc.positions.data_ptr(),
        dc.locs.data_ptr(), kw.get("commit"), kw.get("W", 0), kw.get("B", 0),
        kw.get("pools", pools), None, flags=kw.get("flags", 0))[0]
    assert raw(commit=dc.commit.data_ptr()) == dk.E_INVALID               # commit without W
    assert raw(W=4, B=2) == dk.E_INVALID                                  # W without commit
    assert raw(commit=dc.commit.data_ptr(), W=4, B=3) == dk.E_INVALID     # B*W != T
    assert raw(pools=pools[:1]) == dk.E_INVALID                           # wrong pool count
    assert raw(T=-1) == dk.E_INVALID
    assert raw(commit=dc.commit.data_ptr(), W=4, B=2, flags=2) == dk.E_INVALID  # unknown flag
    with pytest.raises(ValueError):
        dk.ctx_kv_write(pack, dc.x, dc.positions, dc.locs, pools, commit_lens=dc.commit)
    # the binding's own checks: index dtypes and lengths, the activation dtype
    with pytest.raises(ValueError):
        dk.ctx_kv_write(pack, dc.x, dc.positions.to(torch.int32), dc.locs, pools,
                        commit_lens=dc.commit, locs_row_width=4)
    with pytest.raises(ValueError):
        dk.ctx_kv_write(pack, dc.x, dc.positions, dc.locs[:7], pools, commit_lens=dc.commit,
                        locs_row_width=4)
    with pytest.raises(ValueError):
        dk.ctx_kv_write(pack, dc.x, dc.positions, dc.locs, pools,
                        commit_lens=dc.commit.to(torch.int32), locs_row_width=4)
    with pytest.raises(ValueError):
        dk.ctx_kv_write(pack, dc.x.to(torch.float16), dc.positions, dc.locs, pools,
                        commit_lens=dc.commit, locs_row_width=4)
    with pytest.raises(ValueError):
        dk.ctx_kv_write(pack, dc.x, dc.positions[::2].repeat_interleave(2)[:8].contiguous()
                        .cpu(), dc.locs, pools, commit_lens=dc.commit, locs_row_width=4)
    torch.cuda.synchronize()
    assert len(dc.touched_slots(0, "k")) == 0


def test_k_split_workspace_is_required():
    """A K-split write without a large enough workspace is E_INVALID and
    enqueues nothing."""
    case = W.make_case(T=64, H=1024, L=1, NH=1, D=128, slots=128, seed=47)
    dc = DeviceCase(case)
    pack = dc.pack()
    need = pack.workspace_bytes(case.T, False)
    assert need > 0 and pack.plan(case.T, False)["kernel"] == "stream_ksplit"
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    raw = lambda ws, n: dk.ctx_kv_write_raw(
        pack, dc.x.data_ptr(), case.T, case.H, dc.positions.data_ptr(), dc.locs.data_ptr(),
        None, 0, 0, dc.pool_descs(), None, workspace=ws, workspace_bytes=n)[0]
    assert raw(None, 0) == dk.E_INVALID
    assert raw(small.data_ptr(), small.numel()) == dk.E_INVALID
    torch.cuda.synchronize()
    assert len(dc.touched_slots(0, "k")) == 0


def _validate_case(**kw):
    return W.make_case(T=24, H=64, L=2, NH=1, D=64, row_width=8, commit_range=(1, 8),
                       slots=40, P=64, seed=48, **kw)


@pytest.mark.parametrize("what", ["position", "slot", "duplicate"])
def test_validate_mode_reports_range_errors(what):
    """Validate mode: an out-of-table position, a slot past the pool, or two
    stored rows naming one slot return E_RANGE with the cause and write
    nothing."""
    case = _validate_case()
    case.commit_lens[:] = 8
    if what == "position":
        case.positions[9] = case.P
        cause = dk.RANGE_POSITION
    elif what == "slot":
        case.locs[17] = case.slots
        cause = dk.RANGE_SLOT
    else:
        case.locs[20] = case.locs[2]
        cause = dk.RANGE_DUPLICATE
    dc = DeviceCase(case)
    pack = dc.pack()
    say(f"[case] validate mode: {what}")
    with pytest.raises(dk.RangeError) as e:
        dc.write(pack, validate=True)
    assert e.value.cause == cause
    torch.cuda.synchronize()
    assert len(dc.touched_slots(0, "k")) == 0 and len(dc.touched_slots(1, "v")) == 0


def test_validate_mode_ignores_rows_that_are_not_stored():
    """Rows past a request's commit length or with a negative slot are not
    checked (they are never stored): a duplicate or bad position there passes,
    and the write then matches the oracle."""
    case = _validate_case()
    case.commit_lens[:] = [3, 8, 5]
    case.locs[6] = case.locs[0]          # truncated column of request 0
    case.positions[7] = 10 ** 6          # truncated too
    case.locs[12] = -1
    case.positions[12] = -5              # negative slot: skipped
    dc, pack, _ = _run(case, "validate: unchecked rows")
    dc.reset_pools()
    assert dc.write(pack, validate=True)
    torch.cuda.synchronize()
    check_slot_sets(dc)
    compare_rows(dc, None, "validate mode")
    assert dc.range_errors() == 0


def test_fallback_logging(capfd, monkeypatch):
    """DSPARK_LOG=1 prints the reason of the first write fallback of a pack."""
    monkeypatch.setenv("DSPARK_LOG", "1")
    case = W.make_case(T=8, H=64, L=1, NH=1, D=64, slots=16, seed=49)
    dc = DeviceCase(case)
    pack = dc.pack()
    bad = dc.pool_descs()
    bad[0].k_stride1 = 2 * case.D
    assert dk.ctx_kv_write(pack, dc.x, dc.positions, dc.locs, bad) is False
    assert dk.ctx_kv_write(pack, dc.x, dc.positions, dc.locs, bad) is False
    err = capfd.readouterr().err
    assert err.count("dspark_ctx_kv_write fell back") == 1
    assert "pool dtype, layout or alignment" in err or "KV pool dtype" in err


def test_rope_tables_by_content():
    case = W.make_case(T=8, H=64, L=2, NH=1, D=64, slots=16, seed=30)
    dc = DeviceCase(case)
    descs = dc.layer_descs()
    same = dc.table.clone()                       # another pointer, same content
    descs[1] = dk.layer_desc(dc.qkv_w[1], dc.k_norm[1], case.eps, case.q_size, case.kv, case.D,
                             same)
    assert dk.pack_ctx_kv(descs, case.H, dk.BF16) is not None
    other = same.clone()
    other[5, 3] += 1e-3                           # different content
    descs[1] = dk.layer_desc(dc.qkv_w[1], dc.k_norm[1], case.eps, case.q_size, case.kv, case.D,
                             other)
    assert dk.pack_ctx_kv(descs, case.H, dk.BF16) is None
    assert dk.FALLBACK_REASONS[dk.last_fallback_reason] == "ROPE"


@pytest.mark.parametrize("T,H,kernel", [(96, 192, "stream"), (96, 1024, "stream_ksplit"),
                                         (4200, 256, "tiled")],
                         ids=["plain", "k_split", "tiled"])
def test_graph_replays_match_eager(T, H, kernel):
    """The write captured in a HIP graph (as the benchmark times it) gives the
    eager result on every replay, with eager work and syncs between replays.
    At H = 1024 K is split over workgroups: two launches per write, sharing
    one caller workspace across replays. At 4200 rows (on 256 compute units)
    the LDS-tiled kernel runs."""
    case = W.make_case(T=T, H=H, L=2, NH=2, D=128, row_width=8, slots=8192, seed=31)
    dc, pack, _ = _run(case, "eager reference")
    k_ref, v_ref = dc.pools_host()
    ws = dc.workspace(pack)
    assert (ws is not None) == (H == 1024)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert pack.plan(T, True)["kernel"] == kernel
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    dc.reset_pools()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            assert dc.write(pack, workspace=ws)
    for rep in range(4):
        for p in dc.pk + dc.pv:
            p.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        k, v = dc.pools_host()
        assert all(np.array_equal(a, b) for a, b in zip(k + v, k_ref + v_ref)), rep


def test_adaptive_plan_switches_modes_between_graph_replays():
    """The adaptive plan captured once in a HIP graph: the commit lengths are
    device data, so replays alternate between a window that fits the K-split
    splits (about half committed) and a fully committed one (K whole), each
    replay matching the eager result of its own commit lengths."""
    case = W.make_case(T=512, H=1024, L=5, NH=4, D=128, row_width=8, commit_range=(1, 9),
                       slots=700, seed=57)
    half = case.commit_lens.copy()
    full = np.full(64, 8, dtype=np.int64)
    refs = {}
    for name, lens in (("half", half), ("full", full)):
        case.commit_lens = lens
        dc, pack, _ = _run(case, f"eager, {name} committed")
        refs[name] = dc.pools_host()
    assert pack.plan(case.T, True)["adaptive"] or \
        torch.cuda.get_device_properties(0).multi_processor_count != 256
    ws = dc.workspace(pack)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    dc.reset_pools()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            assert dc.write(pack, workspace=ws)
    for rep, name in enumerate(["half", "full", "half", "full"]):
        dc.commit.copy_(torch.from_numpy(half if name == "half" else full))
        for p in dc.pk + dc.pv:
            p.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        k, v = dc.pools_host()
        k_ref, v_ref = refs[name]
        assert all(np.array_equal(a, b) for a, b in zip(k + v, k_ref + v_ref)), (rep, name)
