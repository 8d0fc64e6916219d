"""Element offsets past 2^31: the write, the producer, the QK op, verify and
the draft attention
with operand row strides padded so that the last rows start beyond 2^31
elements of their buffers (4-21 GB device tensors), while the values the
oracle computes stay small. A 32-bit offset anywhere on these paths would
read or write the wrong rows; every stored row is compared with the oracle
to the usual tolerance (exactly for verify), and padding columns the calls
must not touch are checked on the device.
"""

import numpy as np
import pytest
import torch

import speculative_decoding_draft_stacked_amd as dk
from speculative_decoding_draft_stacked_amd import workloads as W
from speculative_decoding_draft_stacked_amd.harness import DeviceCase
from oracle import ctx_kv_oracle as O
from oracle import draft_attention_oracle as A
from oracle import main_proj_oracle as M
from oracle import qk_norm_rope_oracle as Q
from oracle import verify_oracle as V

from gpu_util import TOL, check_slot_sets, compare_rows, say

pytestmark = pytest.mark.gpu
_T = {"bf16": torch.bfloat16, "fp16": torch.float16}
_BIG = 1 << 31


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    dk.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _dev16(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(_T[dtype]).cuda()


def _padded(rows_bits, stride, dtype, fill=-7):
    """A [rows, stride] device buffer holding rows_bits in its first columns
    (the rest set to `fill`), and the [rows, width] view of them."""
    n, width = rows_bits.shape
    full = torch.full((n, stride), fill, dtype=torch.int16, device="cuda")
    full[:, :width] = torch.from_numpy(np.ascontiguousarray(rows_bits).view(np.int16)).cuda()
    return full, full.view(_T[dtype])[:, :width]


def _untouched(full, width, fill=-7):
    """The padding columns of a padded buffer still hold `fill` (checked on the
    device, first and last 64 columns of every row)."""
    pad = full[:, width:]
    return bool((pad[:, :64] == fill).all()) and bool((pad[:, -64:] == fill).all())


def test_write_with_offsets_past_2_31():
    """65536 tokens through the LDS-tiled kernel: ctx_hidden rows 40960
    elements apart (the last row starts at 2.7e9) and pool rows 32768
    elements apart (the last slot at 2.1e9)."""
    case = W.make_case(T=65536, H=64, L=1, NH=1, D=128, slots=65600, seed=91)
    stride = 40960
    assert (case.T - 1) * stride > _BIG
    dc = DeviceCase(case, pool_row_pad=32768 - 128)
    assert (case.slots - 1) * 32768 > _BIG
    x_full, dc.x = _padded(case.x, stride, case.dtype)
    pack = dc.pack()
    say(f"[large] write: plan {pack.plan(case.T, False)}")
    assert dc.write(pack)
    torch.cuda.synchronize()
    check_slot_sets(dc)
    st = compare_rows(dc, None, "large offsets")
    assert dc.range_errors() == 0
    assert _untouched(x_full, case.H)
    say(f"  ok: {st}")
    pack.free()


def test_producer_with_offsets_past_2_31():
    """65536 tokens through the producer's tiled projection and row norm:
    aux rows 40960 + 128 elements apart, ctx rows 40960 apart."""
    c = W.make_proj_case(T=65536, H=128, n_aux=1, seed=92)
    aux_full, aux = _padded(c.aux, 40960 + 128, c.dtype)
    ctx_full, ctx = _padded(np.zeros((c.T, c.H), np.uint16), 40960, c.dtype)
    assert (c.T - 1) * 40960 > _BIG
    w = _dev16(c.w, c.dtype)
    g = _dev16(c.g, c.dtype)
    pack = dk.pack_main_proj(w, g, c.eps)
    assert pack is not None
    ws = torch.empty(max(pack.workspace_bytes(c.T), 16), dtype=torch.uint8, device="cuda")
    dk.main_proj_norm(pack, aux, ctx, ws)
    torch.cuda.synchronize()
    got = O.decode(ctx.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), c.dtype)
    want = M.combine_hidden_states(c.aux, c.w, c.g, c.g_dtype, c.eps, c.dtype)
    rtol, atol = TOL[c.dtype]
    bad = np.abs(got - want) > atol + rtol * np.abs(want)
    assert np.all(np.isfinite(got)) and not bad.any(), np.argwhere(bad)[:3]
    assert _untouched(ctx_full, c.H) and _untouched(aux_full, c.aux.shape[1])
    pack.free()


def test_qk_with_offsets_past_2_31():
    """65536 tokens of the in-place QK op on rows 32768 + 256 elements apart."""
    c = W.make_qk_case(T=65536, NHQ=2, NHK=1, D=64, seed=93)
    width = (c.NHQ + 2 * c.NHK) * c.D
    stride = 32768 + width
    full, qkv = _padded(c.qkv, stride, c.dtype)
    assert (c.T - 1) * stride > _BIG
    pos = torch.from_numpy(c.positions).cuda()
    q_w, k_w = _dev16(c.q_w, c.dtype), _dev16(c.k_w, c.dtype)
    table = torch.from_numpy(c.table).cuda()
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    assert dk.table_qk_norm_rope(qkv, pos, q_w, k_w, table, c.NHQ, c.NHK, c.D, c.eps,
                                 range_errors=err)
    torch.cuda.synchronize()
    got = qkv.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    want = c.qkv.copy()
    skipped = Q.qk_norm_rope_inplace(want, c.positions, c.q_w, c.k_w, c.weight_dtype, c.table,
                                     c.NHQ, c.NHK, c.D, c.eps, c.dtype)
    assert skipped == 0 and int(err.item()) == 0
    nh = (c.NHQ + c.NHK) * c.D
    assert np.array_equal(got[:, nh:], want[:, nh:]), "value heads changed"
    g, wv = O.decode(got[:, :nh], c.dtype), O.decode(want[:, :nh], c.dtype)
    rtol, atol = TOL[c.dtype]
    bad = np.abs(g - wv) > atol + rtol * np.abs(wv)
    assert not bad.any(), np.argwhere(bad)[:3]
    assert _untouched(full, width)


def test_verify_with_offsets_past_2_31():
    """65536 requests with draft and target rows 40960 int64 entries apart."""
    c = W.make_verify_case(B=65536, K=7, vocab=151936, seed=94)
    stride = 40960
    dd = torch.full((c.B, stride), -3, dtype=torch.int64, device="cuda")
    tt = torch.full((c.B, stride), -3, dtype=torch.int64, device="cuda")
    dd[:, :c.K] = torch.from_numpy(c.draft).cuda()
    tt[:, :c.K + 1] = torch.from_numpy(c.target).cuda()
    assert (c.B - 1) * stride > _BIG
    acc = torch.full((c.B,), -7, dtype=torch.int64, device="cuda")
    bon = torch.full((c.B,), -7, dtype=torch.int64, device="cuda")
    dk.verify_accept(dd[:, :c.K], tt[:, :c.K + 1], acc, bon)
    torch.cuda.synchronize()
    ea, eb = V.accept_and_bonus(c.draft, c.target)
    assert np.array_equal(acc.cpu().numpy(), ea)
    assert np.array_equal(bon.cpu().numpy(), eb)


def test_attention_with_pool_offsets_past_2_31():
    """Two requests of 3000 prefix keys gathered from pools whose slots are
    40960 elements apart (a fifth of the 65600 slots start past 2^31)."""
    c = W.make_attn_case(B=2, block=8, nhq=4, nhk=1, D=128, prefix=[3000, 3000], slots=65600,
                         seed=95)
    stride = 40960
    assert (c.slots - 1) * stride > _BIG
    assert int(np.sum(c.kv_indices * stride > _BIG)) > 100
    row = c.nhk * c.D
    kfull, kp = _padded(c.k_pool.reshape(c.slots, row), stride, c.dtype)
    vfull, vp = _padded(c.v_pool.reshape(c.slots, row), stride, c.dtype)
    q = _dev16(c.q, c.dtype)
    ke, ve = _dev16(c.k_ext, c.dtype), _dev16(c.v_ext, c.dtype)
    indptr = torch.from_numpy(c.kv_indptr).cuda()
    indices = torch.from_numpy(c.kv_indices).cuda()
    out = torch.full(c.q.shape, -7, dtype=torch.int16, device="cuda").view(_T[c.dtype])
    n = dk.draft_attention_workspace_bytes(c.B, c.block, c.nhq, c.nhk, c.D, c.max_prefix)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    assert dk.draft_attention(q, ke, ve, kp.unflatten(1, (c.nhk, c.D)),
                              vp.unflatten(1, (c.nhk, c.D)), indptr, indices, out, c.block,
                              c.sm_scale, c.max_prefix, ws, err)
    torch.cuda.synchronize()
    got = O.decode(out.view(torch.int16).cpu().numpy().view(np.uint16), c.dtype)
    want, skipped = A.draft_attention(c.q, c.k_ext, c.v_ext, c.k_pool, c.v_pool, c.kv_indptr,
                                      c.kv_indices, c.block, c.nhq, c.nhk, c.sm_scale, c.dtype)
    assert skipped == 0 and int(err.item()) == 0
    rtol, atol = TOL[c.dtype]
    bad = np.abs(got - want) > atol + rtol * np.abs(want)
    assert np.all(np.isfinite(got)) and not bad.any(), np.argwhere(bad)[:3]
    assert _untouched(kfull, row) and _untouched(vfull, row)

