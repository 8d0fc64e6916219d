"""Host-only checks of the C ABI: the library loads, exports every function
include/dspark.h declares, and its eligibility rules and argument checks behave
as documented. Nothing here dereferences a device pointer or launches work."""

import ctypes
import os
import re
import subprocess
import sys

import pytest

import speculative_decoding_draft_stacked_amd as dk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "dspark.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    assert _declared() == sorted(dk.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = dk.lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_struct_layouts_match_c(tmp_path):
    """The ctypes mirrors have the C compiler's size and field offsets."""
    fields = {"dspark_layer_desc": dk.LayerDesc, "dspark_pool_desc": dk.PoolDesc,
              "dspark_attn_desc": dk.AttnDesc, "dspark_write_plan": dk.WritePlan}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "dspark.h"', "int main(void) {"]
    for cname, py in fields.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    for line in out.splitlines():
        cname, field, value = line.split()
        py = fields[cname]
        got = ctypes.sizeof(py) if field == "size" else getattr(py, field).offset
        assert got == int(value), (cname, field)


def test_status_and_reason_strings():
    assert dk.status_str(dk.OK) == "ok"
    assert "fallback" in dk.status_str(dk.FALLBACK)
    assert "out of range" in dk.status_str(dk.E_RANGE)
    assert dk.fallback_str(5) == "QKV bias present in some layers only"
    assert dk.fallback_str(1234) == "unknown reason"
    assert "same slot" in dk.range_str(dk.RANGE_DUPLICATE)
    assert "rotary table" in dk.range_str(dk.RANGE_POSITION)
    assert dk.range_str(99) == "unknown cause"


# Fake (never dereferenced) device addresses, 16-byte aligned.
def _layer(i=0, **kw):
    H, D, NH = 256, 64, 2
    base = dict(qkv_weight=0x10000000 + i * 0x100000, w_rows=H + 2 * NH * D, w_row_stride=H,
                w_col_stride=1, w_dtype=dk.BF16, qkv_bias=None, k_norm_weight=0x20000000 + i * 256,
                k_norm_dtype=dk.BF16, k_norm_eps=1e-6, q_size=H, kv_size=NH * D, head_dim=D,
                has_kv_scale=0, rope_cos_sin=0x30000000, rope_dtype=dk.FP32, rope_max_pos=4096,
                rope_dim=D, rope_is_neox=1)
    base.update(kw)
    return dk.LayerDesc(**base)


def _elig(layers, hidden=256, dtype=dk.BF16):
    return dk.check_eligibility(layers, hidden, dtype)


def test_eligible_layers():
    assert _elig([_layer(i) for i in range(5)]) == (dk.OK, 0)
    assert _elig([_layer(i, qkv_bias=0x40000000 + i * 4096) for i in range(3)]) == (dk.OK, 0)
    fp16 = [_layer(i, w_dtype=dk.FP16, k_norm_dtype=dk.FP32) for i in range(2)]
    assert _elig(fp16, dtype=dk.FP16) == (dk.OK, 0)


# The fallback trio of the stacked path (sglang PR #31986 parity test: quantized
# weight, eps mismatch, bias mismatch) plus the stricter checks of the fused
# bundle (sglang PR #31847).
@pytest.mark.parametrize("mutate,reason", [
    (lambda ls: ls[1].__setattr__("w_dtype", dk.QUANTIZED), "NOT_SLICEABLE"),
    (lambda ls: ls[2].__setattr__("k_norm_eps", 1e-5), "EPS_MISMATCH"),
    (lambda ls: ls[1].__setattr__("qkv_bias", 0x40000000), "MIXED_BIAS"),
    (lambda ls: ls[0].__setattr__("w_col_stride", 2), "NOT_SLICEABLE"),
    (lambda ls: ls[0].__setattr__("w_rows", 256 + 100), "NOT_SLICEABLE"),
    (lambda ls: ls[1].__setattr__("has_kv_scale", 1), "KV_SCALE"),
    (lambda ls: (ls[2].__setattr__("kv_size", 192), ls[2].__setattr__("w_rows", 1024)), "SHAPE"),
    (lambda ls: [(l.__setattr__("kv_size", 96), l.__setattr__("w_rows", 1024)) for l in ls], "SHAPE"),
    (lambda ls: ls[1].__setattr__("rope_is_neox", 0), "ROPE"),
    (lambda ls: ls[1].__setattr__("rope_dim", 32), "ROPE"),
    (lambda ls: ls[0].__setattr__("rope_dtype", dk.BF16), "ROPE"),
    (lambda ls: ls[2].__setattr__("rope_max_pos", 2048), "ROPE"),
    (lambda ls: ls[0].__setattr__("k_norm_dtype", dk.QUANTIZED), "DTYPE"),
])
def test_fallback_reasons(mutate, reason):
    layers = [_layer(i) for i in range(3)]
    mutate(layers)
    st, r = _elig(layers)
    assert st == dk.FALLBACK and dk.FALLBACK_REASONS[r] == reason


def test_fallback_shapes_and_counts():
    assert _elig([]) == (dk.FALLBACK, 1)
    assert _elig([_layer(i) for i in range(33)])[1] == 2
    # head_dim outside the kernels' coverage
    l32 = [_layer(0, head_dim=32, rope_dim=32, kv_size=64)]
    assert dk.FALLBACK_REASONS[_elig(l32)[1]] == "SHAPE"
    # hidden not a multiple of 8
    odd = [_layer(0, w_row_stride=260)]
    assert dk.FALLBACK_REASONS[_elig(odd, hidden=258)[1]] == "SHAPE"
    # activation dtype fp32 is not a supported GEMM input
    assert dk.FALLBACK_REASONS[_elig([_layer(0)], dtype=dk.FP32)[1]] == "DTYPE"
    # weight dtype must equal the activation dtype
    assert dk.FALLBACK_REASONS[_elig([_layer(0)], dtype=dk.FP16)[1]] == "NOT_SLICEABLE"


def test_invalid_arguments():
    assert _elig([_layer(0)], hidden=0)[0] == dk.E_INVALID
    assert _elig([_layer(0, qkv_weight=None)])[0] == dk.E_INVALID
    lib = dk.lib()
    assert lib.dspark_check_eligibility(None, 2, 256, dk.BF16, None) == dk.E_INVALID
    out = ctypes.c_void_p(123)
    # NULL out pointer, and NULL pack for every pack-taking call
    assert lib.dspark_pack_ctx_kv(None, 1, 256, dk.BF16, None, None, None) == dk.E_INVALID
    assert lib.dspark_ctx_kv_write(None, None, 4, 256, None, None, None, 0, 0, None, 0, None, 0,
                                   None, 0, None, None) == dk.E_INVALID
    n = ctypes.c_int64()
    plan = dk.WritePlan()
    assert lib.dspark_ctx_kv_plan(None, 4, 0, ctypes.byref(plan)) == dk.E_INVALID
    assert lib.dspark_ctx_kv_workspace_bytes(None, 4, 0, ctypes.byref(n)) == dk.E_INVALID
    assert lib.dspark_pack_info(None, None, None, None, None, None, None) == dk.E_INVALID
    lib.dspark_pack_free(None)  # no-op
    # ineligible layers: pack reports fallback before touching the device
    reason = ctypes.c_int32()
    arr = (dk.LayerDesc * 2)(_layer(0), _layer(1, k_norm_eps=1.0))
    assert lib.dspark_pack_ctx_kv(arr, 2, 256, dk.BF16, None, ctypes.byref(out),
                                  ctypes.byref(reason)) == dk.FALLBACK
    assert out.value is None and reason.value == 4


_LOG_SNIPPET = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
import speculative_decoding_draft_stacked_amd as dk
from tests.test_boundary_cpu import _layer
out, reason = ctypes.c_void_p(0), ctypes.c_int32()
arr = (dk.LayerDesc * 2)(_layer(0), _layer(1, qkv_bias=0x40000000))
st = dk.lib().dspark_pack_ctx_kv(arr, 2, 256, dk.BF16, None, ctypes.byref(out),
                                 ctypes.byref(reason))
print(st, reason.value)
"""


@pytest.mark.parametrize("value,logged", [("1", True), ("0", False), ("", False)])
def test_pack_fallback_logging(value, logged):
    """DSPARK_LOG set (not "0") prints the reason of a pack fallback on stderr;
    the pages name silent fallback as a risk."""
    env = dict(os.environ, DSPARK_LOG=value)
    r = subprocess.run([sys.executable, "-c", _LOG_SNIPPET.format(root=ROOT)], env=env,
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == [str(dk.FALLBACK), "5"]
    line = "dspark: dspark_pack_ctx_kv fell back: QKV bias present in some layers only"
    assert (line in r.stderr) == logged


# ------------------------------------------------ in-place table QK norm + rotation

def _qk(T=5, stride=512, D=128, act=dk.BF16, wdt=None, eps=1e-6, P=10, nhq=2, nhk=1):
    """Call with NULL device pointers: only host-side checks may run."""
    r = ctypes.c_int32(-7)
    st = dk.lib().dspark_table_qk_norm_rope(None, T, stride, None, nhq, nhk, D, act, None, None,
                                             act if wdt is None else wdt, eps, None, P, None,
                                             None, ctypes.byref(r))
    return st, r.value


def test_qk_empty_call_is_ok_and_enqueues_nothing():
    assert _qk(T=0) == (dk.OK, 0)


@pytest.mark.parametrize("kw,reason", [
    (dict(D=96), 6), (dict(D=256), 6),                          # SHAPE
    (dict(act=dk.FP32), 7), (dict(act=dk.QUANTIZED), 7),       # DTYPE
    (dict(act=dk.BF16, wdt=dk.FP16), 7), (dict(act=dk.FP16, wdt=dk.BF16), 7),
])
def test_qk_fallbacks(kw, reason):
    assert _qk(**kw) == (dk.FALLBACK, reason)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(nhq=0), dict(nhk=-1), dict(stride=3 * 128 - 8), dict(stride=3 * 128 + 4),
    dict(eps=-1e-6), dict(eps=float("nan")), dict(eps=float("inf")), dict(P=0),
    dict(),  # NULL pointers with tokens to process
])
def test_qk_invalid_arguments(kw):
    assert _qk(**kw)[0] == dk.E_INVALID


def test_qk_weight_dtype_may_be_fp32():
    # passes the dtype checks and stops at the NULL pointers
    assert _qk(wdt=dk.FP32) == (dk.E_INVALID, 0)
    assert _qk(act=dk.FP16, wdt=dk.FP32) == (dk.E_INVALID, 0)


# ------------------------------------------------ verify accept length + bonus

def _verify(B=4, K=7, ds=7, ts=8, d=None, t=None, acc=None, bon=None):
    """NULL device pointers: only host-side checks may run."""
    return dk.lib().dspark_verify_accept(d, ds, t, ts, B, K, acc, bon, None)


def test_verify_empty_is_ok():
    assert _verify(B=0) == dk.OK


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(K=-1), dict(ds=6), dict(ts=7), dict(),  # last: NULL pointers with work
])
def test_verify_invalid_arguments(kw):
    assert _verify(**kw) == dk.E_INVALID


# ------------------------------------------------------------ context producer

def _proj_pack(out_f=256, in_f=768, stride=768, wdt=dk.BF16, gdt=dk.BF16, eps=1e-6,
               act=dk.BF16, w=16, g=16):
    """Host-side checks only: fake non-NULL pointers are never dereferenced
    before a check fails."""
    h = ctypes.c_void_p(0)
    r = ctypes.c_int32(-7)
    st = dk.lib().dspark_pack_main_proj(w, out_f, in_f, stride, wdt, g, gdt, eps, act, None,
                                        ctypes.byref(h), ctypes.byref(r))
    return st, r.value, h.value


@pytest.mark.parametrize("kw,reason", [
    (dict(act=dk.FP32, wdt=dk.FP32), 7), (dict(wdt=dk.FP16), 3), (dict(gdt=dk.FP16), 7),
    (dict(out_f=200), 6), (dict(in_f=770, stride=776), 6), (dict(stride=772), 6), (dict(w=24), 6),
])
def test_proj_pack_fallbacks(kw, reason):
    st, r, h = _proj_pack(**kw)
    assert (st, r, h) == (dk.FALLBACK, reason, None)


@pytest.mark.parametrize("kw", [
    dict(w=None), dict(g=None), dict(out_f=0), dict(in_f=-8), dict(stride=760),
    dict(eps=-1.0), dict(eps=float("nan")),
])
def test_proj_pack_invalid(kw):
    assert _proj_pack(**kw)[0] == dk.E_INVALID


def test_proj_calls_reject_null_pack():
    n = ctypes.c_int64(5)
    lib = dk.lib()
    assert lib.dspark_main_proj_workspace_bytes(None, 4, ctypes.byref(n)) == dk.E_INVALID
    assert lib.dspark_main_proj_norm(None, 16, 4, 768, 16, 256, 16, 1 << 20, None) == dk.E_INVALID
    lib.dspark_main_proj_free(None)  # no-op



# ------------------------------------------------------------ draft attention

def _attn(B=2, block=8, nhq=8, nhk=2, D=128, dtype=dk.BF16, max_prefix=100, ws=None, wsb=0,
          **fields):
    base = dict(q_token_stride=1024, q_head_stride=128, ext_token_stride=256,
                ext_head_stride=128, pool_slot_stride=256, pool_head_stride=128, num_slots=64)
    base.update(fields)
    desc = dk.AttnDesc(**base)
    r = ctypes.c_int32(-7)
    st = dk.lib().dspark_draft_attention(ctypes.byref(desc), B, block, nhq, nhk, D, dtype, 0.1,
                                         max_prefix, ws, wsb, None, None, ctypes.byref(r))
    return st, r.value


def test_attn_fallbacks_and_empty():
    assert _attn(D=96) == (dk.FALLBACK, 6)
    assert _attn(dtype=dk.FP32) == (dk.FALLBACK, 7)
    assert _attn(B=0) == (dk.OK, 0)


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(block=0), dict(nhq=6, nhk=4), dict(max_prefix=-1),
    dict(),  # NULL tensors with work to do
])
def test_attn_invalid(kw):
    assert _attn(**kw)[0] == dk.E_INVALID


def test_attn_workspace_size_formula():
    """One fp32 record of 32 x (D + 2) per request, KV head, 32-row tile and
    split (the block's own keys are one more split than the prefix needs)."""
    n = dk.draft_attention_workspace_bytes(2, 8, 8, 2, 128, 0)
    assert n == 2 * 2 * 1 * 1 * 32 * 130 * 4  # no prefix: one split
    m = dk.draft_attention_workspace_bytes(2, 8, 8, 2, 128, 100000)
    assert m % (2 * 2 * 32 * 130 * 4) == 0 and m > n
