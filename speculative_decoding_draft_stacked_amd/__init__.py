"""Python binding of libdspark (the DSpark cross-layer context-KV write on MI355X).

Argument marshalling only: every step of the write runs in the HIP library.
Torch tensors are accepted for convenience; only their device pointers,
strides, dtypes and the current stream are read here. If the library is not
built, every call raises.

Entry points mirror the C ABI in include/dspark.h:
  check_eligibility(layers, hidden, act_dtype)      -> (status, reason)
  pack_ctx_kv(layers, hidden, act_dtype, stream)    -> Pack | None (None = fallback)
  Pack.plan(T, has_commit), Pack.workspace_bytes(T, has_commit)
  ctx_kv_write(pack, ctx_hidden, positions, locs, pools, commit_lens=None,
               locs_row_width=None, workspace=None, range_errors=None,
               validate=False, stream=None)         -> True (enqueued) | False (fallback)
Misuse (wrong index dtypes, shapes, devices or layouts) raises ValueError
before anything reaches the library; DSPARK_E_RANGE from validate mode raises
RangeError.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdspark.so")

OK, FALLBACK, E_INVALID, E_RANGE, E_DEVICE, E_NOMEM, E_TOO_LARGE = 0, 1, -1, -2, -3, -4, -5
BF16, FP16, FP32, QUANTIZED = 0, 1, 2, 99
RANGE_NONE, RANGE_POSITION, RANGE_SLOT, RANGE_DUPLICATE = 0, 1, 2, 3
WRITE_VALIDATE = 1
KERNEL_STREAM, KERNEL_STREAM_KSPLIT, KERNEL_TILED = 0, 1, 2
KERNEL_NAMES = {KERNEL_STREAM: "stream", KERNEL_STREAM_KSPLIT: "stream_ksplit",
                KERNEL_TILED: "tiled"}
MAX_LAYERS = 32
FALLBACK_REASONS = {
    0: "NONE", 1: "NO_LAYERS", 2: "TOO_MANY_LAYERS", 3: "NOT_SLICEABLE", 4: "EPS_MISMATCH",
    5: "MIXED_BIAS", 6: "SHAPE", 7: "DTYPE", 8: "KV_SCALE", 9: "ROPE", 10: "POOL_LAYOUT",
}
EXPORTS = [
    "dspark_check_eligibility", "dspark_pack_ctx_kv", "dspark_ctx_kv_plan",
    "dspark_ctx_kv_workspace_bytes", "dspark_ctx_kv_write", "dspark_ctx_kv_write_static",
    "dspark_pack_info",
    "dspark_pack_buffers", "dspark_pack_free", "dspark_status_str", "dspark_fallback_str",
    "dspark_range_str", "dspark_table_qk_norm_rope",
    "dspark_verify_accept", "dspark_pack_main_proj", "dspark_main_proj_workspace_bytes",
    "dspark_main_proj_norm", "dspark_main_proj_free", "dspark_draft_attention_workspace_bytes",
    "dspark_draft_attention",
]


class LayerDesc(ctypes.Structure):
    """Mirror of dspark_layer_desc."""

    _fields_ = [
        ("qkv_weight", ctypes.c_void_p),
        ("w_rows", ctypes.c_int64),
        ("w_row_stride", ctypes.c_int64),
        ("w_col_stride", ctypes.c_int64),
        ("w_dtype", ctypes.c_int32),
        ("qkv_bias", ctypes.c_void_p),
        ("k_norm_weight", ctypes.c_void_p),
        ("k_norm_dtype", ctypes.c_int32),
        ("k_norm_eps", ctypes.c_double),
        ("q_size", ctypes.c_int64),
        ("kv_size", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("has_kv_scale", ctypes.c_int32),
        ("rope_cos_sin", ctypes.c_void_p),
        ("rope_dtype", ctypes.c_int32),
        ("rope_max_pos", ctypes.c_int64),
        ("rope_dim", ctypes.c_int64),
        ("rope_is_neox", ctypes.c_int32),
    ]


class PoolDesc(ctypes.Structure):
    """Mirror of dspark_pool_desc."""

    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("num_slots", ctypes.c_int64),
        ("k_stride0", ctypes.c_int64),
        ("k_stride1", ctypes.c_int64),
        ("k_stride2", ctypes.c_int64),
        ("v_stride0", ctypes.c_int64),
        ("v_stride1", ctypes.c_int64),
        ("v_stride2", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
    ]


class WritePlan(ctypes.Structure):
    """Mirror of dspark_write_plan."""

    _fields_ = [
        ("kernel", ctypes.c_int32),
        ("token_tile", ctypes.c_int32),
        ("workgroups", ctypes.c_int64),
        ("reduce_workgroups", ctypes.c_int64),
        ("k_parts", ctypes.c_int32),
        ("compacts", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64),
        ("token_splits", ctypes.c_int64),
        ("adaptive", ctypes.c_int64),
    ]


class RangeError(ValueError):
    """DSPARK_E_RANGE from the write's validate mode; ``cause`` is a RANGE_* code."""

    def __init__(self, cause: int, message: str):
        super().__init__(message)
        self.cause = cause


class AttnDesc(ctypes.Structure):
    """Mirror of dspark_attn_desc."""

    _fields_ = [
        ("q", ctypes.c_void_p),
        ("q_token_stride", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64),
        ("k_ext", ctypes.c_void_p),
        ("v_ext", ctypes.c_void_p),
        ("ext_token_stride", ctypes.c_int64),
        ("ext_head_stride", ctypes.c_int64),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("pool_slot_stride", ctypes.c_int64),
        ("pool_head_stride", ctypes.c_int64),
        ("num_slots", ctypes.c_int64),
        ("kv_indptr", ctypes.c_void_p),
        ("kv_indices", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("out_token_stride", ctypes.c_int64),
        ("out_head_stride", ctypes.c_int64),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m speculative_decoding_draft_stacked_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        p_i32, p_i64 = ctypes.POINTER(i32), ctypes.POINTER(i64)
        L.dspark_check_eligibility.argtypes = [ctypes.POINTER(LayerDesc), i32, i64, i32, p_i32]
        L.dspark_pack_ctx_kv.argtypes = [ctypes.POINTER(LayerDesc), i32, i64, i32, vp,
                                         ctypes.POINTER(vp), p_i32]
        L.dspark_ctx_kv_plan.argtypes = [vp, i64, i32, ctypes.POINTER(WritePlan)]
        L.dspark_ctx_kv_workspace_bytes.argtypes = [vp, i64, i32, p_i64]
        L.dspark_ctx_kv_write.argtypes = [vp, vp, i64, i64, vp, vp, vp, i64, i64,
                                          ctypes.POINTER(PoolDesc), i32, vp, i64, vp,
                                          ctypes.c_uint32, vp, p_i32]
        L.dspark_ctx_kv_write_static.argtypes = [vp, vp, i64, i64, vp, vp, vp, i64, i64,
                                                 ctypes.POINTER(PoolDesc), i32, vp,
                                                 ctypes.c_uint32, vp, p_i32]
        L.dspark_pack_info.argtypes = [vp, p_i32, p_i64, p_i64, p_i64, p_i32, p_i32]
        L.dspark_pack_buffers.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                          ctypes.POINTER(vp)]
        L.dspark_table_qk_norm_rope.argtypes = [vp, i64, i64, vp, i32, i32, i32, i32, vp, vp,
                                                i32, ctypes.c_double, vp, i64, vp, vp, p_i32]
        L.dspark_verify_accept.argtypes = [vp, i64, vp, i64, i64, i32, vp, vp, vp]
        L.dspark_pack_main_proj.argtypes = [vp, i64, i64, i64, i32, vp, i32, ctypes.c_double,
                                            i32, vp, ctypes.POINTER(vp), p_i32]
        L.dspark_main_proj_workspace_bytes.argtypes = [vp, i64, p_i64]
        L.dspark_main_proj_norm.argtypes = [vp, vp, i64, i64, vp, i64, vp, i64, vp]
        L.dspark_draft_attention_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i64, p_i64]
        L.dspark_draft_attention.argtypes = [ctypes.POINTER(AttnDesc), i64, i32, i32, i32, i32,
                                             i32, ctypes.c_double, i64, vp, i64, vp, vp, p_i32]
        L.dspark_main_proj_free.argtypes = [vp]
        L.dspark_main_proj_free.restype = None
        L.dspark_pack_free.argtypes = [vp]
        L.dspark_pack_free.restype = None
        L.dspark_status_str.argtypes = [ctypes.c_int]
        L.dspark_status_str.restype = ctypes.c_char_p
        L.dspark_fallback_str.argtypes = [ctypes.c_int]
        L.dspark_fallback_str.restype = ctypes.c_char_p
        L.dspark_range_str.argtypes = [ctypes.c_int]
        L.dspark_range_str.restype = ctypes.c_char_p
        for name in ("dspark_check_eligibility", "dspark_pack_ctx_kv", "dspark_ctx_kv_write",
                     "dspark_ctx_kv_write_static",
                     "dspark_ctx_kv_plan", "dspark_ctx_kv_workspace_bytes",
                     "dspark_pack_info", "dspark_pack_buffers",
                     "dspark_table_qk_norm_rope", "dspark_verify_accept",
                     "dspark_pack_main_proj", "dspark_main_proj_workspace_bytes",
                     "dspark_main_proj_norm", "dspark_draft_attention_workspace_bytes",
                     "dspark_draft_attention"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().dspark_status_str(status).decode()


def fallback_str(reason: int) -> str:
    return lib().dspark_fallback_str(reason).decode()


def range_str(cause: int) -> str:
    return lib().dspark_range_str(cause).decode()


def _raise_for(status: int, what: str):
    if status == E_INVALID:
        raise ValueError(f"{what}: {status_str(status)}")
    if status < 0:
        raise RuntimeError(f"{what}: {status_str(status)} ({status})")


def _layers_array(layers: Sequence[LayerDesc]):
    arr = (LayerDesc * max(len(layers), 1))(*layers)
    return arr


def check_eligibility(layers: Sequence[LayerDesc], hidden: int, act_dtype: int):
    """(status, reason) of dspark_check_eligibility; host-only."""
    reason = ctypes.c_int32(-1)
    st = lib().dspark_check_eligibility(_layers_array(layers), len(layers), hidden, act_dtype,
                                        ctypes.byref(reason))
    return st, reason.value


class Pack:
    """Owner of a dspark_ctx_kv_pack handle. Keeps the tensors the pack
    references (the rotary table) alive while it exists."""

    def __init__(self, handle: int, keep=()):
        self.handle = handle
        self._keep = tuple(keep)

    @property
    def as_parameter(self):
        if not self.handle:
            raise ValueError("pack already freed")
        return ctypes.c_void_p(self.handle)

    def info(self) -> dict:
        L, H, kv, D, dt, b = (ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64(),
                              ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32())
        _raise_for(lib().dspark_pack_info(self.as_parameter, ctypes.byref(L), ctypes.byref(H),
                                          ctypes.byref(kv), ctypes.byref(D), ctypes.byref(dt),
                                          ctypes.byref(b)), "dspark_pack_info")
        return dict(num_layers=L.value, hidden=H.value, kv_size=kv.value, head_dim=D.value,
                    act_dtype=dt.value, has_bias=bool(b.value))

    def buffers(self):
        w, b, k = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        _raise_for(lib().dspark_pack_buffers(self.as_parameter, ctypes.byref(w), ctypes.byref(b),
                                             ctypes.byref(k)), "dspark_pack_buffers")
        return w.value, b.value, k.value

    def plan(self, num_tokens: int, has_commit: bool) -> dict:
        """dspark_ctx_kv_plan: which kernels a write of num_tokens rows runs."""
        p = WritePlan()
        _raise_for(lib().dspark_ctx_kv_plan(self.as_parameter, num_tokens, int(has_commit),
                                            ctypes.byref(p)), "dspark_ctx_kv_plan")
        return dict(kernel=KERNEL_NAMES.get(p.kernel, str(p.kernel)), token_tile=p.token_tile,
                    workgroups=p.workgroups, reduce_workgroups=p.reduce_workgroups,
                    k_parts=p.k_parts, compacts=bool(p.compacts),
                    workspace_bytes=p.workspace_bytes, token_splits=p.token_splits,
                    adaptive=bool(p.adaptive))

    def workspace_bytes(self, num_tokens: int, has_commit: bool) -> int:
        n = ctypes.c_int64(0)
        _raise_for(lib().dspark_ctx_kv_workspace_bytes(self.as_parameter, num_tokens,
                                                       int(has_commit), ctypes.byref(n)),
                   "dspark_ctx_kv_workspace_bytes")
        return n.value

    def free(self):
        if self.handle:
            lib().dspark_pack_free(ctypes.c_void_p(self.handle))
            self.handle = 0
        self._keep = ()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def _stream(stream) -> Optional[int]:
    """A hipStream_t as an integer: torch streams, raw integers or None (current torch stream)."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def pack_ctx_kv(layers: Sequence[LayerDesc], hidden: int, act_dtype: int, stream=None):
    """Pack the stacked parameters. Returns a Pack, or None when the layers are
    not eligible (the caller then runs its per-layer path); `last_fallback_reason`
    holds the reason."""
    global last_fallback_reason
    h = ctypes.c_void_p()
    reason = ctypes.c_int32(0)
    st = lib().dspark_pack_ctx_kv(_layers_array(layers), len(layers), hidden, act_dtype,
                                  _stream(stream), ctypes.byref(h), ctypes.byref(reason))
    last_fallback_reason = reason.value
    if st == FALLBACK:
        return None
    _raise_for(st, "dspark_pack_ctx_kv")
    # the pack references layer 0's rotary table: keep its tensor alive
    return Pack(h.value, keep=getattr(layers[0], "_tensors", ()) if len(layers) else ())


last_fallback_reason = 0


def ctx_kv_write_raw(pack: Pack, ctx_hidden: int, num_tokens: int, hidden_row_stride: int,
                     positions: int, locs: int, commit_lens: Optional[int], locs_row_width: int,
                     num_requests: int, pools: Sequence[PoolDesc], stream,
                     workspace: Optional[int] = None, workspace_bytes: int = 0,
                     range_errors: Optional[int] = None, flags: int = 0) -> tuple:
    """dspark_ctx_kv_write on raw device pointers; returns (status, detail)."""
    arr = (PoolDesc * max(len(pools), 1))(*pools)
    detail = ctypes.c_int32(0)
    st = lib().dspark_ctx_kv_write(pack.as_parameter, ctx_hidden, num_tokens, hidden_row_stride,
                                   positions, locs, commit_lens, locs_row_width, num_requests,
                                   arr, len(pools), workspace, workspace_bytes, range_errors,
                                   flags, _stream(stream), ctypes.byref(detail))
    return st, detail.value


# ------------------------------------------------------------------ torch plumbing

def _dtype_code(t) -> int:
    import torch
    return {torch.bfloat16: BF16, torch.float16: FP16, torch.float32: FP32}.get(t.dtype, QUANTIZED)


def layer_desc(qkv_weight, k_norm_weight, eps: float, q_size: int, kv_size: int, head_dim: int,
               cos_sin_cache, qkv_bias=None, has_kv_scale: bool = False,
               is_neox: bool = True, rotary_dim: Optional[int] = None) -> LayerDesc:
    """Descriptor of one layer from its tensors (pointers and strides only).
    The descriptor holds a reference to the rotary table, which a pack built
    from it keeps alive."""
    if cos_sin_cache.dim() != 2:
        raise ValueError("cos_sin_cache must be [max_position, rotary_dim]")
    d = LayerDesc(
        qkv_weight=qkv_weight.data_ptr(), w_rows=qkv_weight.shape[0],
        w_row_stride=qkv_weight.stride(0), w_col_stride=qkv_weight.stride(1),
        w_dtype=_dtype_code(qkv_weight),
        qkv_bias=None if qkv_bias is None else qkv_bias.data_ptr(),
        k_norm_weight=k_norm_weight.data_ptr(), k_norm_dtype=_dtype_code(k_norm_weight),
        k_norm_eps=eps, q_size=q_size, kv_size=kv_size, head_dim=head_dim,
        has_kv_scale=int(has_kv_scale), rope_cos_sin=cos_sin_cache.data_ptr(),
        rope_dtype=_dtype_code(cos_sin_cache), rope_max_pos=cos_sin_cache.shape[0],
        rope_dim=cos_sin_cache.shape[1] if rotary_dim is None else rotary_dim,
        rope_is_neox=int(is_neox),
    )
    d._tensors = (cos_sin_cache,)
    return d


def pool_desc(k_buf, v_buf) -> PoolDesc:
    """Descriptor of one layer's pool from its [slots, NH, D] K and V buffers."""
    return PoolDesc(k=k_buf.data_ptr(), v=v_buf.data_ptr(), num_slots=k_buf.shape[0],
                    k_stride0=k_buf.stride(0), k_stride1=k_buf.stride(1),
                    k_stride2=k_buf.stride(2), v_stride0=v_buf.stride(0),
                    v_stride1=v_buf.stride(1), v_stride2=v_buf.stride(2),
                    dtype=_dtype_code(k_buf) if _dtype_code(k_buf) == _dtype_code(v_buf)
                    else QUANTIZED)


_ACT_TORCH = {BF16: "bfloat16", FP16: "float16"}


def _check_index(name: str, t, n: int, device) -> None:
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int64:
        raise ValueError(f"{name} must be an int64 tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.numel() != n or (n and not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous tensor of {n} elements")


def ctx_kv_write(pack: Pack, ctx_hidden, positions, locs, pools: Sequence[PoolDesc],
                 commit_lens=None, locs_row_width: Optional[int] = None, workspace=None,
                 range_errors=None, validate: bool = False, stream=None) -> bool:
    """Enqueue the write. True when enqueued, False on fallback (nothing
    written). ValueError on misuse: commit_lens without locs_row_width, index
    tensors that are not contiguous int64 of the right length, ctx_hidden of
    another dtype than the pack's or without unit column stride, tensors on
    another device. ``workspace`` is a uint8 device tensor of at least
    pack.workspace_bytes(T, commit) bytes (allocated here when None and
    needed); ``range_errors`` an int64 device tensor of one element that counts
    rows skipped for an out-of-range position or slot. With validate=True the
    index arrays are checked first (the stream is synchronised) and a bad row
    raises RangeError."""
    import torch
    if (commit_lens is None) != (locs_row_width is None):
        raise ValueError("commit_lens and locs_row_width must be passed together")
    info = pack.info()
    if ctx_hidden.dim() != 2 or ctx_hidden.stride(1) != 1:
        raise ValueError("ctx_hidden must be [T, hidden] with unit column stride")
    if str(ctx_hidden.dtype).replace("torch.", "") != _ACT_TORCH.get(info["act_dtype"]):
        raise ValueError(f"ctx_hidden is {ctx_hidden.dtype}, the pack's activation dtype is "
                         f"{_ACT_TORCH.get(info['act_dtype'])}")
    if ctx_hidden.shape[1] != info["hidden"]:
        raise ValueError(f"ctx_hidden has {ctx_hidden.shape[1]} columns, the pack {info['hidden']}")
    dev = ctx_hidden.device
    T = ctx_hidden.shape[0]
    _check_index("positions", positions, T, dev)
    _check_index("locs", locs, T, dev)
    W, B = 0, 0
    if commit_lens is not None:
        W = int(locs_row_width)
        if W <= 0 or T % W:
            raise ValueError("locs_row_width must be positive and divide the row count")
        B = T // W
        _check_index("commit_lens", commit_lens, B, dev)
    if range_errors is not None:
        _check_index("range_errors", range_errors, 1, dev)
    need = pack.workspace_bytes(T, commit_lens is not None)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None and workspace.device != dev:
        raise ValueError(f"workspace is on {workspace.device}, expected {dev}")
    st, detail = ctx_kv_write_raw(
        pack, ctx_hidden.data_ptr(), T, ctx_hidden.stride(0), positions.data_ptr(),
        locs.data_ptr(), None if commit_lens is None else commit_lens.data_ptr(), W, B, pools,
        stream, None if workspace is None else workspace.data_ptr(),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        None if range_errors is None else range_errors.data_ptr(),
        WRITE_VALIDATE if validate else 0)
    if st == FALLBACK:
        return False
    if st == E_RANGE:
        raise RangeError(detail, f"dspark_ctx_kv_write: {range_str(detail)}")
    _raise_for(st, "dspark_ctx_kv_write")
    return True


def ctx_kv_write_static(pack: Pack, ctx_hidden, positions, locs, pools: Sequence[PoolDesc],
                        commit_lens=None, locs_row_width: Optional[int] = None,
                        range_errors=None, stream=None) -> bool:
    """dspark_ctx_kv_write_static: the write with the library's static scratch
    instead of a caller workspace (allocates nothing). Same checks and
    results as ctx_kv_write; calls that overlap on one device race."""
    if (commit_lens is None) != (locs_row_width is None):
        raise ValueError("commit_lens and locs_row_width must be passed together")
    info = pack.info()
    if ctx_hidden.dim() != 2 or ctx_hidden.stride(1) != 1:
        raise ValueError("ctx_hidden must be [T, hidden] with unit column stride")
    if str(ctx_hidden.dtype).replace("torch.", "") != _ACT_TORCH.get(info["act_dtype"]):
        raise ValueError("ctx_hidden is not in the pack's activation dtype")
    if ctx_hidden.shape[1] != info["hidden"]:
        raise ValueError(f"ctx_hidden has {ctx_hidden.shape[1]} columns, the pack {info['hidden']}")
    dev = ctx_hidden.device
    T = ctx_hidden.shape[0]
    _check_index("positions", positions, T, dev)
    _check_index("locs", locs, T, dev)
    W, B = 0, 0
    if commit_lens is not None:
        W = int(locs_row_width)
        if W <= 0 or T % W:
            raise ValueError("locs_row_width must be positive and divide the row count")
        B = T // W
        _check_index("commit_lens", commit_lens, B, dev)
    if range_errors is not None:
        _check_index("range_errors", range_errors, 1, dev)
    arr = (PoolDesc * max(len(pools), 1))(*pools)
    detail = ctypes.c_int32(0)
    st = lib().dspark_ctx_kv_write_static(
        pack.as_parameter, ctx_hidden.data_ptr(), T, ctx_hidden.stride(0), positions.data_ptr(),
        locs.data_ptr(), None if commit_lens is None else commit_lens.data_ptr(), W, B, arr,
        len(pools), None if range_errors is None else range_errors.data_ptr(), 0,
        _stream(stream), ctypes.byref(detail))
    if st == FALLBACK:
        return False
    _raise_for(st, "dspark_ctx_kv_write_static")
    return True


def table_qk_norm_rope_raw(qkv: int, num_tokens: int, row_stride: int, positions: int,
                           num_q_heads: int, num_k_heads: int, head_dim: int, act_dtype: int,
                           q_norm_weight: int, k_norm_weight: int, norm_weight_dtype: int,
                           eps: float, cos_sin: int, rope_max_pos: int,
                           range_errors: Optional[int], stream) -> tuple:
    """dspark_table_qk_norm_rope on raw device pointers; returns (status, reason)."""
    reason = ctypes.c_int32(0)
    st = lib().dspark_table_qk_norm_rope(qkv, num_tokens, row_stride, positions, num_q_heads,
                                         num_k_heads, head_dim, act_dtype, q_norm_weight,
                                         k_norm_weight, norm_weight_dtype, eps, cos_sin,
                                         rope_max_pos, range_errors, _stream(stream),
                                         ctypes.byref(reason))
    return st, reason.value


def table_qk_norm_rope(qkv, positions, q_norm_weight, k_norm_weight, cos_sin_cache,
                       num_q_heads: int, num_k_heads: int, head_dim: int, eps: float,
                       range_errors=None, stream=None) -> bool:
    """Enqueue the in-place QK norm + rotation on ``qkv`` [T, row_stride]. True
    when enqueued, False on fallback (nothing changed); ValueError on misuse.
    ``range_errors`` is an optional int64 device tensor of one element that
    counts tokens skipped for a position outside the table. ValueError also for
    positions that are not a contiguous int64 tensor of T entries, a table that
    is not a contiguous fp32 [P, head_dim] tensor, norm weights of fewer than
    head_dim contiguous entries, or tensors on another device."""
    import torch
    if qkv.dim() != 2 or qkv.stride(1) != 1:
        raise ValueError("qkv must be [T, row_stride] with unit column stride")
    dev = qkv.device
    _check_index("positions", positions, qkv.shape[0], dev)
    if range_errors is not None:
        _check_index("range_errors", range_errors, 1, dev)
    if (cos_sin_cache.dtype != torch.float32 or cos_sin_cache.dim() != 2
            or cos_sin_cache.shape[1] != head_dim or not cos_sin_cache.is_contiguous()
            or cos_sin_cache.device != dev):
        raise ValueError("cos_sin_cache must be a contiguous fp32 [max_position, head_dim] "
                         "tensor on qkv's device")
    for name, w in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        if w.numel() < head_dim or not w.is_contiguous() or w.device != dev:
            raise ValueError(f"{name} must be a contiguous tensor of head_dim entries on "
                             "qkv's device")
    st, reason = table_qk_norm_rope_raw(
        qkv.data_ptr(), qkv.shape[0], qkv.stride(0), positions.data_ptr(), num_q_heads,
        num_k_heads, head_dim, _dtype_code(qkv), q_norm_weight.data_ptr(),
        k_norm_weight.data_ptr(),
        _dtype_code(q_norm_weight) if _dtype_code(q_norm_weight) == _dtype_code(k_norm_weight)
        else QUANTIZED, eps, cos_sin_cache.data_ptr(), cos_sin_cache.shape[0],
        None if range_errors is None else range_errors.data_ptr(), stream)
    if st == FALLBACK:
        return False
    _raise_for(st, "dspark_table_qk_norm_rope")
    return True


def verify_accept_raw(draft: Optional[int], draft_row_stride: int, target: int,
                      target_row_stride: int, num_requests: int, num_drafts: int, accept: int,
                      bonus: int, stream) -> int:
    """dspark_verify_accept on raw device pointers; returns the status."""
    return lib().dspark_verify_accept(draft, draft_row_stride, target, target_row_stride,
                                      num_requests, num_drafts, accept, bonus, _stream(stream))


def verify_accept(draft, target, accept, bonus, stream=None) -> None:
    """Enqueue accept lengths and bonus tokens: ``draft`` int64 [B, K],
    ``target`` int64 [B, K + 1] (unit column stride), ``accept`` and ``bonus``
    int64 [B] outputs. ValueError on misuse."""
    import torch
    for name, t in (("draft", draft), ("target", target), ("accept", accept), ("bonus", bonus)):
        if t.dtype != torch.int64:
            raise ValueError(f"{name} must be int64")
    if draft.dim() != 2 or target.dim() != 2 or (draft.numel() and draft.stride(1) != 1) or \
            target.stride(1) != 1:
        raise ValueError("draft and target must be [B, K] / [B, K + 1] with unit column stride")
    B, K = draft.shape
    if target.shape[0] != B or target.shape[1] != K + 1 or accept.numel() < B or bonus.numel() < B:
        raise ValueError("shape mismatch")
    st = verify_accept_raw(draft.data_ptr() if K else None, draft.stride(0) if K else 0,
                           target.data_ptr(), target.stride(0), B, K, accept.data_ptr(),
                           bonus.data_ptr(), stream)
    _raise_for(st, "dspark_verify_accept")


class ProjPack:
    """A packed context producer (owns device buffers until free())."""

    def __init__(self, handle: int, out_features: int, in_features: int):
        self.handle = handle
        self.out_features = out_features
        self.in_features = in_features

    @property
    def as_parameter(self):
        return ctypes.c_void_p(self.handle)

    def workspace_bytes(self, num_tokens: int) -> int:
        n = ctypes.c_int64(0)
        _raise_for(lib().dspark_main_proj_workspace_bytes(self.as_parameter, num_tokens,
                                                          ctypes.byref(n)),
                   "dspark_main_proj_workspace_bytes")
        return n.value

    def free(self):
        if self.handle:
            lib().dspark_main_proj_free(self.as_parameter)
            self.handle = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def pack_main_proj(weight, norm_weight, eps: float, stream=None):
    """Pack main_proj ([out, in] weight, unit column stride) and main_norm's
    weight. Returns a ProjPack, or None on fallback (reason in
    ``last_fallback_reason``)."""
    global last_fallback_reason
    if weight.dim() != 2 or weight.stride(1) != 1:
        raise ValueError("weight must be [out_features, in_features] with unit column stride")
    h = ctypes.c_void_p(0)
    reason = ctypes.c_int32(0)
    st = lib().dspark_pack_main_proj(weight.data_ptr(), weight.shape[0], weight.shape[1],
                                     weight.stride(0), _dtype_code(weight),
                                     norm_weight.data_ptr(), _dtype_code(norm_weight), eps,
                                     _dtype_code(weight), _stream(stream), ctypes.byref(h),
                                     ctypes.byref(reason))
    last_fallback_reason = reason.value
    if st == FALLBACK:
        return None
    _raise_for(st, "dspark_pack_main_proj")
    return ProjPack(h.value, weight.shape[0], weight.shape[1])


def main_proj_norm(pack: ProjPack, aux_hidden, ctx_hidden, workspace, stream=None) -> None:
    """Enqueue ctx_hidden = main_norm(main_proj(aux_hidden)); ``workspace`` is a
    device tensor of at least pack.workspace_bytes(T) bytes."""
    if aux_hidden.stride(1) != 1 or ctx_hidden.stride(1) != 1:
        raise ValueError("aux_hidden and ctx_hidden need unit column stride")
    T = aux_hidden.shape[0]
    if ctx_hidden.shape[0] != T:
        raise ValueError("token counts differ")
    st = lib().dspark_main_proj_norm(pack.as_parameter, aux_hidden.data_ptr(), T,
                                     aux_hidden.stride(0), ctx_hidden.data_ptr(),
                                     ctx_hidden.stride(0), workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(stream))
    _raise_for(st, "dspark_main_proj_norm")


def draft_attention_workspace_bytes(num_requests: int, block: int, num_q_heads: int,
                                    num_kv_heads: int, head_dim: int, max_prefix: int) -> int:
    n = ctypes.c_int64(0)
    _raise_for(lib().dspark_draft_attention_workspace_bytes(num_requests, block, num_q_heads,
                                                            num_kv_heads, head_dim, max_prefix,
                                                            ctypes.byref(n)),
               "dspark_draft_attention_workspace_bytes")
    return n.value


def draft_attention(q, k_ext, v_ext, k_pool, v_pool, kv_indptr, kv_indices, out, block: int,
                    sm_scale: float, max_prefix: int, workspace, range_errors=None,
                    stream=None) -> bool:
    """Enqueue the draft attention: q / out [B*block, NHQ, D], k_ext / v_ext
    [B*block, NHK, D], pools [slots, NHK, D] (unit head-dim stride, same layout
    for K and V), int64 kv_indptr [B+1] and kv_indices. True when enqueued,
    False on fallback; ValueError on misuse."""
    for t in (q, k_ext, v_ext, k_pool, v_pool, out):
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError("attention tensors are [rows, heads, head_dim], unit last stride")
    if k_ext.stride() != v_ext.stride() or k_pool.stride() != v_pool.stride():
        raise ValueError("K and V must share a layout")
    B = kv_indptr.numel() - 1
    desc = AttnDesc(q=q.data_ptr(), q_token_stride=q.stride(0), q_head_stride=q.stride(1),
                    k_ext=k_ext.data_ptr(), v_ext=v_ext.data_ptr(),
                    ext_token_stride=k_ext.stride(0), ext_head_stride=k_ext.stride(1),
                    k_pool=k_pool.data_ptr(), v_pool=v_pool.data_ptr(),
                    pool_slot_stride=k_pool.stride(0), pool_head_stride=k_pool.stride(1),
                    num_slots=k_pool.shape[0], kv_indptr=kv_indptr.data_ptr(),
                    kv_indices=kv_indices.data_ptr(), out=out.data_ptr(),
                    out_token_stride=out.stride(0), out_head_stride=out.stride(1))
    reason = ctypes.c_int32(0)
    st = lib().dspark_draft_attention(ctypes.byref(desc), B, block, q.shape[1], k_ext.shape[1],
                                      q.shape[2], _dtype_code(q), sm_scale, max_prefix,
                                      workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(),
                                      None if range_errors is None else range_errors.data_ptr(),
                                      _stream(stream), ctypes.byref(reason))
    if st == FALLBACK:
        return False
    _raise_for(st, "dspark_draft_attention")
    return True
