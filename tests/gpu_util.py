"""Helpers for the GPU tests: move a synthetic case to the device, run the HIP
write through the C ABI, and compare the pools with the CPU oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import speculative_decoding_draft_stacked_amd as dk
from oracle import ctx_kv_oracle as O

from speculative_decoding_draft_stacked_amd.harness import DeviceCase  # noqa: F401

TOL = {"bf16": (2e-2, 2e-2), "fp16": (5e-3, 5e-3)}  # (rtol, atol), sglang PR #31986 parity test


_hip = None


def device_to_host(ptr: int, nbytes: int) -> np.ndarray:
    """Synchronous copy of a raw device byte range into a host array (hipMemcpy)."""
    global _hip
    import ctypes
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    out = np.empty(nbytes, dtype=np.uint8)
    torch.cuda.synchronize()
    assert _hip.hipMemcpy(out.ctypes.data, ptr, nbytes, 2) == 0  # hipMemcpyDeviceToHost
    return out


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def expected_slots(case) -> np.ndarray:
    valid = O.valid_rows(case.locs, case.commit_lens, case.row_width)
    return np.sort(case.locs[valid])


def check_slot_sets(dc: DeviceCase):
    """The written (layer, slot) set equals {(l, locs[t]) : valid(t)} exactly."""
    want = expected_slots(dc.case)
    for l in range(dc.case.L):
        for which in ("k", "v"):
            got = np.sort(dc.touched_slots(l, which))
            assert np.array_equal(got, want), (l, which, len(got), len(want))


def compare_rows(dc: DeviceCase, rows=None, label="") -> dict:
    """Elementwise |gpu - oracle| <= atol + rtol*|oracle| on the given rows (all
    valid rows by default); returns bit-exact diagnostics."""
    c = dc.case
    valid = O.valid_rows(c.locs, c.commit_lens, c.row_width)
    if rows is None:
        rows = np.nonzero(valid)[0]
    rows = np.asarray([t for t in rows if valid[t]], dtype=np.int64)
    if len(rows) == 0:
        return {"rows": 0}
    ok_k, ok_v = O.rows_kv(c, rows)
    rtol, atol = TOL[c.dtype]
    stats = {"rows": len(rows), "exact": 0, "total": 0, "max_abs": 0.0}
    for l in range(c.L):
        for which, want in (("k", ok_k[l]), ("v", ok_v[l])):
            got = dc.rows_at(l, which, c.locs[rows])
            g = O.decode(got, c.dtype)
            w = O.decode(want, c.dtype)
            assert np.all(np.isfinite(g)), (label, l, which, "non-finite / unwritten")
            err = np.abs(g - w)
            bad = err > atol + rtol * np.abs(w)
            if bad.any():
                i = np.argwhere(bad)[0]
                raise AssertionError(
                    f"{label} layer {l} {which}: {int(bad.sum())} elements out of tolerance; "
                    f"first at row {rows[i[0]]} head {i[1]} d {i[2]}: gpu {g[tuple(i)]} "
                    f"oracle {w[tuple(i)]}")
            stats["exact"] += int(np.sum(got == want))
            stats["total"] += got.size
            stats["max_abs"] = max(stats["max_abs"], float(err.max()))
    stats["exact_frac"] = stats["exact"] / stats["total"]
    return stats
