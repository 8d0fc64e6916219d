"""Device plumbing for synthetic cases: puts a workloads.Case on cuda:0 as
torch tensors, builds the C-ABI descriptors, packs and runs the write.

Torch only allocates memory and supplies the stream here; the write itself is
the HIP library's."""

from __future__ import annotations

import numpy as np
import torch

import speculative_decoding_draft_stacked_amd as dk

TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
ACT = {"bf16": dk.BF16, "fp16": dk.FP16}


def _f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit patterns -> float32 values (exact widening)."""
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    return bits.view(np.float16).astype(np.float32)


def _dev16(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda").view(TORCH_DT[dtype])


class DeviceCase:
    """A Case's tensors on cuda:0 plus sentinel-filled pools."""

    def __init__(self, case, k_norm_fp32: bool = False, pool_row_pad: int = 0):
        self.case = case
        dt = case.dtype
        self.x = _dev16(case.x, dt)
        self.qkv_w = [_dev16(w, dt) for w in case.qkv_w]
        self.qkv_b = None if case.qkv_b is None else [_dev16(b, dt) for b in case.qkv_b]
        if k_norm_fp32:
            self.k_norm = [torch.from_numpy(_f32(g, dt)).cuda()
                           for g in case.k_norm_w]
        else:
            self.k_norm = [_dev16(g, dt) for g in case.k_norm_w]
        self.table = torch.from_numpy(case.table).cuda()
        self.positions = torch.from_numpy(case.positions).cuda()
        self.locs = torch.from_numpy(case.locs).cuda()
        self.commit = None if case.commit_lens is None else torch.from_numpy(case.commit_lens).cuda()
        self.pool_row_pad = pool_row_pad
        self.err = torch.zeros(1, dtype=torch.int64, device="cuda")  # range-error counter
        self.reset_pools()

    def reset_pools(self):
        c = self.case
        shape = (c.slots, c.NH, c.D)

        def pool():
            if self.pool_row_pad:
                big = torch.full((c.slots, c.NH * c.D + self.pool_row_pad), -1, dtype=torch.int16,
                                 device="cuda")
                return big[:, : c.NH * c.D].view(TORCH_DT[c.dtype]).view(shape)
            return torch.full(shape, -1, dtype=torch.int16, device="cuda").view(TORCH_DT[c.dtype])

        self.pk = [pool() for _ in range(c.L)]
        self.pv = [pool() for _ in range(c.L)]

    def layer_descs(self):
        c = self.case
        return [dk.layer_desc(self.qkv_w[l], self.k_norm[l], c.eps, c.q_size, c.kv, c.D,
                              self.table, qkv_bias=None if self.qkv_b is None else self.qkv_b[l])
                for l in range(c.L)]

    def pool_descs(self):
        return [dk.pool_desc(self.pk[l], self.pv[l]) for l in range(self.case.L)]

    def pack(self):
        p = dk.pack_ctx_kv(self.layer_descs(), self.case.H, ACT[self.case.dtype])
        assert p is not None, dk.fallback_str(dk.last_fallback_reason)
        return p

    def workspace(self, pack):
        """A device workspace of the size the write needs (None when it needs none)."""
        n = pack.workspace_bytes(self.case.T, self.commit is not None)
        return torch.empty(n, dtype=torch.uint8, device="cuda") if n else None

    def write(self, pack, workspace=None, validate: bool = False) -> bool:
        c = self.case
        return dk.ctx_kv_write(pack, self.x, self.positions, self.locs, self.pool_descs(),
                               commit_lens=self.commit,
                               locs_row_width=c.row_width if self.commit is not None else None,
                               workspace=workspace if workspace is not None
                               else self.workspace(pack),
                               range_errors=self.err, validate=validate)

    def range_errors(self) -> int:
        """Reads and clears the count of rows skipped for an out-of-range
        position or slot (per row and layer)."""
        torch.cuda.synchronize()
        n = int(self.err.item())
        self.err.zero_()
        return n

    def pools_host(self):
        torch.cuda.synchronize()
        k = [p.contiguous().view(torch.int16).cpu().numpy().view(np.uint16) for p in self.pk]
        v = [p.contiguous().view(torch.int16).cpu().numpy().view(np.uint16) for p in self.pv]
        return k, v

    def touched_slots(self, layer: int, which: str) -> np.ndarray:
        """Slots whose row holds any word other than the sentinel (computed on the device)."""
        p = (self.pk if which == "k" else self.pv)[layer]
        hit = (p.view(torch.int16) != -1).flatten(1).any(dim=1)
        return torch.nonzero(hit).flatten().cpu().numpy()

    def rows_at(self, layer: int, which: str, slots: np.ndarray) -> np.ndarray:
        p = (self.pk if which == "k" else self.pv)[layer]
        idx = torch.from_numpy(np.asarray(slots, dtype=np.int64)).cuda()
        return p.view(torch.int16)[idx].cpu().numpy().view(np.uint16)


