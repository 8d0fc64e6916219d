"""One draft step's operations chained on the device through the C ABI, each
reading what the previous one left in device memory, against the oracles
chained on the CPU from the same seeded inputs (no oracle input comes from
the device):

    aux hidden --producer--> ctx_hidden --stacked write--> per-layer K/V pools
    draft QKV --in-place QK norm + rotation--> queries, the block's own K/V
    queries + own K/V + one layer's pool (the requests' slots) --draft attention--> out

This checks the data contract between the operations (the producer's row
layout is the write's input, the write's pool layout and slots are what the
attention gathers, the QK op's in-place rows are the attention's strided
query and key/value views) besides each one's arithmetic.

Tolerance: each stage, and the end of the chain, within |gpu - oracle| <=
atol + rtol*|oracle| with the write's (rtol, atol). Beyond each operation's
own rounding differences, the chains differ where an earlier stage rounded an
element to the neighbouring dtype number: a ctx ulp moves a K/V element by
far less than its own ulp through the write's small weights (std 0.02), and a
K ulp moves a score by about |q_i| times that ulp, far below the score gaps
that decide the outputs. sm_scale is set large in two cases so that each
output follows its few best keys (a wrong slot, head or layer then moves it
by O(1), where an average over thousands of keys would hide it).
"""

import dataclasses

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

from gpu_util import TOL, say

pytestmark = pytest.mark.gpu
_T = {"bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "no GPU visible"
    dk.lib()


def _dev16(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(_T[dtype]).cuda()


def _host16(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_chain(s):
    """The CPU oracles chained: (ctx values, K pools, V pools, QKV patterns
    after the QK op, attention values, skipped slots)."""
    p, dt = s.proj, s.dtype
    ctx = M.combine_hidden_states(p.aux, p.w, p.g, p.g_dtype, p.eps, dt)
    write = dataclasses.replace(s.write, x=O.encode(ctx, dt))
    pk, pv = W.sentinel_pools(write)
    O.ctx_kv_write(write, pk, pv)
    q = s.qk
    qkv = q.qkv.copy()
    Q.qk_norm_rope_inplace(qkv, q.positions, q.q_w, q.k_w, q.weight_dtype, q.table, q.NHQ, q.NHK,
                           q.D, q.eps, dt)
    nq, nk = q.NHQ * q.D, q.NHK * q.D
    rows = qkv.shape[0]
    out, skipped = A.draft_attention(
        qkv[:, :nq].reshape(rows, q.NHQ, q.D), qkv[:, nq:nq + nk].reshape(rows, q.NHK, q.D),
        qkv[:, nq + nk:nq + 2 * nk].reshape(rows, q.NHK, q.D), pk[s.layer], pv[s.layer],
        s.kv_indptr, s.kv_indices, s.block, q.NHQ, q.NHK, s.sm_scale, dt)
    return ctx, pk, pv, qkv, out, skipped


class DeviceStep:
    """The step's device buffers; run() enqueues the four operations on the
    current stream, in order, with no host synchronisation between them."""

    def __init__(self, s):
        self.s = s
        p, q, dt = s.proj, s.qk, s.dtype
        self.aux = _dev16(p.aux, dt)
        self.w = _dev16(p.w, dt)
        self.g = torch.from_numpy(p.g).cuda() if p.g_dtype == "fp32" else _dev16(p.g, dt)
        self.proj = dk.pack_main_proj(self.w, self.g, p.eps)
        assert self.proj is not None
        self.proj_ws = torch.empty(max(self.proj.workspace_bytes(p.T), 16), dtype=torch.uint8,
                                   device="cuda")
        self.ctx = torch.empty((p.T, p.H), dtype=_T[dt], device="cuda")
        self.dc = DeviceCase(s.write)
        self.dc.x = self.ctx  # the write reads the producer's output in place
        self.pack = self.dc.pack()
        self.write_ws = self.dc.workspace(self.pack)
        self.qkv0 = _dev16(q.qkv, dt)  # pristine draft rows
        self.qkv = self.qkv0.clone()
        self.pos = torch.from_numpy(q.positions).cuda()
        self.q_w, self.k_w = _dev16(q.q_w, dt), _dev16(q.k_w, dt)
        nq, nk = q.NHQ * q.D, q.NHK * q.D
        self.q = self.qkv[:, :nq].unflatten(1, (q.NHQ, q.D))
        self.k_ext = self.qkv[:, nq:nq + nk].unflatten(1, (q.NHK, q.D))
        self.v_ext = self.qkv[:, nq + nk:nq + 2 * nk].unflatten(1, (q.NHK, q.D))
        self.indptr = torch.from_numpy(s.kv_indptr).cuda()
        self.indices = torch.from_numpy(s.kv_indices).cuda()
        self.max_prefix = int(np.max(s.prefix))
        n = dk.draft_attention_workspace_bytes(s.B, s.block, q.NHQ, q.NHK, q.D, self.max_prefix)
        self.attn_ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
        self.attn_err = torch.zeros(1, dtype=torch.int64, device="cuda")
        self.qk_err = torch.zeros(1, dtype=torch.int64, device="cuda")
        self.out = torch.empty((s.B * s.block, q.NHQ, q.D), dtype=_T[dt], device="cuda")

    def reset(self):
        """Inputs back to their drawn state, outputs to junk, in place (a
        captured graph keeps these buffers' addresses); eager work."""
        self.ctx.view(torch.int16).fill_(-7)
        for p in self.dc.pk + self.dc.pv:
            p.view(torch.int16).fill_(-1)
        self.qkv.copy_(self.qkv0)
        self.out.view(torch.int16).fill_(-7)
        self.attn_err.zero_()
        self.qk_err.zero_()
        self.dc.err.zero_()

    def run(self):
        s, q = self.s, self.s.qk
        dk.main_proj_norm(self.proj, self.aux, self.ctx, self.proj_ws)
        assert self.dc.write(self.pack, workspace=self.write_ws)
        assert dk.table_qk_norm_rope(self.qkv, self.pos, self.q_w, self.k_w, self.dc.table,
                                     q.NHQ, q.NHK, q.D, q.eps, range_errors=self.qk_err)
        assert dk.draft_attention(self.q, self.k_ext, self.v_ext, self.dc.pk[s.layer],
                                  self.dc.pv[s.layer], self.indptr, self.indices, self.out,
                                  s.block, s.sm_scale, self.max_prefix, self.attn_ws,
                                  self.attn_err)

    def results(self):
        ks, vs = self.dc.pools_host()
        return (_host16(self.ctx), ks, vs, _host16(self.qkv), _host16(self.out),
                int(self.attn_err.item()), int(self.qk_err.item()), int(self.dc.err.item()))


def _within(label, got_bits, want, dt):
    g = O.decode(got_bits, dt)
    assert np.all(np.isfinite(g)), f"{label}: non-finite output"
    rtol, atol = TOL[dt]
    err = np.abs(g - want)
    bad = err > atol + rtol * np.abs(want)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{label}: {int(bad.sum())} out of tolerance; first at {i}: "
                             f"gpu {g[i]} oracle {want[i]}")
    exact = float(np.mean(O.encode(want, dt) == got_bits))
    say(f"  {label}: ok, exact_frac {exact:.4f}, max_abs {float(err.max()):.3g}")


def _check(s, dev, ref):
    ctx_o, pk_o, pv_o, qkv_o, out_o, skipped_o = ref
    ctx, ks, vs, qkv, out, attn_err, qk_err, write_err = dev
    dt, q = s.dtype, s.qk
    assert skipped_o == 0 and attn_err == 0 and qk_err == 0 and write_err == 0
    _within("ctx_hidden", ctx, ctx_o, dt)
    for l in range(s.write.L):
        for name, got, want in (("K", ks[l], pk_o[l]), ("V", vs[l], pv_o[l])):
            written = np.any(want != W.SENTINEL, axis=(1, 2))
            assert np.array_equal(np.any(got != W.SENTINEL, axis=(1, 2)), written), \
                f"layer {l} {name}: written slot set differs"
            assert np.array_equal(np.sort(np.nonzero(written)[0]), np.sort(s.write.locs))
            _within(f"layer {l} {name} pool", got[written], O.decode(want[written], dt), dt)
    nh = (q.NHQ + q.NHK) * q.D
    _within("QK-normed query/key heads", qkv[:, :nh], O.decode(qkv_o[:, :nh], dt), dt)
    assert np.array_equal(qkv[:, nh:], qkv_o[:, nh:]), "value heads changed"
    _within("attention", out, out_o, dt)


CASES = {
    # four requests (prefixes of 37, 64, 1 and 100 tokens), blocks of 8, G = 4:
    # streaming write and producer kernels; sm_scale 1 makes each output
    # follow its few best keys, so a wrong slot, head or layer shows
    "bf16_d128": dict(B=4, block=8, prefix=[37, 64, 1, 100], H=512, NH=2, NHQ=8, D=128,
                      sm_scale=1.0),
    # head_dim 64, fp16, one layer's pool of three, longer prefixes
    "fp16_d64": dict(B=3, block=4, prefix=[300, 129, 33], H=768, L=3, NH=4, NHQ=16, D=64,
                     dtype="fp16", sm_scale=0.5),
    # a prefill-sized producer and write (tiled kernels) under a short draft
    "tiled_prefill": dict(B=2, block=8, prefix=[2500, 2100], H=1024, NH=2, NHQ=4, D=128,
                          P=8192, sm_scale=1.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_chain(name):
    s = W.make_draft_step(name=name, seed=sum(map(ord, name)), **CASES[name])
    say(f"[step] {name}: B={s.B} block={s.block} prefix={s.prefix.tolist()} H={s.proj.H} "
        f"L={s.write.L} heads {s.qk.NHQ}/{s.qk.NHK} D={s.qk.D} {s.dtype}")
    dev = DeviceStep(s)
    dev.reset()
    dev.run()
    got = dev.results()
    _check(s, got, oracle_chain(s))


def test_chain_in_one_graph():
    """The four operations captured as one HIP graph replay to the eager
    chain's bits, every replay (inputs restored and outputs reset by eager
    work between replays)."""
    s = W.make_draft_step(name="graph", seed=77, **CASES["bf16_d128"])
    dev = DeviceStep(s)
    dev.reset()
    dev.run()
    eager = dev.results()
    _check(s, eager, oracle_chain(s))
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    dev.reset()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            dev.run()
    for rep in range(3):
        dev.reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dev.results()
        for a, b in zip(got, eager):
            if isinstance(a, list):
                assert all(np.array_equal(x, y) for x, y in zip(a, b)), rep
            elif isinstance(a, np.ndarray):
                assert np.array_equal(a, b), rep
            else:
                assert a == b, rep


@pytest.mark.parametrize("i", range(6))
def test_random_chain(i):
    """Seeded sweep of whole chains: request count, block length, prefixes,
    hidden size, layer count, KV heads, grouping, head_dim and dtype drawn per
    case (sm_scale 1 so that outputs follow their best keys)."""
    rng = np.random.default_rng(8100 + i)
    B = int(rng.integers(1, 6))
    D = int(rng.choice([64, 128]))
    NH = int(rng.choice([1, 2, 4]))
    kw = dict(B=B, block=int(rng.integers(1, 17)),
              prefix=[int(x) for x in rng.integers(1, 600, size=B)],
              H=int(rng.integers(2, 9)) * 128, L=int(rng.integers(1, 4)), NH=NH,
              NHQ=NH * int(rng.choice([1, 2, 4])), D=D,
              dtype="fp16" if rng.random() < 0.4 else "bf16", sm_scale=1.0)
    s = W.make_draft_step(name=f"chain{i}", seed=8100 + i, **kw)
    say(f"[chain {i}] {kw}")
    dev = DeviceStep(s)
    dev.reset()
    dev.run()
    _check(s, dev.results(), oracle_chain(s))

