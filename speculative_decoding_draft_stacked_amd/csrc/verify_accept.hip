// Accept length and bonus token of the verify step, for gfx950.
//
// Method: sglang PR #31847 ("[spec decoding] support inkling dspark",
// implementation breakdown step 2, compute_dflash_correct_drafts_and_bonus):
// for each request the accepted drafts are the longest prefix of its K drafted
// tokens equal to the target's tokens at the same positions, i.e. the first
// mismatching position (K when none), and the bonus token is the target's token
// at that position.
//
// Mapping. Each request takes a group of LPR lanes, the smallest power of two
// >= K (at most 64), so a wave holds 64 / LPR requests. Every lane compares one
// position; one ballot gives the mismatch bits of the whole wave, and the count
// of trailing zeros of a group's bits is its first mismatch. Requests with
// K > 64 take a whole wave and walk the positions 64 at a time, stopping at
// the first chunk that has a mismatch. Exact integer work, no rounding.
#include "internal.h"

namespace dspark {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void verify_accept_kernel(const VerifyArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lpr = a.lanes_per_request;
  const int seg = lane / lpr;
  const int sl = lane % lpr;
  const int64_t b = wave * (64 / lpr) + seg;
  const bool live = b < a.B;
  const int64_t* d = a.draft + (live ? b : 0) * a.draft_stride;
  const int64_t* t = a.target + (live ? b : 0) * a.target_stride;
  int acc = a.K;
  for (int c0 = 0; c0 < a.K; c0 += lpr) {  // one pass unless K > 64 (then lpr = 64)
    const int i = c0 + sl;
    const bool mism = live && i < a.K && d[i] != t[i];
    const unsigned long long m = __ballot(mism);
    const unsigned long long mine =
        lpr == 64 ? m : (m >> (seg * lpr)) & ((1ull << lpr) - 1ull);
    if (mine) {  // uniform over the group; with lpr == 64, over the wave
      acc = c0 + __builtin_ctzll(mine);
      break;
    }
  }
  if (live && sl == 0) {
    a.accept[b] = acc;
    a.bonus[b] = t[acc];
  }
}

}  // namespace

hipError_t launch_verify_accept(const VerifyArgs& in, hipStream_t stream) {
  if (in.B <= 0) return hipSuccess;
  VerifyArgs a = in;
  int lpr = 1;
  while (lpr < a.K && lpr < 64) lpr <<= 1;
  a.lanes_per_request = lpr;
  const int64_t waves = (a.B + 64 / lpr - 1) / (64 / lpr);
  const int64_t blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(verify_accept_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dspark
