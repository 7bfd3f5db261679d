// kappa-gram evidence, recency-ordered retrieval and candidate gather.
// SwitchSD write-up §2.5 (dual gate: probe AND an earlier occurrence of the
// kappa-gram ending at the current token), paper §3.3 "Copy-Based Speculative
// Generation" and write-up §2.6 (up to W continuations of up to D tokens,
// ranked by recency).
//
// One 1024-lane workgroup per sequence scans end positions from the newest
// (n-2) backwards in chunks of 8192.  A chunk of ids (plus a kappa-1 halo) is
// staged in LDS with coalesced loads; lane t tests positions top-8t .. top-8t-7,
// so lane order equals recency order.  Matches are compacted in that order by a
// workgroup prefix sum over per-lane counts, and the scan stops as soon as W
// matches are known.  The candidate gather then copies L_w = min(D, n-1-p_w)
// ids after each match.
#include "common.h"
#include "kernels.h"
#include "switchsd.h"

namespace ssd {

constexpr int kKgThreads = 1024;
constexpr int kKgPer = 8;
constexpr int kKgChunk = kKgThreads * kKgPer;

__global__ __launch_bounds__(kKgThreads) void kgram_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ cu_len, int kappa, int W, int D,
    const uint8_t* __restrict__ fire, int32_t* __restrict__ match_end, int32_t* __restrict__ n_match,
    int32_t* __restrict__ cand, int32_t* __restrict__ cand_len, uint8_t* __restrict__ copy_gate) {
  __shared__ int s_ids[kKgChunk + SSD_MAX_KAPPA];
  __shared__ int s_suffix[SSD_MAX_KAPPA];
  __shared__ int s_list[SSD_MAX_W];
  __shared__ int s_wave[kKgThreads / kWave];
  const int b = blockIdx.x, t = threadIdx.x;
  const int base = cu_len[b];
  const int n = cu_len[b + 1] - base;
  const bool active = (fire == nullptr || fire[b] != 0) && n >= kappa + 1;
  int found = 0;
  if (active) {
    if (t < kappa) s_suffix[t] = ids[base + n - kappa + t];
    const int lo = kappa - 1;
    for (int top = n - 2; top >= lo && found < W; top -= kKgChunk) {
      const int cbeg = max(lo, top - kKgChunk + 1);
      const int lbase = cbeg - kappa + 1;
      const int cnt = top - lbase + 1;
      // stage the chunk: every thread issues all of its loads before storing any
      int tmp[kKgPer + 1];
#pragma unroll
      for (int u = 0; u <= kKgPer; ++u) {
        const int i = t + u * kKgThreads;
        tmp[u] = i < cnt ? ids[base + lbase + i] : 0;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u <= kKgPer; ++u) {
        const int i = t + u * kKgThreads;
        if (i < cnt) s_ids[i] = tmp[u];
      }
      __syncthreads();
      unsigned mask = 0;
      const int p0 = top - t * kKgPer;
#pragma unroll
      for (int i = 0; i < kKgPer; ++i) {
        const int p = p0 - i;
        if (p >= cbeg) {
          bool m = true;
          for (int qq = 0; qq < kappa; ++qq) {
            if (s_ids[p - qq - lbase] != s_suffix[kappa - 1 - qq]) { m = false; break; }
          }
          if (m) mask |= 1u << i;
        }
      }
      int total;
      int rank = found + block_excl_scan<kKgThreads>(__popc(mask), s_wave, total);
      while (mask) {
        const int i = __ffs(mask) - 1;
        mask &= mask - 1;
        if (rank < W) s_list[rank] = p0 - i;
        ++rank;
      }
      found += total;
    }
  }
  __syncthreads();
  const int M = min(found, W);
  for (int w = t; w < W; w += kKgThreads) {
    const int p = w < M ? s_list[w] : -1;
    match_end[static_cast<size_t>(b) * W + w] = p;
    cand_len[static_cast<size_t>(b) * W + w] = w < M ? min(D, n - 1 - p) : 0;
  }
  for (int e = t; e < W * D; e += kKgThreads) {
    const int w = e / D, j = e - w * D;
    int v = -1;
    if (w < M) {
      const int p = s_list[w];
      if (j < min(D, n - 1 - p)) v = ids[base + p + 1 + j];
    }
    cand[static_cast<size_t>(b) * W * D + e] = v;
  }
  if (t == 0) {
    n_match[b] = M;
    copy_gate[b] = M > 0 ? 1 : 0;
  }
}

hipError_t launch_kgram(const int32_t* ids, const int32_t* cu_len, int B, int kappa, int W, int D,
                        const uint8_t* fire, int32_t* match_end, int32_t* n_match, int32_t* cand,
                        int32_t* cand_len, uint8_t* copy_gate, hipStream_t s) {
  hipLaunchKernelGGL(kgram_kernel, dim3(B), dim3(kKgThreads), 0, s, ids, cu_len, kappa, W, D, fire,
                     match_end, n_match, cand, cand_len, copy_gate);
  return hipGetLastError();
}

}  // namespace ssd
