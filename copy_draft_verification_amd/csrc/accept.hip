// Longest accepted continuation at T = 0 (SwitchSD paper §3.3: the longest
// validated continuation is kept; greedy verification stops at the first
// disagreement with the target's argmax).
//
// One wavefront per sequence.  For candidate w, lane j tests
// cand[w][j] == pred(w, j-1); a ballot turns the tests into a bit mask and the
// run of ones from bit 0 is the accepted length a_w.  A wave reduction then
// picks the largest a_w, lowest w on ties, and the token after it.
#include "common.h"
#include "kernels.h"

namespace ssd {

__global__ __launch_bounds__(kWave) void accept_kernel(
    const int32_t* __restrict__ cand, const int32_t* __restrict__ cand_len,
    const uint8_t* __restrict__ copy_gate, const int32_t* __restrict__ argmax, int W, int D,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ best_w, int32_t* __restrict__ best_len,
    int32_t* __restrict__ next_token) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int R = 1 + W * D;
  const int32_t* am = argmax + static_cast<size_t>(b) * R;
  if (copy_gate[b] == 0) {
    for (int w = lane; w < W; w += kWave) accept_len[static_cast<size_t>(b) * W + w] = 0;
    if (lane == 0) {
      best_w[b] = -1;
      best_len[b] = 0;
      next_token[b] = -1;
    }
    return;
  }
  int my_a = 0;
  for (int w = 0; w < W; ++w) {
    int L = cand_len[static_cast<size_t>(b) * W + w];
    L = L < 0 ? 0 : (L > D ? D : L);
    bool ok = false;
    if (lane < L) {
      const int prev = lane == 0 ? am[0] : am[1 + w * D + lane - 1];
      ok = cand[(static_cast<size_t>(b) * W + w) * D + lane] == prev;
    }
    const unsigned long long m = __ballot(ok);
    const unsigned long long inv = ~m;
    int a = inv == 0ull ? kWave : __ffsll(static_cast<long long>(inv)) - 1;
    a = min(a, L);
    if (lane == w) my_a = a;
  }
  int bv = lane < W ? my_a : -1, bi = lane;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int ov = __shfl_xor(bv, o, kWave), oi = __shfl_xor(bi, o, kWave);
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
  }
  if (lane < W) accept_len[static_cast<size_t>(b) * W + lane] = my_a;
  if (lane == 0) {
    best_w[b] = bi;
    best_len[b] = bv;
    next_token[b] = bv == 0 ? am[0] : am[1 + bi * D + bv - 1];
  }
}

hipError_t launch_accept(const int32_t* cand, const int32_t* cand_len, const uint8_t* copy_gate,
                         const int32_t* argmax, int B, int W, int D, int32_t* accept_len,
                         int32_t* best_w, int32_t* best_len, int32_t* next_token, hipStream_t s) {
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(kWave), 0, s, cand, cand_len, copy_gate, argmax,
                     W, D, accept_len, best_w, best_len, next_token);
  return hipGetLastError();
}

}  // namespace ssd
