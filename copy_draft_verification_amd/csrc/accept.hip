// Longest accepted continuation at T = 0 (SwitchSD paper §3.3: the longest
// validated continuation is kept; greedy verification stops at the first
// disagreement with the target's argmax).
//
// One wavefront per sequence (accept_seq).
#include "accept_seq.h"
#include "common.h"
#include "kernels.h"
#include "switchsd.h"

namespace ssd {

__global__ __launch_bounds__(kWave) void accept_kernel(
    const int32_t* __restrict__ cand, const int32_t* __restrict__ cand_len,
    const uint8_t* __restrict__ copy_gate, const int32_t* __restrict__ argmax, int W, int D,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ best_w, int32_t* __restrict__ best_len,
    int32_t* __restrict__ next_token) {
  __shared__ int s_pred[SSD_MAX_W][kWave];
  const int b = blockIdx.x;
  accept_seq(b, threadIdx.x, cand, cand_len, copy_gate, argmax + static_cast<size_t>(b) * (1 + W * D), W,
             D, accept_len, best_w, best_len, next_token, s_pred);
}

hipError_t launch_accept(const int32_t* cand, const int32_t* cand_len, const uint8_t* copy_gate,
                         const int32_t* argmax, int B, int W, int D, int32_t* accept_len,
                         int32_t* best_w, int32_t* best_len, int32_t* next_token, hipStream_t s) {
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(kWave), 0, s, cand, cand_len, copy_gate, argmax,
                     W, D, accept_len, best_w, best_len, next_token);
  return hipGetLastError();
}

}  // namespace ssd
