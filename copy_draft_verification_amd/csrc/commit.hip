// Commit of the accepted draft into the target's KV cache (SwitchSD paper §3.3:
// the longest validated continuation extends the context; greedy decoding then
// adds the target's own next token, which becomes the next anchor).
//
// The verification pass already holds the accepted tokens' keys and values:
// workgroup (b, j) copies row j of candidate best_w[b] (K and V, Hkv*d elements
// each, in 16-byte pieces) to cache row cache_off[b] + j, and writes token j of
// the context extension.  Nothing is written for a closed gate, an out-of-range
// best_w / best_len, or a commit that would not fit in the cache.
#include "common.h"
#include "kernels.h"

namespace ssd {

__global__ __launch_bounds__(256) void commit_kernel(
    const uint4* __restrict__ k_cand, const uint4* __restrict__ v_cand,
    const int32_t* __restrict__ cand, const int32_t* __restrict__ best_w,
    const int32_t* __restrict__ best_len, const int32_t* __restrict__ next_token, int W, int D,
    int row_chunks, uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, long long cache_rows,
    const long long* __restrict__ cache_off, int32_t* __restrict__ tokens_out,
    int32_t* __restrict__ n_tokens_out) {
  const int b = blockIdx.x, j = blockIdx.y;
  const int w = best_w[b], L = best_len[b];
  const long long off = cache_off[b];
  const bool open = w >= 0;
  const bool valid = open && w < W && L >= 0 && L <= D && off >= 0 && off + L <= cache_rows;
  if (valid && j < L) {
    const size_t src = (static_cast<size_t>(b) * W * D + static_cast<size_t>(w) * D + j) * row_chunks;
    const size_t dst = static_cast<size_t>(off + j) * row_chunks;
    for (int c = threadIdx.x; c < row_chunks; c += blockDim.x) {
      k_cache[dst + c] = k_cand[src + c];
      v_cache[dst + c] = v_cand[src + c];
    }
  }
  if (threadIdx.x == 0) {
    int t = -1;
    if (valid && j < L) t = cand[(static_cast<size_t>(b) * W + w) * D + j];
    else if (valid && j == L) t = next_token[b];
    tokens_out[static_cast<size_t>(b) * (D + 1) + j] = t;
  }
  if (j == 0 && threadIdx.x == 1) {
    tokens_out[static_cast<size_t>(b) * (D + 1) + D] = (valid && L == D) ? next_token[b] : -1;
    n_tokens_out[b] = valid ? L + 1 : (open ? -1 : 0);
  }
}

hipError_t launch_commit(const void* k_cand, const void* v_cand, const int32_t* cand,
                         const int32_t* best_w, const int32_t* best_len, const int32_t* next_token,
                         int B, int W, int D, int row_bytes, void* k_cache, void* v_cache,
                         long long cache_rows, const long long* cache_off, int32_t* tokens_out,
                         int32_t* n_tokens_out, hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(B, D), dim3(256), 0, s, static_cast<const uint4*>(k_cand),
                     static_cast<const uint4*>(v_cand), cand, best_w, best_len, next_token, W, D,
                     row_bytes / 16, static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache),
                     cache_rows, cache_off, tokens_out, n_tokens_out);
  return hipGetLastError();
}

}  // namespace ssd
