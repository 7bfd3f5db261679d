// Verification at temperature T > 0: the candidate trie and the acceptance walk
// (the LM head's sampling epilogue and its tile reduction live with the LM head).
// SwitchSD paper §3.3 "Overall Framework" (verification is delegated to the
// target and keeps speculative decoding's guarantee) and §2 "Speculative
// Decoding"; VIA-SD page "Draft-Verify and Lossy Acceptance" (lossless setting:
// a drafted token is accepted by its relative likelihood, a rejected one is
// replaced by a draw from the residual distribution).
//
// A copy candidate is a point-mass draft, so its token c is accepted with
// probability p(c).  Candidates with equal prefixes share a node of a trie; at a
// node, the distinct child tokens are tried in order of their lowest candidate
// with the probability left after the children rejected before them,
// p(x) / (1 - tried); when all are rejected (or there is none) the next token is
// a Gumbel-max draw from p without the tried children.  p is softmax(logits / T)
// of the node's row: the anchor row for the root, else row (r, j-1) with r the
// lowest candidate of the node's group.
//
// Random numbers: Philox4x32-10 keyed by the 64-bit seed.  Residual draw at
// global row g, token x: counter (x/4, g, 0, 0), word x%4.  Acceptance test of
// child k at row g: counter (k, g, 1, 0), word 0.
#include <limits.h>

#include "common.h"
#include "kernels.h"
#include "switchsd.h"

namespace ssd {

// One workgroup per sequence.  The trie follows from the common-prefix lengths
// lcp(v, w) of the candidates (a W x W table in LDS): the group of candidate w
// after j+1 tokens is {v : lcp(v, w) >= j+1}, and its lowest member rep_j(w)
// names it.  Candidate w's token j is a child of the node whose group has prefix
// length j (the anchor row for j = 0, else row (prep, j-1), prep = lowest v with
// lcp(v, w) >= j) exactly when w = rep_j(w) (the first candidate of its token
// group); row (w, j) is itself a node exactly then.  Every (candidate, depth)
// item is independent given the table, so the work is spread over the threads;
// every row's n_children and every child slot k < n_children is written once.
constexpr int kTrieThreads = 256;
__global__ __launch_bounds__(kTrieThreads) void trie_kernel(const int32_t* __restrict__ cand,
                                                            const int32_t* __restrict__ cand_len,
                                                            const uint8_t* __restrict__ copy_gate,
                                                            int W, int D,
                                                            int32_t* __restrict__ n_children,
                                                            int32_t* __restrict__ children,
                                                            int32_t* __restrict__ child_w,
                                                            float* __restrict__ child_logit) {
  __shared__ int s_tok[SSD_MAX_W * SSD_MAX_D];
  __shared__ int s_prep[SSD_MAX_W * SSD_MAX_D];
  __shared__ uint8_t s_first[SSD_MAX_W * SSD_MAX_D];
  __shared__ uint8_t s_lcp[SSD_MAX_W * SSD_MAX_W];
  __shared__ int s_L[SSD_MAX_W];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int R = 1 + W * D, WD = W * D;
  const size_t base = static_cast<size_t>(b) * R;
  const bool gate = copy_gate[b] != 0;
  for (int w = tid; w < W; w += kTrieThreads) {
    int L = gate ? cand_len[static_cast<size_t>(b) * W + w] : 0;
    s_L[w] = L < 0 ? 0 : (L > D ? D : L);
  }
  for (int i = tid; i < WD; i += kTrieThreads) s_tok[i] = cand[static_cast<size_t>(b) * WD + i];
  __syncthreads();
  for (int pq = tid; pq < W * W; pq += kTrieThreads) {
    const int v = pq / W, w = pq - v * W;
    const int n = min(s_L[v], s_L[w]);
    int q = 0;
    while (q < n && s_tok[v * D + q] == s_tok[w * D + q]) ++q;
    s_lcp[pq] = static_cast<uint8_t>(q);
  }
  __syncthreads();
  for (int i = tid; i < WD; i += kTrieThreads) {
    const int w = i / D, j = i - w * D;
    int rep = W, prep = -1;
    for (int v = 0; v < W; ++v) {
      const int l = s_lcp[v * W + w];
      if (rep == W && l > j) rep = v;
      if (j > 0 && prep < 0 && l >= j) prep = v;
    }
    s_first[i] = (j < s_L[w] && rep == w) ? 1 : 0;
    s_prep[i] = prep;
  }
  __syncthreads();
  for (int i = tid; i < WD; i += kTrieThreads) {
    const int w = i / D, j = i - w * D;
    const bool first = s_first[i] != 0;
    if (first) {
      const int prep = s_prep[i];
      int k = 0;
      for (int v = 0; v < w; ++v)
        if (s_first[v * D + j] && s_prep[v * D + j] == prep) ++k;
      const int prow = j == 0 ? 0 : 1 + prep * D + (j - 1);
      const size_t slot = (base + prow) * W + k;
      children[slot] = s_tok[i];
      child_w[slot] = w;
      child_logit[slot] = -INFINITY;
    }
    // row (w, j) is the node after tokens 0..j of w when w leads its token group;
    // its children are the group's tokens at depth j + 1
    int nc = 0;
    if (first && j + 1 < D)
      for (int v = 0; v < W; ++v)
        if (s_first[v * D + j + 1] && s_prep[v * D + j + 1] == w) ++nc;
    n_children[base + 1 + i] = nc;
  }
  if (tid == 0) {
    int nc = 0;
    for (int v = 0; v < W; ++v) nc += s_first[v * D];
    n_children[base] = nc;
  }
}

// One thread per sequence walks the trie from the anchor row.
__global__ __launch_bounds__(kWave) void accept_sample_kernel(
    const int32_t* __restrict__ n_children, const int32_t* __restrict__ child_w,
    const float* __restrict__ child_logit, const float* __restrict__ lse,
    const int32_t* __restrict__ resample, const uint8_t* __restrict__ copy_gate, int B, int W,
    int D, uint32_t k0, uint32_t k1, int32_t* __restrict__ best_w, int32_t* __restrict__ best_len,
    int32_t* __restrict__ next_token) {
  const int b = blockIdx.x * kWave + threadIdx.x;
  if (b >= B) return;
  if (!copy_gate[b]) {
    best_w[b] = -1;
    best_len[b] = 0;
    next_token[b] = -1;
    return;
  }
  const int R = 1 + W * D;
  int row = 0, j = 0, bw = 0, nxt = -1;
  for (int depth = 0; depth <= D; ++depth) {
    const size_t g = static_cast<size_t>(b) * R + row;
    const int nc = min(max(n_children[g], 0), W);
    const float l = lse[g];
    float tried = 0.f;
    bool moved = false;
    for (int k = 0; k < nc; ++k) {
      const float p = __expf(child_logit[g * W + k] - l);
      const float r = p == 0.f ? 0.f : p / fmaxf(1.f - tried, p);
      const float u = word_uniform(philox4x32_10(k, static_cast<uint32_t>(g), 1, 0, k0, k1).x);
      if (u < r) {
        const int w = min(max(child_w[g * W + k], 0), W - 1);
        if (j >= D) break;
        bw = w;
        row = 1 + w * D + j;
        ++j;
        moved = true;
        break;
      }
      tried += p;
    }
    if (!moved) {
      nxt = resample[g];
      break;
    }
  }
  best_w[b] = bw;
  best_len[b] = j;
  next_token[b] = nxt;
}

hipError_t launch_trie(const int32_t* cand, const int32_t* cand_len, const uint8_t* copy_gate,
                       int B, int W, int D, int32_t* n_children, int32_t* children,
                       int32_t* child_w, float* child_logit, hipStream_t s) {
  hipLaunchKernelGGL(trie_kernel, dim3(B), dim3(kTrieThreads), 0, s, cand, cand_len, copy_gate, W,
                     D, n_children, children, child_w, child_logit);
  return hipGetLastError();
}

hipError_t launch_accept_sample(const int32_t* n_children, const int32_t* child_w,
                                const float* child_logit, const float* lse,
                                const int32_t* resample, const uint8_t* copy_gate, int B, int W,
                                int D, unsigned long long seed, int32_t* best_w,
                                int32_t* best_len, int32_t* next_token, hipStream_t s) {
  hipLaunchKernelGGL(accept_sample_kernel, dim3((B + kWave - 1) / kWave), dim3(kWave), 0, s,
                     n_children, child_w, child_logit, lse, resample, copy_gate, B, W, D,
                     static_cast<uint32_t>(seed & 0xffffffffu), static_cast<uint32_t>(seed >> 32),
                     best_w, best_len, next_token);
  return hipGetLastError();
}

}  // namespace ssd
