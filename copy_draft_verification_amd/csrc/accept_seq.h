// Longest accepted continuation at T = 0 (SwitchSD paper §3.3: the longest
// validated continuation is kept; greedy verification stops at the first
// disagreement with the target's argmax), computed by one wavefront per sequence.
// For candidate w, lane j tests cand[w][j] == pred(w, j-1); a ballot turns the
// tests into a bit mask and the run of ones from bit 0 is the accepted length a_w.
// A wave reduction then picks the largest a_w, lowest w on ties, and the token
// after it.  Used by the accept kernel and by the argmax launch that follows the
// greedy LM head when it accepts as well.
#pragma once
#include "common.h"
#include "switchsd.h"

namespace ssd {

// Candidates are handled 16 at a time: every lane issues its loads for the 16
// candidates first (candidate token j and the prediction it is checked against),
// then the ballots run.  Lane j <= D keeps pred(w, j-1) in LDS, so the token after
// the accepted prefix is an LDS read rather than another global load.
constexpr int kAcGroup = 16;

// What the accept reads before it needs the argmax: the gate, the candidate
// lengths (lane w) and the first group's candidate tokens.  Issued on its own, it
// lets a caller overlap these loads with the loads of the argmax itself.
struct AcceptPre {
  int gate, len_lane;
  int c[kAcGroup];
};

// Candidate token j (= lane) of candidates w0 .. w0+15 of sequence b, -1 past W or D.
// Unconditional loads from clamped (in-bounds) indices, then selects: predicated
// loads would become branches, each ending in a wait for every load before it.
__device__ __forceinline__ void accept_load_cand(const int32_t* __restrict__ cand, int b, int lane,
                                                 int W, int D, int w0, int (&c)[kAcGroup]) {
  const int32_t* cb = cand + static_cast<size_t>(b) * W * D;
#pragma unroll
  for (int u = 0; u < kAcGroup; ++u) {
    const int w = w0 + u;
    const bool cv = w < W && lane < D;
    const int cx = cb[cv ? w * D + lane : 0];
    c[u] = cv ? cx : -1;
  }
}

__device__ __forceinline__ AcceptPre accept_prefetch(int b, int lane, const int32_t* __restrict__ cand,
                                                     const int32_t* __restrict__ cand_len,
                                                     const uint8_t* __restrict__ copy_gate, int W, int D) {
  // the arrays are fixed-size, so the reads are in bounds whatever the gate says
  AcceptPre pre;
  pre.gate = copy_gate[b];
  const int len_raw = cand_len[static_cast<size_t>(b) * W + (lane < W ? lane : 0)];
  pre.len_lane = lane < W ? len_raw : 0;
  accept_load_cand(cand, b, lane, W, D, 0, pre.c);
  return pre;
}

// Sequence b, by the calling wavefront (lane = its lane), from its prefetched
// inputs.  am: the argmax of sequence b's 1 + W*D rows (global memory or LDS);
// s_pred: this wave's SSD_MAX_W x 64 ints of LDS.
__device__ __forceinline__ void accept_run(
    const AcceptPre& pre, int b, int lane, const int32_t* __restrict__ cand,
    const int32_t* __restrict__ am, int W, int D, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ best_w, int32_t* __restrict__ best_len, int32_t* __restrict__ next_token,
    int (*s_pred)[kWave]) {
  int c[kAcGroup], pv[kAcGroup];
#pragma unroll
  for (int u = 0; u < kAcGroup; ++u) c[u] = pre.c[u];
  // pred(w, lane-1): the anchor's argmax for lane 0, else row (w, lane-1)
  auto load_pred = [&](int w0) {
#pragma unroll
    for (int u = 0; u < kAcGroup; ++u) {
      const int w = w0 + u;
      const bool pvv = w < W && lane <= D;
      const int pi = (pvv && lane > 0) ? 1 + w * D + lane - 1 : 0;
      const int px = am[pi];
      pv[u] = pvv ? px : -1;
    }
  };
  load_pred(0);
  if (pre.gate == 0) {
    for (int w = lane; w < W; w += kWave) accept_len[static_cast<size_t>(b) * W + w] = 0;
    if (lane == 0) {
      best_w[b] = -1;
      best_len[b] = 0;
      next_token[b] = -1;
    }
    return;
  }
  int my_a = 0;
  for (int w0 = 0; w0 < W; w0 += kAcGroup) {
    if (w0 > 0) {
      accept_load_cand(cand, b, lane, W, D, w0, c);
      load_pred(w0);
    }
#pragma unroll
    for (int u = 0; u < kAcGroup; ++u) {
      const int w = w0 + u;
      if (w >= W) break;
      int L = __shfl(pre.len_lane, w, kWave);
      L = L < 0 ? 0 : (L > D ? D : L);
      const bool ok = lane < L && c[u] == pv[u];
      const unsigned long long m = __ballot(ok);
      const unsigned long long inv = ~m;
      int a = inv == 0ull ? kWave : __ffsll(static_cast<long long>(inv)) - 1;
      a = min(a, L);
      if (lane == w) my_a = a;
      s_pred[w][lane] = pv[u];
    }
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
    // pred(bi, bv-1) sits in lane bv of row bi (lanes 0..min(D, 63) were filled)
    next_token[b] = bv < kWave ? s_pred[bi][bv] : am[1 + bi * D + bv - 1];
  }
}

__device__ __forceinline__ void accept_seq(
    int b, int lane, const int32_t* __restrict__ cand, const int32_t* __restrict__ cand_len,
    const uint8_t* __restrict__ copy_gate, const int32_t* __restrict__ am, int W, int D,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ best_w, int32_t* __restrict__ best_len,
    int32_t* __restrict__ next_token, int (*s_pred)[kWave]) {
  const AcceptPre pre = accept_prefetch(b, lane, cand, cand_len, copy_gate, W, D);
  accept_run(pre, b, lane, cand, am, W, D, accept_len, best_w, best_len, next_token, s_pred);
}

}  // namespace ssd
