// The verification pass as a full target forward: embedding, decoder layers,
// final norm, LM head.  SwitchSD paper §3.3 "Parallel Verification with
// Block-Triangular Attention" verifies the anchor and all W candidates in one
// target forward; the layer is the Llama-family pre-norm layer of the paper's
// targets (§4.1), with synthetic weights:
//   h = RMSNorm(x) g_attn; q, k, v = W_qkv h; RoPE(q, k); a = attention;
//   x += W_o a; h = RMSNorm(x) g_mlp; x += W_down (silu(W_gate h) * W_up h).
// Positions: anchor row n - 1, candidate token j at n + j; RoPE turns adjacent
// pairs (2i, 2i+1) of a head by pos * base^(-2i/d).
//
// Rows are the verification rows [B][R] (R = 1 + W*D); only real rows (open
// gate, row 0 or j < L_w) are computed, through the compact row list of the
// LM-head workspace.  The residual stream x is fp32; the normalised states h,
// q / k / v, the attention output and the MLP activation are bf16.  The
// projections run on the LM-head kernel's main loop: split-K partial sums for
// W_qkv, W_o and W_down (reduced by the kernels below, which also apply RoPE, or
// the residual add and the next RMSNorm in one pass), silu(gate) * up fused into the
// gate / up projection.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "switchsd.h"

namespace ssd {

constexpr int kFwThreads = 256;

// Sum of v over the workgroup (kThreads threads); every thread gets it.
template <int kThreads = kFwThreads>
__device__ __forceinline__ float block_sum(float v, float* s_part) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  if (lane == 0) s_part[wv] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) t += s_part[i];
  __syncthreads();
  return t;
}

// h[grow] = bf16(x[grow] / sqrt(mean(x^2) + eps) * g), x already in `xv`
// (this thread's elements k = tid + i * kFwThreads).
template <int kPer>
__device__ __forceinline__ void write_norm(const float (&xv)[kPer], int hid, float eps,
                                           const uint16_t* __restrict__ g, uint16_t* __restrict__ hrow,
                                           float* s_part) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int k = threadIdx.x + i * kFwThreads;
    if (k < hid) ss += xv[i] * xv[i];
  }
  const float tot = block_sum(ss, s_part);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(hid) + eps);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int k = threadIdx.x + i * kFwThreads;
    if (k < hid) hrow[k] = f32_to_bf16(xv[i] * inv * bf16_to_f32(g[k]));
  }
}

constexpr int kFwMaxPer = 8192 / kFwThreads;  // hidden <= 8192

// Row tokens to the residual stream, then the first RMSNorm.  One workgroup per
// compact row.
__global__ __launch_bounds__(kFwThreads) void fwd_embed_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ cu_len,
    const int32_t* __restrict__ cand, const uint16_t* __restrict__ embed, int V, int R, int WD,
    int hid, const int32_t* __restrict__ row_list, const int32_t* __restrict__ n_rows,
    const uint16_t* __restrict__ g, float eps, float* __restrict__ x, uint16_t* __restrict__ hbuf) {
  __shared__ float s_part[kFwThreads / kWave];
  const int ci = blockIdx.x;
  if (ci >= *n_rows) return;
  const int grow = row_list[ci], b = grow / R, r = grow - b * R;
  int tok = r == 0 ? ids[cu_len[b + 1] - 1] : cand[static_cast<size_t>(b) * WD + (r - 1)];
  const bool ok = tok >= 0 && tok < V;
  const uint16_t* e = embed + static_cast<size_t>(ok ? tok : 0) * hid;
  float xv[kFwMaxPer];
#pragma unroll
  for (int i = 0; i < kFwMaxPer; ++i) {
    const int k = threadIdx.x + i * kFwThreads;
    xv[i] = (k < hid && ok) ? bf16_to_f32(e[k]) : 0.f;
    if (k < hid) x[static_cast<size_t>(grow) * hid + k] = xv[i];
  }
  write_norm<kFwMaxPer>(xv, hid, eps, g, hbuf + static_cast<size_t>(grow) * hid, s_part);
}

// Split-K sums of the W_qkv projection, RoPE on q and k, and the scatter: q to
// [B][R][Hq][d]; a candidate row's k and v to the candidate blocks
// [B][W*D][Hkv][d] (the anchor's key and value are prefix entry n - 1).  Grid:
// (compact row, slice of 512 features); each thread owns one pair of features and
// issues its loads for up to eight splits at a time before adding them.
constexpr int kSplitBatch = 8;
__global__ __launch_bounds__(kFwThreads) void fwd_qkv_finish_kernel(
    const float* __restrict__ part, int splits, int part_rows, int Hq, int Hkv, int d,
    const int32_t* __restrict__ cu_len, int R, int D, int WD, double log2_base,
    const int32_t* __restrict__ row_list, const int32_t* __restrict__ n_rows,
    uint16_t* __restrict__ q, uint16_t* __restrict__ k_cand, uint16_t* __restrict__ v_cand) {
  const int ci = blockIdx.x;
  if (ci >= *n_rows) return;
  const int N = (Hq + 2 * Hkv) * d;
  const int e = 2 * (blockIdx.y * kFwThreads + threadIdx.x);
  if (e >= N) return;
  const int grow = row_list[ci], b = grow / R, r = grow - b * R;
  const int n = cu_len[b + 1] - cu_len[b];
  const int pos = r == 0 ? n - 1 : n + (r - 1) % D;
  const size_t stride = static_cast<size_t>(part_rows) * N;
  const float* p0 = part + static_cast<size_t>(ci) * N + e;
  float v0 = 0.f, v1 = 0.f;
  for (int s0 = 0; s0 < splits; s0 += kSplitBatch) {
    float2 pv[kSplitBatch];
#pragma unroll
    for (int u = 0; u < kSplitBatch; ++u)
      pv[u] = s0 + u < splits ? *reinterpret_cast<const float2*>(p0 + (s0 + u) * stride) : make_float2(0.f, 0.f);
#pragma unroll
    for (int u = 0; u < kSplitBatch; ++u) {
      v0 += pv[u].x;
      v1 += pv[u].y;
    }
  }
  const int head = e / d, i = (e - head * d) >> 1;
  if (head < Hq + Hkv) {  // q or k: rotate the pair
    const double ang = static_cast<double>(pos) * exp2(-(2.0 * i / d) * log2_base);
    double sn, cs;
    sincos(ang, &sn, &cs);
    const float c = static_cast<float>(cs), sg = static_cast<float>(sn);
    const float r0 = v0 * c - v1 * sg, r1 = v0 * sg + v1 * c;
    v0 = r0;
    v1 = r1;
  }
  const uint32_t packed = f32_to_bf16(v0) | static_cast<uint32_t>(f32_to_bf16(v1)) << 16;
  if (head < Hq) {
    *reinterpret_cast<uint32_t*>(q + static_cast<size_t>(grow) * Hq * d + e) = packed;
  } else if (r > 0) {
    const bool is_k = head < Hq + Hkv;
    const int kvh = is_k ? head - Hq : head - Hq - Hkv;
    uint16_t* dst = (is_k ? k_cand : v_cand) +
                    ((static_cast<size_t>(b) * WD + (r - 1)) * Hkv + kvh) * d + (e - head * d);
    *reinterpret_cast<uint32_t*>(dst) = packed;
  }
}

// x[grow] += the split partials (added in split order), then
// h[grow] = RMSNorm(x[grow]) g.  One 1024-thread workgroup per compact row;
// thread t owns features 4t + 4096p (p < 2), and the loads of up to eight splits
// are in flight before any is added.
constexpr int kRnThreads = 1024;
constexpr int kRnPass = 8192 / (4 * kRnThreads);  // hidden <= 8192
__global__ __launch_bounds__(kRnThreads) void fwd_residual_norm_kernel(
    const float* __restrict__ part, int splits, int part_rows, int hid,
    const int32_t* __restrict__ row_list, const int32_t* __restrict__ n_rows,
    const uint16_t* __restrict__ g, float eps, float* __restrict__ x, uint16_t* __restrict__ hbuf) {
  __shared__ float s_part[kRnThreads / kWave];
  const int ci = blockIdx.x;
  if (ci >= *n_rows) return;
  const int grow = row_list[ci];
  const size_t stride = static_cast<size_t>(part_rows) * hid;
  float* const xr = x + static_cast<size_t>(grow) * hid;
  float4 acc[kRnPass];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < kRnPass; ++p) {
    const int k = 4 * (threadIdx.x + p * kRnThreads);
    if (k >= hid) continue;
    const float* p0 = part + static_cast<size_t>(ci) * hid + k;
    float4 a = *reinterpret_cast<const float4*>(xr + k);
    for (int s0 = 0; s0 < splits; s0 += kSplitBatch) {
      float4 pv[kSplitBatch];
#pragma unroll
      for (int u = 0; u < kSplitBatch; ++u)
        pv[u] = s0 + u < splits ? *reinterpret_cast<const float4*>(p0 + (s0 + u) * stride)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < kSplitBatch; ++u) {
        a.x += pv[u].x;
        a.y += pv[u].y;
        a.z += pv[u].z;
        a.w += pv[u].w;
      }
    }
    *reinterpret_cast<float4*>(xr + k) = a;
    ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    acc[p] = a;
  }
  const float tot = block_sum<kRnThreads>(ss, s_part);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(hid) + eps);
  uint16_t* const hr = hbuf + static_cast<size_t>(grow) * hid;
#pragma unroll
  for (int p = 0; p < kRnPass; ++p) {
    const int k = 4 * (threadIdx.x + p * kRnThreads);
    if (k >= hid) continue;
    const float4 a = acc[p];
    // the gain vector carries no alignment promise beyond its element size
    const uint32_t h0 = f32_to_bf16(a.x * inv * bf16_to_f32(g[k]));
    const uint32_t h1 = f32_to_bf16(a.y * inv * bf16_to_f32(g[k + 1]));
    const uint32_t h2 = f32_to_bf16(a.z * inv * bf16_to_f32(g[k + 2]));
    const uint32_t h3 = f32_to_bf16(a.w * inv * bf16_to_f32(g[k + 3]));
    *reinterpret_cast<uint2*>(hr + k) = make_uint2(h0 | h1 << 16, h2 | h3 << 16);
  }
}

// a[grow][f] = silu(sum of the gate partials) * (sum of the up partials), bf16.
// Grid: (compact row, slice of 1024 features), four features per thread.
__global__ __launch_bounds__(kFwThreads) void fwd_swiglu_finish_kernel(
    const float* __restrict__ part, int splits, int part_rows, int inter,
    const int32_t* __restrict__ row_list, const int32_t* __restrict__ n_rows,
    uint16_t* __restrict__ a) {
  const int ci = blockIdx.x;
  if (ci >= *n_rows) return;
  const int f = 4 * (blockIdx.y * kFwThreads + threadIdx.x);
  if (f >= inter) return;
  const size_t ld = 2 * static_cast<size_t>(inter), stride = static_cast<size_t>(part_rows) * ld;
  const float* p0 = part + static_cast<size_t>(ci) * ld + f;
  float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
  for (int s = 0; s < splits; ++s) {
    const float4 pg = *reinterpret_cast<const float4*>(p0 + s * stride);
    const float4 pu = *reinterpret_cast<const float4*>(p0 + s * stride + inter);
    g.x += pg.x; g.y += pg.y; g.z += pg.z; g.w += pg.w;
    u.x += pu.x; u.y += pu.y; u.z += pu.z; u.w += pu.w;
  }
  auto act = [](float gv, float uv) { return f32_to_bf16(gv / (1.0f + __expf(-gv)) * uv); };
  *reinterpret_cast<uint2*>(a + static_cast<size_t>(row_list[ci]) * inter + f) =
      make_uint2(act(g.x, u.x) | static_cast<uint32_t>(act(g.y, u.y)) << 16,
                 act(g.z, u.z) | static_cast<uint32_t>(act(g.w, u.w)) << 16);
}

__global__ __launch_bounds__(256) void fwd_zero_kernel(uint32_t* __restrict__ p, size_t n_words) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n_words;
       i += static_cast<size_t>(gridDim.x) * 256)
    p[i] = 0u;
}

// Splits of K (into multiples of 256) so that about one workgroup per CU runs:
// more splits only add partial-sum traffic.
int fwd_splits(const LmPlan& p, int K) {
  const int base = p.vtiles * p.mchunks, units = K / 256;
  int best = 1;
  for (int s = 1; s <= 32 && s <= units; ++s)
    if (units % s == 0 && base * s <= 288) best = s;
  return best;
}

namespace {
size_t al(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

FwdLayout fwd_layout(int B, int max_n, int W, int D, int Hq, int Hkv, int d, int inter, int V) {
  FwdLayout L;
  const int R = 1 + W * D, rows = B * R, hid = Hq * d;
  L.attn = attn_plan(B, max_n, R, Hq, Hkv, true);
  L.lm = lm_plan(rows, V, true);
  L.p_qkv = gemm_plan(rows, (Hq + 2 * Hkv) * d, false);
  L.p_o = gemm_plan(rows, hid, false);
  L.p_gu = gemm_plan(rows, inter, true);
  L.p_down = gemm_plan(rows, hid, false);
  L.s_qkv = fwd_splits(L.p_qkv, hid);
  L.s_o = fwd_splits(L.p_o, hid);
  L.s_down = fwd_splits(L.p_down, inter);
  L.s_gu = fwd_splits(L.p_gu, hid);
  const size_t part = static_cast<size_t>(rows) *
      std::max({static_cast<size_t>(L.s_qkv) * (Hq + 2 * Hkv) * d, static_cast<size_t>(L.s_o) * hid,
                static_cast<size_t>(L.s_down) * hid, static_cast<size_t>(L.s_gu) * 2 * inter});
  size_t o = 0;
  L.off_lm = o;      o += al(lm_workspace_bytes(L.lm, rows));
  L.off_attn = o;    o += al(attn_workspace_bytes(L.attn, B, R, Hq, d));
  L.off_x = o;       o += al(sizeof(float) * rows * hid);
  L.off_h = o;       o += al(2ull * rows * hid);
  L.off_q = o;       o += al(2ull * rows * Hq * d);
  L.off_kc = o;      o += al(2ull * B * W * D * Hkv * d);
  L.off_vc = o;      o += al(2ull * B * W * D * Hkv * d);
  L.off_att = o;     o += al(2ull * rows * Hq * d);
  L.off_a = o;       o += al(2ull * rows * inter);
  L.off_part = o;    o += al(sizeof(float) * part);
  L.bytes = o;
  return L;
}

hipError_t launch_forward(const int32_t* ids, const int32_t* cu_len, const int32_t* cand,
                          const int32_t* cand_len, const uint8_t* copy_gate, const void* embed,
                          const FwdLayer* layers, int n_layers, const void* final_norm,
                          const void* lm_head, int B, int W, int D, int Hq, int Hkv, int d,
                          int inter, int V, float rope_base, float eps, const FwdLayout& L,
                          void* ws, int32_t* argmax_out, float* x_out, hipEvent_t ev_begin,
                          hipEvent_t ev_end, hipStream_t s) {
  const int R = 1 + W * D, rows = B * R, hid = Hq * d, WD = W * D;
  char* w = static_cast<char*>(ws);
  void* lmws = w + L.off_lm;
  float* ws_attn = reinterpret_cast<float*>(w + L.off_attn);
  float* x = x_out ? x_out : reinterpret_cast<float*>(w + L.off_x);
  auto* hb = reinterpret_cast<uint16_t*>(w + L.off_h);
  auto* qb = reinterpret_cast<uint16_t*>(w + L.off_q);
  auto* kc = reinterpret_cast<uint16_t*>(w + L.off_kc);
  auto* vc = reinterpret_cast<uint16_t*>(w + L.off_vc);
  auto* att = reinterpret_cast<uint16_t*>(w + L.off_att);
  auto* ab = reinterpret_cast<uint16_t*>(w + L.off_a);
  auto* part = reinterpret_cast<float*>(w + L.off_part);
  const LmWsView lv = lm_ws_view(lmws, rows);
  if (ev_begin && hipEventRecord(ev_begin, s) != hipSuccess) return hipErrorInvalidValue;
  hipError_t e = launch_compact_rows(lmws, rows, R, W, D, cand_len, copy_gate, s);
  if (e != hipSuccess) return e;
  // q of rows that are not real and candidate keys / values past L_w are read by
  // the attention but never written by the layers: start them at zero
  hipLaunchKernelGGL(fwd_zero_kernel, dim3(256), dim3(256), 0, s, reinterpret_cast<uint32_t*>(qb),
                     static_cast<size_t>(rows) * Hq * d / 2);
  hipLaunchKernelGGL(fwd_zero_kernel, dim3(256), dim3(256), 0, s, reinterpret_cast<uint32_t*>(kc),
                     static_cast<size_t>(B) * WD * Hkv * d / 2);
  hipLaunchKernelGGL(fwd_zero_kernel, dim3(256), dim3(256), 0, s, reinterpret_cast<uint32_t*>(vc),
                     static_cast<size_t>(B) * WD * Hkv * d / 2);
  if (x_out)
    hipLaunchKernelGGL(fwd_zero_kernel, dim3(256), dim3(256), 0, s, reinterpret_cast<uint32_t*>(x),
                       static_cast<size_t>(rows) * hid);
  const uint16_t* g0 = static_cast<const uint16_t*>(n_layers > 0 ? layers[0].attn_norm : final_norm);
  hipLaunchKernelGGL(fwd_embed_kernel, dim3(rows), dim3(kFwThreads), 0, s, ids, cu_len, cand,
                     static_cast<const uint16_t*>(embed), V, R, WD, hid, lv.row_list, lv.n_rows, g0,
                     eps, x, hb);
  const double log2_base = log2(static_cast<double>(rope_base));
  // x += the split partials of the last projection, then h = RMSNorm(x) g
  auto residual_finish = [&](int splits, const uint16_t* g) {
    hipLaunchKernelGGL(fwd_residual_norm_kernel, dim3(rows), dim3(kRnThreads), 0, s, part, splits,
                       rows, hid, lv.row_list, lv.n_rows, g, eps, x, hb);
  };
  const float scale = 1.0f / sqrtf(static_cast<float>(d));
  for (int l = 0; l < n_layers; ++l) {
    const FwdLayer& ly = layers[l];
    e = launch_gemm(hb, ly.wqkv, rows, hid, (Hq + 2 * Hkv) * d, L.p_qkv, L.s_qkv, false, lmws, part,
                    nullptr, (Hq + 2 * Hkv) * d, s);
    if (e != hipSuccess) return e;
    const int nqkv = (Hq + 2 * Hkv) * d;
    hipLaunchKernelGGL(fwd_qkv_finish_kernel, dim3(rows, (nqkv / 2 + kFwThreads - 1) / kFwThreads),
                       dim3(kFwThreads), 0, s, part, L.s_qkv, rows, Hq, Hkv, d, cu_len, R, D, WD,
                       log2_base, lv.row_list, lv.n_rows, qb, kc, vc);
    e = launch_attention(qb, ly.k_cache, ly.v_cache, cu_len, kc, vc, cand_len, copy_gate, B, W, D, Hq,
                         Hkv, d, true, scale, L.attn, att, ws_attn, s);
    if (e != hipSuccess) return e;
    e = launch_gemm(att, ly.wo, rows, hid, hid, L.p_o, L.s_o, false, lmws, part, nullptr, hid, s);
    if (e != hipSuccess) return e;
    residual_finish(L.s_o, static_cast<const uint16_t*>(ly.mlp_norm));
    if (L.s_gu > 1) {  // split-K: gate and up partials, then silu(gate) * up
      e = launch_gemm_pair(hb, ly.w_gate_up, rows, hid, inter, L.p_gu, L.s_gu, lmws, part, s);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(fwd_swiglu_finish_kernel, dim3(rows, (inter / 4 + kFwThreads - 1) / kFwThreads),
                         dim3(kFwThreads), 0, s, part, L.s_gu, rows, inter, lv.row_list, lv.n_rows, ab);
    } else {  // enough workgroups without splitting: silu(gate) * up in the epilogue
      e = launch_gemm(hb, ly.w_gate_up, rows, hid, inter, L.p_gu, 1, true, lmws, nullptr, ab, inter, s);
      if (e != hipSuccess) return e;
    }
    e = launch_gemm(ab, ly.w_down, rows, inter, hid, L.p_down, L.s_down, false, lmws, part, nullptr,
                    hid, s);
    if (e != hipSuccess) return e;
    const uint16_t* gn = static_cast<const uint16_t*>(l + 1 < n_layers ? layers[l + 1].attn_norm : final_norm);
    residual_finish(L.s_down, gn);
  }
  e = launch_lmhead(hb, lm_head, rows, hid, V, true, L.lm, nullptr, lmws, nullptr, nullptr, s);
  if (e != hipSuccess) return e;
  e = launch_argmax_finish(lmws, B, R, argmax_out, nullptr, s);
  if (e == hipSuccess && ev_end && hipEventRecord(ev_end, s) != hipSuccess) return hipErrorInvalidValue;
  return e;
}

}  // namespace ssd
