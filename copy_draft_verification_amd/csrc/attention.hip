// Block-triangular verification attention (SwitchSD paper §3.3 "Parallel
// Verification with Block-Triangular Attention"; write-up §2.6).
//
// Every query row of a sequence sees the whole prefix; row (w, j) additionally
// sees candidate keys (w, 0..j).  The pass is split accordingly:
//   1. prefix sweep: a dense, unmasked attention of all real rows against the
//      prefix K/V, split over key ranges (flash-decoding style partials m, l, o
//      in the exp2 domain).  bf16 runs on 32x32x16 MFMA with the g query heads
//      of one KV head packed into the M dimension (g*R rows share one K/V
//      stream); fp32 runs on the vector ALU.
//   2. merge: per (row, head) the split partials are combined and the row's own
//      candidate triangle (at most D keys) is folded in exactly, then the
//      normalised output is written.  Rows that are not real are written as 0.
// No mask is ever materialised: the candidate triangle lives only in the
// merge's loop bound j.
#include "common.h"
#include "kernels.h"

namespace ssd {

// ----------------------------------------------------------------- bf16 MFMA
constexpr int kAttD = 128;          // head dim of the MFMA path
constexpr int kKB = 64;             // keys per LDS block
constexpr int kKStride = kAttD + 8; // bf16 per K row in LDS (272 B: conflict-free b128 reads)
constexpr int kVtStride = kKB + 4;  // bf16 per V^T row in LDS (136 B: conflict-free b64 reads)
constexpr int kAttRowsPerBlock = 128;

__global__ __launch_bounds__(256, 2) void attn_prefix_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pre,
    const uint16_t* __restrict__ v_pre, const int32_t* __restrict__ cu_len,
    const uint8_t* __restrict__ copy_gate, int B, int R, int Hq, int Hkv, int nsplit, int chunk,
    float scale_log2, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kKB * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[kAttD * kVtStride];

  const int qtile = blockIdx.x;
  const int b = blockIdx.y / Hkv, kvh = blockIdx.y - b * Hkv;
  const int split = blockIdx.z;
  if (copy_gate[b] == 0) return;
  const int base = cu_len[b];
  const int n_b = cu_len[b + 1] - base;
  const int k0 = split * chunk;
  if (k0 >= n_b) return;
  const int k1 = split == nsplit - 1 ? n_b : min(k0 + chunk, n_b);

  const int g = Hq / Hkv, G = R * g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int h = lane >> 5, l32 = lane & 31;
  const int i_row = qtile * kAttRowsPerBlock + wave * 32 + l32;  // this lane's query row (B operand column)
  const bool row_ok = i_row < G;
  const int r_row = row_ok ? i_row / g : 0, hh = row_ok ? i_row - (i_row / g) * g : 0;

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[row][16s + 8h .. +7]
  bf16x8 qf[8];
  {
    const uint16_t* qp = q + ((static_cast<size_t>(b) * R + r_row) * Hq + kvh * g + hh) * kAttD + 8 * h;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qp + 16 * s) : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8, u);
    }
  }

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // staging registers for the next K / V block
  uint4 kreg[4], vreg[4];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = tid + c * 256;          // 1024 chunks of 16 B
      const int key = idx >> 4, part = idx & 15;
      const int t = kb + key;
      kreg[c] = t < k1 ? *reinterpret_cast<const uint4*>(
                             k_pre + ((static_cast<size_t>(base) + t) * Hkv + kvh) * kAttD + part * 8)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = tid + c * 256;          // 512 (key pair, d chunk) items
      const int kp = idx >> 4, dc = idx & 15;
      const int t0 = kb + 2 * kp;
      vreg[2 * c] = t0 < k1 ? *reinterpret_cast<const uint4*>(
                                  v_pre + ((static_cast<size_t>(base) + t0) * Hkv + kvh) * kAttD + dc * 8)
                            : make_uint4(0, 0, 0, 0);
      vreg[2 * c + 1] = t0 + 1 < k1 ? *reinterpret_cast<const uint4*>(
                                          v_pre + ((static_cast<size_t>(base) + t0 + 1) * Hkv + kvh) * kAttD + dc * 8)
                                    : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = tid + c * 256;
      const int key = idx >> 4, part = idx & 15;
      *reinterpret_cast<uint4*>(&k_lds[key * kKStride + part * 8]) = kreg[c];
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = tid + c * 256;
      const int kp = idx >> 4, dc = idx & 15;
      const uint32_t* a = reinterpret_cast<const uint32_t*>(&vreg[2 * c]);
      const uint32_t* bb = reinterpret_cast<const uint32_t*>(&vreg[2 * c + 1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // d = dc*8 + 2e (low halves) and dc*8 + 2e + 1 (high halves)
        const uint32_t lo = (a[e] & 0xffffu) | (bb[e] << 16);
        const uint32_t hi = (a[e] >> 16) | (bb[e] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(&vt_lds[(dc * 8 + 2 * e) * kVtStride + 2 * kp]) = lo;
        *reinterpret_cast<uint32_t*>(&vt_lds[(dc * 8 + 2 * e + 1) * kVtStride + 2 * kp]) = hi;
      }
    }
  };

  load_block(k0);
  for (int kb = k0; kb < k1; kb += kKB) {
    __syncthreads();
    store_block();
    __syncthreads();
    if (kb + kKB < k1) load_block(kb + kKB);

    // S^T[key][row] for two 32-key subtiles
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4 u = *reinterpret_cast<const uint4*>(&k_lds[(kt * 32 + l32) * kKStride + 16 * s + 8 * h]);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), qf[s], sacc[kt], 0, 0, 0);
      }
    }
    // online softmax over this block (exp2 domain); lanes l and l^32 share a row
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + kt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const float sv = key < k1 ? sacc[kt][r] * scale_log2 : -INFINITY;
        sacc[kt][r] = sv;
        mloc = fmaxf(mloc, sv);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[kt][8 * s2 + e] - m_new);
          psum += p;
          pf[kt][s2][e] = static_cast<__bf16>(p);
        }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    // O^T[d][row] += V^T[d][keys] P^T[keys][row]; key order of a P fragment element e
    // for lane half h: kt*32 + 16*s2 + 8*(e/4) + 4*h + e%4 (the S^T output layout)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const uint16_t* vr = &vt_lds[(dt * 32 + l32) * kVtStride + kt * 32 + 16 * s2 + 4 * h];
          const uint2 lo = *reinterpret_cast<const uint2*>(vr);
          const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
          const uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), pf[kt][s2], oacc[dt], 0, 0, 0);
        }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (!row_ok) return;
  const size_t po = ((static_cast<size_t>(split) * B + b) * R + r_row) * Hq + kvh * g + hh;
  if (h == 0) {
    ws_m[po] = m_run;
    ws_l[po] = l_tot;
  }
  float* op = ws_o + po * kAttD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = dt * 32 + 8 * rq + 4 * h;
      *reinterpret_cast<float4*>(op + d0) =
          make_float4(oacc[dt][4 * rq], oacc[dt][4 * rq + 1], oacc[dt][4 * rq + 2], oacc[dt][4 * rq + 3]);
    }
}

// ----------------------------------------------------------------- fp32 VALU
// One wavefront per (row, head); lanes hold d/64 output elements each.
template <int DPL>
__global__ __launch_bounds__(256) void attn_prefix_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k_pre, const float* __restrict__ v_pre,
    const int32_t* __restrict__ cu_len, const uint8_t* __restrict__ copy_gate,
    const int32_t* __restrict__ cand_len, int B, int R, int Hq, int Hkv, int W, int D, int nsplit,
    int chunk, float scale_log2, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o) {
  constexpr int d = DPL * kWave;
  const int b = blockIdx.y, split = blockIdx.z;
  const int rh = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (rh >= R * Hq || copy_gate[b] == 0) return;
  const int r = rh / Hq, hq = rh - r * Hq;
  if (!real_row(r, D, cand_len + static_cast<size_t>(b) * W, true)) return;
  const int base = cu_len[b];
  const int n_b = cu_len[b + 1] - base;
  const int k0 = split * chunk;
  if (k0 >= n_b) return;
  const int k1 = split == nsplit - 1 ? n_b : min(k0 + chunk, n_b);
  const int kv = hq / (Hq / Hkv);
  float qv[DPL], o[DPL];
  const float* qp = q + ((static_cast<size_t>(b) * R + r) * Hq + hq) * d;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    qv[e] = qp[lane + kWave * e];
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int t = k0; t < k1; ++t) {
    const size_t kvo = ((static_cast<size_t>(base) + t) * Hkv + kv) * d;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) part += qv[e] * k_pre[kvo + lane + kWave * e];
    const float s = wave_sum(part) * scale_log2;
    const float m_new = fmaxf(m, s);
    const float a = exp2f(m - m_new), p = exp2f(s - m_new);
    l = l * a + p;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = o[e] * a + p * v_pre[kvo + lane + kWave * e];
    m = m_new;
  }
  const size_t po = ((static_cast<size_t>(split) * B + b) * R + r) * Hq + hq;
  if (lane == 0) {
    ws_m[po] = m;
    ws_l[po] = l;
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) ws_o[po * d + lane + kWave * e] = o[e];
}

// ----------------------------------------------------------------- merge + triangle
template <typename T, int DPL>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cand, const T* __restrict__ v_cand,
    const int32_t* __restrict__ cu_len, const int32_t* __restrict__ cand_len,
    const uint8_t* __restrict__ copy_gate, int B, int R, int Hq, int Hkv, int W, int D, int nsplit,
    int chunk, float scale_log2, const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o, T* __restrict__ out) {
  constexpr int d = DPL * kWave;
  const size_t item = static_cast<size_t>(blockIdx.x) * 4 + threadIdx.x / kWave;  // (b, r, hq)
  const int lane = threadIdx.x & (kWave - 1);
  if (item >= static_cast<size_t>(B) * R * Hq) return;
  const int hq = static_cast<int>(item % Hq);
  const int r = static_cast<int>((item / Hq) % R);
  const int b = static_cast<int>(item / (static_cast<size_t>(Hq) * R));
  T* op = out + item * d;  // out[b][r][hq*d + ...] == out + ((b*R + r)*Hq + hq)*d
  if (!real_row(r, D, cand_len + static_cast<size_t>(b) * W, copy_gate[b] != 0)) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) store_f32(op, lane + kWave * e, 0.f);
    return;
  }
  const int n_b = cu_len[b + 1] - cu_len[b];
  const int nsp = min(nsplit, (n_b + chunk - 1) / chunk);
  float M = -INFINITY;
  for (int s = 0; s < nsp; ++s)
    M = fmaxf(M, ws_m[((static_cast<size_t>(s) * B + b) * R + r) * Hq + hq]);
  float L = 0.f, o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  for (int s = 0; s < nsp; ++s) {
    const size_t po = ((static_cast<size_t>(s) * B + b) * R + r) * Hq + hq;
    const float f = __builtin_amdgcn_exp2f(ws_m[po] - M);
    L += f * ws_l[po];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] += f * ws_o[po * d + lane + kWave * e];
  }
  if (r > 0) {
    // own-candidate triangle: keys (w, 0..j)
    const int w = (r - 1) / D, j = (r - 1) - w * D;
    const int kv = hq / (Hq / Hkv);
    float qv[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) qv[e] = load_f32(q, item * d + lane + kWave * e);
    for (int jj = 0; jj <= j; ++jj) {
      const size_t kvo = ((static_cast<size_t>(b) * W * D + w * D + jj) * Hkv + kv) * d;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) part += qv[e] * load_f32(k_cand, kvo + lane + kWave * e);
      const float sc = wave_sum(part) * scale_log2;
      const float m_new = fmaxf(M, sc);
      const float a = exp2f(M - m_new), p = exp2f(sc - m_new);
      L = L * a + p;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = o[e] * a + p * load_f32(v_cand, kvo + lane + kWave * e);
      M = m_new;
    }
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int e = 0; e < DPL; ++e) store_f32(op, lane + kWave * e, o[e] * inv);
}

// ----------------------------------------------------------------- host side
AttnPlan attn_plan(int B, int max_n, int R, int Hq, int Hkv, bool bf16) {
  AttnPlan p;
  const int g = Hq / Hkv;
  int units, min_keys, target;
  if (bf16) {
    p.qtiles = (R * g + kAttRowsPerBlock - 1) / kAttRowsPerBlock;
    units = B * Hkv * p.qtiles;
    min_keys = 512;
    target = 512;
  } else {
    p.qtiles = (R * Hq + 3) / 4;
    units = B * p.qtiles;
    min_keys = 256;
    target = 1024;
  }
  int ns = (target + units - 1) / units;
  int cap = max_n / min_keys;
  if (cap < 1) cap = 1;
  if (ns > cap) ns = cap;
  if (ns < 1) ns = 1;
  int ch = (max_n + ns - 1) / ns;
  ch = (ch + kKB - 1) / kKB * kKB;
  if (ch < kKB) ch = kKB;
  p.nsplit = ns;
  p.chunk = ch;
  return p;
}

size_t attn_workspace_bytes(const AttnPlan& p, int B, int R, int Hq, int d) {
  const size_t rows = static_cast<size_t>(p.nsplit) * B * R * Hq;
  return rows * sizeof(float) * (2 + static_cast<size_t>(d));
}

hipError_t launch_attention(const void* q, const void* k_pre, const void* v_pre,
                            const int32_t* cu_len, const void* k_cand, const void* v_cand,
                            const int32_t* cand_len, const uint8_t* copy_gate, int B, int W,
                            int D, int Hq, int Hkv, int d, bool bf16, float scale,
                            const AttnPlan& plan, void* attn_out, float* ws, hipStream_t s) {
  const int R = 1 + W * D;
  const size_t rows = static_cast<size_t>(plan.nsplit) * B * R * Hq;
  float* ws_m = ws;
  float* ws_l = ws + rows;
  float* ws_o = ws + 2 * rows;
  const float scale_log2 = scale * kLog2e;
  const size_t items = static_cast<size_t>(B) * R * Hq;
  const dim3 mgrid(static_cast<unsigned>((items + 3) / 4));
  if (bf16) {
    hipLaunchKernelGGL(attn_prefix_bf16_kernel, dim3(plan.qtiles, B * Hkv, plan.nsplit), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_pre),
                       static_cast<const uint16_t*>(v_pre), cu_len, copy_gate, B, R, Hq, Hkv,
                       plan.nsplit, plan.chunk, scale_log2, ws_m, ws_l, ws_o);
    hipLaunchKernelGGL((attn_merge_kernel<uint16_t, 2>), mgrid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cand),
                       static_cast<const uint16_t*>(v_cand), cu_len, cand_len, copy_gate, B, R, Hq,
                       Hkv, W, D, plan.nsplit, plan.chunk, scale_log2, ws_m, ws_l, ws_o,
                       static_cast<uint16_t*>(attn_out));
  } else {
    const dim3 pgrid(plan.qtiles, B, plan.nsplit);
    if (d == 64) {
      hipLaunchKernelGGL(attn_prefix_f32_kernel<1>, pgrid, dim3(256), 0, s,
                         static_cast<const float*>(q), static_cast<const float*>(k_pre),
                         static_cast<const float*>(v_pre), cu_len, copy_gate, cand_len, B, R, Hq,
                         Hkv, W, D, plan.nsplit, plan.chunk, scale_log2, ws_m, ws_l, ws_o);
      hipLaunchKernelGGL((attn_merge_kernel<float, 1>), mgrid, dim3(256), 0, s,
                         static_cast<const float*>(q), static_cast<const float*>(k_cand),
                         static_cast<const float*>(v_cand), cu_len, cand_len, copy_gate, B, R,
                         Hq, Hkv, W, D, plan.nsplit, plan.chunk, scale_log2, ws_m, ws_l, ws_o,
                         static_cast<float*>(attn_out));
    } else {
      hipLaunchKernelGGL(attn_prefix_f32_kernel<2>, pgrid, dim3(256), 0, s,
                         static_cast<const float*>(q), static_cast<const float*>(k_pre),
                         static_cast<const float*>(v_pre), cu_len, copy_gate, cand_len, B, R, Hq,
                         Hkv, W, D, plan.nsplit, plan.chunk, scale_log2, ws_m, ws_l, ws_o);
      hipLaunchKernelGGL((attn_merge_kernel<float, 2>), mgrid, dim3(256), 0, s,
                         static_cast<const float*>(q), static_cast<const float*>(k_cand),
                         static_cast<const float*>(v_cand), cu_len, cand_len, copy_gate, B, R,
                         Hq, Hkv, W, D, plan.nsplit, plan.chunk, scale_log2, ws_m, ws_l, ws_o,
                         static_cast<float*>(attn_out));
    }
  }
  return hipGetLastError();
}

}  // namespace ssd
