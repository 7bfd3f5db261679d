// LM-head projection + greedy argmax for every verification row (SwitchSD
// paper §3.3: one target forward pass verifies all candidates; write-up §3.1:
// T = 0, so each row's verdict is the argmax of its logits).
//
// logits[row][v] = sum_k O[row][k] * lm_head[v][k].  The weight matrix (V x hid,
// K-contiguous) is the dominant HBM stream, so each workgroup owns a 256-wide
// vocabulary tile and streams it exactly once while every row of the row chunk
// (up to 224 rows, the whole verify batch of one sequence) is multiplied
// against it: the rows are the MFMA N dimension (B operand, staged in LDS),
// the vocabulary is the M dimension (A operand, loaded straight from HBM into
// registers one k-step ahead).  The epilogue reduces each row over the tile to
// a (max, lowest index) pair without writing logits; a second tiny kernel
// reduces the tiles.  An fp32 variant on the vector ALU serves fp32 inputs.
#include <limits.h>

#include "common.h"
#include "kernels.h"

namespace ssd {

constexpr int kLmVT = 256;               // vocabulary per workgroup (4 waves x 64)
constexpr int kLmMC = 224;               // rows per chunk (7 MFMA tiles of 32)
constexpr int kLmMT = kLmMC / 32;        // row tiles
constexpr int kLmKS = 64;                // k per iteration (4 MFMA k-steps)
constexpr int kLmOStride = kLmKS + 8;    // bf16 per LDS row (144 B)
constexpr int kLmOChunks = kLmMC * (kLmKS / 8);  // 16-byte chunks per O stage (1792)
constexpr int kLmOPer = kLmOChunks / 256;        // per thread (7)

__global__ __launch_bounds__(256, 1) void lmhead_bf16_kernel(
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ Wt, int rows, int K, int V,
    float* __restrict__ logits_out, int2* __restrict__ part, int vtiles) {
  __shared__ __attribute__((aligned(16))) uint16_t o_lds[2][kLmMC * kLmOStride];
  __shared__ float red_v[4][kLmMC];
  __shared__ int red_i[4][kLmMC];

  const int mc = blockIdx.x;            // row chunk varies fastest: chunks of one tile run together
  const int vt = blockIdx.y;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int h = lane >> 5, l32 = lane & 31;
  const int row0 = mc * kLmMC;
  const int vbase = vt * kLmVT + wave * 64;

  // A operand rows (vocabulary) of this lane; out-of-range rows read row V-1
  const uint16_t* ap[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    int v = vbase + a * 32 + l32;
    v = v < V ? v : V - 1;
    ap[a] = Wt + static_cast<size_t>(v) * K + 8 * h;
  }

  f32x16 acc[2][kLmMT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < kLmMT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][t][r] = 0.f;

  uint4 afrag[2][4], anext[2][4], ostage[kLmOPer];
  auto load_a = [&](uint4 (&dst)[2][4], int kk) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int s = 0; s < 4; ++s) dst[a][s] = *reinterpret_cast<const uint4*>(ap[a] + kk + 16 * s);
  };
  auto load_o = [&](int kk) {
#pragma unroll
    for (int c = 0; c < kLmOPer; ++c) {
      const int idx = tid + c * 256;
      const int rr = idx >> 3, part8 = idx & 7;
      const int row = row0 + rr;
      ostage[c] = row < rows ? *reinterpret_cast<const uint4*>(O + static_cast<size_t>(row) * K + kk + part8 * 8)
                             : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_o = [&](int buf) {
#pragma unroll
    for (int c = 0; c < kLmOPer; ++c) {
      const int idx = tid + c * 256;
      const int rr = idx >> 3, part8 = idx & 7;
      *reinterpret_cast<uint4*>(&o_lds[buf][rr * kLmOStride + part8 * 8]) = ostage[c];
    }
  };

  const int nit = K / kLmKS;
  load_o(0);
  store_o(0);
  load_a(afrag, 0);
  for (int it = 0; it < nit; ++it) {
    const int buf = it & 1;
    __syncthreads();
    const bool more = it + 1 < nit;
    if (more) {
      load_a(anext, (it + 1) * kLmKS);
      load_o((it + 1) * kLmKS);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int t = 0; t < kLmMT; ++t) {
        const uint4 u = *reinterpret_cast<const uint4*>(&o_lds[buf][(t * 32 + l32) * kLmOStride + 16 * s + 8 * h]);
        const bf16x8 bfr = __builtin_bit_cast(bf16x8, u);
#pragma unroll
        for (int a = 0; a < 2; ++a)
          acc[a][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, afrag[a][s]), bfr,
                                                              acc[a][t], 0, 0, 0);
      }
    }
    if (more) {
      store_o(buf ^ 1);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int s = 0; s < 4; ++s) afrag[a][s] = anext[a][s];
    }
  }

  // epilogue: per row (this lane's column l32 of each row tile) best over the tile
#pragma unroll
  for (int t = 0; t < kLmMT; ++t) {
    const int row = row0 + t * 32 + l32;
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = vbase + a * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const float x = acc[a][t][r];
        if (v < V && better(x, v, bv, bi)) { bv = x; bi = v; }
        if (logits_out && v < V && row < rows) logits_out[static_cast<size_t>(row) * V + v] = x;
      }
    const float ov = __shfl_xor(bv, 32, kWave);
    const int oi = __shfl_xor(bi, 32, kWave);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    if (h == 0) {
      red_v[wave][t * 32 + l32] = bv;
      red_i[wave][t * 32 + l32] = bi;
    }
  }
  __syncthreads();
  for (int i = tid; i < kLmMC; i += 256) {
    const int row = row0 + i;
    if (row >= rows) continue;
    float bv = red_v[0][i];
    int bi = red_i[0][i];
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (better(red_v[w][i], red_i[w][i], bv, bi)) { bv = red_v[w][i]; bi = red_i[w][i]; }
    part[static_cast<size_t>(vt) * rows + row] = make_int2(__float_as_int(bv), bi);
  }
}

// fp32: thread per vocabulary column, 32 rows per workgroup, O staged in LDS.
constexpr int kLmF32Rows = 32;
__global__ __launch_bounds__(256) void lmhead_f32_kernel(
    const float* __restrict__ O, const float* __restrict__ Wt, int rows, int K, int V,
    float* __restrict__ logits_out, int2* __restrict__ part, int vtiles) {
  __shared__ float o_lds[kLmF32Rows][64];
  __shared__ float red_v[4][kLmF32Rows];
  __shared__ int red_i[4][kLmF32Rows];
  const int mc = blockIdx.x, vt = blockIdx.y;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int row0 = mc * kLmF32Rows;
  const int v = vt * 256 + tid;
  const float* wr = Wt + static_cast<size_t>(v < V ? v : V - 1) * K;
  float acc[kLmF32Rows];
#pragma unroll
  for (int i = 0; i < kLmF32Rows; ++i) acc[i] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 64) {
    const int kc = min(64, K - k0);
    __syncthreads();
    for (int e = tid; e < kLmF32Rows * 64; e += 256) {
      const int rr = e / 64, kk = e % 64;
      const int row = row0 + rr;
      o_lds[rr][kk] = (row < rows && kk < kc) ? O[static_cast<size_t>(row) * K + k0 + kk] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < kc; ++kk) {
      const float wv = wr[k0 + kk];
#pragma unroll
      for (int i = 0; i < kLmF32Rows; ++i) acc[i] += o_lds[i][kk] * wv;
    }
  }
#pragma unroll
  for (int i = 0; i < kLmF32Rows; ++i) {
    const int row = row0 + i;
    if (logits_out && v < V && row < rows) logits_out[static_cast<size_t>(row) * V + v] = acc[i];
    float bv = v < V ? acc[i] : -INFINITY;
    int bi = v < V ? v : INT_MAX;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) {
      red_v[wave][i] = bv;
      red_i[wave][i] = bi;
    }
  }
  __syncthreads();
  if (tid < kLmF32Rows) {
    const int row = row0 + tid;
    if (row < rows) {
      float bv = red_v[0][tid];
      int bi = red_i[0][tid];
      for (int w = 1; w < 4; ++w)
        if (better(red_v[w][tid], red_i[w][tid], bv, bi)) { bv = red_v[w][tid]; bi = red_i[w][tid]; }
      part[static_cast<size_t>(vt) * rows + row] = make_int2(__float_as_int(bv), bi);
    }
  }
}

__global__ __launch_bounds__(256) void argmax_reduce_kernel(
    const int2* __restrict__ part, int vtiles, int rows, int R, int W, int D,
    const int32_t* __restrict__ cand_len, const uint8_t* __restrict__ copy_gate,
    int32_t* __restrict__ argmax_out) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int b = row / R, r = row - b * R;
  if (!real_row(r, D, cand_len + static_cast<size_t>(b) * W, copy_gate[b] != 0)) {
    argmax_out[row] = -1;
    return;
  }
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int t = 0; t < vtiles; ++t) {
    const int2 p = part[static_cast<size_t>(t) * rows + row];
    const float v = __int_as_float(p.x);
    if (better(v, p.y, bv, bi)) { bv = v; bi = p.y; }
  }
  argmax_out[row] = bi;
}

LmPlan lm_plan(int rows, int V, bool bf16) {
  LmPlan p;
  p.vtiles = (V + 255) / 256;
  p.mchunks = bf16 ? (rows + kLmMC - 1) / kLmMC : (rows + kLmF32Rows - 1) / kLmF32Rows;
  return p;
}

size_t lm_workspace_bytes(const LmPlan& p, int rows) {
  return static_cast<size_t>(p.vtiles) * rows * sizeof(int2);
}

hipError_t launch_lmhead(const void* attn_out, const void* lm_head, int rows, int hid, int V,
                         bool bf16, const LmPlan& plan, float* logits_out, void* ws,
                         hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t s) {
  int2* part = static_cast<int2*>(ws);
  if (ev_begin && hipEventRecord(ev_begin, s) != hipSuccess) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(lmhead_bf16_kernel, dim3(plan.mchunks, plan.vtiles), dim3(256), 0, s,
                       static_cast<const uint16_t*>(attn_out), static_cast<const uint16_t*>(lm_head),
                       rows, hid, V, logits_out, part, plan.vtiles);
  else
    hipLaunchKernelGGL(lmhead_f32_kernel, dim3(plan.mchunks, plan.vtiles), dim3(256), 0, s,
                       static_cast<const float*>(attn_out), static_cast<const float*>(lm_head), rows,
                       hid, V, logits_out, part, plan.vtiles);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev_end && hipEventRecord(ev_end, s) != hipSuccess) return hipErrorInvalidValue;
  return e;
}

hipError_t launch_argmax_reduce(const void* ws, const LmPlan& plan, int rows, int R, int W, int D,
                                const int32_t* cand_len, const uint8_t* copy_gate,
                                int32_t* argmax_out, hipStream_t s) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3((rows + 255) / 256), dim3(256), 0, s,
                     static_cast<const int2*>(ws), plan.vtiles, rows, R, W, D, cand_len, copy_gate,
                     argmax_out);
  return hipGetLastError();
}

}  // namespace ssd
