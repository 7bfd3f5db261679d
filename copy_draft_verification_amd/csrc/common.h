// Device helpers shared by the gfx950 kernels of the copy-speculation path.
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// A compile-time int as a value (selects unrolled steps and stages).
template <int N> using IntC = std::integral_constant<int, N>;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p, size_t i);
template <> __device__ __forceinline__ float load_f32<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

template <typename T> __device__ __forceinline__ void store_f32(T* p, size_t i, float v);
template <> __device__ __forceinline__ void store_f32<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void store_f32<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = f32_to_bf16(v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Eight consecutive elements of a bf16 (one 16-byte load) or fp32 (two) row.
template <typename T> struct Chunk8;
template <> struct Chunk8<uint16_t> {
  uint4 v;
  __device__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  // Streaming read (nontemporal hint): for data read once, so that it does not
  // displace reused lines in the caches.
  __device__ void load_stream(const uint16_t* p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    v = make_uint4(t.x, t.y, t.z, t.w);
  }
  // Buffer load: an offset past the buffer's size returns zeros.
  template <int kPolicy>
  __device__ void load_buf(__amdgpu_buffer_rsrc_t res, int off) {
    v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(res, off, 0, kPolicy));
  }
  __device__ float at(int e) const {
    const uint32_t w = (&v.x)[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <> struct Chunk8<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ void load_stream(const float* p) {
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
    a = make_float4(x[0], x[1], x[2], x[3]);
    b = make_float4(y[0], y[1], y[2], y[3]);
  }
  template <int kPolicy>
  __device__ void load_buf(__amdgpu_buffer_rsrc_t res, int off) {
    a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(res, off, 0, kPolicy));
    b = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(res, off + 16, 0, kPolicy));
  }
  __device__ float at(int e) const { return e < 4 ? (&a.x)[e] : (&b.x)[e - 4]; }
};

// Philox4x32-10 block function (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): counter (c0..c3), key (k0, k1) -> four
// 32-bit words.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // one 32 x 32 -> 64-bit multiply per product (v_mad_u64_u32) instead of a
    // separate high and low multiply
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
    c0 = static_cast<uint32_t>(p1 >> 32) ^ c1 ^ k0;
    c1 = static_cast<uint32_t>(p1);
    c2 = static_cast<uint32_t>(p0 >> 32) ^ c3 ^ k1;
    c3 = static_cast<uint32_t>(p0);
  }
  return make_uint4(c0, c1, c2, c3);
}

// 32-bit word -> (floor(w / 512) + 1/2) / 2^23, in (0, 1) and exact in binary32.
__device__ __forceinline__ float word_uniform(uint32_t w) {
  return fmaf(static_cast<float>(w >> 9), 0x1p-23f, 0x1p-24f);
}

// Gumbel noise -ln(-ln u) from two hardware base-2 logarithms (v_log_f32):
// with e = -log2 u, -ln(-ln u) = -ln2 * log2(e) - ln(ln 2).  u >= 2^-24 and
// e >= 8.5e-8 are normal floats, so the instruction needs no denormal scaling.
// Measured on every u of the grid, -ln u from v_log_f32 is within 3.2 ulp
// (relative) near u = 1 included, where -ln u is tiny and the noise largest; the
// noise is within a few 1e-7 of the exact value.
__device__ __forceinline__ float gumbel_of(uint32_t w) {
  const float e = -__builtin_amdgcn_logf(word_uniform(w));
  return fmaf(-0.69314718f, __builtin_amdgcn_logf(e), 0.36651292f);
}

// (max, sum of 2^(x - max)) pairs of a base-2 log-sum-exp, merged.
__device__ __forceinline__ void lse2_merge(float& m, float& s, float om, float os) {
  const float nm = fmaxf(m, om);
  if (nm == -INFINITY) return;
  s = (m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f(m - nm)) +
      (om == -INFINITY ? 0.f : os * __builtin_amdgcn_exp2f(om - nm));
  m = nm;
}

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format, no
// swizzle, offset addressing): loads past num_records return zero.
constexpr int kBufFlags = 0x00020000;

// Cache-policy operand of the buffer load builtins: the nontemporal bit, for data
// streamed once from HBM.
constexpr int kNonTemporal = 2;

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory
// operations of this wave are outstanding; the other counters are not waited on.
constexpr int waitcnt_vm(int n) {
  return ((n >> 4) & 3) << 14 | 0xf << 8 | 0x7 << 4 | (n & 0xf);
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also fences global
// memory, which makes the compiler wait for every outstanding global load (the
// register prefetches included) before the barrier; here only LDS operations are
// drained.  The memory clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Maxima of MFMA results without the canonicalising maximum the compiler puts in
// front of every fmaxf input (which doubles a maximum tree).  In IEEE mode
// v_max_f32 / v_max3_f32 return the other operand for a quiet NaN, as fmaxf does;
// callers pass MFMA results or -inf, never signalling NaNs.
__device__ __forceinline__ float vmax2_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// (value, index) order used by every argmax: larger value wins, equal values
// go to the lower index.  NaN never wins.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Is row r (0 <= r < 1 + W*D) of sequence b a real query row?
__device__ __forceinline__ bool real_row(int r, int D, const int32_t* cand_len_b, bool gate) {
  if (!gate) return false;
  if (r == 0) return true;
  int w = (r - 1) / D, j = (r - 1) - w * D;
  int L = cand_len_b[w];
  L = L < 0 ? 0 : (L > D ? D : L);
  return j < L;
}

// Exclusive prefix sum of v over a workgroup of NT threads (NT / 64 waves), in
// thread order; `total` receives the sum.  s_wave holds NT / 64 ints of LDS.
// Contains two workgroup barriers: every thread of the workgroup must call it.
// With kLdsOnly the barriers order LDS only (lds_barrier), so global loads the
// caller has in flight stay in flight across the scan.
template <int NT, bool kLdsOnly = false>
__device__ __forceinline__ int block_excl_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) s_wave[wv] = incl;
  if constexpr (kLdsOnly) lds_barrier(); else __syncthreads();
  int woff = 0, tot = 0;
  for (int i = 0; i < NT / kWave; ++i) {
    const int c = s_wave[i];
    if (i < wv) woff += c;
    tot += c;
  }
  if constexpr (kLdsOnly) lds_barrier(); else __syncthreads();
  total = tot;
  return woff + incl - v;
}

// Compact list of the real verification rows of B*R rows (R per sequence), in row
// order: row_list[k] = k-th real row, inv[row] = its position or -1, *n_rows = the
// count.  Run by every thread of one workgroup of NT threads; s_wave holds NT / 64
// ints of LDS.
// It also zeroes the greedy LM head's per-row argmax keys (keys; may be null).
template <int NT>
__device__ void compact_rows_body(int rows, int R, int W, int D, const int32_t* __restrict__ cand_len,
                                  const uint8_t* __restrict__ copy_gate, int32_t* __restrict__ row_list,
                                  int32_t* __restrict__ inv, int32_t* __restrict__ n_rows, int* s_wave,
                                  unsigned long long* __restrict__ keys) {
  if (keys != nullptr)
    for (int i = static_cast<int>(threadIdx.x); i < rows; i += NT) keys[i] = 0ull;
  int base = 0;
  for (int r0 = 0; r0 < rows; r0 += NT) {
    const int row = r0 + static_cast<int>(threadIdx.x);
    bool real = false;
    if (row < rows) {
      const int b = row / R;
      real = real_row(row - b * R, D, cand_len + static_cast<size_t>(b) * W, copy_gate[b] != 0);
    }
    int total;
    const int pos = base + block_excl_scan<NT>(real ? 1 : 0, s_wave, total);
    if (row < rows) {
      inv[row] = real ? pos : -1;
      if (real) row_list[pos] = row;
    }
    base += total;
  }
  if (threadIdx.x == 0) *n_rows = base;
}

}  // namespace ssd
