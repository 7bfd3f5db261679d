// Offline calibration of the copy-intent probe: copy-mode labels of whole
// contexts, probe logits at every position of every layer, and per layer the
// F1-optimal threshold and the ROC AUC, then the layer choice.
// SwitchSD paper §3.2 "Problem Formulation" (a position is copy-mode when it lies
// in a verbatim run of at least n_train = 5 tokens that occurs earlier) and
// "Layer and Threshold Selection" (layer by F1, threshold by F1); §4.3.3 reports
// the F1-optimal threshold and the AUC.
//
// Labels.  A position is labelled exactly when an n_train-window containing it
// also starts at an earlier position of the same context.  An open-addressing
// table keyed by (context, window) keeps, per distinct window, its first start
// (atomicMin over packed (context << 32 | start), so the result does not depend
// on the order of the inserts); a second pass flags each window whose table
// entry is an earlier start, a third ORs the flags over the n_train windows that
// contain each position.  Every output byte is written exactly once.
//
// Probe logits.  z[l][i] = w_l . H[l][i] is a batched GEMV that streams the
// states once from HBM with nontemporal loads (each state is read once); w_l
// sits in LDS, shared by the 8 waves of a workgroup; one wave reduces one row.
//
// Sweep.  Per layer the (score, label) pairs are sorted by descending score
// (a bitonic network over a power of two of at least 1024 keys, padded with keys
// that sort last: chunks of up to 8192 per workgroup in registers, wave shuffles
// and LDS, longer strides as separate global passes), then one workgroup walks the sorted keys carrying the running
// counts.  At the last element of each group of equal scores it evaluates the
// threshold t = that score (copy predicted when z >= t): TP = positives so far,
// FP = negatives so far.  F1 = 2TP / (2TP + FP + FN) is compared exactly as a
// fraction of integers; a tie keeps the earlier (higher) threshold.  The
// Mann-Whitney statistic 2U adds, per group, p_g * (2 * negatives below + n_g).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace ssd {

// ---------------------------------------------------------------- labels
constexpr int kLbThreads = 256;
constexpr unsigned long long kEmptySlot = ~0ull;

// Context of global position a: the largest b with cu_len[b] <= a.
__device__ __forceinline__ int context_of(const int32_t* __restrict__ cu_len, int B, int a) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_len[mid] <= a) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014) as the mixing step of the window hash.
__device__ __forceinline__ unsigned long long mix64(unsigned long long x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

__device__ __forceinline__ unsigned long long window_hash(const int32_t* __restrict__ ids, int b,
                                                          int a, int n_train) {
  unsigned long long h = mix64(static_cast<unsigned long long>(b) + 0x9e3779b97f4a7c15ull);
  for (int q = 0; q < n_train; ++q) h = mix64(h ^ static_cast<uint32_t>(ids[a + q]));
  return h;
}

// Same context and same n_train tokens?
__device__ __forceinline__ bool same_window(const int32_t* __restrict__ ids, unsigned long long x,
                                            unsigned long long y, int n_train) {
  if ((x >> 32) != (y >> 32)) return false;
  const int ax = static_cast<int>(x & 0xffffffffu), ay = static_cast<int>(y & 0xffffffffu);
  for (int q = 0; q < n_train; ++q)
    if (ids[ax + q] != ids[ay + q]) return false;
  return true;
}

__global__ __launch_bounds__(kLbThreads) void labels_clear_kernel(unsigned long long* table,
                                                                  long long cap) {
  const long long i = static_cast<long long>(blockIdx.x) * kLbThreads + threadIdx.x;
  if (i < cap) table[i] = kEmptySlot;
}

__global__ __launch_bounds__(kLbThreads) void labels_insert_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ cu_len, int B, int total_n,
    int n_train, unsigned long long* __restrict__ table, long long mask) {
  const int a = blockIdx.x * kLbThreads + threadIdx.x;
  if (a >= total_n) return;
  const int b = context_of(cu_len, B, a);
  if (a + n_train > min(cu_len[b + 1], total_n)) return;
  const unsigned long long key = static_cast<unsigned long long>(b) << 32 | static_cast<uint32_t>(a);
  long long slot = static_cast<long long>(window_hash(ids, b, a, n_train) & mask);
  // The table holds at least twice as many slots as windows, so an empty slot is
  // always reached; the bound only guarantees that the loop ends.
  for (long long probe = 0; probe <= mask; ++probe) {
    unsigned long long cur = table[slot];
    if (cur == kEmptySlot) {
      cur = atomicCAS(&table[slot], kEmptySlot, key);
      if (cur == kEmptySlot) return;
    }
    // A slot only ever holds keys of one window, so even a stale read names it.
    if (same_window(ids, cur, key, n_train)) {
      atomicMin(&table[slot], key);
      return;
    }
    slot = (slot + 1) & mask;
  }
}

__global__ __launch_bounds__(kLbThreads) void labels_repeat_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ cu_len, int B, int total_n,
    int n_train, const unsigned long long* __restrict__ table, long long mask,
    uint8_t* __restrict__ repeat) {
  const int a = blockIdx.x * kLbThreads + threadIdx.x;
  if (a >= total_n) return;
  const int b = context_of(cu_len, B, a);
  uint8_t r = 0;
  if (a + n_train <= min(cu_len[b + 1], total_n)) {
    const unsigned long long key = static_cast<unsigned long long>(b) << 32 | static_cast<uint32_t>(a);
    long long slot = static_cast<long long>(window_hash(ids, b, a, n_train) & mask);
    for (long long probe = 0; probe <= mask; ++probe) {
      const unsigned long long cur = table[slot];
      if (cur == kEmptySlot) break;   // unreachable: every window was inserted
      if (same_window(ids, cur, key, n_train)) {
        r = static_cast<int>(cur & 0xffffffffu) < a ? 1 : 0;
        break;
      }
      slot = (slot + 1) & mask;
    }
  }
  repeat[a] = r;
}

__global__ __launch_bounds__(kLbThreads) void labels_mark_kernel(
    const int32_t* __restrict__ cu_len, int B, int total_n, int n_train,
    const uint8_t* __restrict__ repeat, uint8_t* __restrict__ labels) {
  const int i = blockIdx.x * kLbThreads + threadIdx.x;
  if (i >= total_n) return;
  const int b = context_of(cu_len, B, i);
  const int lo = max(cu_len[b], i - n_train + 1);
  uint8_t v = 0;
  for (int a = lo; a <= i; ++a) v |= repeat[a];
  labels[i] = v;
}

long long label_table_slots(long long total_n) {
  long long cap = 256;
  while (cap < 2 * total_n) cap <<= 1;
  return cap;
}

size_t labels_workspace_bytes(long long total_n) {
  const size_t table = static_cast<size_t>(label_table_slots(total_n)) * 8;
  return table + (static_cast<size_t>(total_n) + 255) / 256 * 256;
}

hipError_t launch_copy_labels(const int32_t* ids, const int32_t* cu_len, int B, int total_n,
                              int n_train, uint8_t* labels, void* ws, hipStream_t s) {
  const long long cap = label_table_slots(total_n);
  auto* table = static_cast<unsigned long long*>(ws);
  auto* repeat = reinterpret_cast<uint8_t*>(table + cap);
  const int grid = (total_n + kLbThreads - 1) / kLbThreads;
  hipLaunchKernelGGL(labels_clear_kernel, dim3(static_cast<unsigned>((cap + kLbThreads - 1) / kLbThreads)),
                     dim3(kLbThreads), 0, s, table, cap);
  hipLaunchKernelGGL(labels_insert_kernel, dim3(grid), dim3(kLbThreads), 0, s, ids, cu_len, B,
                     total_n, n_train, table, cap - 1);
  hipLaunchKernelGGL(labels_repeat_kernel, dim3(grid), dim3(kLbThreads), 0, s, ids, cu_len, B,
                     total_n, n_train, table, cap - 1, repeat);
  hipLaunchKernelGGL(labels_mark_kernel, dim3(grid), dim3(kLbThreads), 0, s, cu_len, B, total_n,
                     n_train, repeat, labels);
  return hipGetLastError();
}

// ---------------------------------------------------------------- probe logits
constexpr int kPlThreads = 512;
constexpr int kPlRowsPerWave = 16;
constexpr int kPlRows = kPlRowsPerWave * (kPlThreads / kWave);   // rows per workgroup
constexpr int kPlUnroll = 8;                                     // 16-byte loads in flight per lane
constexpr int kPlFastHid = kWave * kPlUnroll * 8;                // widest row of one round of loads

template <typename T>
__global__ __launch_bounds__(kPlThreads) void probe_logits_kernel(const T* __restrict__ h,
                                                                  const float* __restrict__ w,
                                                                  long long N, int hid,
                                                                  float* __restrict__ z) {
  extern __shared__ __align__(16) float s_w[];
  const int l = blockIdx.y;
  const float* wl = w + static_cast<size_t>(l) * hid;
  // zero past hid up to kPlFastHid, so that the lanes of the fast path that load
  // past a row (zeros) add exactly 0
  for (int k = threadIdx.x; k < max(hid, kPlFastHid); k += kPlThreads) s_w[k] = k < hid ? wl[k] : 0.f;
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const T* hl = h + static_cast<size_t>(l) * N * hid;
  if ((hid & 7) == 0 && hid <= kPlFastHid) {
    // A row is one round of loads: the next row's loads are issued before this
    // row's FMAs, so each wave keeps a row in flight while it computes.  Each row
    // is read as a buffer of hid elements: every lane issues all kPlUnroll loads,
    // those past the row return zeros, and no load sits behind a lane-dependent
    // branch (which would make the compiler wait for every load in flight
    // before any FMA).
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    auto row_u = [&](int m) {
      return static_cast<long long>(blockIdx.x) * kPlRows + m * (kPlThreads / kWave) + wvu;
    };
    // Row r >= N (there is no next row) is issued too, as a buffer of size 0:
    // its loads return zeros without touching memory, and every row is followed
    // by the same number of loads, so the compiler's wait before the FMAs
    // leaves the next row's loads in flight.
    auto load_row = [&](Chunk8<T> (&dst)[kPlUnroll], long long r) {
      const bool ok = r < N;
      const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<T*>(hl + (ok ? static_cast<size_t>(r) * hid : 0)), 0,
          ok ? hid * static_cast<int>(sizeof(T)) : 0, kBufFlags);
#pragma unroll
      for (int u = 0; u < kPlUnroll; ++u)
        dst[u].template load_buf<kNonTemporal>(res, (u * kWave + lane) * 8 * static_cast<int>(sizeof(T)));
    };
    // Row m computes from one buffer while row m+1 loads into the other; the
    // loop is unrolled by two so that the buffers swap roles without a copy (a
    // register copy would wait for the loads in flight).
    auto row = [&](int m, const Chunk8<T> (&cur)[kPlUnroll], Chunk8<T> (&nxt)[kPlUnroll]) -> bool {
      const long long r = row_u(m);
      if (r >= N) return false;
      load_row(nxt, m + 1 < kPlRowsPerWave ? row_u(m + 1) : N);
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < kPlUnroll; ++u) {
        const int c = u * kWave + lane;
        const float4 w0 = reinterpret_cast<const float4*>(s_w)[2 * c];
        const float4 w1 = reinterpret_cast<const float4*>(s_w)[2 * c + 1];
        acc = fmaf(w0.x, cur[u].at(0), acc);
        acc = fmaf(w0.y, cur[u].at(1), acc);
        acc = fmaf(w0.z, cur[u].at(2), acc);
        acc = fmaf(w0.w, cur[u].at(3), acc);
        acc = fmaf(w1.x, cur[u].at(4), acc);
        acc = fmaf(w1.y, cur[u].at(5), acc);
        acc = fmaf(w1.z, cur[u].at(6), acc);
        acc = fmaf(w1.w, cur[u].at(7), acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) z[static_cast<size_t>(l) * N + r] = acc;
      return true;
    };
    static_assert(kPlRowsPerWave % 2 == 0, "rows come in pairs");
    Chunk8<T> b0[kPlUnroll], b1[kPlUnroll];
    load_row(b0, row_u(0));
    for (int m = 0; m < kPlRowsPerWave; m += 2) {
      if (!row(m, b0, b1)) break;
      if (!row(m + 1, b1, b0)) break;
    }
    return;
  }
  for (int m = 0; m < kPlRowsPerWave; ++m) {
    const long long r = static_cast<long long>(blockIdx.x) * kPlRows + m * (kPlThreads / kWave) + wv;
    if (r >= N) break;
    const T* hr = hl + static_cast<size_t>(r) * hid;
    float acc = 0.f;
    if ((hid & 7) == 0) {
      const int nch = hid >> 3;
      for (int c0 = 0; c0 < nch; c0 += kWave * kPlUnroll) {
        Chunk8<T> hv[kPlUnroll];
#pragma unroll
        for (int u = 0; u < kPlUnroll; ++u) {
          const int c = c0 + u * kWave + lane;
          if (c < nch) hv[u].load_stream(hr + 8 * c);
        }
#pragma unroll
        for (int u = 0; u < kPlUnroll; ++u) {
          const int c = c0 + u * kWave + lane;
          if (c < nch) {
            const float4 w0 = reinterpret_cast<const float4*>(s_w)[2 * c];
            const float4 w1 = reinterpret_cast<const float4*>(s_w)[2 * c + 1];
            acc = fmaf(w0.x, hv[u].at(0), acc);
            acc = fmaf(w0.y, hv[u].at(1), acc);
            acc = fmaf(w0.z, hv[u].at(2), acc);
            acc = fmaf(w0.w, hv[u].at(3), acc);
            acc = fmaf(w1.x, hv[u].at(4), acc);
            acc = fmaf(w1.y, hv[u].at(5), acc);
            acc = fmaf(w1.z, hv[u].at(6), acc);
            acc = fmaf(w1.w, hv[u].at(7), acc);
          }
        }
      }
    } else {
      for (int k = lane; k < hid; k += kWave) acc = fmaf(s_w[k], load_f32(hr, k), acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) z[static_cast<size_t>(l) * N + r] = acc;
  }
}

hipError_t launch_probe_logits(const void* h, bool bf16, const float* w, int L, long long N,
                               int hid, float* z, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((N + kPlRows - 1) / kPlRows), L);
  const size_t lds = static_cast<size_t>(std::max(hid, kPlFastHid)) * sizeof(float);
  if (bf16)
    hipLaunchKernelGGL(probe_logits_kernel<uint16_t>, grid, dim3(kPlThreads), lds, s,
                       static_cast<const uint16_t*>(h), w, N, hid, z);
  else
    hipLaunchKernelGGL(probe_logits_kernel<float>, grid, dim3(kPlThreads), lds, s,
                       static_cast<const float*>(h), w, N, hid, z);
  return hipGetLastError();
}

// ---------------------------------------------------------------- sweep
constexpr int kSwThreads = 1024;
constexpr int kSwChunk = kSwThreads * 8;   // largest chunk sorted by one workgroup (64 KiB of LDS)
constexpr int kScThreads = 512;  // workgroup of the scan (one per layer)
constexpr int kSwPer = 8;        // keys per thread per pass of the scan
constexpr unsigned long long kPadKey = ~0ull;

// 32-bit key that orders scores descending (ascending key = descending z);
// -0 and +0 are one score.
__device__ __forceinline__ uint32_t desc_key(float z) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~ord;
}

__device__ __forceinline__ float key_score(uint32_t k) {
  const uint32_t ord = ~k;
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

__global__ __launch_bounds__(256) void sweep_keys_kernel(const float* __restrict__ z,
                                                         const uint8_t* __restrict__ labels,
                                                         int N, int Np,
                                                         unsigned long long* __restrict__ keys) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= Np) return;
  const int l = blockIdx.y;
  unsigned long long k = kPadKey;
  if (i < N)
    k = static_cast<unsigned long long>(desc_key(z[static_cast<size_t>(l) * N + i])) << 32 |
        (labels[i] ? 1u : 0u);
  keys[static_cast<size_t>(l) * Np + i] = k;
}

// Compare-exchange of the bitonic network's stage (k, j) for pair p: the pair is
// (lo, lo + j), sorted ascending when bit k of lo (global index) is clear.
__device__ __forceinline__ int pair_lo(int p, int j) { return ((p & ~(j - 1)) << 1) | (p & (j - 1)); }

__device__ __forceinline__ void cmp_swap(unsigned long long& a, unsigned long long& b, bool up) {
  const unsigned long long lo = a < b ? a : b, hi = a < b ? b : a;
  a = up ? lo : hi;
  b = up ? hi : lo;
}

// Strides below E stay inside one thread's E keys.
template <int E, int J>
__device__ __forceinline__ void reg_stage(unsigned long long (&r)[E], int gi0, int k) {
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((e & J) == 0) cmp_swap(r[e], r[e | J], ((gi0 + e) & k) == 0);
}

// One chunk of 1024 * E keys per workgroup (E = 1, 2, 4 or 8); thread t holds
// keys E*t .. E*t+E-1 in registers.  Strides below E are exchanged in registers,
// E .. 32*E between lanes of a wave (shuffles, no barrier), 64*E and up through
// LDS, where key i sits at (i % E) * 1024 + i / E so that the lanes of a wave
// touch consecutive words.  k_merge == 0: sort the chunk with every stage k up
// to the chunk size.  Otherwise finish the merge of size k_merge (larger than
// the chunk) with the strides below the chunk size.
template <int E>
__global__ __launch_bounds__(kSwThreads) void sort_local_kernel(unsigned long long* __restrict__ keys,
                                                                int Np, int k_merge) {
  constexpr int C = kSwThreads * E;
  __shared__ unsigned long long s[C];
  const int t = threadIdx.x;
  const int base = blockIdx.x * C;
  unsigned long long* kl = keys + static_cast<size_t>(blockIdx.y) * Np + base;
  unsigned long long r[E];
#pragma unroll
  for (int e = 0; e < E; ++e) r[e] = kl[t * E + e];
  const int gi0 = base + t * E;
  const int k0 = k_merge ? k_merge : 2, k1 = k_merge ? k_merge : C;
  for (int k = k0; k <= k1; k <<= 1) {
    int j = (k_merge ? C : k) >> 1;
    if (j >= E * kWave) {
#pragma unroll
      for (int e = 0; e < E; ++e) s[e * kSwThreads + t] = r[e];
      __syncthreads();
      for (; j >= E * kWave; j >>= 1) {
        const int js = j / E;
#pragma unroll
        for (int q = 0; q < (E + 1) / 2; ++q) {
          const int p = t + q * kSwThreads;
          if (p < C / 2) {
            const int e = p / (kSwThreads / 2), pm = p % (kSwThreads / 2);
            const int mlo = pair_lo(pm, js);
            unsigned long long a = s[e * kSwThreads + mlo], b = s[e * kSwThreads + mlo + js];
            cmp_swap(a, b, ((base + mlo * E + e) & k) == 0);
            s[e * kSwThreads + mlo] = a;
            s[e * kSwThreads + mlo + js] = b;
          }
        }
        __syncthreads();
      }
#pragma unroll
      for (int e = 0; e < E; ++e) r[e] = s[e * kSwThreads + t];
      __syncthreads();
    }
    for (; j >= E; j >>= 1) {
      const int m = j / E;
      const bool lower = (t & m) == 0;
      const bool up = (gi0 & k) == 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const unsigned long long b = __shfl_xor(r[e], m, kWave);
        const unsigned long long mn = r[e] < b ? r[e] : b, mx = r[e] < b ? b : r[e];
        r[e] = (lower == up) ? mn : mx;
      }
    }
    if constexpr (E > 4) { if (j >= 4) reg_stage<E, 4>(r, gi0, k); }
    if constexpr (E > 2) { if (j >= 2) reg_stage<E, 2>(r, gi0, k); }
    if constexpr (E > 1) { if (j >= 1) reg_stage<E, 1>(r, gi0, k); }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) kl[t * E + e] = r[e];
}

__global__ __launch_bounds__(256) void sort_global_kernel(unsigned long long* __restrict__ keys,
                                                          int Np, int k, int j) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= Np / 2) return;
  unsigned long long* kl = keys + static_cast<size_t>(blockIdx.y) * Np;
  const int lo = pair_lo(p, j), hi = lo + j;
  const bool up = (lo & k) == 0;
  const unsigned long long a = kl[lo], b = kl[hi];
  if (up ? a > b : a < b) {
    kl[lo] = b;
    kl[hi] = a;
  }
}

// Exclusive max-scan of v over the workgroup (thread order); `total` gets the max.
template <int NT>
__device__ __forceinline__ unsigned long long block_excl_max(unsigned long long v,
                                                             unsigned long long* s_wave,
                                                             unsigned long long& total) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  unsigned long long incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned long long t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl = t > incl ? t : incl;
  }
  unsigned long long excl = __shfl_up(incl, 1, kWave);
  if (lane == 0) excl = 0;
  if (lane == kWave - 1) s_wave[wv] = incl;
  __syncthreads();
  unsigned long long woff = 0, tot = 0;
  for (int i = 0; i < NT / kWave; ++i) {
    const unsigned long long c = s_wave[i];
    if (i < wv) woff = c > woff ? c : woff;
    tot = c > tot ? c : tot;
  }
  __syncthreads();
  total = tot;
  return woff > excl ? woff : excl;
}

// Is F1 of (tp_a, den_a) higher than of (tp_b, den_b)?  F1 = 2 tp / den.
__device__ __forceinline__ bool f1_higher(int tp_a, long long den_a, int tp_b, long long den_b) {
  return static_cast<long long>(tp_a) * den_b > static_cast<long long>(tp_b) * den_a;
}

__global__ __launch_bounds__(kScThreads) void sweep_scan_kernel(
    const unsigned long long* __restrict__ keys, int N, int Np, float* __restrict__ thr_out,
    int32_t* __restrict__ counts_out, long long* __restrict__ u2_out, float* __restrict__ auc_out) {
  __shared__ int s_wave[kScThreads / kWave];
  __shared__ unsigned long long s_wave64[kScThreads / kWave];
  __shared__ int s_tp[kScThreads], s_idx[kScThreads];
  __shared__ long long s_den[kScThreads], s_u2[kScThreads];
  const int l = blockIdx.x, t = threadIdx.x;
  const unsigned long long* kl = keys + static_cast<size_t>(l) * Np;

  int pc = 0;
  for (int i = t; i < N; i += kScThreads) pc += static_cast<int>(kl[i] & 1u);
  int POS;
  block_excl_scan<kScThreads>(pc, s_wave, POS);
  const long long NEG = static_cast<long long>(N) - POS;

  // Group starts are packed as ((start + 1) << 32 | positives before the start);
  // both fields grow with the start, so the latest start is the max.
  int carry_cp = 0;
  unsigned long long carry_start = 0;
  int best_tp = 0, best_idx = 0x7fffffff;
  long long best_den = 1, u2 = 0;
  for (int c0 = 0; c0 < N; c0 += kScThreads * kSwPer) {
    const int i0 = c0 + t * kSwPer;
    unsigned long long kk[kSwPer + 2];   // [0] = key before i0, [1..kSwPer] mine, [kSwPer+1] after
#pragma unroll
    for (int e = 0; e < kSwPer + 2; ++e) {
      const int i = i0 - 1 + e;
      kk[e] = (i >= 0 && i < N) ? kl[i] : kPadKey;
    }
    int my_pos = 0;
#pragma unroll
    for (int e = 1; e <= kSwPer; ++e) my_pos += (i0 + e - 1 < N) ? static_cast<int>(kk[e] & 1u) : 0;
    int chunk_pos;
    const int cp0 = carry_cp + block_excl_scan<kScThreads>(my_pos, s_wave, chunk_pos);
    unsigned long long my_start = 0;
    {
      int cp = cp0;
#pragma unroll
      for (int e = 1; e <= kSwPer; ++e) {
        const int i = i0 + e - 1;
        if (i < N) {
          if (i == 0 || (kk[e - 1] >> 32) != (kk[e] >> 32))
            my_start = static_cast<unsigned long long>(i + 1) << 32 | static_cast<uint32_t>(cp);
          cp += static_cast<int>(kk[e] & 1u);
        }
      }
    }
    unsigned long long chunk_start;
    unsigned long long cur = block_excl_max<kScThreads>(my_start, s_wave64, chunk_start);
    cur = cur > carry_start ? cur : carry_start;
    int cp = cp0;
#pragma unroll
    for (int e = 1; e <= kSwPer; ++e) {
      const int i = i0 + e - 1;
      if (i < N) {
        if (i == 0 || (kk[e - 1] >> 32) != (kk[e] >> 32))
          cur = static_cast<unsigned long long>(i + 1) << 32 | static_cast<uint32_t>(cp);
        cp += static_cast<int>(kk[e] & 1u);
        if (i == N - 1 || (kk[e + 1] >> 32) != (kk[e] >> 32)) {
          const long long s_i = static_cast<long long>(cur >> 32) - 1;
          const long long pg = cp - static_cast<long long>(cur & 0xffffffffu);
          const long long ng = (i - s_i + 1) - pg;
          const long long cn = static_cast<long long>(i) + 1 - cp;   // negatives with z >= t
          u2 += pg * (2 * (NEG - cn) + ng);
          if (cp > 0) {
            const long long den = static_cast<long long>(cp) + cn + POS;   // 2TP + FP + FN
            if (f1_higher(cp, den, best_tp, best_den)) {
              best_tp = cp;
              best_den = den;
              best_idx = i;
            }
          }
        }
      }
    }
    carry_cp += chunk_pos;
    carry_start = chunk_start > carry_start ? chunk_start : carry_start;
  }

  s_tp[t] = best_tp;
  s_den[t] = best_den;
  s_idx[t] = best_idx;
  s_u2[t] = u2;
  __syncthreads();
  for (int o = kScThreads / 2; o > 0; o >>= 1) {
    if (t < o) {
      const int tb = s_tp[t + o], ib = s_idx[t + o];
      const long long db = s_den[t + o];
      if (f1_higher(tb, db, s_tp[t], s_den[t]) ||
          (!f1_higher(s_tp[t], s_den[t], tb, db) && ib < s_idx[t])) {
        s_tp[t] = tb;
        s_den[t] = db;
        s_idx[t] = ib;
      }
      s_u2[t] += s_u2[t + o];
    }
    __syncthreads();
  }
  if (t == 0) {
    const int tp = s_tp[0], idx = s_idx[0];
    const bool found = tp > 0;
    thr_out[l] = found ? key_score(static_cast<uint32_t>(kl[idx] >> 32)) : INFINITY;
    const int fp = found ? idx + 1 - tp : 0;
    counts_out[4 * l + 0] = tp;
    counts_out[4 * l + 1] = fp;
    counts_out[4 * l + 2] = POS - tp;
    counts_out[4 * l + 3] = POS;
    u2_out[l] = s_u2[0];
    auc_out[l] = (POS > 0 && NEG > 0)
                     ? static_cast<float>(static_cast<double>(s_u2[0]) / (2.0 * POS * static_cast<double>(NEG)))
                     : NAN;
  }
}

// Layer with the highest F1 (the lowest layer on ties) and tau = sigma(t).  One
// wave: each lane keeps the best of its layers, then a butterfly keeps the best
// of all (ties to the lower layer).
__global__ __launch_bounds__(kWave) void select_layer_kernel(const float* __restrict__ thr,
                                                             const int32_t* __restrict__ counts, int L,
                                                             int32_t* __restrict__ best_layer,
                                                             float* __restrict__ tau) {
  const int lane = threadIdx.x;
  int bl = 0x7fffffff, btp = 0;
  long long bden = 1;
  for (int l = lane; l < L; l += kWave) {
    const int tp = counts[4 * l];
    const long long den = 2ll * tp + counts[4 * l + 1] + counts[4 * l + 2];
    if (bl == 0x7fffffff || f1_higher(tp, den, btp, bden)) {
      bl = l;
      btp = tp;
      bden = den;
    }
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int ol = __shfl_xor(bl, o, kWave), otp = __shfl_xor(btp, o, kWave);
    const long long oden = __shfl_xor(bden, o, kWave);
    const bool take = ol != 0x7fffffff &&
                      (bl == 0x7fffffff || f1_higher(otp, oden, btp, bden) ||
                       (!f1_higher(btp, bden, otp, oden) && ol < bl));
    if (take) {
      bl = ol;
      btp = otp;
      bden = oden;
    }
  }
  if (lane == 0) {
    const double t = thr[bl];
    *best_layer = bl;
    *tau = static_cast<float>(isinf(t) ? (t > 0 ? 1.0 : 0.0) : 1.0 / (1.0 + exp(-t)));
  }
}

int sweep_padded(long long N) {
  int Np = kSwThreads;
  while (Np < N) Np <<= 1;
  return Np;
}

size_t calibrate_workspace_bytes(int L, long long N) {
  return static_cast<size_t>(L) * static_cast<size_t>(sweep_padded(N)) * 8;
}

hipError_t launch_calibrate(const float* z, const uint8_t* labels, int L, int N, float* thr_out,
                            int32_t* counts_out, long long* u2_out, float* auc_out,
                            int32_t* best_layer, float* tau, void* ws, hipStream_t s) {
  const int Np = sweep_padded(N);
  auto* keys = static_cast<unsigned long long*>(ws);
  hipLaunchKernelGGL(sweep_keys_kernel, dim3((Np + 255) / 256, L), dim3(256), 0, s, z, labels, N, Np, keys);
  const int chunk = Np < kSwChunk ? Np : kSwChunk;
  const dim3 lgrid(Np / chunk, L);
  auto local = [&](int k_merge) {
    switch (chunk / kSwThreads) {
      case 1: hipLaunchKernelGGL(sort_local_kernel<1>, lgrid, dim3(kSwThreads), 0, s, keys, Np, k_merge); break;
      case 2: hipLaunchKernelGGL(sort_local_kernel<2>, lgrid, dim3(kSwThreads), 0, s, keys, Np, k_merge); break;
      case 4: hipLaunchKernelGGL(sort_local_kernel<4>, lgrid, dim3(kSwThreads), 0, s, keys, Np, k_merge); break;
      default: hipLaunchKernelGGL(sort_local_kernel<8>, lgrid, dim3(kSwThreads), 0, s, keys, Np, k_merge); break;
    }
  };
  local(0);
  for (int k = 2 * chunk; k <= Np; k <<= 1) {
    for (int j = k >> 1; j >= chunk; j >>= 1)
      hipLaunchKernelGGL(sort_global_kernel, dim3((Np / 2 + 255) / 256, L), dim3(256), 0, s, keys, Np, k, j);
    local(k);
  }
  hipLaunchKernelGGL(sweep_scan_kernel, dim3(L), dim3(kScThreads), 0, s, keys, N, Np, thr_out,
                     counts_out, u2_out, auc_out);
  hipLaunchKernelGGL(select_layer_kernel, dim3(1), dim3(64), 0, s, thr_out, counts_out, L, best_layer, tau);
  return hipGetLastError();
}

}  // namespace ssd
