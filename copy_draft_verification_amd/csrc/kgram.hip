// kappa-gram evidence, recency-ordered retrieval and candidate gather.
// SwitchSD write-up §2.5 (dual gate: probe AND an earlier occurrence of the
// kappa-gram ending at the current token), paper §3.3 "Copy-Based Speculative
// Generation" and write-up §2.6 (up to W continuations of up to D tokens,
// ranked by recency).
//
// One workgroup per sequence (1024 lanes for fewer than 512 sequences, else 256)
// scans end positions from the newest (n-2) backwards in chunks of 8 per lane
// (8192 or 2048).  A chunk of ids (plus a kappa-1 halo) is
// copied from HBM straight into LDS by buffer-to-LDS loads, which hold no
// registers while in flight; two LDS stages let the next chunk's loads run
// while the current chunk is tested, and a context of up to two chunks is
// entirely in flight at once.  The barriers of the loop order LDS only, which
// leaves those loads outstanding.  Lane t tests positions top-8t .. top-8t-7
// from its eight ids (two 16-byte LDS reads), so lane order equals recency
// order.  Matches are compacted in that order by a workgroup prefix sum over
// per-lane counts, and the scan stops as soon as W matches are known.  The
// candidate gather then copies L_w = min(D, n-1-p_w) ids after each match, from
// LDS where the chunk the scan ended in (or the kappa-gram suffix) holds them.
#include "common.h"
#include "kernels.h"
#include "switchsd.h"

namespace ssd {

constexpr int kKgPer = 8;  // end positions per lane and chunk
constexpr int kKgPad = 8;  // LDS slots before the staged ids (the lowest lane reads from 1 below)
static_assert(kKgPad % 4 == 0 && kKgPad >= kKgPer - 1, "pad keeps 16-byte reads in the array");
// Geometry of a workgroup of NT lanes.  Staged ids per chunk: the chunk's end
// positions, the kappa-1 ids before the oldest of them, and up to 3 more below
// those, so that the staged range starts at a position congruent to top-7 (mod 4)
// and every lane's eight ids (top-8t-7 .. top-8t) sit on a 16-byte boundary of LDS.
template <int NT>
struct KgGeom {
  static constexpr int kChunk = NT * kKgPer;                       // end positions per chunk
  static constexpr int kStage = kChunk + (SSD_MAX_KAPPA - 1) + 3;  // staged ids per chunk
  static constexpr int kLoads = (kStage + NT - 1) / NT;            // loads per lane and chunk (9)
  static constexpr int kSlots = kKgPad + kLoads * NT;              // ints per LDS stage
  static_assert(kLoads <= 31, "vmcnt holds two chunks' loads");
};
// Workgroup sizes: 1024 lanes when there are few contexts (each context's scan is
// the latency of the launch), 256 when there are many (eight workgroups per CU, so
// some are always streaming while others test or write).
constexpr int kKgWide = 1024;
constexpr int kKgNarrow = 256;
constexpr int kKgNarrowFrom = 512;  // contexts from which the narrow workgroups run

// LDS reads of the stages, written as asm that waits for its own result.  The
// compiler cannot tell which LDS a pending buffer-to-LDS copy writes, so before a
// plain read of one stage it would wait for every copy in flight, the other
// stage's included; the stage being read has already been waited for (fixed
// wait count + barrier).
using i32x4 = __attribute__((ext_vector_type(4))) int;
__device__ __forceinline__ uint32_t lds_addr(const int* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) int*)p));
}
__device__ __forceinline__ int lds_ld(const int* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
// The outputs are early-clobber: the first read's destination must not share a
// register with the address, which the second read takes when it issues, and LDS
// data can land before that (nothing orders a register read after an LDS load
// still in flight to the same register).
__device__ __forceinline__ void lds_ld8(const int* p, i32x4& a, i32x4& b) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(b) : "v"(lds_addr(p)) : "memory");
}

// The probe of sequence b, computed by the whole workgroup (paper §3.2 "Layer and
// Threshold Selection", write-up §2.3): z = w . h_b in fp32 (each thread sums
// eight consecutive k per chunk, then a wave sum and a sum over the waves in wave
// order), fire = z >= thr.  Thread 0 writes z_out[b] (if given) and fire_out[b].
// Returns fire to every thread.
template <int NT>
__device__ __forceinline__ bool probe_in_block(const KgProbe& pr, int b, float* s_part, int* s_fire) {
  const int t = threadIdx.x;
  float acc = 0.f;
  if ((pr.hidden & 7) == 0) {
    const int nch = pr.hidden >> 3;
    for (int c = t; c < nch; c += NT) {
      float hv[8];
      if (pr.bf16) {
        Chunk8<uint16_t> x;
        x.load(static_cast<const uint16_t*>(pr.h) + static_cast<size_t>(b) * pr.hidden + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = x.at(e);
      } else {
        Chunk8<float> x;
        x.load(static_cast<const float*>(pr.h) + static_cast<size_t>(b) * pr.hidden + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = x.at(e);
      }
      Chunk8<float> wv;
      wv.load(pr.w + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += wv.at(e) * hv[e];
    }
  } else {
    for (int k = t; k < pr.hidden; k += NT) {
      const float hk = pr.bf16 ? bf16_to_f32(static_cast<const uint16_t*>(pr.h)[static_cast<size_t>(b) * pr.hidden + k])
                               : static_cast<const float*>(pr.h)[static_cast<size_t>(b) * pr.hidden + k];
      acc += pr.w[k] * hk;
    }
  }
  acc = wave_sum(acc);
  if ((t & (kWave - 1)) == 0) s_part[t / kWave] = acc;
  __syncthreads();
  if (t == 0) {
    float z = 0.f;
    for (int i = 0; i < NT / kWave; ++i) z += s_part[i];
    const bool f = z >= pr.thr;
    if (pr.z_out) pr.z_out[b] = z;
    pr.fire_out[b] = f ? 1 : 0;
    *s_fire = f ? 1 : 0;
  }
  __syncthreads();
  return *s_fire != 0;
}

// Eight waves per SIMD: two 1024-lane workgroups per CU (2 x 72 KB of LDS) or eight
// 256-lane ones (8 x 19 KB); while some compare, the others' loads are in flight.  With pr.h set, the workgroup first
// computes its sequence's probe (probe_in_block) while its first chunk copies are
// in flight, and scans only if the probe fired; `fire` is then not read.
template <int NT>
__global__ __launch_bounds__(NT, 8) void kgram_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ cu_len, int kappa, int W, int D,
    const uint8_t* __restrict__ fire, int32_t* __restrict__ match_end, int32_t* __restrict__ n_match,
    int32_t* __restrict__ cand, int32_t* __restrict__ cand_len, uint8_t* __restrict__ copy_gate,
    KgProbe pr) {
  // the two stages, read through the asm helpers above
  __shared__ int s_suffix[SSD_MAX_KAPPA];
  __shared__ int s_list[SSD_MAX_W];
  using G = KgGeom<NT>;
  constexpr int kKgChunk = G::kChunk, kKgLoads = G::kLoads, kKgSlots = G::kSlots;
  __shared__ int s_wave[NT / kWave];
  __shared__ float s_part[NT / kWave];
  __shared__ int s_fire;
  __shared__ __attribute__((aligned(16))) int st0[kKgSlots];
  __shared__ __attribute__((aligned(16))) int st1[kKgSlots];
  const int b = blockIdx.x, t = threadIdx.x;
  const int base = cu_len[b];
  const int n = cu_len[b + 1] - base;
  const bool fused = pr.h != nullptr;
  const bool active = (fused || fire == nullptr || fire[b] != 0) && n >= kappa + 1;
  if (fused && !active) probe_in_block<NT>(pr, b, s_part, &s_fire);
  int found = 0;
  // the chunk the scan ended in: its stage still holds positions g_abase .. g_top
  const int* g_stage = st0;
  int g_abase = 0, g_top = -1;
  if (active) {
    const int lo = kappa - 1;
    // the LDS destination of a buffer-to-LDS load (M0) must be wave-uniform
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    if (t < kappa) s_suffix[t] = ids[base + n - kappa + t];
    // first staged position of the chunk whose newest end position is top
    auto stage_lo = [&](int top) {
      const int lbase = max(lo, top - kKgChunk + 1) - (kappa - 1);
      return lbase - ((lbase - (top - (kKgPer - 1))) & 3);
    };
    // The sequence's ids as a buffer: loads past its last id return zero.  A
    // staged position below 0 (at most 3 of them, lanes 0..2 of the first load)
    // reads id 0 instead; positions below the halo are never compared.  Staged
    // index i lands in stage slot kKgPad + i; every lane issues kKgLoads loads
    // per chunk, so the wave's load count per chunk is fixed.  The ids are read
    // once, so the copies carry the nontemporal hint: with the default policy a
    // stream of buffer-to-LDS copies tops out near 4.6 TB/s on this part, with the
    // hint near 7 TB/s.
    const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(ids + base), 0, n * 4, kBufFlags);
    // Loads of a chunk that does not exist (top < lo) are still issued, with an
    // offset past the buffer: they return zeros without touching memory, and every
    // chunk is followed by exactly kKgLoads loads of this wave, so one fixed wait
    // count serves every chunk.
    constexpr int kOutOfRange = 0x7ffffff0;
    // Slots past the chunk's staged count (ids above top, which the previous chunk
    // already read) take the out-of-range offset too: no memory is touched.
    auto issue = [&](int* stage, int top) {
      const bool past = top < lo;
      const int abase = past ? 0 : stage_lo(top);
      const int i0 = abase + t, room = past ? 0 : top - abase + 1 - t;
#pragma unroll
      for (int u = 0; u < kKgLoads; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            res, (__attribute__((address_space(3))) void*)(stage + kKgPad + u * NT + wave * kWave),
            4, u * NT >= room ? kOutOfRange : u == 0 ? max(i0, 0) * 4 : (i0 + u * NT) * 4,
            0, 0, kNonTemporal);
    };
    // Test the chunk whose newest end position is top, staged in `stage`; false
    // when the scan is over.  On return the stage may be reloaded (the scan ends
    // with a barrier that follows every read of it).
    auto chunk = [&](int* stage, int top) -> bool {
      // this wave's loads of the chunk have landed (the next chunk's may not)...
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kKgLoads));
      // ...and every wave's
      lds_barrier();
      const int cbeg = max(lo, top - kKgChunk + 1);
      const int abase = stage_lo(top);
      const int s_last = s_suffix[kappa - 1];
      const int s_prev = kappa >= 2 ? s_suffix[kappa - 2] : 0;
      unsigned mask = 0;
      const int p0 = top - t * kKgPer;
      if (p0 >= cbeg) {
        // ids of positions p0-7 .. p0; positions below cbeg are never matched
        const int s0 = kKgPad + p0 - (kKgPer - 1) - abase;
        i32x4 ra, rb;
        lds_ld8(stage + s0, ra, rb);
        const int v[kKgPer] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
        for (int i = 0; i < kKgPer; ++i) {
          const int p = p0 - i;  // its id is v[7 - i]
          bool m = p >= cbeg && v[kKgPer - 1 - i] == s_last;
          // the id before it is still in registers, except for the lane's oldest position
          if (i < kKgPer - 1 && kappa >= 2) m = m && v[kKgPer - 2 - i] == s_prev;
          if (m) {
            for (int qq = i < kKgPer - 1 ? 2 : 1; qq < kappa; ++qq)
              if (lds_ld(stage + kKgPad + p - qq - abase) != s_suffix[kappa - 1 - qq]) { m = false; break; }
          }
          if (m) mask |= 1u << i;
        }
      }
      int total;
      int rank = found + block_excl_scan<NT, true>(__popc(mask), s_wave, total);
      while (mask) {
        const int i = __ffs(mask) - 1;
        mask &= mask - 1;
        if (rank < W) s_list[rank] = p0 - i;
        ++rank;
      }
      found += total;
      const int nt = top - kKgChunk;
      if (nt < lo || found >= W) {
        g_stage = stage;
        g_abase = abase;
        g_top = top;
        return false;
      }
      issue(stage, nt - kKgChunk);
      return true;
    };
    int top = n - 2;
    issue(st0, top);
    issue(st1, top - kKgChunk);
    // fused probe: computed while the first copies are in flight; a closed probe
    // retrieves nothing
    const bool fired = !fused || probe_in_block<NT>(pr, b, s_part, &s_fire);
    for (; fired;) {
      if (!chunk(st0, top)) break;
      top -= kKgChunk;
      if (!chunk(st1, top)) break;
      top -= kKgChunk;
    }
    // a scan that stopped early may still have the next chunk's loads in
    // flight: they must land before the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  const int M = min(found, W);
  for (int w = t; w < W; w += NT) {
    const int p = w < M ? s_list[w] : -1;
    match_end[static_cast<size_t>(b) * W + w] = p;
    cand_len[static_cast<size_t>(b) * W + w] = w < M ? min(D, n - 1 - p) : 0;
  }
  // Candidate gather: id q = p+1+j from the last chunk's stage when it holds q,
  // from the suffix for the newest kappa positions, else from memory (matches of
  // earlier, newer chunks whose stage has been reloaded).
  for (int e = t; e < W * D; e += NT) {
    const int w = e / D, j = e - w * D;
    int v = -1;
    if (w < M) {
      const int p = s_list[w];
      if (j < min(D, n - 1 - p)) {
        const int q = p + 1 + j;
        if (q >= g_abase && q <= g_top) v = lds_ld(g_stage + kKgPad + q - g_abase);
        else if (q >= n - kappa) v = s_suffix[q - (n - kappa)];
        else v = ids[base + q];
      }
    }
    cand[static_cast<size_t>(b) * W * D + e] = v;
  }
  if (t == 0) {
    n_match[b] = M;
    copy_gate[b] = M > 0 ? 1 : 0;
  }
}

hipError_t launch_kgram(const int32_t* ids, const int32_t* cu_len, int B, int kappa, int W, int D,
                        const uint8_t* fire, int32_t* match_end, int32_t* n_match, int32_t* cand,
                        int32_t* cand_len, uint8_t* copy_gate, hipStream_t s, const KgProbe* probe) {
  const KgProbe pr = probe != nullptr ? *probe : KgProbe{};
  if (B < kKgNarrowFrom)
    hipLaunchKernelGGL(kgram_kernel<kKgWide>, dim3(B), dim3(kKgWide), 0, s, ids, cu_len, kappa, W, D, fire,
                       match_end, n_match, cand, cand_len, copy_gate, pr);
  else
    hipLaunchKernelGGL(kgram_kernel<kKgNarrow>, dim3(B), dim3(kKgNarrow), 0, s, ids, cu_len, kappa, W, D,
                       fire, match_end, n_match, cand, cand_len, copy_gate, pr);
  return hipGetLastError();
}

}  // namespace ssd
