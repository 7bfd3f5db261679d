// LM-head projection + greedy argmax for every verification row (SwitchSD
// paper §3.3: one target forward pass verifies all candidates; write-up §3.1:
// T = 0, so each row's verdict is the argmax of its logits).
//
// logits[row][v] = sum_k O[row][k] * lm_head[v][k].  The weight matrix (V x hid)
// is the dominant HBM stream, so each workgroup owns a 256-wide vocabulary tile
// and streams it exactly once while every row of the row chunk (up to 224 rows,
// the whole verify batch of one sequence) is multiplied against it: the rows are
// the MFMA N dimension (B operand, staged in LDS), the vocabulary is the M
// dimension (A operand, loaded straight from HBM into registers, three k-steps
// ahead, from the packed layout in which each wave's fragments of a k-step are
// one contiguous 8 KB run).  The epilogue reduces each row over the tile to a
// (max, lowest index) pair without writing logits and folds it into the row's
// 64-bit key by an atomic max; a one-wave-per-sequence launch turns the keys into
// argmax indices (and may run the accept).  The same main loop, with other epilogues, serves the sampling
// verification and the projections of the forward.  An fp32 variant on the
// vector ALU serves fp32 inputs (plain [V][hid] weights).
#include <limits.h>

#include <type_traits>
#include <utility>

#include "accept_seq.h"
#include "common.h"
#include "kernels.h"

namespace ssd {

// bf16 path.  Workgroup = 4 waves = 256 vocabulary entries (64 per wave, two
// 32-wide MFMA tiles) x one chunk of 224 rows (seven tiles of 32).
// v_mfma_f32_32x32x16_bf16: A = 32 vocabulary x 16 k (this lane: vocabulary l32,
// k 8h..8h+7 of the step), B = 16 k x 32 rows (same lane/k pairing), D = 32 x 32
// with lane (l32, h) holding vocabulary 8(r/4) + 4h + r%4 of row l32 in element r.
// The k order inside a step is the same on both sides, so the lane-to-k
// assignment does not change the contraction.
//
// Memory pipeline (one iteration = 64 k):
//  * weights: straight from HBM into registers (the A operand), in four register
//    slots;
//  * rows: copied from global memory into LDS by buffer-to-LDS loads, into four
//    LDS stages.
// With several row chunks both streams run three iterations ahead, the same
// distance, because a wave's loads complete in issue order: a short-latency row
// load issued after a weight load cannot be consumed before that weight load has
// landed.  With one row chunk (kPairSync below) the weights run three iterations
// ahead and the rows two.
constexpr int kLmWaves = 4;
constexpr int kLmVA = 2;                          // A tiles (32 vocabulary) per wave
constexpr int kLmVT = kLmWaves * kLmVA * 32;      // vocabulary per workgroup (256)
constexpr int kLmNT = 7;                          // row tiles of 32 per chunk
constexpr int kLmMC = kLmNT * 32;                 // rows per chunk (224)
constexpr int kLmKS = 64;                         // k per iteration (four MFMA k-steps)
constexpr int kLmStage = kLmMC * kLmKS;           // bf16 per LDS stage (224 rows x 128 B, no padding)
constexpr int kLmBlocks = kLmMC / 8;              // 1 KB load blocks per stage (8 rows each)
constexpr int kLmBlocksPerWave = kLmBlocks / kLmWaves;  // 7
constexpr int kLmSlots = 4;                       // weight register slots = LDS stages
constexpr int kLmKAlign = kLmKS * kLmSlots;       // the hidden size must be a multiple of this
constexpr int kLmBAhead = 4;                      // LDS reads of B fragments in flight
constexpr int kLmIssueAt = 4;                     // MFMA pair after which the next loads start (full tiles)
constexpr int kLmXcds = 8;                        // XCDs; workgroups are dealt round-robin
constexpr int kLmXcdSlots = 32;                   // concurrent workgroups per XCD (one per CU)
constexpr int kPastEnd = -1;                      // iteration index of a load past the K range
// Packed weight layout (ssd_pack_weight, ssd_pack_gate_up): per (256-row tile,
// k-slab), a 32 KB block; in it, per wave, the 8 KB of A fragments the wave loads
// for that slab, one 1 KB run per (tile a, k-step s), lane-major.  A wave's
// weight loads then stream one contiguous 8 KB run per iteration.  For the gate /
// up pair, tile row 64w + 32a + l is feature 128t + 32w + l of the gate (a = 0) or
// of the up matrix (a = 1).
constexpr int kPkWaveBytes = kLmVA * 4 * kWave * 16;       // 8 KB
constexpr int kPkSlabBytes = kLmWaves * kPkWaveBytes;      // 32 KB
// loads a wave issues per iteration: row blocks, then weight fragments
constexpr int kLmLoadsPerIter = kLmBlocksPerWave + kLmVA * 4;
static_assert(kLmBlocks % kLmWaves == 0, "row blocks split evenly over the waves");
static_assert(kLmLoadsPerIter * 3 <= 63, "vmcnt holds the loads of three iterations");

template <typename F, int... Ts>
__device__ __forceinline__ void for_each_tile(F& f, std::integer_sequence<int, Ts...>) {
  (f(IntC<Ts>{}), ...);
}

// Row r of a stage keeps its eight 16-byte k chunks in swizzled order:
// logical chunk c sits at position c ^ ((r >> 1) & 7).  Sixteen consecutive rows
// read at one logical chunk then cover all 64 LDS banks once.
__device__ __forceinline__ int lm_swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// GEMM epilogues of the decoder layers (same main loop).  Lane (l32, h) holds,
// per A tile a and register r, output feature vbase + 32a + 8(r/4) + 4h + r%4 of
// compact row row0 + 32t + l32 (SwiGLU: feature vbase + 8(r/4) + 4h + r%4, with
// the gate in A tile 0 and the up projection in A tile 1).
//  * kEpiPartial: this split's partial sums, fp32, dense by compact row:
//    part[split][row][feature], four consecutive features per 16-byte store.
//    kEpiPartialHalf: the same for one A tile per wave (a 128-row half tile).
//  * kEpiSwiGLU: silu(gate) * up, bf16, at out[global row][feature].
//  * kEpiPair: the gate and up partial sums of this split, fp32:
//    part[split][row][feature] and part[split][row][N + feature].
template <int kEpi, int kVA>
__device__ __forceinline__ void gemm_epilogue(const f32x16 (&acc)[kVA][kLmNT], int row0, int rows,
                                              int vbase, int V, int h, int l32, const GemmArgs& ga) {
#pragma unroll
  for (int t = 0; t < kLmNT; ++t) {
    const int row = row0 + t * 32 + l32;
    if (row >= rows) continue;
    if constexpr (kEpi == kEpiPair) {
      // gate partials at [f], up partials at [N + f]
      float* pr = ga.part + (static_cast<size_t>(blockIdx.y) * ga.part_rows + row) * ga.ld;
#pragma unroll
      for (int a = 0; a < kLmVA; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = vbase + 8 * q + 4 * h;
          float* dst = pr + a * V + f;
          if (f + 3 < V)
            *reinterpret_cast<float4*>(dst) =
                make_float4(acc[a][t][4 * q], acc[a][t][4 * q + 1], acc[a][t][4 * q + 2], acc[a][t][4 * q + 3]);
          else
            for (int i = 0; i < 4; ++i)
              if (f + i < V) dst[i] = acc[a][t][4 * q + i];
        }
    } else if constexpr (kEpi == kEpiPartial || kEpi == kEpiPartialHalf) {
      float* pr = ga.part + (static_cast<size_t>(blockIdx.y) * ga.part_rows + row) * ga.ld;
#pragma unroll
      for (int a = 0; a < kVA; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int v = vbase + a * 32 + 8 * q + 4 * h;
          if (v + 3 < V)
            *reinterpret_cast<float4*>(pr + v) =
                make_float4(acc[a][t][4 * q], acc[a][t][4 * q + 1], acc[a][t][4 * q + 2], acc[a][t][4 * q + 3]);
          else
            for (int i = 0; i < 4; ++i)
              if (v + i < V) pr[v + i] = acc[a][t][4 * q + i];
        }
    } else {
      uint16_t* orow = ga.out + static_cast<size_t>(ga.row_list[row]) * ga.ld;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = vbase + 8 * q + 4 * h;
        uint16_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc[0][t][4 * q + i], u = acc[1][t][4 * q + i];
          o[i] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
        }
        if (f + 3 < V)
          *reinterpret_cast<uint2*>(orow + f) =
              make_uint2(o[0] | static_cast<uint32_t>(o[1]) << 16, o[2] | static_cast<uint32_t>(o[3]) << 16);
        else
          for (int i = 0; i < 4; ++i)
            if (f + i < V) orow[f + i] = o[i];
      }
    }
  }
}

// Sampling epilogue (T > 0).  Per row and this workgroup's vocabulary tile:
// the base-2 log-sum-exp pair (max, sum 2^(t2 - max)) of t2 = log2(e) * logit / T
// over every token,
// and the best t + Gumbel noise over the tokens that are not children of the
// row's trie node (the residual draw's candidates).  The children's t values are
// stored for the acceptance tests.  Lane (l32, h) holds, per A tile a and
// register r, token vbase + 32a + 8(r/4) + 4h + r%4: groups of four consecutive
// tokens, one Philox block each.
__device__ __forceinline__ void sample_epilogue(
    const f32x16 (&acc)[kLmVA][kLmNT], int row0, int rows, int vbase, int V, int vt, int vtiles,
    int wave, int tid, int l32, int h, const int32_t* __restrict__ row_list, const SampleArgs& sa,
    float (&red_y)[kLmWaves][kLmMC], int (&red_x)[kLmWaves][kLmMC],
    float (&red_m)[kLmWaves][kLmMC], float (&red_s)[kLmWaves][kLmMC], float4* __restrict__ part) {
  // The rows' trie data first, for all seven row tiles at once and before any
  // store, so that the three dependent loads (row list, child count, child
  // tokens) cost three memory latencies rather than three per tile.
  int growv[kLmNT], ncv[kLmNT];
  uint32_t exclv[kLmNT];
#pragma unroll
  for (int t = 0; t < kLmNT; ++t) {
    const int row = row0 + t * 32 + l32;
    growv[t] = row < rows ? row_list[row] : -1;
  }
#pragma unroll
  for (int t = 0; t < kLmNT; ++t)
    ncv[t] = growv[t] >= 0 ? min(max(sa.n_children[growv[t]], 0), sa.W) : 0;
  // children that fall on this lane's 32 tokens, as a bit mask over (a, r).  The
  // first four child slots of every tile's row are loaded unconditionally (slot
  // indices clamped into the row's W slots) so that all 28 loads are in flight
  // together; rows with more children (the anchor's) finish in a loop.
  auto child_bit = [&](int c) -> uint32_t {
    const int dd = c - vbase;
    if (dd >= 0 && dd < kLmVA * 32 && ((dd >> 2) & 1) == h) {
      const int rem = dd & 31;
      return 1u << ((dd >> 5) * 16 + ((rem >> 3) << 2) + (rem & 3));
    }
    return 0u;
  };
  constexpr int kFastKids = 4;
  int cfast[kLmNT][kFastKids];
#pragma unroll
  for (int t = 0; t < kLmNT; ++t) {
    const int32_t* ch = sa.children + static_cast<size_t>(growv[t] < 0 ? 0 : growv[t]) * sa.W;
#pragma unroll
    for (int k = 0; k < kFastKids; ++k) cfast[t][k] = ch[min(k, sa.W - 1)];
  }
#pragma unroll
  for (int t = 0; t < kLmNT; ++t) {
    uint32_t excl = 0;
#pragma unroll
    for (int k = 0; k < kFastKids; ++k)
      if (k < ncv[t]) excl |= child_bit(cfast[t][k]);
    const int32_t* ch = sa.children + static_cast<size_t>(growv[t] < 0 ? 0 : growv[t]) * sa.W;
    for (int k = kFastKids; k < ncv[t]; ++k) excl |= child_bit(ch[k]);
    exclv[t] = excl;
  }
  const float inv_t2 = sa.inv_t * kLog2e;
  const bool full = vbase + kLmVA * 32 <= V;  // every value of the tile is a token
  // token index of position p = 16 a + r of this lane
  auto tok = [&](int p) { return vbase + (p >> 4) * 32 + 8 * ((p & 15) >> 2) + 4 * h + (p & 3); };
  // one call per row tile with a compile-time tile index, so that the
  // accumulators stay in registers (a loop this large is not unrolled)
  auto tile = [&](auto Tc) {
    constexpr int t = decltype(Tc)::value;
    const int grow = growv[t], nc = ncv[t];
    const uint32_t excl = exclv[t];
    const int32_t* ch = sa.children + static_cast<size_t>(grow < 0 ? 0 : grow) * sa.W;
    // Scans over the lane's 32 values in four interleaved chains (short dependent
    // chains without holding a second copy of the values, which would not fit beside
    // the accumulators): the maximum of t2 = log2(e) t, the sum of 2^(t2 - max), and
    // the best t + Gumbel noise over the tokens that are not children, first
    // position on ties.  Values past V take no part (-inf); children take no part
    // in the residual draw.
    constexpr int kN = kLmVA * 16;
    float v32[kN];
#pragma unroll
    for (int p = 0; p < kN; ++p)
      v32[p] = (full | (tok(p) < V)) ? acc[p >> 4][t][p & 15] * inv_t2 : -INFINITY;
    auto max4 = [&]() {
      float c[4] = {v32[0], v32[1], v32[2], v32[3]};
#pragma unroll
      for (int p = 4; p < kN; ++p) c[p & 3] = fmaxf(c[p & 3], v32[p]);
      return fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));
    };
    float m = max4();
    // a lane without a valid value keeps m = -inf and s = 0
    const float mref = m == -INFINITY ? 0.f : m;
    float sc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < kN; ++p) sc[p & 3] += __builtin_amdgcn_exp2f(v32[p] - mref);
    float s = (sc[0] + sc[1]) + (sc[2] + sc[3]);
#pragma unroll
    for (int a = 0; a < kLmVA; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int x0 = vbase + a * 32 + 8 * q + 4 * h;
        const uint4 wd = philox4x32_10(static_cast<uint32_t>(x0 >> 2), static_cast<uint32_t>(grow), 0, 0,
                                       sa.k0, sa.k1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = a * 16 + 4 * q + i;
          const bool draw = (full | (x0 + i < V)) & (((excl >> p) & 1u) == 0u);
          const float g = gumbel_of(i == 0 ? wd.x : i == 1 ? wd.y : i == 2 ? wd.z : wd.w);
          v32[p] = draw ? acc[a][t][4 * q + i] * sa.inv_t + g : -INFINITY;
        }
      }
    const float ymax = max4();
    // first position holding ymax: per chain the lowest matching position, then the least
    int pc[4] = {kN, kN, kN, kN};
#pragma unroll
    for (int p = kN - 1; p >= 0; --p) pc[p & 3] = v32[p] == ymax ? p : pc[p & 3];
    const int pb = min(min(pc[0], pc[1]), min(pc[2], pc[3]));
    // -inf marks both "no draw" and a drawn -inf: report only a drawn position
    bool found = pb < kN;
#pragma unroll
    for (int i = 0; i < kN; ++i)
      if (i == pb) found = found & (full | (tok(i) < V)) & (((excl >> i) & 1u) == 0u);
    float by = found ? ymax : -INFINITY;
    int bx = found ? tok(pb) : INT_MAX;
    // the children's t values go to their slots (rare: few lanes hold a child)
    if (excl != 0u && grow >= 0) {
#pragma unroll
      for (int p = 0; p < kN; ++p)
        if ((excl >> p) & 1u) {
          const int x = tok(p);
          const float tv = acc[p >> 4][t][p & 15] * sa.inv_t;
          for (int k = 0; k < nc; ++k)
            if (ch[k] == x) sa.child_logit[static_cast<size_t>(grow) * sa.W + k] = tv;
        }
    }
    {
      const float om = __shfl_xor(m, 32, kWave), os = __shfl_xor(s, 32, kWave);
      const float oy = __shfl_xor(by, 32, kWave);
      const int ox = __shfl_xor(bx, 32, kWave);
      lse2_merge(m, s, om, os);
      if (better(oy, ox, by, bx)) { by = oy; bx = ox; }
    }
    if (h == 0) {
      red_m[wave][t * 32 + l32] = m;
      red_s[wave][t * 32 + l32] = s;
      red_y[wave][t * 32 + l32] = by;
      red_x[wave][t * 32 + l32] = bx;
    }
  };
  for_each_tile(tile, std::make_integer_sequence<int, kLmNT>{});
  __syncthreads();
  for (int i = tid; i < kLmMC; i += 256) {
    const int row = row0 + i;
    if (row >= rows) continue;
    float m = red_m[0][i], s = red_s[0][i], by = red_y[0][i];
    int bx = red_x[0][i];
#pragma unroll
    for (int w = 1; w < kLmWaves; ++w) {
      lse2_merge(m, s, red_m[w][i], red_s[w][i]);
      if (better(red_y[w][i], red_x[w][i], by, bx)) { by = red_y[w][i]; bx = red_x[w][i]; }
    }
    part[static_cast<size_t>(row) * vtiles + vt] = make_float4(m, s, by, __int_as_float(bx));
  }
}

// 64-bit argmax key of a (value, index) pair: the value's bits made
// order-preserving in the high half (-0 taken as +0, so that equal values tie), the
// complemented index in the low half.  The unsigned maximum of keys is then the
// largest value with the lowest index, the order of `better`.  0 stands for no
// value (every value NaN or past V); no real pair maps to it, since its high half
// would be a NaN's.
__device__ __forceinline__ unsigned long long argmax_key(float v, int i) {
  if (i == INT_MAX) return 0ull;
  uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(u) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(i));
}

// Greedy epilogue: per row (this lane's column l32 of each row tile), the best
// (value, lowest index) over this workgroup's tile, combined over the four waves,
// then folded into the key of the row's global index (thread i of the workgroup
// holds grow = the global row of chunk row i, or -1) by a device-wide 64-bit atomic
// max.
__device__ __forceinline__ void argmax_epilogue(
    const f32x16 (&acc)[kLmVA][kLmNT], int row0, int rows, int vbase, int V, int wave, int tid,
    int l32, int h, const int32_t* __restrict__ row_list, float* __restrict__ logits_out,
    float (&red_v)[kLmWaves][kLmMC], int (&red_i)[kLmWaves][kLmMC], unsigned long long* __restrict__ keys,
    int grow) {
  // Debug output, on its own path: inside the scan below, a store per value behind
  // its own test made the epilogue a chain of about 1400 branches, 16 us per
  // workgroup even with logits_out null.
  if (logits_out != nullptr) {
#pragma unroll
    for (int t = 0; t < kLmNT; ++t) {
      const int row = row0 + t * 32 + l32;
      if (row >= rows) continue;
      float* lr = logits_out + static_cast<size_t>(row_list[row]) * V;
#pragma unroll
      for (int a = 0; a < kLmVA; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int v = vbase + a * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (v < V) lr[v] = acc[a][t][r];
        }
    }
  }
  // Per row tile, this lane's 32 values: their maximum by a tree of v_max3 (which
  // never returns a NaN against a number, so NaN never wins), then the first
  // position holding it (positions rise with the token index, so the first is the
  // lowest); values past V take no part.  A linear scan with `better` was a
  // dependent chain through every value (with && and ||, a few branches per value:
  // 16 us per workgroup; branch-free, still 6.6 us at one wave per SIMD).
  constexpr int kN = kLmVA * 16;
  const bool full = vbase + kLmVA * 32 <= V;  // every value of the tile is a token
  // token index of position p = 16 a + r of this lane
  auto tok = [&](int p) { return vbase + (p >> 4) * 32 + 8 * ((p & 15) >> 2) + 4 * h + (p & 3); };
#pragma unroll
  for (int t = 0; t < kLmNT; ++t) {
    float xs[kN];
#pragma unroll
    for (int a = 0; a < kLmVA; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) xs[a * 16 + r] = acc[a][t][r];
    if (!full) {
#pragma unroll
      for (int p = 0; p < kN; ++p) xs[p] = tok(p) < V ? xs[p] : -INFINITY;
    }
    static_assert(kN == 32, "the max tree below is written for 32 values");
    float t1[11];
#pragma unroll
    for (int i = 0; i < 10; ++i) t1[i] = vmax3_raw(xs[3 * i], xs[3 * i + 1], xs[3 * i + 2]);
    t1[10] = vmax2_raw(xs[30], xs[31]);
    const float t20 = vmax3_raw(t1[0], t1[1], t1[2]), t21 = vmax3_raw(t1[3], t1[4], t1[5]);
    const float t22 = vmax3_raw(t1[6], t1[7], t1[8]), t23 = vmax2_raw(t1[9], t1[10]);
    const float mx = vmax2_raw(vmax3_raw(t20, t21, t22), t23);
    // the first position holding it, by a descending chain of selects
    int pbest = kN;
#pragma unroll
    for (int p = kN - 1; p >= 0; --p) pbest = xs[p] == mx ? p : pbest;
    // A position past V holds -inf: it can equal mx only when every value is -inf
    // or NaN, and then it must not be reported.  Every value NaN: mx is NaN and no
    // position matches.  Either way the lane offers (-inf, none), which any value
    // of another lane beats.
    const bool found = (pbest < kN) & (full | (tok(pbest) < V));
    float bv = found ? mx : -INFINITY;
    int bi = found ? tok(pbest) : INT_MAX;
    const float ov = __shfl_xor(bv, 32, kWave);
    const int oi = __shfl_xor(bi, 32, kWave);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    if (h == 0) {
      red_v[wave][t * 32 + l32] = bv;
      red_i[wave][t * 32 + l32] = bi;
    }
  }
  __syncthreads();
  static_assert(kLmMC <= kLmWaves * kWave, "one thread per chunk row");
  if (grow >= 0) {
    const int i = tid;
    float bv = red_v[0][i];
    int bi = red_i[0][i];
#pragma unroll
    for (int w = 1; w < kLmWaves; ++w)
      if (better(red_v[w][i], red_i[w][i], bv, bi)) { bv = red_v[w][i]; bi = red_i[w][i]; }
    __hip_atomic_fetch_max(keys + grow, argmax_key(bv, bi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// kOnce: every weight of the launch is read by one workgroup only (a single row
// chunk), so the weight loads carry the nontemporal hint, which streams faster
// from HBM; with several row chunks the chunks of one tile share it through L2,
// and the default policy keeps it there.
// kRows: the weights are the plain row-major [N][K] matrix instead of the packed
// layout (greedy launch only): each A-fragment load then gathers 16 bytes from each
// of 32 rows, where the packed layout reads 1 KB contiguous.  The four k-steps of
// a slab read the same 128-byte line of each row, so these loads keep the default
// cache policy, which holds the line in the vector cache from one step to the next.
template <int kEpi, bool kOnce, bool kRows = false>
__global__ __launch_bounds__(256, 1) void lmhead_bf16_kernel(
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ Wt, int total_rows, int K, int V,
    const int32_t* __restrict__ row_list, const int32_t* __restrict__ n_rows,
    float* __restrict__ logits_out, void* __restrict__ part_out, int vtiles, int mchunks, int sv,
    int sm, SampleArgs sa, GemmArgs ga) {
  constexpr bool kSample = kEpi == kEpiSample;
  constexpr bool kSwiGLU = kEpi == kEpiSwiGLU || kEpi == kEpiPair;   // packed gate / up pair
  // A tiles per wave: one for a half tile (rows 64w + 32 hh .. + 31 of a packed tile)
  constexpr int kVA = kEpi == kEpiPartialHalf ? 1 : kLmVA;
  constexpr int kLoadsPerIter = kLmBlocksPerWave + kVA * 4;
  __shared__ __attribute__((aligned(1024))) uint16_t st0[kLmStage];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[kLmStage];
  __shared__ __attribute__((aligned(1024))) uint16_t st2[kLmStage];
  __shared__ __attribute__((aligned(1024))) uint16_t st3[kLmStage];
  __shared__ float red_v[kLmWaves][kLmMC];
  __shared__ int red_i[kLmWaves][kLmMC];
  __shared__ float red_m[kSample ? kLmWaves : 1][kLmMC];
  __shared__ float red_s[kSample ? kLmWaves : 1][kLmMC];

  // XCD-aware tile order.  Workgroups are dealt round-robin over the XCDs (block L
  // runs on XCD L % 8).  Super-tiles of sv vocabulary tiles x sm row chunks (about
  // one XCD's worth of concurrent workgroups) are dealt to XCDs whole, so the
  // workgroups resident together on an XCD share their weights and rows in its L2.
  const int xcd = static_cast<int>(blockIdx.x % kLmXcds), li = static_cast<int>(blockIdx.x / kLmXcds);
  const int per = sv * sm;
  const int super = (li / per) * kLmXcds + xcd;
  const int n_sm = (mchunks + sm - 1) / sm;
  const int vt = (super / n_sm) * sv + (li % per) / sm;
  const int mc = (super % n_sm) * sm + (li % per) % sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  // wave index in a scalar register: the LDS destination of a buffer-to-LDS load
  // (M0) must be wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  // rows of this chunk are compact indices row0.. into the list of real rows
  const int rows = *n_rows;
  if (vt >= vtiles || mc >= mchunks || mc * kLmMC >= rows) return;
  const int h = lane >> 5, l32 = lane & 31;
  const int row0 = mc * kLmMC;
  // greedy: the global row of chunk row tid, for the epilogue (loaded now, used last)
  int grow = -1;
  if constexpr (kEpi == kEpiArgmax)
    if (tid < kLmMC && row0 + tid < rows) grow = row_list[row0 + tid];
  // the gate / up GEMM takes its two A tiles from two matrices (the same 32
  // features of each), so a workgroup covers 128 features instead of 256; a
  // half-tile workgroup covers rows 64w + 32hh .. + 31 of packed tile vt / 2
  const int ptile = kVA == 1 ? vt >> 1 : vt, hh = kVA == 1 ? vt & 1 : 0;
  const int vbase = kSwiGLU ? vt * (kLmVT / kLmVA) + wave * 32
                            : ptile * kLmVT + wave * kLmVA * 32 + hh * 32;
  // split-K: this workgroup contracts k0 .. k0 + kc of the hidden dimension
  const int kc = ga.kc > 0 ? ga.kc : K;
  const int k0 = static_cast<int>(blockIdx.y) * kc;

  // Buffer resources: this workgroup's weight tile (K / 64 packed slabs of 32 KB,
  // zero rows past N) and its row chunk of O.  Reads whose per-lane offset is past
  // the range return zero (rows past `rows`, prefetches past the K range), so the
  // pipeline needs no guards.
  const int o_bytes = total_rows * K * 2;
  static_assert(!kRows || (kEpi == kEpiArgmax && kVA == kLmVA), "row-major weights: greedy launch only");
  // rows of the tile past N (plain layout: past the end of the matrix) read as zero
  const int tile_rows = kRows ? max(0, min(kLmVT, V - ptile * kLmVT)) : kLmVT;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Wt + static_cast<size_t>(ptile) * kLmVT * K), 0, K * tile_rows * 2, kBufFlags);
  int aoff[kVA];
#pragma unroll
  for (int a = 0; a < kVA; ++a)
    aoff[a] = kRows ? (wave * 64 + (a + hh) * 32 + (lane & 31)) * K * 2 + (lane >> 5) * 16
                    : wave * kPkWaveBytes + (a + hh) * 4 * kWave * 16 + lane * 16;
  // per k-step (16 k) and k-slab (64 k) strides of the A-fragment loads
  constexpr int kStepBytes = kRows ? 32 : kWave * 16;
  constexpr int kSlabBytes = kRows ? kLmKS * 2 : kPkSlabBytes;
  const __amdgpu_buffer_rsrc_t ores =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(O), 0, o_bytes, kBufFlags);
  // Row blocks of this wave: block b = wave*7 + j holds stage rows 8b..8b+7; lane i
  // fills stage row 8b + i/8 at swizzled position i%8 from O row
  // row_list[row0 + 8b + i/8].  Stage rows past the last real row read past the end
  // of O, which returns zero.
  int ooff[kLmBlocksPerWave];
#pragma unroll
  for (int j = 0; j < kLmBlocksPerWave; ++j) {
    const int sr = 8 * (wave * kLmBlocksPerWave + j) + (lane >> 3);
    const int ci = row0 + sr;
    const int orow = ci < rows ? row_list[ci] : -1;
    ooff[j] = orow < 0 ? o_bytes : (orow * K + lm_swz(sr, lane & 7) * 8) * 2;
  }

  f32x16 acc[kVA][kLmNT];
#pragma unroll
  for (int a = 0; a < kVA; ++a)
#pragma unroll
    for (int t = 0; t < kLmNT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][t][r] = 0.f;

  uint4 aw[kLmSlots][kVA][4];
  // The loop issues loads ahead of their use; the issues that fall past this
  // workgroup's K range (it == kPastEnd) take a per-lane offset beyond every
  // buffer's num_records, so they return zeros without touching memory instead
  // of fetching the next range's data.
  constexpr int kOutOfRange = 0x7ffffff0;
  // Iteration it contracts k-slab (it + rot) mod nit: the workgroups resident
  // together start at different slabs of their tiles, so their streams do not all
  // hit the same column range of the weight rows (and the same HBM channels) at
  // once.
  const int nit = kc / kLmKS;
  const int rot = vt % nit;
  auto slab = [&](int it) {   // global k-slab index (k0 is a multiple of 64)
    const int r = it + rot;
    return k0 / kLmKS + (r >= nit ? r - nit : r);
  };
  auto load_a = [&](uint4 (&dst)[kVA][4], int it) {
    const bool past = it == kPastEnd;
    // slab block of iteration it; run (a, s) of this wave, 16 B per lane
    const int so = past ? 0 : slab(it) * kSlabBytes;
#pragma unroll
    for (int a = 0; a < kVA; ++a)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        dst[a][s] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       wres, past ? kOutOfRange : aoff[a] + s * kStepBytes, so, (kOnce && !kRows) ? kNonTemporal : 0));
  };
  auto load_o = [&](uint16_t* stage, int it) {
    const bool past = it == kPastEnd;
    const int ko = past ? 0 : slab(it) * kLmKS * 2;
#pragma unroll
    for (int j = 0; j < kLmBlocksPerWave; ++j) {
      const int b = wave * kLmBlocksPerWave + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ores, (__attribute__((address_space(3))) void*)(stage + b * 512), 16,
          past ? kOutOfRange : ooff[j], ko, 0, 0);
    }
  };
  // 28 B fragments per iteration (k-step s major, row tile t minor), each feeding two
  // MFMAs.  The LDS reads run kLmBAhead fragments ahead of their use; the
  // scheduling groups pin that order (first kLmBAhead reads, then two MFMAs and one
  // read at a time) so that the compiler does not sink the reads next to their use.
  //
  // With kInterleave, issue_next issues the next iteration's loads from inside the
  // MFMA stream: one load after each MFMA pair from pair kLmIssueAt on, so that the
  // first MFMAs after the barrier wait only on their own B fragments, and the loads'
  // issue slots fall under MFMAs already in the matrix pipeline.  That makes the
  // greedy LM head 7-9% faster (batch 1 and batch 32), the gate / up projection 8%
  // and the split-K projections on half tiles 3-4% faster, the latter with the
  // loads starting after pair 10 (their 11 loads per iteration against 14 MFMA
  // pairs; after pair 4 they were slower).  The sampling epilogue is 3-4% slower
  // with it, so it issues its loads before the MFMAs.
  constexpr bool kInterleave = kEpi == kEpiArgmax || kEpi == kEpiPair || kEpi == kEpiPartialHalf;
  constexpr int kIssueAt = kEpi == kEpiPartialHalf ? 10 : kLmIssueAt;
  // kPairSync: one barrier per two iterations.  At the start of an even iteration
  // each wave waits for its rows and weights of iterations it and it+1, and one
  // barrier makes every wave's rows of both visible and frees the stages of it-2
  // and it-1; odd iterations have neither wait nor barrier.  Each step issues the
  // rows of it+2 and the weights of it+3 (a register slot is free as soon as its
  // own wave is done with it, a stage only after the barrier), spread evenly over
  // the step's 28 MFMA pairs.  In the greedy launch with one row chunk (batch 1)
  // the barrier per two iterations is 8% faster than one per iteration (244
  // against 266 us at 201 rows, same box); with several chunks (batch 32: 6.27
  // against 5.78 ms) it is 8% slower, so those keep a barrier per iteration.  At
  // batch 1, same box: all loads of it+2 and it+3 in the even step, two after each
  // MFMA pair from pair 2, 205 us (the vector memory path took the burst at the
  // cost of MFMA issue); the weights of both in the even step and the rows of both
  // in the odd one, each spread, 189 us; this schedule, 185 us (193 against 185 on
  // another box).
  constexpr bool kPairSync = kEpi == kEpiArgmax && kOnce;
  // compute: iteration `it` on `w` and `stage`; issue_next() issues kNL loads,
  // placed among the MFMAs from pair kAt on (kNL = 0: issue_next is not called):
  // with kSpread evenly over the remaining pairs, else kPer after each pair.
  auto compute = [&](auto NL_c, const uint4 (&w)[kVA][4], const uint16_t* stage, auto&& issue_next) {
    constexpr int kNL = decltype(NL_c)::value;
    constexpr bool kSpread = kPairSync;
    constexpr int kPer = kNL > kLoadsPerIter ? 2 : 1;               // loads per MFMA pair
    constexpr int kAt = kSpread ? 0 : kIssueAt;
    constexpr int NB = 4 * kLmNT;
    static_assert(kSpread ? kNL <= NB : kAt + (kNL + kPer - 1) / kPer <= NB,
                  "the loads fit between the MFMA pairs");
    const uint16_t* ob = stage + l32 * kLmKS;
    const int sw = (l32 >> 1) & 7;
    auto frag = [&](int j) {
      const int s = j / kLmNT, t = j % kLmNT;
      return *reinterpret_cast<const uint4*>(ob + t * 32 * kLmKS + (((2 * s + h) ^ sw) << 3));
    };
    uint4 bq[kLmBAhead + 1];
#pragma unroll
    for (int i = 0; i < kLmBAhead; ++i) bq[i] = frag(i);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int s = i / kLmNT, t = i % kLmNT;
      if (kNL > 0 && i == kAt) issue_next();
      if (i + kLmBAhead < NB) bq[(i + kLmBAhead) % (kLmBAhead + 1)] = frag(i + kLmBAhead);
      const bf16x8 bfr = __builtin_bit_cast(bf16x8, bq[i % (kLmBAhead + 1)]);
#pragma unroll
      for (int a = 0; a < kVA; ++a)
        acc[a][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w[a][s]), bfr,
                                                            acc[a][t], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kLmBAhead, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, kVA, 0);      // MFMAs
      if (i + kLmBAhead < NB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if constexpr (kSpread) {                                    // global loads
        const int cnt = i >= kAt ? ((i + 1 - kAt) * kNL) / (NB - kAt) - ((i - kAt) * kNL) / (NB - kAt) : 0;
        if (cnt == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      } else if (kNL > 0 && i >= kAt && (i - kAt) * kPer < kNL) {
        if (kPer == 2 && kNL - (i - kAt) * kPer >= 2)
          __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
  };
  uint16_t* const stages[kLmSlots] = {st0, st1, st2, st3};

  // Step U of the unrolled loop works on iteration it (it % 4 == U): wait until this
  // wave's rows and weights of iteration it have landed (everything but the two
  // newer iterations' loads), barrier so every wave's row blocks are in LDS and
  // stage (U+3)%4 is no longer read, then compute iteration it and issue iteration
  // it+3 (before the MFMAs, or among them with kInterleave).
  auto step = [&](auto U_c, int it) {
    constexpr int U = decltype(U_c)::value;
    if constexpr (kPairSync) {
      // Every step issues the rows of it+2, into the stage of it-2 (every wave left
      // it before the last barrier), then the weights of it+3, into this wave's
      // register slot of it-1.  At an even step everything up to the rows of it+1
      // has landed once only the newest weights (those of it+2, from the odd step
      // before) are outstanding.
      auto issue_next = [&]() {
        load_o(stages[(U + 2) % kLmSlots], it + 2 < nit ? it + 2 : kPastEnd);
        load_a(aw[(U + 3) % kLmSlots], it + 3 < nit ? it + 3 : kPastEnd);
      };
      if constexpr (U % 2 == 0) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kVA * 4));
        lds_barrier();
      }
      compute(IntC<kLoadsPerIter>{}, aw[U], stages[U], issue_next);
      return;
    }
    // s_waitcnt as a builtin, so that the compiler's own wait tracking knows it
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kLoadsPerIter));
    lds_barrier();
    // iteration it+3 goes into stage and slot (U+3) % 4, which iteration it does not read
    auto issue_rows = [&]() { load_o(stages[(U + 3) % kLmSlots], it + 3 < nit ? it + 3 : kPastEnd); };
    auto issue_weights = [&]() { load_a(aw[(U + 3) % kLmSlots], it + 3 < nit ? it + 3 : kPastEnd); };
    if constexpr (kInterleave) {
      // no scheduling barrier inside the MFMA stream: the group barriers place the loads
      compute(IntC<kLoadsPerIter>{}, aw[U], stages[U], [&]() {
        issue_rows();
        issue_weights();
      });
    } else {
      issue_rows();
      __builtin_amdgcn_sched_barrier(0);  // keep the issue order: rows, then weights
      issue_weights();
      __builtin_amdgcn_sched_barrier(0);
      compute(IntC<0>{}, aw[U], stages[U], [] {});
    }
  };
  load_o(st0, 0);
  load_a(aw[0], 0);
  __builtin_amdgcn_sched_barrier(0);
  load_o(st1, 1);
  load_a(aw[1], 1);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!kPairSync) {
    load_o(st2, 2);
    load_a(aw[2], 2);
  } else {
    load_a(aw[2], 2);  // the weights run three iterations ahead, the rows two
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int it0 = 0; it0 < nit; it0 += kLmSlots) {
    step(IntC<0>{}, it0);
    step(IntC<1>{}, it0 + 1);
    step(IntC<2>{}, it0 + 2);
    step(IntC<3>{}, it0 + 3);
  }
  // the last three iterations' loads (past the end: zeros) must land before the
  // workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if constexpr (kEpi == kEpiPartial || kEpi == kEpiPartialHalf || kSwiGLU) {
    gemm_epilogue<kEpi, kVA>(acc, row0, rows, vbase, V, h, l32, ga);
  } else if constexpr (kSample) {
    sample_epilogue(acc, row0, rows, vbase, V, vt, vtiles, wave, tid, l32, h, row_list, sa,
                    red_v, red_i, reinterpret_cast<float(&)[kLmWaves][kLmMC]>(red_m),
                    reinterpret_cast<float(&)[kLmWaves][kLmMC]>(red_s), static_cast<float4*>(part_out));
  } else {
    argmax_epilogue(acc, row0, rows, vbase, V, wave, tid, l32, h, row_list, logits_out, red_v, red_i,
                    static_cast<unsigned long long*>(part_out), grow);
  }
}


// fp32: thread per vocabulary column, 32 rows per workgroup.  Per 64-wide slice of
// the contraction, each thread loads its column's 64 weights as sixteen 16-byte
// loads in flight together and the workgroup loads the slice of its 32 rows of O;
// both go to LDS, the weights transposed so that a thread's piece c sits beside its
// neighbours'.  The contraction loop reads one weight piece per step and the rows as
// broadcasts; it is kept rolled (the code runs once per workgroup, and a fully
// unrolled body costs more in instruction fetches than it saves).  The logits then
// pass through LDS so that each wave scans eight rows with lanes on consecutive
// columns; the argmax folds into the per-row keys as in the bf16 kernel (workgroup
// best, then a device-wide 64-bit atomic max).
constexpr int kLmF32Rows = 32;
constexpr int kLmF32VT = 256;  // vocabulary per workgroup (one column per thread)
constexpr int kLmF32KC = 64;   // contraction slice
__global__ __launch_bounds__(256) void lmhead_f32_kernel(
    const float* __restrict__ O, const float* __restrict__ Wt, int K, int V,
    const int32_t* __restrict__ row_list, const int32_t* __restrict__ n_rows, int cap,
    float* __restrict__ logits_out, unsigned long long* __restrict__ keys) {
  constexpr int kC = kLmF32KC / 4;                        // 16-byte pieces per slice row
  constexpr int kStage = kLmF32Rows * kC / 256;           // O pieces per thread and slice (2)
  static_assert(kC * kLmF32VT * 16 >= kLmF32Rows * kLmF32VT * 4, "logits fit the weight stage");
  __shared__ float4 s_w[kC][kLmF32VT];                    // weights; later the tile's logits
  __shared__ float4 o_lds[kLmF32Rows][kC];
  __shared__ int s_grow[kLmF32Rows];                      // the chunk's attention rows
  const int mc = blockIdx.x, vt = blockIdx.y;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int row0 = mc * kLmF32Rows;
  const int v = vt * kLmF32VT + tid;
  const float4* wr = reinterpret_cast<const float4*>(Wt + static_cast<size_t>(v < V ? v : V - 1) * K);
  // The first slice's weights and the staged rows' list entries are requested
  // with the row count, not after it: entries past the count (stale, or never
  // written) are clamped into [0, cap) and their sums are never used.
  int grow[kStage], rows;
  {
    float4 w4[kC];
#pragma unroll
    for (int c = 0; c < kC; ++c) w4[c] = wr[c];
#pragma unroll
    for (int u = 0; u < kStage; ++u) grow[u] = row_list[min(row0 + (tid + 256 * u) / kC, cap - 1)];
    rows = *n_rows;  // compact rows; O row of compact row i is row_list[i]
    __builtin_amdgcn_sched_barrier(0);  // all of them in flight before the first wait
#pragma unroll
    for (int c = 0; c < kC; ++c) s_w[c][tid] = w4[c];
    // an empty use, so that the list loads stay ahead of the exit test below
#pragma unroll
    for (int u = 0; u < kStage; ++u) asm volatile("" ::"v"(grow[u]));
  }
  if (row0 >= rows) return;
  const float4* orow[kStage];
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int e = tid + 256 * u;
    const int g = min(max(grow[u], 0), cap - 1);
    orow[u] = reinterpret_cast<const float4*>(O + static_cast<size_t>(g) * K) + e % kC;
    if (e % kC == 0) s_grow[e / kC] = g;  // for the epilogue (read after its barriers)
  }
  float acc[kLmF32Rows];
#pragma unroll
  for (int i = 0; i < kLmF32Rows; ++i) acc[i] = 0.f;
  for (int k0 = 0; k0 < K; k0 += kLmF32KC) {
    if (k0 > 0) {
      __syncthreads();  // the previous slice has been read
      float4 w4[kC];
#pragma unroll
      for (int c = 0; c < kC; ++c) w4[c] = wr[k0 / 4 + c];
#pragma unroll
      for (int c = 0; c < kC; ++c) s_w[c][tid] = w4[c];
    }
    float4 ox[kStage];
#pragma unroll
    for (int u = 0; u < kStage; ++u) ox[u] = orow[u][k0 / 4];
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      const int e = tid + 256 * u;
      o_lds[e / kC][e % kC] = ox[u];
    }
    __syncthreads();
#pragma unroll 1
    for (int c = 0; c < kC; ++c) {
      const float4 w = s_w[c][tid];
#pragma unroll
      for (int i = 0; i < kLmF32Rows; ++i) {
        const float4 o = o_lds[i][c];
        acc[i] += o.x * w.x + o.y * w.y + o.z * w.z + o.w * w.w;
      }
    }
  }
  __syncthreads();
  float* s_l = reinterpret_cast<float*>(&s_w[0][0]);  // [row][column]
#pragma unroll
  for (int i = 0; i < kLmF32Rows; ++i) s_l[i * kLmF32VT + tid] = acc[i];
  __syncthreads();
  for (int i = wave; i < kLmF32Rows && row0 + i < rows; i += 4) {
    const int grow = s_grow[i];
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int u = 0; u < kLmF32VT / kWave; ++u) {
      const int col = lane + kWave * u, vc = vt * kLmF32VT + col;
      const float x = s_l[i * kLmF32VT + col];
      if (logits_out && vc < V) logits_out[static_cast<size_t>(grow) * V + vc] = x;
      // NaN logits and columns past V take no part; columns rise with u, so only a
      // larger value replaces the best
      if (vc < V && x > bv) { bv = x; bi = vc; }
      if (vc < V && bi == INT_MAX && x == -INFINITY) bi = vc;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0)
      __hip_atomic_fetch_max(keys + grow, argmax_key(bv, bi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Real rows (open gate, row 0 or j < L_w) in row order: row_list[i] = row of the
// i-th real row, inv[row] = i or -1, n_rows = count.  One workgroup scans all rows.
constexpr int kCompactThreads = 1024;
// ----------------------------------------------------------------- weight packing
// One thread per 16-byte chunk of the packed layout.  Chunk c, decomposed as
// (tile vt, slab, wave, run a*4 + s, lane = 32h + l32), holds tile row
// 64*wave + 32a + l32 at k = slab*64 + 16s + 8h .. +7: the A fragment lane
// (l32, h) of that wave loads for tile a, k-step s.  The tile row is weight row
// 256vt + 64*wave + 32a + l32 of w, or, for a pair (w2 != null), feature
// 128vt + 32*wave + l32 of w (a = 0) or w2 (a = 1).  Rows past N are zero.
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint16_t* __restrict__ w,
                                                          const uint16_t* __restrict__ w2, int N,
                                                          int K, uint16_t* __restrict__ packed,
                                                          size_t n_chunks) {
  const int nslab = K / kLmKS;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t c = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < n_chunks; c += stride) {
    const int lane = static_cast<int>(c % kWave);
    size_t t = c / kWave;
    const int run = static_cast<int>(t % (kLmVA * 4));
    t /= kLmVA * 4;
    const int wave = static_cast<int>(t % kLmWaves);
    t /= kLmWaves;
    const int slab = static_cast<int>(t % nslab);
    const size_t vt = t / nslab;
    const int a = run / 4;
    const size_t row = w2 ? vt * (kLmVT / kLmVA) + wave * 32 + (lane & 31)
                          : vt * kLmVT + wave * kLmVA * 32 + a * 32 + (lane & 31);
    const uint16_t* src = (w2 && a == 1) ? w2 : w;
    const int k = slab * kLmKS + (run % 4) * 16 + (lane >> 5) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < static_cast<size_t>(N)) v = *reinterpret_cast<const uint4*>(src + row * K + k);
    *reinterpret_cast<uint4*>(packed + c * 8) = v;
  }
}

__global__ __launch_bounds__(kCompactThreads) void compact_rows_kernel(
    int rows, int R, int W, int D, const int32_t* __restrict__ cand_len,
    const uint8_t* __restrict__ copy_gate, int32_t* __restrict__ row_list,
    int32_t* __restrict__ inv, int32_t* __restrict__ n_rows, unsigned long long* __restrict__ keys) {
  __shared__ int s_wave[kCompactThreads / kWave];
  compact_rows_body<kCompactThreads>(rows, R, W, D, cand_len, copy_gate, row_list, inv, n_rows, s_wave,
                                     keys);
}

// One wave per sequence: the argmax of each of its R rows from the row's key (the
// low half of a nonzero key is the complemented index; 0, the value the keys start
// from, stays on rows that are not real and on real rows whose logits are all NaN:
// -1); then, when asked, the sequence's accept on those rows, which reads them
// from LDS.
__global__ __launch_bounds__(kWave) void argmax_finish_kernel(
    const unsigned long long* __restrict__ keys, int R, int32_t* __restrict__ argmax_out,
    AcceptArgs acc) {
  __shared__ int s_am[1 + SSD_MAX_W * SSD_MAX_D];
  __shared__ int s_pred[SSD_MAX_W][kWave];
  const int b = blockIdx.x, lane = threadIdx.x;
  // Only the low halves are read: a key's low half is the complemented index, and
  // the key 0 (no value) has low half 0, whose complement is the -1 reported then.
  const uint32_t* kb = reinterpret_cast<const uint32_t*>(keys + static_cast<size_t>(b) * R);
  int32_t* ob = argmax_out + static_cast<size_t>(b) * R;
  constexpr int kU = 8;  // keys in flight per lane
  uint32_t k[kU];
  auto load_keys = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int r = r0 + u * kWave + lane;
      k[u] = kb[2 * static_cast<size_t>(r < R ? r : R - 1)];
    }
  };
  load_keys(0);
  // the accept's own inputs are requested with the first keys (one wait for both)
  AcceptPre pre{};
  if (acc.cand != nullptr) {
    pre = accept_prefetch(b, lane, acc.cand, acc.cand_len, acc.copy_gate, acc.W, acc.D);
    asm volatile("" ::"v"(pre.gate), "v"(pre.len_lane));
#pragma unroll
    for (int u = 0; u < kAcGroup; ++u) asm volatile("" ::"v"(pre.c[u]));
  }
  for (int r0 = 0; r0 < R; r0 += kU * kWave) {
    if (r0 > 0) load_keys(r0);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int r = r0 + u * kWave + lane;
      if (r >= R) break;
      const int v = static_cast<int>(~k[u]);
      ob[r] = v;
      s_am[r] = v;
    }
  }
  if (acc.cand == nullptr) return;
  __syncthreads();
  accept_run(pre, b, lane, acc.cand, s_am, acc.W, acc.D, acc.accept_len, acc.best_w, acc.best_len,
             acc.next_token, s_pred);
}

// One wave per row: merges the row's per-tile (max, sum-exp, best score, best
// token) over the vocabulary tiles into lse = logsumexp(logits / T) and the
// residual draw.  The (max, sum) pairs are in base 2: max of t*log2(e) and the
// sum of 2^(t*log2(e) - max).  Rows that are not real get lse = -inf and draw -1.
__global__ __launch_bounds__(256) void sample_reduce_kernel(const float4* __restrict__ part,
                                                            int vtiles, int rows,
                                                            const int32_t* __restrict__ inv,
                                                            float* __restrict__ lse,
                                                            int32_t* __restrict__ resample) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (row >= rows) return;
  const int ci = inv[row];
  if (ci < 0) {
    if (lane == 0) {
      lse[row] = -INFINITY;
      resample[row] = -1;
    }
    return;
  }
  float m = -INFINITY, s = 0.f, by = -INFINITY;
  int bx = INT_MAX;
  const float4* pr = part + static_cast<size_t>(ci) * vtiles;
  for (int t0 = 0; t0 < vtiles; t0 += 4 * kWave) {
    float4 p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * kWave + lane;
      p[u] = t < vtiles ? pr[t] : make_float4(-INFINITY, 0.f, -INFINITY, __int_as_float(INT_MAX));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      lse2_merge(m, s, p[u].x, p[u].y);
      const int x = __float_as_int(p[u].w);
      if (better(p[u].z, x, by, bx)) { by = p[u].z; bx = x; }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, kWave), os = __shfl_xor(s, o, kWave);
    const float oy = __shfl_xor(by, o, kWave);
    const int ox = __shfl_xor(bx, o, kWave);
    lse2_merge(m, s, om, os);
    if (better(oy, ox, by, bx)) { by = oy; bx = ox; }
  }
  if (lane == 0) {
    lse[row] = (m + log2f(s)) * 0.69314718f;   // base-2 pair -> natural log-sum-exp
    resample[row] = bx == INT_MAX ? -1 : bx;
  }
}

namespace {
// bf16 tiling of `vtiles` vocabulary (feature) tiles over the row chunks
LmPlan plan_for(int rows, int vtiles) {
  LmPlan p;
  p.vtiles = vtiles;
  p.mchunks = (rows + kLmMC - 1) / kLmMC;
  p.sm = p.mchunks < 8 ? p.mchunks : 8;
  p.sv = kLmXcdSlots / p.sm;
  // narrow matrices: smaller super-tiles, so that every XCD gets some
  const int spread = (vtiles + kLmXcds - 1) / kLmXcds;
  if (p.sv > spread) p.sv = spread;
  const int n_super = ((p.vtiles + p.sv - 1) / p.sv) * ((p.mchunks + p.sm - 1) / p.sm);
  p.blocks = kLmXcds * ((n_super + kLmXcds - 1) / kLmXcds) * p.sv * p.sm;
  return p;
}
}  // namespace

LmPlan lm_plan(int rows, int V, bool bf16) {
  if (bf16) return plan_for(rows, (V + kLmVT - 1) / kLmVT);
  LmPlan p;
  p.vtiles = (V + kLmF32VT - 1) / kLmF32VT;
  p.mchunks = (rows + kLmF32Rows - 1) / kLmF32Rows;
  // super-tiles of one XCD's worth of workgroups (bf16 path)
  p.sm = p.mchunks < 8 ? p.mchunks : 8;
  p.sv = kLmXcdSlots / p.sm;
  const int n_super = ((p.vtiles + p.sv - 1) / p.sv) * ((p.mchunks + p.sm - 1) / p.sm);
  p.blocks = kLmXcds * ((n_super + kLmXcds - 1) / kLmXcds) * p.sv * p.sm;
  return p;
}

// LM-head workspace: [n_rows (256 B)] [row_list: rows ints] [inv: rows ints]
// [tile partials: rows x vtiles x 16 B], each region 256-byte aligned.
namespace {
size_t al256(size_t x) { return (x + 255) / 256 * 256; }
struct LmWs {
  int32_t* n_rows;
  int32_t* row_list;
  int32_t* inv;
  int2* part;
  unsigned long long* keys;  // greedy (both dtypes): a key per row at the start of the partials region
};
LmWs lm_ws(void* ws, int rows) {
  char* p = static_cast<char*>(ws);
  LmWs w;
  w.n_rows = reinterpret_cast<int32_t*>(p);
  p += 256;
  w.row_list = reinterpret_cast<int32_t*>(p);
  p += al256(sizeof(int32_t) * rows);
  w.inv = reinterpret_cast<int32_t*>(p);
  p += al256(sizeof(int32_t) * rows);
  w.part = reinterpret_cast<int2*>(p);
  w.keys = reinterpret_cast<unsigned long long*>(p);
  return w;
}
}  // namespace

// The partials region: 16 bytes per (row, tile) when sampling (max, sum-exp, best
// score, best token); a greedy launch uses only its first 8 bytes per row (the keys).
LmWsView lm_ws_view(void* ws, int rows) {
  const LmWs w = lm_ws(ws, rows);
  return LmWsView{w.n_rows, w.row_list, w.inv, w.keys};
}

size_t lm_workspace_bytes(const LmPlan& p, int rows) {
  return 256 + 2 * al256(sizeof(int32_t) * rows) + static_cast<size_t>(p.vtiles) * rows * sizeof(float4);
}

// Launch the bf16 kernel with epilogue kEpi; the nontemporal weight loads when the
// launch has one row chunk.
template <int kEpi, bool kRows = false, typename... Args>
static void launch_bf16(const LmPlan& plan, dim3 grid, hipStream_t s, Args... args) {
  if (plan.mchunks == 1)
    hipLaunchKernelGGL((lmhead_bf16_kernel<kEpi, true, kRows>), grid, dim3(256), 0, s, args...);
  else
    hipLaunchKernelGGL((lmhead_bf16_kernel<kEpi, false, kRows>), grid, dim3(256), 0, s, args...);
}

hipError_t launch_compact_rows(void* ws, int rows, int R, int W, int D, const int32_t* cand_len,
                               const uint8_t* copy_gate, hipStream_t s) {
  const LmWs w = lm_ws(ws, rows);
  hipLaunchKernelGGL(compact_rows_kernel, dim3(1), dim3(kCompactThreads), 0, s, rows, R, W, D,
                     cand_len, copy_gate, w.row_list, w.inv, w.n_rows, w.keys);
  return hipGetLastError();
}

hipError_t launch_lmhead(const void* attn_out, const void* lm_head, int rows, int hid, int V,
                         bool bf16, const LmPlan& plan, float* logits_out, void* ws,
                         hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t s,
                         const SampleArgs* sample, bool rows_layout) {
  const LmWs w = lm_ws(ws, rows);
  if (rows_layout && (!bf16 || sample != nullptr)) return hipErrorInvalidValue;
  if (ev_begin && hipEventRecord(ev_begin, s) != hipSuccess) return hipErrorInvalidValue;
  if (rows_layout)
    launch_bf16<kEpiArgmax, true>(plan, dim3(plan.blocks), s,
                       static_cast<const uint16_t*>(attn_out), static_cast<const uint16_t*>(lm_head),
                       rows, hid, V, w.row_list, w.n_rows, logits_out, static_cast<void*>(w.keys),
                       plan.vtiles, plan.mchunks, plan.sv, plan.sm, SampleArgs{}, GemmArgs{});
  else if (bf16 && sample)
    launch_bf16<kEpiSample>(plan, dim3(plan.blocks), s,
                       static_cast<const uint16_t*>(attn_out), static_cast<const uint16_t*>(lm_head),
                       rows, hid, V, w.row_list, w.n_rows, logits_out, static_cast<void*>(w.part),
                       plan.vtiles, plan.mchunks, plan.sv, plan.sm, *sample, GemmArgs{});
  else if (bf16)
    launch_bf16<kEpiArgmax>(plan, dim3(plan.blocks), s,
                       static_cast<const uint16_t*>(attn_out), static_cast<const uint16_t*>(lm_head),
                       rows, hid, V, w.row_list, w.n_rows, logits_out, static_cast<void*>(w.keys),
                       plan.vtiles, plan.mchunks, plan.sv, plan.sm, SampleArgs{}, GemmArgs{});
  else
    hipLaunchKernelGGL(lmhead_f32_kernel, dim3(plan.mchunks, plan.vtiles), dim3(256), 0, s,
                       static_cast<const float*>(attn_out), static_cast<const float*>(lm_head), hid,
                       V, w.row_list, w.n_rows, rows, logits_out, w.keys);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev_end && hipEventRecord(ev_end, s) != hipSuccess) return hipErrorInvalidValue;
  return e;
}

size_t packed_weight_bytes(int N, int K, bool pair) {
  const int tile = pair ? kLmVT / kLmVA : kLmVT;   // rows (features) per 256-row packed tile
  return static_cast<size_t>((N + tile - 1) / tile) * kLmVT * K * 2;
}

int lm_k_align() { return kLmKAlign; }

hipError_t launch_pack_weight(const void* w, const void* w2, int N, int K, void* packed,
                              hipStream_t s) {
  const size_t n_chunks = packed_weight_bytes(N, K, w2 != nullptr) / 16;
  const size_t want = (n_chunks + 255) / 256;
  const int blocks = static_cast<int>(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(pack_weight_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const uint16_t*>(w), static_cast<const uint16_t*>(w2), N, K,
                     static_cast<uint16_t*>(packed), n_chunks);
  return hipGetLastError();
}

hipError_t launch_argmax_finish(void* ws, int B, int R, int32_t* argmax_out, const AcceptArgs* accept,
                                hipStream_t s) {
  const LmWs w = lm_ws(ws, B * R);
  hipLaunchKernelGGL(argmax_finish_kernel, dim3(B), dim3(kWave), 0, s, w.keys, R, argmax_out,
                     accept != nullptr ? *accept : AcceptArgs{});
  return hipGetLastError();
}

hipError_t launch_sample_reduce(void* ws, const LmPlan& plan, int rows, float* lse,
                                int32_t* resample, hipStream_t s) {
  const LmWs w = lm_ws(ws, rows);
  hipLaunchKernelGGL(sample_reduce_kernel, dim3((rows + 3) / 4), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(w.part), plan.vtiles, rows, w.inv, lse, resample);
  return hipGetLastError();
}

}  // namespace ssd

namespace ssd {

LmPlan gemm_plan(int rows, int N, bool swiglu) {
  if (swiglu) return plan_for(rows, (N + kLmVT / kLmVA - 1) / (kLmVT / kLmVA));
  // A projection whose 256-row tiles fill fewer than half the CUs needs many
  // K splits to keep every CU streaming, and each split writes a full tile of
  // fp32 partial sums.  Half tiles (one A tile per wave) give twice the tiles,
  // so half the splits and half the partial sums.
  const int full = (N + kLmVT - 1) / kLmVT;
  const int mchunks = (rows + kLmMC - 1) / kLmMC;
  const bool half = full * mchunks < 128;
  LmPlan p = plan_for(rows, half ? 2 * full : full);
  p.half = half ? 1 : 0;
  return p;
}

hipError_t launch_gemm(const void* rows_in, const void* w, int total_rows, int K, int N,
                       const LmPlan& plan, int splits, bool swiglu, const void* lm_ws_ptr, float* part,
                       uint16_t* out, int ld, hipStream_t s) {
  const LmWs lw = lm_ws(const_cast<void*>(lm_ws_ptr), total_rows);
  GemmArgs ga{};
  ga.kc = K / splits;
  ga.part = part;
  ga.part_rows = total_rows;
  ga.ld = ld;
  ga.out = out;
  ga.row_list = lw.row_list;
  const dim3 grid(plan.blocks, splits);
  if (swiglu)
    launch_bf16<kEpiSwiGLU>(plan, grid, s,
                       static_cast<const uint16_t*>(rows_in), static_cast<const uint16_t*>(w), total_rows,
                       K, N, lw.row_list, lw.n_rows, nullptr, nullptr, plan.vtiles, plan.mchunks,
                       plan.sv, plan.sm, SampleArgs{}, ga);
  else if (plan.half)
    launch_bf16<kEpiPartialHalf>(plan, grid, s,
                       static_cast<const uint16_t*>(rows_in), static_cast<const uint16_t*>(w), total_rows,
                       K, N, lw.row_list, lw.n_rows, nullptr, nullptr, plan.vtiles, plan.mchunks,
                       plan.sv, plan.sm, SampleArgs{}, ga);
  else
    launch_bf16<kEpiPartial>(plan, grid, s,
                       static_cast<const uint16_t*>(rows_in), static_cast<const uint16_t*>(w), total_rows,
                       K, N, lw.row_list, lw.n_rows, nullptr, nullptr, plan.vtiles, plan.mchunks,
                       plan.sv, plan.sm, SampleArgs{}, ga);
  return hipGetLastError();
}

hipError_t launch_gemm_pair(const void* rows_in, const void* w_gate_up, int total_rows, int K, int N,
                            const LmPlan& plan, int splits, const void* lm_ws_ptr, float* part,
                            hipStream_t s) {
  const LmWs lw = lm_ws(const_cast<void*>(lm_ws_ptr), total_rows);
  GemmArgs ga{};
  ga.kc = K / splits;
  ga.part = part;
  ga.part_rows = total_rows;
  ga.ld = 2 * N;
  ga.row_list = lw.row_list;
  launch_bf16<kEpiPair>(plan, dim3(plan.blocks, splits), s,
                     static_cast<const uint16_t*>(rows_in), static_cast<const uint16_t*>(w_gate_up),
                     total_rows, K, N, lw.row_list, lw.n_rows, nullptr, nullptr, plan.vtiles,
                     plan.mchunks, plan.sv, plan.sm, SampleArgs{}, ga);
  return hipGetLastError();
}

}  // namespace ssd
