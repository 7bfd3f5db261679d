// Block-triangular verification attention (SwitchSD paper §3.3 "Parallel
// Verification with Block-Triangular Attention"; write-up §2.6).
//
// Every query row of a sequence sees the whole prefix; row (w, j) additionally
// sees candidate keys (w, 0..j).  The pass is split accordingly:
//   1. prefix sweep: attention of all real rows against key ranges ("slots",
//      flash-decoding style partials m, l, o in the exp2 domain).  bf16 runs on
//      32x32x16 MFMA with the g query heads of one KV head packed together (g*R
//      rows share one K/V stream); the prefix is split into ranges, and one more
//      slot holds the W*D candidate keys, where each row's visible range
//      (w*D .. w*D + j) is applied to the scores in registers.  fp32 runs the
//      prefix ranges on the vector ALU.
//   2. merge: per (row, head) the partials are combined and the normalised
//      output is written (fp32: the row's own candidate triangle, at most D keys,
//      is folded in exactly here).  Rows that are not real are written as 0.
// No mask is ever materialised in memory.
#include "common.h"
#include "kernels.h"

namespace ssd {

// ----------------------------------------------------------------- bf16 MFMA
constexpr int kAttD = 128;          // head dim of the MFMA path
constexpr int kKB = 64;             // keys per LDS block
constexpr int kAttWaves = 8;        // one 32-row MFMA tile per wave, two waves per SIMD
constexpr int kAttThreads = kAttWaves * kWave;
constexpr int kAttRowsPerBlock = kAttWaves * 32;                 // 256 (row, head) rows
constexpr int kStage = kKB * kAttD;                              // bf16 per K or V stage (16 KB)
constexpr int kDmaPerWave = kStage * 2 / 16 / kWave / kAttWaves; // 16-byte copies per wave and stage (2)
constexpr int kXcds = 8;            // workgroups are dealt round-robin over the 8 XCDs
constexpr float kFreeRange = 32.f;  // scores may exceed the running max by 2^32 before it moves
constexpr int kAhead = 2;           // LDS fragment reads in flight ahead of their MFMA
constexpr int kOutOfRange = 0x7ffffff0;
constexpr int kPersistCus = 256;    // persistent grid: one workgroup per CU

// LDS layouts (16-byte chunks, 16 per 256-byte key row, no padding).  The LDS
// serves 64 banks of 4 bytes (256 bytes) per cycle and a 256-byte row starts at
// bank 0, so the accesses served together must fall on distinct chunk positions:
//  * K: chunk c of key k sits at position c ^ (k & 15).  The S MFMA's A operand
//    reads one chunk of 32 consecutive keys; every 16 consecutive lanes hit the 16
//    positions of a row once.
//  * V: chunk c of key k sits at position c ^ 4(k & 3).  A transposing read of the
//    O MFMA's A operand takes, per half wave, the four chunks of a 32-wide d tile
//    of 4 consecutive keys; the 16 chunks land on the 16 positions once.
__device__ __forceinline__ int k_pos(int key, int c) { return c ^ (key & 15); }
__device__ __forceinline__ int v_pos(int key, int c) { return c ^ ((key & 3) << 2); }

using v4i16 = __attribute__((ext_vector_type(4))) short;
using lds_v4i16 = __attribute__((address_space(3))) v4i16;
using bf16x2 = __attribute__((ext_vector_type(2))) __bf16;

// What one wave needs to stream the workgroup's key range.
struct AttnCtx {
  __amdgpu_buffer_rsrc_t kres, vres;
  int key_bytes;             // bytes per key (all kv heads)
  int k0;                    // first key of the range
  int wave, lane, l32, h;
  int koff[kDmaPerWave], voff[kDmaPerWave];  // this lane's copy offsets within a block
};

// Copy keys key0 .. key0+63 of K (or V) into an LDS stage: this wave's share, two
// 1 KB copies at the offsets dma_offsets computed.
template <bool kV>
__device__ __forceinline__ void dma_stage(const AttnCtx& c, uint16_t* st, int key0, bool past) {
  const int kb = key0 * c.key_bytes;   // wave-uniform
#pragma unroll
  for (int u = 0; u < kDmaPerWave; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        kV ? c.vres : c.kres,
        (__attribute__((address_space(3))) void*)(st + (c.wave * kDmaPerWave + u) * kWave * 8), 16,
        past ? kOutOfRange : kb + (kV ? c.voff[u] : c.koff[u]), 0, 0, 0);
}

// This lane's offsets of its copies within a block (see dma_stage): unit p of the
// stage is key p / 16 at position p % 16, which receives that key's chunk at the
// position (the swizzles are involutions).
__device__ __forceinline__ void dma_offsets(AttnCtx& c, int kvo) {
#pragma unroll
  for (int u = 0; u < kDmaPerWave; ++u) {
    const int p = (c.wave * kDmaPerWave + u) * kWave + c.lane;
    const int key = p >> 4, pos = p & 15;
    c.koff[u] = key * c.key_bytes + kvo + k_pos(key, pos) * 16;
    c.voff[u] = key * c.key_bytes + kvo + v_pos(key, pos) * 16;
  }
}

// S MFMA A operand: keys 32 kt + l32, d chunk 2 s + h (d 16 s + 8 h .. + 7).
__device__ __forceinline__ bf16x8 k_frag(const uint16_t* st, int i, int l32, int h) {
  const int kt = i & 1, s = i >> 1;
  const int key = kt * 32 + l32;
  return *reinterpret_cast<const bf16x8*>(st + key * kAttD + k_pos(key, 2 * s + h) * 8);
}

// O MFMA A operand V^T for key step ks (16 keys) and d tile dt: lane (l32, h) gets d
// = 32 dt + l32 and keys 16 ks + {4h .. 4h+3, 8+4h .. 8+4h+3}, the order in which the
// S accumulator holds them (elements 8 s2 .. 8 s2 + 7 of subtile ks / 2, s2 = ks % 2).
// Two transposing reads: in read t, 16-lane group G sends lane 4e + c to key
// 16 ks + 8 t + 4 (G >> 1) + e, d 32 dt + 16 (G & 1) + 4 c .. + 3; the read returns to
// lane i of the group column i & 3 of lanes (i >> 2) + 4e, e = 0..3.
__device__ __forceinline__ bf16x8 v_frag(const uint16_t* st, int ks, int dt, int lane) {
  const int G = lane >> 4, i = lane & 15, e = i >> 2, cc = i & 3;
  const int d0 = dt * 32 + 16 * (G & 1) + 4 * cc;
  const int ch = d0 >> 3, sub = d0 & 7;
  v4i16 r[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = ks * 16 + 8 * t + 4 * (G >> 1) + e;
    r[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(st + key * kAttD + v_pos(key, ch) * 8 + sub));
  }
  struct Two { v4i16 a, b; } two{r[0], r[1]};
  return __builtin_bit_cast(bf16x8, two);
}

// The wave's tile: 32 (row, head) rows.
struct AttnRows {
  bf16x8 q[8];            // B operand of S^T = K Q^T: Q[row][16 s + 8 h .. + 7]
  f32x16 o[4];            // O^T[d][row], d tile dt
  float m, l;             // running max (scaled, base 2) and this lane's half of the sum
  float alpha;            // pending rescale of o (applied before the next O MFMAs)
  bool pend;
};

// Row maximum of a block of scores (both halves of the row), scaled.
// The scores are MFMA results or -inf, so the raw maximum instructions serve.
__device__ __forceinline__ float block_max(const f32x16 (&s)[2], float scale) {
  float t1[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int a = 3 * i, b = a + 1, c = a + 2;
    t1[i] = vmax3_raw(s[a >> 4][a & 15], s[b >> 4][b & 15], s[c >> 4][c & 15]);
  }
  t1[10] = vmax2_raw(s[1][14], s[1][15]);
  const float t2 = vmax3_raw(vmax3_raw(t1[0], t1[1], t1[2]), vmax3_raw(t1[3], t1[4], t1[5]),
                             vmax3_raw(t1[6], t1[7], t1[8]));
  float mx = vmax3_raw(t2, t1[9], t1[10]);
  mx = vmax2_raw(mx, __shfl_xor(mx, 32, kWave));
  return mx * scale;   // scale > 0: the max commutes with it
}

// Moves the running max when the block's scores exceed it by more than 2^range
// (always for the first block with a visible key): l is rescaled at once, o before
// it next accumulates (O MFMAs still pending use the old max).
__device__ __forceinline__ void move_max(AttnRows& R, float mb, float range) {
  const bool need = mb > R.m + range || (R.m == -INFINITY && mb != -INFINITY);
  if (__ballot(need)) {
    const float m_new = need ? mb : R.m;
    const float a = R.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(R.m - m_new);
    R.m = m_new;
    R.l *= a;
    R.alpha = R.pend ? R.alpha * a : a;
    R.pend = true;
  }
}

__device__ __forceinline__ void apply_pending(AttnRows& R) {
  if (R.pend) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) R.o[dt][r] *= R.alpha;
    R.pend = false;
  }
}

// p = 2^(scale s - m) in place (a row without a visible key yet has m = -inf: it
// exponentiates against 0, its scores are -inf and every p is 0).
__device__ __forceinline__ void exp_in_place(f32x16 (&s)[2], float scale, float m) {
  const float nm = m == -INFINITY ? 0.f : -m;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], scale, nm));
}

// Pack probabilities to the O MFMA's bf16 B operand; returns the sum of the packed
// values (dot products with (1, 1)), the half-row sum this lane contributes to l.
__device__ __forceinline__ float pack_p(const f32x16 (&s)[2], bf16x8 (&p)[2][2]) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float sum = 0.f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      uint32_t w[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const bf16x2 pr = {static_cast<__bf16>(s[kt][8 * s2 + 2 * e2]),
                           static_cast<__bf16>(s[kt][8 * s2 + 2 * e2 + 1])};
        w[e2] = __builtin_bit_cast(uint32_t, pr);
        sum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, sum, false);
      }
      p[kt][s2] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
  return sum;
}

// Scores of keys a row may not see become -inf: keys at or past k1 and, in the
// candidate slot, keys outside [vis_lo, vis_hi] (the row's own candidate prefix).
// kb is the block's first key; lane half h holds keys kb + 32 kt + 8 (r / 4) + 4 h + r % 4.
__device__ __forceinline__ void mask_block(f32x16 (&s)[2], int kb, int k1, int h, bool cand,
                                           int vis_lo, int vis_hi) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + kt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      const bool vis = key < k1 && (!cand || (key >= vis_lo && key <= vis_hi));
      s[kt][r] = vis ? s[kt][r] : -INFINITY;
    }
}

// S^T of the tile from one K stage: 16 fragments, one MFMA each.
__device__ __forceinline__ void s_mfmas(const uint16_t* kst, const AttnRows& R, f32x16 (&s)[2],
                                        int l32, int h) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
  bf16x8 f[kAhead + 1];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) f[i] = k_frag(kst, i, l32, h);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + kAhead < 16) f[(i + kAhead) % (kAhead + 1)] = k_frag(kst, i + kAhead, l32, h);
    s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i % (kAhead + 1)], R.q[i >> 1], s[i & 1], 0, 0, 0);
  }
}

// O^T += V^T P^T from one V stage: 16 fragments (4 key steps x 4 d tiles).
__device__ __forceinline__ void o_mfmas(const uint16_t* vst, AttnRows& R, const bf16x8 (&p)[2][2],
                                        int lane) {
  bf16x8 f[kAhead + 1];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) f[i] = v_frag(vst, i >> 2, i & 3, lane);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int ks = i >> 2, dt = i & 3;
    if (i + kAhead < 16) {
      const int j = i + kAhead;
      f[j % (kAhead + 1)] = v_frag(vst, j >> 2, j & 3, lane);
    }
    R.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i % (kAhead + 1)], p[ks >> 1][ks & 1], R.o[dt], 0, 0, 0);
  }
}

// The worker: the wave's tile (kRows) or none (the wave still issues its share of
// every copy and passes every barrier) over the workgroup's key range.
//
// The range's 64-key blocks run in a two-block pipeline.  Iteration j: the running max is
// checked against block j's scores; then, while the vector ALU exponentiates them,
// the matrix core runs the O MFMAs of block j-1 and the S MFMAs of block j+1, and
// block j's probabilities are packed once block j-1's O MFMAs hold no reference to
// the packed buffer.  Copies: iteration j copies K of block j+4 and V of block j+2
// (four stages each); K of block j+1 and V of block j-1 are read in iteration j,
// and a stage is rewritten only after the barrier that follows its last read.
// Blocks past the last one are copied as zeros (offsets past the buffers) and their
// products are discarded; keys past the last one of the buffer read as zero too.
//
// Masks: in a partial last block of the prefix, keys past the range; in the
// candidate slot, every key outside the row's own candidate prefix.  Both are
// applied to the block's scores before the running max sees them.
template <bool kRows>
__device__ __forceinline__ void attn_worker(const AttnCtx& c, AttnRows& R, uint16_t* k0s,
                                            uint16_t* k1s, uint16_t* k2s, uint16_t* k3s,
                                            uint16_t* v0s, uint16_t* v1s, uint16_t* v2s,
                                            uint16_t* v3s, int nb, int k1, int vis_lo, int vis_hi,
                                            bool cand, float scale) {
  uint16_t* const ks[4] = {k0s, k1s, k2s, k3s};
  uint16_t* const vs[4] = {v0s, v1s, v2s, v3s};
  const int k0 = c.k0;
  auto issue = [&](auto Kc, auto Vc, int xk, int xv) {
    dma_stage<false>(c, ks[decltype(Kc)::value], k0 + xk * kKB, xk >= nb);
    dma_stage<true>(c, vs[decltype(Vc)::value], k0 + xv * kKB, xv < 0 || xv >= nb);
  };
  constexpr int kPer = 2 * kDmaPerWave;   // copies per wave per issue slot
  if (nb > 0) {
    f32x16 s[2][2];                       // scores of block x in s[x % 2]
    // packed probabilities of the block whose O MFMAs are next; zero for block -1,
    // whose V stage is zeros
    bf16x8 p[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int a2 = 0; a2 < 2; ++a2) p[a][a2] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    // issue slots -4 .. -1: K of blocks 0..3, V of blocks -2..1
    issue(IntC<0>{}, IntC<2>{}, 0, -2);
    issue(IntC<1>{}, IntC<3>{}, 1, -1);
    issue(IntC<2>{}, IntC<0>{}, 2, 0);
    issue(IntC<3>{}, IntC<1>{}, 3, 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * kPer));
    lds_barrier();
    if constexpr (kRows) s_mfmas(k0s, R, s[0], c.l32, c.h);
    // iteration j (U = j % 4): reads K of j+1 (stage (U+1) % 4), V of j-1 (stage
    // (U+3) % 4); copies K of j+4 into stage U and V of j+2 into stage (U+2) % 4
    auto iter = [&](auto Uc, int j) {
      constexpr int U = decltype(Uc)::value;
      constexpr int cur = U & 1, nxt = cur ^ 1;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kPer));
      lds_barrier();
      issue(IntC<U>{}, IntC<(U + 2) % 4>{}, j + 4, j + 2);
      if constexpr (kRows) {
        apply_pending(R);                 // a max moved by block j-1: before its O MFMAs
        const bool live = j < nb;
        if (live && (cand || k0 + (j + 1) * kKB > k1))
          mask_block(s[cur], k0 + j * kKB, k1, c.h, cand, vis_lo, vis_hi);
        if (live) move_max(R, block_max(s[cur], scale), kFreeRange);
        exp_in_place(s[cur], scale, R.m);
        o_mfmas(vs[(U + 3) % 4], R, p, c.lane);
        s_mfmas(ks[(U + 1) % 4], R, s[nxt], c.l32, c.h);
        const float sum = pack_p(s[cur], p);
        R.l += live ? sum : 0.f;
        // schedule: each O MFMA with its fragment's two transposing reads and two
        // vector instructions, each S MFMA with its fragment read and four, so that
        // block j's exponentials and packing spread over the whole MFMA stream
        // (with four per O MFMA they all landed among the O MFMAs and the S MFMAs ran
        // bare: 2-4% slower at batch 32 and at the 70B share)
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i + kAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i + kAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
    };
    for (int j0 = 0; j0 <= nb; j0 += 4) {
      iter(IntC<0>{}, j0);
      if (j0 + 1 > nb) break;
      iter(IntC<1>{}, j0 + 1);
      if (j0 + 2 > nb) break;
      iter(IntC<2>{}, j0 + 2);
      if (j0 + 3 > nb) break;
      iter(IntC<3>{}, j0 + 3);
    }
    if constexpr (kRows) apply_pending(R);
    // the copies of blocks past the range still in flight land before the
    // workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// One work item (see attn_prefix_bf16_kernel): returns at once when it has nothing
// to contribute.
__device__ __forceinline__ void attn_item(
    int idx, int xcd, uint16_t* ks0, uint16_t* ks1, uint16_t* ks2, uint16_t* ks3, uint16_t* vs0,
    uint16_t* vs1, uint16_t* vs2, uint16_t* vs3, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_pre, const uint16_t* __restrict__ v_pre,
    const int32_t* __restrict__ cu_len, const uint16_t* __restrict__ k_cand,
    const uint16_t* __restrict__ v_cand, const uint8_t* __restrict__ copy_gate,
    const int32_t* __restrict__ cand_len, int B, int R, int Hq, int Hkv, int W, int D, int nsplit,
    int chunk, int qtiles, float scale_log2, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o) {
  const int nslots = nsplit + 1;
  const int bkn = B * Hkv, per_x = (bkn + kXcds - 1) / kXcds;
  const int qtile = idx % qtiles;
  const int slot = (idx / qtiles) / per_x, qx = (idx / qtiles) % per_x;
  const int bk = qx * kXcds + xcd;
  if (slot >= nslots || bk >= bkn) return;
  const int b = bk / Hkv, kvh = bk % Hkv;
  if (copy_gate[b] == 0) return;
  const int base = cu_len[b];
  const int n_b = cu_len[b + 1] - base;
  const bool cand = slot == nsplit;
  int k0, k1, nkeys;
  const uint16_t *kp, *vp;
  if (cand) {
    k0 = 0;
    k1 = nkeys = W * D;
    kp = k_cand + static_cast<size_t>(b) * W * D * Hkv * kAttD;
    vp = v_cand + static_cast<size_t>(b) * W * D * Hkv * kAttD;
  } else {
    k0 = slot * chunk;
    if (k0 >= n_b) return;
    k1 = slot == nsplit - 1 ? n_b : min(k0 + chunk, n_b);
    nkeys = n_b;
    kp = k_pre + static_cast<size_t>(base) * Hkv * kAttD;
    vp = v_pre + static_cast<size_t>(base) * Hkv * kAttD;
  }
  const int nb = (k1 - k0 + kKB - 1) / kKB;   // blocks of the range, the last one maybe partial

  const int g = Hq / Hkv, G = R * g;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  // wave index in a scalar register: the LDS destination of a copy must be wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  AttnCtx c;
  // keys of this sequence (or its candidates); keys past the last one read as zero
  // and never touch the memory after it
  c.key_bytes = Hkv * kAttD * 2;
  c.kres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kp), 0, nkeys * c.key_bytes, kBufFlags);
  c.vres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vp), 0, nkeys * c.key_bytes, kBufFlags);
  c.k0 = k0;
  c.wave = wave;
  c.lane = lane;
  c.l32 = lane & 31;
  c.h = lane >> 5;
  dma_offsets(c, kvh * kAttD * 2);

  // this wave's tile; a tile whose rows are all padding (candidates past M, tokens
  // past L_w) does no arithmetic
  const int i_row = qtile * kAttRowsPerBlock + wave * 32 + c.l32;
  const bool row_ok = i_row < G;
  const int r_row = row_ok ? i_row / g : 0, hh = row_ok ? i_row - r_row * g : 0;
  const bool row_real = row_ok && real_row(r_row, D, cand_len + static_cast<size_t>(b) * W, true);
  // a workgroup without a real row has nothing to contribute (the merge reads
  // partials of real rows only)
  if (!__syncthreads_or(row_real)) return;
  const bool has = __ballot(row_real) != 0;
  // candidate mask of this row: keys cw*D .. cw*D + cj (none for the anchor row)
  const int cw = r_row > 0 ? (r_row - 1) / D : -1;
  const int cj = r_row > 0 ? (r_row - 1) - cw * D : -1;
  const int vis_lo = cw >= 0 ? cw * D : 1;
  const int vis_hi = cw >= 0 ? cw * D + cj : 0;

  AttnRows Rw;
  if (!has) {
    attn_worker<false>(c, Rw, ks0, ks1, ks2, ks3, vs0, vs1, vs2, vs3, nb, k1, vis_lo, vis_hi, cand,
                       scale_log2);
    return;
  }
  {
    const uint16_t* qp = q + ((static_cast<size_t>(b) * R + r_row) * Hq + kvh * g + hh) * kAttD + 8 * c.h;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qp + 16 * s) : make_uint4(0, 0, 0, 0);
      Rw.q[s] = __builtin_bit_cast(bf16x8, u);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) Rw.o[dt][r] = 0.f;
    Rw.m = -INFINITY;
    Rw.l = 0.f;
    Rw.alpha = 1.f;
    Rw.pend = false;
  }
  attn_worker<true>(c, Rw, ks0, ks1, ks2, ks3, vs0, vs1, vs2, vs3, nb, k1, vis_lo, vis_hi, cand,
                    scale_log2);
  const float l_tot = Rw.l + __shfl_xor(Rw.l, 32, kWave);
  if (!row_ok) return;
  const size_t po = ((static_cast<size_t>(slot) * B + b) * R + r_row) * Hq + kvh * g + hh;
  if (c.h == 0) {
    ws_m[po] = Rw.m;
    ws_l[po] = l_tot;
  }
  float* op = ws_o + po * kAttD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = dt * 32 + 8 * rq + 4 * c.h;
      *reinterpret_cast<float4*>(op + d0) =
          make_float4(Rw.o[dt][4 * rq], Rw.o[dt][4 * rq + 1], Rw.o[dt][4 * rq + 2], Rw.o[dt][4 * rq + 3]);
    }
}

// One workgroup = 256 query rows (the g query heads of one KV head packed together,
// one tile of 32 per wave) x one key range of one sequence.  Key ranges ("slots")
// 0..nsplit-1 split the prefix; slot nsplit holds the W*D candidate keys, where row
// (w, j) may only see keys (w, 0..j).  Each slot leaves a partial (running max m,
// sum l, unnormalised o) in the workspace, in the exp2 domain; the merge kernel
// combines them.
//
// Grid: the (sequence, kv head, slot) groups are dealt to XCDs so that all row
// tiles of a group share one XCD's L2 (they read the same keys).  With
// compact.row_list set, the grid has one more workgroup, the last, which writes the
// compact list of real rows for the LM head while the others attend.
__global__ __launch_bounds__(kAttThreads, 1) void attn_prefix_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pre,
    const uint16_t* __restrict__ v_pre, const int32_t* __restrict__ cu_len,
    const uint16_t* __restrict__ k_cand, const uint16_t* __restrict__ v_cand,
    const uint8_t* __restrict__ copy_gate, const int32_t* __restrict__ cand_len, int B, int R,
    int Hq, int Hkv, int W, int D, int nsplit, int chunk, int qtiles, float scale_log2,
    float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o, LmWsView compact,
    int* __restrict__ work, int items_x) {
  __shared__ __attribute__((aligned(1024))) uint16_t ks0[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t ks1[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t ks2[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t ks3[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t vs0[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t vs1[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t vs2[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t vs3[kStage];
  if (compact.row_list != nullptr && blockIdx.x == gridDim.x - 1) {
    __shared__ int s_cwave[kAttThreads / kWave];
    compact_rows_body<kAttThreads>(B * R, R, W, D, cand_len, copy_gate, compact.row_list, compact.inv,
                                   compact.n_rows, s_cwave, compact.keys);
    return;
  }

  // XCD-aware work items.  Workgroup L runs on XCD x = L % 8; item idx of that XCD
  // is the (sequence, kv head) pair bk = 8 q + x, so each XCD holds the same kv
  // heads of every sequence and the XCDs get equal work whatever the context
  // lengths.  On an XCD the prefix slots come first and the (short) candidate slots
  // last; the row tiles of one (pair, slot) are consecutive and share the XCD's L2
  // (they read the same keys).  Without `work`, workgroup L takes item L / 8.  With
  // it (a persistent grid), the workgroups of an XCD take its items in order from
  // the XCD's counter work[16 x] (zero at launch) until none is left: items with no
  // real row, or past a context's end, are skipped at once, so the CUs stay busy.
  __shared__ int s_item;
  const int xcd = static_cast<int>(blockIdx.x % kXcds);
  if (work == nullptr) {
    attn_item(static_cast<int>(blockIdx.x / kXcds), xcd, ks0, ks1, ks2, ks3, vs0, vs1, vs2, vs3, q,
              k_pre, v_pre, cu_len, k_cand, v_cand, copy_gate, cand_len, B, R, Hq, Hkv, W, D, nsplit,
              chunk, qtiles, scale_log2, ws_m, ws_l, ws_o);
    return;
  }
  for (;;) {
    __syncthreads();   // the previous item is done with LDS and with s_item
    if (threadIdx.x == 0) s_item = atomicAdd(work + 16 * xcd, 1);
    __syncthreads();
    const int idx = s_item;
    if (idx >= items_x) return;
    attn_item(idx, xcd, ks0, ks1, ks2, ks3, vs0, vs1, vs2, vs3, q, k_pre, v_pre, cu_len, k_cand,
              v_cand, copy_gate, cand_len, B, R, Hq, Hkv, W, D, nsplit, chunk, qtiles, scale_log2,
              ws_m, ws_l, ws_o);
  }
}

// bf16 merge: one wave per (sequence, row, query head).  Combines the prefix slots
// that hold keys of this sequence and the candidate slot (a row without visible
// candidate keys left m = -inf there, which weighs 0), normalises and writes bf16.
// Rows that are not real are written as 0.  The kernel is a chain of dependent
// loads, so every load it needs is issued up front, from slot indices clamped into
// the workspace, and the first round uses them without a branch (a branch would let
// the compiler sink the loads behind it): lane s reads slot s's (m, l), and the
// outputs of the first kMergeBatch slots come with them; further slots take more
// rounds.  Requires B*R*Hq < 2^31 and nsplit + 1 <= 64.
constexpr int kMergeBatch = 8;
__global__ __launch_bounds__(256) void attn_merge_bf16_kernel(
    const int32_t* __restrict__ cu_len, const int32_t* __restrict__ cand_len,
    const uint8_t* __restrict__ copy_gate, int B, int R, int Hq, int W, int D, int nsplit,
    int chunk, const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o, uint16_t* __restrict__ out) {
  const uint32_t item = blockIdx.x * 4u + threadIdx.x / kWave;  // (b, r, hq)
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t per_slot = static_cast<uint32_t>(B) * R * Hq;
  if (item >= per_slot) return;
  const int r = static_cast<int>((item / Hq) % R);
  const int b = static_cast<int>(item / (static_cast<uint32_t>(Hq) * R));
  const int nslot = nsplit + 1;  // the prefix slots, then the candidate slot
  const int w = r > 0 ? (r - 1) / D : 0, j = r > 0 ? (r - 1) - w * D : 0;
  const int gate = copy_gate[b];
  const int lw = cand_len[static_cast<size_t>(b) * W + w];
  const int n_b = cu_len[b + 1] - cu_len[b];
  const size_t pl = static_cast<size_t>(lane < nslot ? lane : nslot - 1) * per_slot + item;
  const float m_l = ws_m[pl], l_l = ws_l[pl];
  float2 ov[kMergeBatch];
  auto load_o = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const size_t s = static_cast<size_t>(min(s0 + u, nslot - 1));
      ov[u] = *reinterpret_cast<const float2*>(ws_o + (s * per_slot + item) * kAttD + 2 * lane);
    }
  };
  load_o(0);
  // every load above is issued before anything waits for one of them
  __builtin_amdgcn_sched_barrier(0);
  // bitwise, so that no branch separates the loads from their use
  const bool real = (gate != 0) & ((r == 0) | (j < min(max(lw, 0), D)));
  const int nsp = min(nsplit, (n_b + chunk - 1) / chunk);
  auto used = [&](int s) { return s < nslot && (s < nsp || s == nsplit); };
  const bool valid = used(lane);
  const float M = wave_max(valid ? m_l : -INFINITY);
  const float f = valid ? __builtin_amdgcn_exp2f(m_l - M) : 0.f;
  const float L = wave_sum(valid ? f * l_l : 0.f);
  float o0 = 0.f, o1 = 0.f;
  auto fold = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int s = s0 + u;
      const float fs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), min(s, kWave - 1)));
      o0 += used(s) ? fs * ov[u].x : 0.f;
      o1 += used(s) ? fs * ov[u].y : 0.f;
    }
  };
  fold(0);
  for (int s0 = kMergeBatch; s0 < nslot; s0 += kMergeBatch) {
    load_o(s0);
    fold(s0);
  }
  const float inv = 1.f / L;
  const uint32_t packed = static_cast<uint32_t>(f32_to_bf16(o0 * inv)) |
                          (static_cast<uint32_t>(f32_to_bf16(o1 * inv)) << 16);
  *reinterpret_cast<uint32_t*>(out + static_cast<size_t>(item) * kAttD + 2 * lane) = real ? packed : 0u;
}

// ----------------------------------------------------------------- fp32 VALU
// A workgroup of four wavefronts takes four consecutive rows of one query head,
// so all four read the same keys: the whole workgroup stages each block of 64 keys
// of K and V in LDS with coalesced 16-byte loads, issuing the next block's loads
// before the current one is used.  Scores: lane = key, a d-long dot product per
// lane against the wave's q (read from LDS as a broadcast), so the running max and
// sum take one wave reduction per 64 keys rather than one per key.  P.V: lane =
// output element, the block's 64 probabilities taken from the score lanes with
// readlane (keys past the range have p = 0 and V = 0).
constexpr int kF32Rows = 4;   // rows (wavefronts) per workgroup
constexpr int kF32Keys = 64;  // keys per LDS block

template <int DPL>
__global__ __launch_bounds__(256) void attn_prefix_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k_pre, const float* __restrict__ v_pre,
    const int32_t* __restrict__ cu_len, const uint8_t* __restrict__ copy_gate,
    const int32_t* __restrict__ cand_len, int B, int R, int Hq, int Hkv, int W, int D, int nsplit,
    int chunk, float scale_log2, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o) {
  constexpr int d = DPL * kWave;
  constexpr int d4 = d / 4;                        // 16-byte chunks per key row
  constexpr int kKs = d4 + 1;                      // padded K row, in chunks
  constexpr int kLd = kF32Keys * d4 / 256;         // chunks per thread per operand
  __shared__ float4 sK[kF32Keys * kKs];
  __shared__ float sV[kF32Keys * d];
  __shared__ float4 sQ[kF32Rows][d4];
  const int b = blockIdx.y, split = blockIdx.z;
  const int rtiles = (R + kF32Rows - 1) / kF32Rows;
  const int hq = blockIdx.x / rtiles;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int r = (blockIdx.x - hq * rtiles) * kF32Rows + wave;
  if (copy_gate[b] == 0) return;
  const int base = cu_len[b];
  const int n_b = cu_len[b + 1] - base;
  const int k0 = split * chunk;
  if (k0 >= n_b) return;
  const int k1 = split == nsplit - 1 ? n_b : min(k0 + chunk, n_b);
  const bool real = r < R && real_row(r, D, cand_len + static_cast<size_t>(b) * W, true);
  if (!__syncthreads_or(real)) return;
  const int kv = hq / (Hq / Hkv);
  if (real && lane < d4)
    sQ[wave][lane] = reinterpret_cast<const float4*>(
        q + ((static_cast<size_t>(b) * R + r) * Hq + hq) * d)[lane];
  // this thread's chunks of a block: chunk f = tid + 256u is key f / d4, column f % d4
  float4 rk[kLd], rv[kLd];
  auto load = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kLd; ++u) {
      const int f = threadIdx.x + 256 * u, t = f / d4, c = f - (f / d4) * d4;
      const bool ok = t0 + t < k1;
      const size_t o = ((static_cast<size_t>(base) + (ok ? t0 + t : k0)) * Hkv + kv) * d4 + c;
      const float4 kx = reinterpret_cast<const float4*>(k_pre)[o];
      const float4 vx = reinterpret_cast<const float4*>(v_pre)[o];
      // component selects (a select of whole float4 values goes through memory)
      rk[u] = make_float4(ok ? kx.x : 0.f, ok ? kx.y : 0.f, ok ? kx.z : 0.f, ok ? kx.w : 0.f);
      rv[u] = make_float4(ok ? vx.x : 0.f, ok ? vx.y : 0.f, ok ? vx.z : 0.f, ok ? vx.w : 0.f);
    }
  };
  load(k0);
  float m = -INFINITY, l = 0.f, o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  for (int t0 = k0; t0 < k1; t0 += kF32Keys) {
    __syncthreads();  // the previous block has been read by every wave
#pragma unroll
    for (int u = 0; u < kLd; ++u) {
      const int f = threadIdx.x + 256 * u, t = f / d4, c = f - (f / d4) * d4;
      sK[t * kKs + c] = rk[u];
      reinterpret_cast<float4*>(sV)[f] = rv[u];
    }
    __syncthreads();
    if (t0 + kF32Keys < k1) load(t0 + kF32Keys);
    if (real) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int c = 0; c < d4; ++c) {
        const float4 kk = sK[lane * kKs + c], qq = sQ[wave][c];
        acc.x += kk.x * qq.x;
        acc.y += kk.y * qq.y;
        acc.z += kk.z * qq.z;
        acc.w += kk.w * qq.w;
      }
      const float s = t0 + lane < k1 ? ((acc.x + acc.y) + (acc.z + acc.w)) * scale_log2 : -INFINITY;
      const float m_new = fmaxf(m, wave_max(s));
      const float a = exp2f(m - m_new), p = exp2f(s - m_new);
      l = l * a + wave_sum(p);
      float pa[DPL][4];
#pragma unroll
      for (int e = 0; e < DPL; ++e) pa[e][0] = pa[e][1] = pa[e][2] = pa[e][3] = 0.f;
#pragma unroll
      for (int t = 0; t < kF32Keys; ++t) {
        const float pt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), t));
#pragma unroll
        for (int e = 0; e < DPL; ++e) pa[e][t & 3] += pt * sV[t * d + lane + kWave * e];
      }
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = o[e] * a + ((pa[e][0] + pa[e][1]) + (pa[e][2] + pa[e][3]));
      m = m_new;
    }
  }
  if (!real) return;
  const size_t po = ((static_cast<size_t>(split) * B + b) * R + r) * Hq + hq;
  if (lane == 0) {
    ws_m[po] = m;
    ws_l[po] = l;
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) ws_o[po * d + lane + kWave * e] = o[e];
}

// ----------------------------------------------------------------- merge + triangle
// fp32 merge: one wave per (sequence, row, query head), laid out as the bf16 merge
// (lane s holds split s's (m, l); every load issued up front and the first round
// used without a branch), then the row's own candidate triangle is folded in
// exactly: keys (w, 0..j), j < D <= 64, lane jj scoring key (w, jj), so one wave max
// and one wave sum fold it in; lane = output element then accumulates the values.
// The anchor row (j = -1) sees no candidate key and passes through unchanged.
template <int DPL>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const float* __restrict__ q, const float* __restrict__ k_cand, const float* __restrict__ v_cand,
    const int32_t* __restrict__ cu_len, const int32_t* __restrict__ cand_len,
    const uint8_t* __restrict__ copy_gate, int B, int R, int Hq, int Hkv, int W, int D, int nsplit,
    int chunk, float scale_log2, const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o, float* __restrict__ out, LmWsView compact) {
  constexpr int d = DPL * kWave, d4 = d / 4;
  if (compact.row_list != nullptr && blockIdx.x == gridDim.x - 1) {
    // one more workgroup: the LM head's compact row list (and zeroed argmax keys)
    __shared__ int s_cwave[256 / kWave];
    compact_rows_body<256>(B * R, R, W, D, cand_len, copy_gate, compact.row_list, compact.inv,
                           compact.n_rows, s_cwave, compact.keys);
    return;
  }
  const uint32_t item = blockIdx.x * 4u + threadIdx.x / kWave;  // (b, r, hq)
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t per_slot = static_cast<uint32_t>(B) * R * Hq;
  if (item >= per_slot) return;
  const int hq = static_cast<int>(item % Hq);
  const int r = static_cast<int>((item / Hq) % R);
  const int b = static_cast<int>(item / (static_cast<uint32_t>(Hq) * R));
  const int kv = hq / (Hq / Hkv);
  const int w = r > 0 ? (r - 1) / D : 0, j = r > 0 ? (r - 1) - w * D : -1;
  const int jc = j < 0 ? 0 : j;
  const size_t row0 = (static_cast<size_t>(b) * W * D + static_cast<size_t>(w) * D) * Hkv + kv;
  const float4* kr = reinterpret_cast<const float4*>(k_cand) +
                     (row0 + static_cast<size_t>(lane <= jc ? lane : 0) * Hkv) * d4;
  const float4* qr = reinterpret_cast<const float4*>(q) + static_cast<size_t>(item) * d4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int c = 0; c < d4; ++c) {
    const float4 kk = kr[c], qq = qr[c];
    acc.x += kk.x * qq.x;
    acc.y += kk.y * qq.y;
    acc.z += kk.z * qq.z;
    acc.w += kk.w * qq.w;
  }
  float vv[kMergeBatch][DPL];
  auto load_v = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float* vr = v_cand + (row0 + static_cast<size_t>(min(j0 + u, jc)) * Hkv) * d;
#pragma unroll
      for (int e = 0; e < DPL; ++e) vv[u][e] = vr[lane + kWave * e];
    }
  };
  load_v(0);
  const int gate = copy_gate[b];
  const int lw = cand_len[static_cast<size_t>(b) * W + w];
  const int n_b = cu_len[b + 1] - cu_len[b];
  const size_t pl = static_cast<size_t>(lane < nsplit ? lane : nsplit - 1) * per_slot + item;
  const float m_l = ws_m[pl], l_l = ws_l[pl];
  float ov[kMergeBatch][DPL];
  auto load_o = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float* src = ws_o + (static_cast<size_t>(min(s0 + u, nsplit - 1)) * per_slot + item) * d;
#pragma unroll
      for (int e = 0; e < DPL; ++e) ov[u][e] = src[lane + kWave * e];
    }
  };
  load_o(0);
  // every load above is issued before anything waits for one of them
  __builtin_amdgcn_sched_barrier(0);
  // bitwise, so that no branch separates the loads from their use
  const bool real = (gate != 0) & ((r == 0) | (j < min(max(lw, 0), D)));
  // prefix splits
  const int nsp = min(nsplit, (n_b + chunk - 1) / chunk);
  const bool valid = lane < nsp;
  const float M = wave_max(valid ? m_l : -INFINITY);
  const float f = valid ? __builtin_amdgcn_exp2f(m_l - M) : 0.f;
  float L = wave_sum(valid ? f * l_l : 0.f), o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  auto fold_o = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int s = s0 + u;
      const float fs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), min(s, kWave - 1)));
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] += s < nsp ? fs * ov[u][e] : 0.f;
    }
  };
  fold_o(0);
  for (int s0 = kMergeBatch; s0 < nsp; s0 += kMergeBatch) {
    load_o(s0);
    fold_o(s0);
  }
  // own-candidate triangle
  const float sc = lane <= j ? ((acc.x + acc.y) + (acc.z + acc.w)) * scale_log2 : -INFINITY;
  const float m_new = fmaxf(M, wave_max(sc));
  const float a = exp2f(M - m_new), p = exp2f(sc - m_new);
  L = L * a + wave_sum(p);
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] *= a;
  auto fold_v = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int jj = j0 + u;
      const float pt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), min(jj, kWave - 1)));
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] += jj <= j ? pt * vv[u][e] : 0.f;
    }
  };
  fold_v(0);
  for (int j0 = kMergeBatch; j0 <= j; j0 += kMergeBatch) {
    load_v(j0);
    fold_v(j0);
  }
  const float inv = 1.f / L;
  float* op = out + static_cast<size_t>(item) * d;  // out[b][r][hq*d + ...]
#pragma unroll
  for (int e = 0; e < DPL; ++e) op[lane + kWave * e] = real ? o[e] * inv : 0.f;
}

// ----------------------------------------------------------------- host side
AttnPlan attn_plan(int B, int max_n, int R, int Hq, int Hkv, bool bf16) {
  AttnPlan p;
  const int g = Hq / Hkv;
  if (bf16) {
    // One workgroup per CU, 256 CUs.  With little work per CU (under 64 key blocks)
    // the split is latency-bound: take as many splits as fit, with the candidate
    // slot, in one round of workgroups.  Otherwise cut the prefix into ranges of at
    // most 4096 keys: long contexts then spread over more CUs (ragged batches balance,
    // and units whose rows are all padding, which exit at once, leave the CUs to
    // the others), at the cost of one more partial slot per range for the merge.
    constexpr int kCus = 256, kMaxBlocks = 64;
    p.qtiles = (R * g + kAttRowsPerBlock - 1) / kAttRowsPerBlock;
    const long long units = static_cast<long long>(B) * Hkv * p.qtiles;
    const int blocks = (max_n + kKB - 1) / kKB;
    int cap = max_n / 256;
    if (cap < 1) cap = 1;
    if (cap > 32) cap = 32;
    int ns;
    const bool latency = units * blocks < static_cast<long long>(kKB) * kCus;
    if (latency) {
      ns = static_cast<int>(kCus / units) - 1;
    } else {
      ns = (blocks + kMaxBlocks - 1) / kMaxBlocks;
    }
    // with enough work the items go to a persistent grid (load balance); a single
    // round of workgroups needs no counters
    p.persist = latency ? 0 : 1;
    if (ns > cap) ns = cap;
    if (ns < 1) ns = 1;
    int ch = (max_n + ns - 1) / ns;
    ch = (ch + kKB - 1) / kKB * kKB;
    if (ch < kKB) ch = kKB;
    p.nsplit = ns;
    p.chunk = ch;
    p.nslots = ns + 1;  // one more slot for the candidate keys
    return p;
  }
  p.qtiles = Hq * ((R + kF32Rows - 1) / kF32Rows);  // workgroups of 4 rows of one head
  const int units = B * p.qtiles;
  const int min_keys = 128, target = 1024;
  int ns = (target + units - 1) / units;
  int cap = max_n / min_keys;
  if (cap < 1) cap = 1;
  if (ns > cap) ns = cap;
  if (ns > kWave) ns = kWave;  // the merge holds one split per lane
  if (ns < 1) ns = 1;
  int ch = (max_n + ns - 1) / ns;
  ch = (ch + kKB - 1) / kKB * kKB;
  if (ch < kKB) ch = kKB;
  p.nsplit = ns;
  p.chunk = ch;
  p.nslots = ns;
  p.persist = 0;
  return p;
}

// Work counters of the persistent grid: one per XCD, 64 bytes apart, after the
// partials.
constexpr size_t kWorkBytes = kXcds * 64;

size_t attn_workspace_bytes(const AttnPlan& p, int B, int R, int Hq, int d) {
  const size_t rows = static_cast<size_t>(p.nslots) * B * R * Hq;
  return rows * sizeof(float) * (2 + static_cast<size_t>(d)) + kWorkBytes;
}

__global__ void attn_work_reset_kernel(int* __restrict__ work) {
  if (threadIdx.x < kXcds) work[16 * threadIdx.x] = 0;
}

hipError_t launch_attention(const void* q, const void* k_pre, const void* v_pre,
                            const int32_t* cu_len, const void* k_cand, const void* v_cand,
                            const int32_t* cand_len, const uint8_t* copy_gate, int B, int W,
                            int D, int Hq, int Hkv, int d, bool bf16, float scale,
                            const AttnPlan& plan, void* attn_out, float* ws, hipStream_t s,
                            const LmWsView* compact) {
  if (plan.nslots > kWave) return hipErrorInvalidValue;  // the merges hold a slot per lane
  const int R = 1 + W * D;
  const size_t rows = static_cast<size_t>(plan.nslots) * B * R * Hq;
  float* ws_m = ws;
  float* ws_l = ws + rows;
  float* ws_o = ws + 2 * rows;
  const float scale_log2 = scale * kLog2e;
  const size_t items = static_cast<size_t>(B) * R * Hq;
  const dim3 mgrid(static_cast<unsigned>((items + 3) / 4));
  const LmWsView cv = compact != nullptr ? *compact : LmWsView{nullptr, nullptr, nullptr, nullptr};
  if (bf16) {
    const int per_xcd = (B * Hkv + kXcds - 1) / kXcds * plan.nslots;
    const int items_x = per_xcd * plan.qtiles;
    int* work = nullptr;
    int grid = kXcds * items_x;
    if (plan.persist) {
      work = reinterpret_cast<int*>(ws + rows * (2 + static_cast<size_t>(d)));
      hipLaunchKernelGGL(attn_work_reset_kernel, dim3(1), dim3(kWave), 0, s, work);
      grid = kPersistCus < grid ? kPersistCus : grid;
    }
    hipLaunchKernelGGL(attn_prefix_bf16_kernel, dim3(grid + (compact != nullptr ? 1 : 0)),
                       dim3(kAttThreads), 0, s, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k_pre), static_cast<const uint16_t*>(v_pre), cu_len,
                       static_cast<const uint16_t*>(k_cand), static_cast<const uint16_t*>(v_cand),
                       copy_gate, cand_len, B, R, Hq, Hkv, W, D, plan.nsplit, plan.chunk, plan.qtiles,
                       scale_log2, ws_m, ws_l, ws_o, cv, work, items_x);
    hipLaunchKernelGGL(attn_merge_bf16_kernel, mgrid, dim3(256), 0, s, cu_len, cand_len, copy_gate,
                       B, R, Hq, W, D, plan.nsplit, plan.chunk, ws_m, ws_l, ws_o,
                       static_cast<uint16_t*>(attn_out));
  } else {
    const dim3 pgrid(plan.qtiles, B, plan.nsplit);
    const dim3 fgrid(mgrid.x + (compact != nullptr ? 1 : 0));
    if (d == 64) {
      hipLaunchKernelGGL(attn_prefix_f32_kernel<1>, pgrid, dim3(256), 0, s,
                         static_cast<const float*>(q), static_cast<const float*>(k_pre),
                         static_cast<const float*>(v_pre), cu_len, copy_gate, cand_len, B, R, Hq,
                         Hkv, W, D, plan.nsplit, plan.chunk, scale_log2, ws_m, ws_l, ws_o);
      hipLaunchKernelGGL(attn_merge_kernel<1>, fgrid, dim3(256), 0, s,
                         static_cast<const float*>(q), static_cast<const float*>(k_cand),
                         static_cast<const float*>(v_cand), cu_len, cand_len, copy_gate, B, R,
                         Hq, Hkv, W, D, plan.nsplit, plan.chunk, scale_log2, ws_m, ws_l, ws_o,
                         static_cast<float*>(attn_out), cv);
    } else {
      hipLaunchKernelGGL(attn_prefix_f32_kernel<2>, pgrid, dim3(256), 0, s,
                         static_cast<const float*>(q), static_cast<const float*>(k_pre),
                         static_cast<const float*>(v_pre), cu_len, copy_gate, cand_len, B, R, Hq,
                         Hkv, W, D, plan.nsplit, plan.chunk, scale_log2, ws_m, ws_l, ws_o);
      hipLaunchKernelGGL(attn_merge_kernel<2>, fgrid, dim3(256), 0, s,
                         static_cast<const float*>(q), static_cast<const float*>(k_cand),
                         static_cast<const float*>(v_cand), cu_len, cand_len, copy_gate, B, R,
                         Hq, Hkv, W, D, plan.nsplit, plan.chunk, scale_log2, ws_m, ws_l, ws_o,
                         static_cast<float*>(attn_out), cv);
    }
  }
  return hipGetLastError();
}

}  // namespace ssd
