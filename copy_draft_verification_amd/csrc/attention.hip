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
constexpr int kAttRowsPerBlock = 128;
constexpr int kXcds = 8;            // workgroups are dealt round-robin over the 8 XCDs
constexpr float kLazyRescale = 8.f; // the running max moves only when exceeded by 2^8
constexpr int kAttAhead = 4;        // LDS fragment reads in flight ahead of their MFMA
constexpr int kAttIssueAt = 2;      // S MFMA after which the next block's loads start

// V^T in LDS: row d holds the block's 64 keys (128 B, no padding) as sixteen 8-byte
// units of 4 keys; unit u sits at position u ^ vt_swz(d).  With this swizzle both the
// transposing writes (16 lanes = 16 rows d = 8*dc + e, one unit) and the MFMA
// A-operand reads (32 lanes = 32 consecutive rows, one unit) hit distinct banks.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) ^ (d >> 3)) & 15; }

// One workgroup = 128 query rows (the g query heads of one KV head packed together)
// x one key range of one sequence.  Key ranges ("slots") 0..nsplit-1 split the
// prefix; slot nsplit holds the W*D candidate keys, where row (w, j) may only see
// keys (w, 0..j): that mask is evaluated in registers from the key and row
// indices.  Each slot leaves a partial (running max m, sum l, unnormalised o) in
// the workspace, in the exp2 domain; the merge kernel combines them.
//
// Grid: the (sequence, kv head, slot) groups are dealt to XCDs so that all row
// tiles of a group share one XCD's L2 (they read the same keys).  With
// compact.row_list set, the grid has one more workgroup, the last, which writes
// the compact list of real rows for the LM head while the others attend.
__global__ __launch_bounds__(256, 2) void attn_prefix_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pre,
    const uint16_t* __restrict__ v_pre, const int32_t* __restrict__ cu_len,
    const uint16_t* __restrict__ k_cand, const uint16_t* __restrict__ v_cand,
    const uint8_t* __restrict__ copy_gate, const int32_t* __restrict__ cand_len, int B, int R,
    int Hq, int Hkv, int W, int D, int nsplit, int chunk, int qtiles, float scale_log2,
    float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o, LmWsView compact) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kKB * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[kAttD * kKB];
  if (compact.row_list != nullptr && blockIdx.x == gridDim.x - 1) {
    __shared__ int s_cwave[256 / kWave];
    compact_rows_body<256>(B * R, R, W, D, cand_len, copy_gate, compact.row_list, compact.inv,
                           compact.n_rows, s_cwave);
    return;
  }

  // XCD-aware decode: block L runs on XCD L % 8; groups g with g % 8 == x run there
  const int nslots = nsplit + 1;
  const int groups = B * Hkv * nslots;
  const int xcd = static_cast<int>(blockIdx.x % kXcds), idx = static_cast<int>(blockIdx.x / kXcds);
  const int qtile = idx % qtiles;
  const int grp = (idx / qtiles) * kXcds + xcd;
  if (grp >= groups) return;
  const int slot = grp % nslots;
  const int b = (grp / nslots) / Hkv, kvh = (grp / nslots) % Hkv;
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
  // keys of this sequence (or its candidates).  The key index goes into the
  // per-lane offset, so keys past the last one fall outside the buffer's range:
  // they read as zero and never touch the memory after it.
  const int key_bytes = Hkv * kAttD * 2;
  const __amdgpu_buffer_rsrc_t kres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kp), 0, nkeys * key_bytes, kBufFlags);
  const __amdgpu_buffer_rsrc_t vres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vp), 0, nkeys * key_bytes, kBufFlags);

  const int g = Hq / Hkv, G = R * g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int h = lane >> 5, l32 = lane & 31;
  const int i_row = qtile * kAttRowsPerBlock + wave * 32 + l32;  // this lane's query row (B operand column)
  const bool row_ok = i_row < G;
  const int r_row = row_ok ? i_row / g : 0, hh = row_ok ? i_row - (i_row / g) * g : 0;
  // A tile whose rows are all padding (candidates past M, tokens past L_w) has
  // nothing to contribute: the merge reads partials of real rows only.
  if (!__syncthreads_or(row_ok && real_row(r_row, D, cand_len + static_cast<size_t>(b) * W, true)))
    return;
  // candidate mask of this row: keys cw*D .. cw*D + cj (none for the anchor row)
  const int cw = r_row > 0 ? (r_row - 1) / D : -1;
  const int cj = r_row > 0 ? (r_row - 1) - cw * D : -1;
  // Keys this row may see in this slot: [vis_lo, vis_hi] and below k1.  In the
  // candidate slot that is its own candidate's keys cw*D .. cw*D + cj (an empty
  // range for the anchor row); in a prefix slot, every key.
  const int vis_lo = !cand ? 0 : (cw >= 0 ? cw * D : 1);
  const int vis_hi = !cand ? INT_MAX : (cw >= 0 ? cw * D + cj : 0);

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

  // Staging of a 64-key block.  K: thread loads 16 B (d chunk tid%16) of keys
  // tid/16 + 16c.  V: thread loads d chunk dc = tid%16 of the four keys 4kq..4kq+3,
  // kq = tid/16, and writes them transposed as eight 8-byte units (one per d).
  const int koff = ((tid >> 4) * Hkv + kvh) * kAttD * 2 + (tid & 15) * 16;
  const int kq = tid >> 4, dc = tid & 15;
  const int voff = ((4 * kq) * Hkv + kvh) * kAttD * 2 + dc * 16;
  uint4 kreg[4], vreg[4];
  // A block past the key range (past = true) is "loaded" with an offset beyond both
  // buffers: zeros, no memory touched, and no branch around the loads.
  constexpr int kOutOfRange = 0x7ffffff0;
  auto load_block = [&](int kb, bool past) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      kreg[c] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     kres, past ? kOutOfRange : koff + (kb + 16 * c) * key_bytes, 0, 0));
#pragma unroll
    for (int k = 0; k < 4; ++k)
      vreg[k] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     vres, past ? kOutOfRange : voff + (kb + k) * key_bytes, 0, 0));
  };
  auto store_block = [&]() {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<uint4*>(&k_lds[((tid >> 4) + 16 * c) * kKStride + (tid & 15) * 8]) = kreg[c];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = dc * 8 + e;
      const uint32_t w0 = (&vreg[0].x)[e >> 1], w1 = (&vreg[1].x)[e >> 1];
      const uint32_t w2 = (&vreg[2].x)[e >> 1], w3 = (&vreg[3].x)[e >> 1];
      uint2 u;
      if (e & 1) {
        u.x = (w0 >> 16) | (w1 & 0xffff0000u);
        u.y = (w2 >> 16) | (w3 & 0xffff0000u);
      } else {
        u.x = (w0 & 0xffffu) | (w1 << 16);
        u.y = (w2 & 0xffffu) | (w3 << 16);
      }
      *reinterpret_cast<uint2*>(&vt_lds[d * kKB + 4 * (kq ^ vt_swz(d))]) = u;
    }
  };

  load_block(k0, false);
  for (int kb = k0; kb < k1; kb += kKB) {
    lds_barrier();  // every wave is done reading the previous block
    store_block();
    lds_barrier();  // this block is in LDS
    // The next block's loads go out from inside the S MFMAs below (one after each
    // of MFMAs kAttIssueAt .. kAttIssueAt+7), so the first MFMAs after the barrier
    // wait only on their K fragments: 3-4.5% faster where a workgroup walks many
    // blocks (batch 32, long contexts).
    const bool next_past = kb + kKB >= k1;

    // S^T[key][row] for two 32-key subtiles.  The two accumulation chains alternate
    // (MFMA i works on subtile i % 2, k-step i / 2), and the K fragments are read
    // kAttAhead MFMAs ahead of their use, so no MFMA waits on its own LDS read.
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
    {
      auto kfrag = [&](int i) {
        return *reinterpret_cast<const uint4*>(&k_lds[((i & 1) * 32 + l32) * kKStride + 16 * (i >> 1) + 8 * h]);
      };
      uint4 kq[kAttAhead + 1];
#pragma unroll
      for (int i = 0; i < kAttAhead; ++i) kq[i] = kfrag(i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i == kAttIssueAt) load_block(kb + kKB, next_past);
        if (i + kAttAhead < 16) kq[(i + kAttAhead) % (kAttAhead + 1)] = kfrag(i + kAttAhead);
        sacc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, kq[i % (kAttAhead + 1)]), qf[i >> 1], sacc[i & 1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kAttAhead, 0);  // DS reads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
        if (i + kAttAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (i >= kAttIssueAt && i < kAttIssueAt + 8)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // a global load
      }
    }
    // Online softmax in the exp2 domain; lanes l and l^32 share a row.  Keys past
    // k1 and candidate keys outside this row's own prefix are masked (only partial
    // prefix blocks and candidate blocks need the test).
    float smax = -INFINITY;
    if (!cand && kb + kKB <= k1) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[kt][r]);
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + kt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool vis = key < k1 && key >= vis_lo && key <= vis_hi;
          sacc[kt][r] = vis ? sacc[kt][r] : -INFINITY;
          smax = fmaxf(smax, sacc[kt][r]);
        }
    }
    smax = fmaxf(smax, __shfl_xor(smax, 32, kWave));
    const float m_blk = smax * scale_log2;  // scale > 0: the max commutes with it
    // Lazy rescale: keep the running max until a block exceeds it by more than 2^8
    // (probabilities then stay <= 256, exact enough in bf16 and fp32).
    const bool need = m_blk > m_run + kLazyRescale;
    if (__ballot(need)) {
      const float m_new = need ? m_blk : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    // a row with no visible key yet keeps m = -inf; exponentiate against 0 then
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    float psum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][8 * s2 + e], scale_log2, neg_m));
          psum += p;
          pf[kt][s2][e] = static_cast<__bf16>(p);
        }
    l_run += psum;
    // O^T[d][row] += V^T[d][keys] P^T[keys][row]; key order of a P fragment element e
    // for lane half h: kt*32 + 16*s2 + 8*(e/4) + 4*h + e%4 (the S^T output layout),
    // i.e. 4-key units 8kt + 4s2 + h (e < 4) and that + 2 (e >= 4)
    // MFMA i = (dt, kt, s2) = (i / 4, i / 2 % 2, i % 2); its two 8-byte V^T reads
    // are issued kAttAhead MFMAs ahead
    {
      auto vfrag = [&](int i) {
        const int d = (i >> 2) * 32 + l32;
        const uint16_t* vr = &vt_lds[d * kKB];
        const int sw = vt_swz(d);
        const int u0 = 8 * ((i >> 1) & 1) + 4 * (i & 1) + h;
        const uint2 lo = *reinterpret_cast<const uint2*>(vr + 4 * (u0 ^ sw));
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 4 * ((u0 + 2) ^ sw));
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
      };
      uint4 vq[kAttAhead + 1];
#pragma unroll
      for (int i = 0; i < kAttAhead; ++i) vq[i] = vfrag(i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + kAttAhead < 16) vq[(i + kAttAhead) % (kAttAhead + 1)] = vfrag(i + kAttAhead);
        oacc[i >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, vq[i % (kAttAhead + 1)]), pf[(i >> 1) & 1][i & 1], oacc[i >> 2], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAttAhead, 0);  // DS reads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
        if (i + kAttAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (!row_ok) return;
  const size_t po = ((static_cast<size_t>(slot) * B + b) * R + r_row) * Hq + kvh * g + hh;
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

// bf16 merge: one wave per (sequence, row, query head).  Combines the prefix slots
// that hold keys of this sequence and the candidate slot (a row without visible
// candidate keys left m = -inf there, which weighs 0), normalises and writes bf16.
// Rows that are not real are written as 0.
__global__ __launch_bounds__(256) void attn_merge_bf16_kernel(
    const int32_t* __restrict__ cu_len, const int32_t* __restrict__ cand_len,
    const uint8_t* __restrict__ copy_gate, int B, int R, int Hq, int W, int D, int nsplit,
    int chunk, const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o, uint16_t* __restrict__ out) {
  const size_t item = static_cast<size_t>(blockIdx.x) * 4 + threadIdx.x / kWave;  // (b, r, hq)
  const int lane = threadIdx.x & (kWave - 1);
  if (item >= static_cast<size_t>(B) * R * Hq) return;
  const int r = static_cast<int>((item / Hq) % R);
  const int b = static_cast<int>(item / (static_cast<size_t>(Hq) * R));
  uint16_t* op = out + item * kAttD;  // out[b][r][hq*d + ...]
  if (!real_row(r, D, cand_len + static_cast<size_t>(b) * W, copy_gate[b] != 0)) {
    *reinterpret_cast<uint32_t*>(op + 2 * lane) = 0u;
    return;
  }
  const int n_b = cu_len[b + 1] - cu_len[b];
  const int nsp = min(nsplit, (n_b + chunk - 1) / chunk);
  const size_t per_slot = static_cast<size_t>(B) * R * Hq;
  const size_t row_item = item;  // == (b*R + r)*Hq + hq
  float M = ws_m[static_cast<size_t>(nsplit) * per_slot + row_item];
  for (int s = 0; s < nsp; ++s) M = fmaxf(M, ws_m[s * per_slot + row_item]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  auto add = [&](size_t po) {
    const float f = __builtin_amdgcn_exp2f(ws_m[po] - M);
    L += f * ws_l[po];
    const float2 v = *reinterpret_cast<const float2*>(ws_o + po * kAttD + 2 * lane);
    o0 += f * v.x;
    o1 += f * v.y;
  };
  for (int s = 0; s < nsp; ++s) add(s * per_slot + row_item);
  add(static_cast<size_t>(nsplit) * per_slot + row_item);
  const float inv = 1.f / L;
  const uint32_t packed = static_cast<uint32_t>(f32_to_bf16(o0 * inv)) |
                          (static_cast<uint32_t>(f32_to_bf16(o1 * inv)) << 16);
  *reinterpret_cast<uint32_t*>(op + 2 * lane) = packed;
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
  p.nslots = bf16 ? ns + 1 : ns;  // bf16: one more slot for the candidate keys
  return p;
}

size_t attn_workspace_bytes(const AttnPlan& p, int B, int R, int Hq, int d) {
  const size_t rows = static_cast<size_t>(p.nslots) * B * R * Hq;
  return rows * sizeof(float) * (2 + static_cast<size_t>(d));
}

hipError_t launch_attention(const void* q, const void* k_pre, const void* v_pre,
                            const int32_t* cu_len, const void* k_cand, const void* v_cand,
                            const int32_t* cand_len, const uint8_t* copy_gate, int B, int W,
                            int D, int Hq, int Hkv, int d, bool bf16, float scale,
                            const AttnPlan& plan, void* attn_out, float* ws, hipStream_t s,
                            const LmWsView* compact) {
  if (compact != nullptr && !bf16) return hipErrorInvalidValue;
  const int R = 1 + W * D;
  const size_t rows = static_cast<size_t>(plan.nslots) * B * R * Hq;
  float* ws_m = ws;
  float* ws_l = ws + rows;
  float* ws_o = ws + 2 * rows;
  const float scale_log2 = scale * kLog2e;
  const size_t items = static_cast<size_t>(B) * R * Hq;
  const dim3 mgrid(static_cast<unsigned>((items + 3) / 4));
  if (bf16) {
    const int groups = B * Hkv * plan.nslots;
    const int per_xcd = (groups + kXcds - 1) / kXcds;
    const LmWsView cv = compact != nullptr ? *compact : LmWsView{nullptr, nullptr, nullptr};
    hipLaunchKernelGGL(attn_prefix_bf16_kernel,
                       dim3(kXcds * per_xcd * plan.qtiles + (compact != nullptr ? 1 : 0)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_pre),
                       static_cast<const uint16_t*>(v_pre), cu_len,
                       static_cast<const uint16_t*>(k_cand), static_cast<const uint16_t*>(v_cand),
                       copy_gate, cand_len, B, R, Hq, Hkv, W, D, plan.nsplit, plan.chunk, plan.qtiles,
                       scale_log2, ws_m, ws_l, ws_o, cv);
    hipLaunchKernelGGL(attn_merge_bf16_kernel, mgrid, dim3(256), 0, s, cu_len, cand_len, copy_gate,
                       B, R, Hq, W, D, plan.nsplit, plan.chunk, ws_m, ws_l, ws_o,
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
