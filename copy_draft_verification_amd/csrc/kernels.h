// Internal launchers (host side) for the copy-speculation kernels.  Each returns
// hipGetLastError() after its launches.  Arguments are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace ssd {

hipError_t launch_probe(const void* h, bool bf16, const float* w, int B, int hidden, float thr,
                        float* z_out, uint8_t* fire_out, hipStream_t s);

// The probe computed inside the retrieval launch (ssd_probe_kgram_retrieve): h [B][hidden]
// (bf16 or fp32), w [hidden], thr = logit(tau); z_out may be null.
struct KgProbe {
  const void* h = nullptr;
  bool bf16 = false;
  const float* w = nullptr;
  int hidden = 0;
  float thr = 0.f;
  float* z_out = nullptr;
  uint8_t* fire_out = nullptr;
};
hipError_t launch_kgram(const int32_t* ids, const int32_t* cu_len, int B, int kappa, int W, int D,
                        const uint8_t* fire, int32_t* match_end, int32_t* n_match, int32_t* cand,
                        int32_t* cand_len, uint8_t* copy_gate, hipStream_t s,
                        const KgProbe* probe = nullptr);

hipError_t launch_accept(const int32_t* cand, const int32_t* cand_len, const uint8_t* copy_gate,
                         const int32_t* argmax, int B, int W, int D, int32_t* accept_len,
                         int32_t* best_w, int32_t* best_len, int32_t* next_token, hipStream_t s);

// Split of the prefix keys over workgroups for block-triangular attention.
struct AttnPlan {
  int nsplit;   // splits of the prefix per (sequence, kv head, row tile)
  int chunk;    // keys per split (multiple of 64); the last split runs to n_b
  int qtiles;   // row tiles per (sequence, kv head)
  int nslots;   // partial slots in the workspace (bf16: nsplit + the candidate slot)
  int persist;  // bf16: a persistent grid takes the work items from per-XCD counters
};
AttnPlan attn_plan(int B, int max_n, int R, int Hq, int Hkv, bool bf16);
size_t attn_workspace_bytes(const AttnPlan& p, int B, int R, int Hq, int d);

// The LM-head workspace's compact row list (written by launch_compact_rows, or by
// launch_attention when it is given one).
struct LmWsView {
  int32_t* n_rows;
  int32_t* row_list;
  int32_t* inv;
  unsigned long long* keys;  // [rows] greedy argmax keys by global row, zeroed with the compaction
};

// With `compact`, one more workgroup of one of the attention launches (bf16: the
// prefix sweep, fp32: the merge) writes the compact list of the B*(1+W*D) rows,
// as launch_compact_rows would, beside the attention instead of after it.
hipError_t launch_attention(const void* q, const void* k_pre, const void* v_pre,
                            const int32_t* cu_len, const void* k_cand, const void* v_cand,
                            const int32_t* cand_len, const uint8_t* copy_gate, int B, int W,
                            int D, int Hq, int Hkv, int d, bool bf16, float scale,
                            const AttnPlan& plan, void* attn_out, float* ws, hipStream_t s,
                            const LmWsView* compact = nullptr);

struct LmPlan {
  int vtiles;   // vocabulary tiles (one workgroup column each)
  int mchunks;  // row chunks
  int sv, sm;   // bf16: super-tile of sv vocabulary tiles x sm row chunks per XCD
  int blocks;   // bf16: workgroups launched (super-tiles dealt round-robin to XCDs)
  int half = 0; // GEMM: tiles are 128-row halves of the packed 256-row tiles
};
LmPlan lm_plan(int rows, int V, bool bf16);
size_t lm_workspace_bytes(const LmPlan& p, int rows);
// packed bf16 weight layout of the LM-head / GEMM kernel: bytes for N rows of K (or
// N features of a gate / up pair), its K alignment, and the packing (w2: the up
// matrix of a pair, else null)
size_t packed_weight_bytes(int N, int K, bool pair);
int lm_k_align();
hipError_t launch_pack_weight(const void* w, const void* w2, int N, int K, void* packed,
                              hipStream_t s);

// Sampling (T > 0) arguments of the LM head's epilogue: 1/T, the Philox key, the
// trie's children per global row, and where the children's logits / T go.
struct SampleArgs {
  float inv_t;
  uint32_t k0, k1;
  int W;
  const int32_t* n_children;  // [B*R]
  const int32_t* children;    // [B*R][W]
  float* child_logit;         // [B*R][W]
};

// Epilogues of the bf16 LM-head / GEMM kernel.
constexpr int kEpiArgmax = 0;   // per (row, tile) best (value, index)
constexpr int kEpiSample = 1;   // per (row, tile) sampling partials
constexpr int kEpiPartial = 2;  // split-K partial sums, fp32
constexpr int kEpiSwiGLU = 3;   // silu(gate) * up, bf16
constexpr int kEpiPair = 4;     // two A matrices (gate, up), split-K partial sums of both
constexpr int kEpiPartialHalf = 5;  // kEpiPartial on one 128-row half of a packed 256-row tile

struct GemmArgs {
  int kc;                     // hidden elements per split (0: all of K)
  float* part;                // kEpiPartial: [splits][part_rows][ld], by compact row
  int part_rows;
  int ld;                     // leading dimension of part / out (elements)
  uint16_t* out;              // kEpiSwiGLU: [global row][ld]
  const int32_t* row_list;    // compact row -> global row
};

// Accept at T = 0 after the greedy argmax (launch_argmax_finish); cand == null: no
// accept.  The arrays of launch_accept.
struct AcceptArgs {
  const int32_t* cand = nullptr;
  const int32_t* cand_len = nullptr;
  const uint8_t* copy_gate = nullptr;
  int W = 0, D = 0;
  int32_t* accept_len = nullptr;
  int32_t* best_w = nullptr;
  int32_t* best_len = nullptr;
  int32_t* next_token = nullptr;
};

// sample != nullptr: sampling partials.  Otherwise greedy: each row's best (value,
// lowest index) is folded into a 64-bit key per row (launch_argmax_finish).
// rows_layout (bf16 greedy only): lm_head is the plain row-major [V][hid] matrix
// instead of the packed layout.
hipError_t launch_lmhead(const void* attn_out, const void* lm_head, int rows, int hid, int V,
                         bool bf16, const LmPlan& plan, float* logits_out, void* ws,
                         hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t s,
                         const SampleArgs* sample = nullptr, bool rows_layout = false);
// Greedy: argmax_out [B][R] from the keys of launch_lmhead (-1 for rows that are
// not real), then, with `accept`, the accept of every sequence; one launch.
hipError_t launch_argmax_finish(void* ws, int B, int R, int32_t* argmax_out, const AcceptArgs* accept,
                                hipStream_t s);

// Lists the real rows (open gate; row 0 or candidate token j < L_w) in the LM-head
// workspace; the LM head then contracts only those rows.
hipError_t launch_compact_rows(void* ws, int rows, int R, int W, int D, const int32_t* cand_len,
                               const uint8_t* copy_gate, hipStream_t s);


// Verification at T > 0: the candidate trie (before the LM head), the reduction of
// the sampling partials into lse / residual draw per row, and the acceptance walk.
hipError_t launch_trie(const int32_t* cand, const int32_t* cand_len, const uint8_t* copy_gate,
                       int B, int W, int D, int32_t* n_children, int32_t* children,
                       int32_t* child_w, float* child_logit, hipStream_t s);
hipError_t launch_sample_reduce(void* ws, const LmPlan& plan, int rows, float* lse,
                                int32_t* resample, hipStream_t s);
hipError_t launch_accept_sample(const int32_t* n_children, const int32_t* child_w,
                                const float* child_logit, const float* lse,
                                const int32_t* resample, const uint8_t* copy_gate, int B, int W,
                                int D, unsigned long long seed, int32_t* best_w,
                                int32_t* best_len, int32_t* next_token, hipStream_t s);

hipError_t launch_commit(const void* k_cand, const void* v_cand, const int32_t* cand,
                         const int32_t* best_w, const int32_t* best_len, const int32_t* next_token,
                         int B, int W, int D, int row_bytes, void* k_cache, void* v_cache,
                         long long cache_rows, const long long* cache_off, int32_t* tokens_out,
                         int32_t* n_tokens_out, hipStream_t s);

// Offline probe calibration: copy-mode labels, batched probe logits, and the
// per-layer F1 / AUC sweep with the layer choice.
size_t labels_workspace_bytes(long long total_n);
hipError_t launch_copy_labels(const int32_t* ids, const int32_t* cu_len, int B, int total_n,
                              int n_train, uint8_t* labels, void* ws, hipStream_t s);
hipError_t launch_probe_logits(const void* h, bool bf16, const float* w, int L, long long N,
                               int hid, float* z, hipStream_t s);
size_t calibrate_workspace_bytes(int L, long long N);
hipError_t launch_calibrate(const float* z, const uint8_t* labels, int L, int N, float* thr_out,
                            int32_t* counts_out, long long* u2_out, float* auc_out,
                            int32_t* best_layer, float* tau, void* ws, hipStream_t s);

// Decoder-layer GEMM on the LM-head kernel's main loop: rows (bf16, gathered
// through the compact row list in the LM-head workspace `lm_ws_ptr`) times
// w^T [N][K], w packed (launch_pack_weight).  splits must divide K into multiples
// of 256.  swiglu: w is a packed gate / up pair, out[global row][f] =
// silu(gate) * up (bf16); otherwise part[split][compact row][n] = partial sums (fp32).
LmPlan gemm_plan(int rows, int N, bool swiglu);
hipError_t launch_gemm(const void* rows_in, const void* w, int total_rows, int K, int N,
                       const LmPlan& plan, int splits, bool swiglu, const void* lm_ws_ptr, float* part,
                       uint16_t* out, int ld, hipStream_t s);
// The gate / up projection (a packed pair) with split-K: part[split][compact row][f] =
// gate partial, part[split][compact row][N + f] = up partial (ld = 2 N).
hipError_t launch_gemm_pair(const void* rows_in, const void* w_gate_up, int total_rows, int K, int N,
                            const LmPlan& plan, int splits, const void* lm_ws_ptr, float* part,
                            hipStream_t s);

LmWsView lm_ws_view(void* ws, int rows);

// Multi-layer verification forward (embedding, decoder layers, final norm, LM head).
// Projections are packed (launch_pack_weight); norms and caches are plain bf16.
struct FwdLayer {
  const void* attn_norm;  // [hid] bf16
  const void* wqkv;       // [(Hq + 2 Hkv) d][hid]: q heads, then k heads, then v heads
  const void* wo;         // [hid][Hq d]
  const void* mlp_norm;   // [hid]
  const void* w_gate_up;  // the pair [inter][hid] gate, [inter][hid] up
  const void* w_down;     // [hid][inter]
  const void* k_cache;    // [sum n][Hkv][d] prefix keys after RoPE
  const void* v_cache;    // [sum n][Hkv][d]
};
struct FwdLayout {
  AttnPlan attn;
  LmPlan lm, p_qkv, p_o, p_gu, p_down;
  int s_qkv, s_o, s_down, s_gu;  // split-K factors
  size_t off_lm, off_attn, off_x, off_h, off_q, off_kc, off_vc, off_att, off_a, off_part, bytes;
};
FwdLayout fwd_layout(int B, int max_n, int W, int D, int Hq, int Hkv, int d, int inter, int V);
hipError_t launch_forward(const int32_t* ids, const int32_t* cu_len, const int32_t* cand,
                          const int32_t* cand_len, const uint8_t* copy_gate, const void* embed,
                          const FwdLayer* layers, int n_layers, const void* final_norm,
                          const void* lm_head, int B, int W, int D, int Hq, int Hkv, int d,
                          int inter, int V, float rope_base, float eps, const FwdLayout& L,
                          void* ws, int32_t* argmax_out, float* x_out, hipEvent_t ev_begin,
                          hipEvent_t ev_end, hipStream_t s);

}  // namespace ssd
