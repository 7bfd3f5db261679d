/*
 * switchsd.h — C ABI of the SwitchSD copy-speculation hot path on MI355X (gfx950).
 *
 * The method is SwitchSD ("To Copy or Not to Copy: Controlling Speculative
 * Decoding via Intrinsic Model Signals", arXiv 2609.20186).  One decoding step
 * of its copy path is four calls, all asynchronous on one HIP stream:
 *
 *   ssd_probe_score     copy-intent probe on the layer-l hidden state
 *   ssd_kgram_retrieve  kappa-gram evidence + up to W recency-ordered candidates
 *                       (ssd_probe_kgram_retrieve: both in one launch)
 *   ssd_blocktri_verify one verification pass: block-triangular attention, then
 *                       LM-head projection and greedy (T = 0) argmax per row
 *   ssd_accept_longest  longest accepted continuation and the token after it
 *                       (ssd_blocktri_verify_accept: verification and accept in
 *                       the verification's launches)
 *
 * and, after accept, ssd_commit_accepted copies the accepted tokens' keys and
 * values into the caller's KV cache and lists the tokens that extend the context.
 * At temperature T > 0, ssd_blocktri_verify_sample and ssd_accept_sample take the
 * place of ssd_blocktri_verify and ssd_accept_longest.  Once, when the model is
 * loaded, ssd_pack_weight (and ssd_pack_gate_up for an MLP's gate / up pair)
 * rearranges the bf16 weight matrices into the layout that the bf16 calls read.
 *
 * Offline, before decoding, three calls calibrate the probe (paper §3.2):
 *
 *   ssd_copy_labels     copy-mode label of every position of whole contexts
 *   ssd_probe_logits    probe logit of every position at every layer
 *   ssd_calibrate       per layer the F1-optimal threshold and ROC AUC, then the
 *                       layer and tau used by ssd_probe_score
 *
 * Conventions shared by every call:
 *  - Pointers to arrays are DEVICE pointers (hipMalloc / torch CUDA tensors);
 *    scalars are passed by value from the host.  Arrays are dense, row-major,
 *    with the layouts stated per argument.
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    synchronizes, keeps no global state, and may be called concurrently on
 *    different streams with disjoint output and workspace buffers.
 *  - Arguments are validated on the host before anything is launched; a call
 *    that returns an error launches nothing.  SSD_ERR_HIP reports a launch
 *    failure (hipGetLastError after the launches).
 *  - Device-side data contracts that the host cannot check are the caller's:
 *    cu_len is non-decreasing with cu_len[0] = 0, every context holds at least
 *    one token, token ids are non-negative.  Violations give wrong results,
 *    never out-of-range accesses outside the arrays described by cu_len.
 *  - bfloat16 arrays hold raw bf16 bit patterns (uint16); float arrays hold
 *    IEEE binary32.
 *
 * Row layout of the verification pass (paper §3.3 "Parallel Verification with
 * Block-Triangular Attention"): per sequence R = 1 + W*D query rows; row 0 is
 * the anchor (newest context token), row 1 + w*D + j is token j of candidate w.
 */
#ifndef SWITCHSD_H
#define SWITCHSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

#define SSD_ABI_VERSION 12

typedef enum {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = 1, /* null pointer, size out of range, tau outside (0,1), ... */
  SSD_ERR_UNSUPPORTED = 2, /* valid but not implemented shape (e.g. bf16 head dim != 128) */
  SSD_ERR_WORKSPACE = 3,   /* workspace missing or smaller than ssd_verify_workspace_bytes */
  SSD_ERR_HIP = 4          /* a kernel launch failed */
} ssd_status_t;

/* SSD_BF16_ROWS: bf16 like SSD_BF16 (bf16 storage, fp32 accumulation), with the
 * LM head given as the plain row-major [V][hid] matrix instead of the packed layout
 * of ssd_pack_weight.  Taken by the T = 0 verification calls only
 * (ssd_blocktri_verify, _noalloc, _accept); its weight stream is slower than the
 * packed layout's, each A-fragment load gathering 16 bytes from each of 32 rows. */
typedef enum { SSD_F32 = 0, SSD_BF16 = 1, SSD_BF16_ROWS = 2 } ssd_dtype_t;

/* Limits checked by validation. */
#define SSD_MAX_W 64      /* candidates per sequence */
#define SSD_MAX_D 64      /* tokens per candidate */
#define SSD_MAX_KAPPA 64  /* kappa-gram length */
#define SSD_MAX_NTRAIN 64 /* copy-label window length (calibration) */
#define SSD_MAX_PROBE_HIDDEN 16384 /* hidden size of the batched probe logits */
#define SSD_MAX_CALIB_N (1 << 28)  /* scored positions per layer (calibration) */
#define SSD_MAX_CALIB_L 65535      /* layers (calibration) */

int ssd_abi_version(void);
const char* ssd_status_string(int status);

/*
 * Copy-intent probe.  Paper §3.2 "Layer and Threshold Selection" and §3.3:
 * copy drafting is allowed only when PR(H_i^(l)) >= tau; write-up §2.3: the
 * probe is a bias-free linear projection trained with binary cross-entropy.
 * Computes z_b = sum_k w_k h_{b,k} (fp32 accumulation) and
 * fire_b = [sigmoid(z_b) >= tau], evaluated as z_b >= ln(tau / (1 - tau)).
 *   h        [B][hidden], dtype h_dtype (the anchor's layer-l state per sequence)
 *   w        [hidden] float (probe direction)
 *   z_out    [B] float, may be NULL
 *   fire_out [B] uint8 (1 = probe fired)
 * Errors: INVALID_ARG for null h/w/fire_out, B < 1, hidden < 1, tau not in (0,1).
 */
ssd_status_t ssd_probe_score(const void* h, ssd_dtype_t h_dtype, const float* w, int32_t B,
                             int32_t hidden, float tau, float* z_out, uint8_t* fire_out,
                             hipStream_t stream);

/*
 * kappa-gram evidence and candidate retrieval.  Write-up §2.5 (dual gate):
 * copying needs the probe to fire AND the kappa-gram ending at the current
 * token to have occurred earlier in the context.  Paper §3.3 "Copy-Based
 * Speculative Generation" / write-up §2.6: up to W continuations of up to D
 * tokens, ranked by recency.
 * For sequence b with ids x[0..n-1] = ids[cu_len[b] .. cu_len[b+1]-1]:
 *   earlier occurrences are end positions p, kappa-1 <= p <= n-2, with
 *   x[p-kappa+1..p] == x[n-kappa..n-1]; the W largest are kept, newest first;
 *   L_w = min(D, n-1-p_w), cand[w][j] = x[p_w+1+j] for j < L_w.
 *   If fire != NULL and fire[b] == 0 nothing is retrieved for b.
 *   ids       [cu_len[B]] int32
 *   cu_len    [B+1] int32 offsets
 *   fire      [B] uint8 or NULL (NULL = every probe fired)
 *   match_end [B][W] int32, -1 padded      n_match [B] int32 = M
 *   cand      [B][W][D] int32, -1 padded   cand_len [B][W] int32 (0 for w >= M)
 *   copy_gate [B] uint8 = fired && M > 0
 * Errors: INVALID_ARG for null pointers (fire excepted), B < 1,
 *   kappa not in [1, SSD_MAX_KAPPA], W not in [1, SSD_MAX_W], D not in [1, SSD_MAX_D].
 * Data contract (device-side, not checked): cu_len is non-decreasing and every
 *   context holds fewer than 2^29 - 2^14 ids (byte offsets inside a context are
 *   32-bit).
 */
ssd_status_t ssd_kgram_retrieve(const int32_t* ids, const int32_t* cu_len, int32_t B,
                                int32_t kappa, int32_t W, int32_t D, const uint8_t* fire,
                                int32_t* match_end, int32_t* n_match, int32_t* cand,
                                int32_t* cand_len, uint8_t* copy_gate, hipStream_t stream);

/*
 * The probe and the retrieval in one launch: exactly ssd_probe_score followed by
 * ssd_kgram_retrieve with fire = fire_out (paper §3.2 "Layer and Threshold
 * Selection" and §3.3; write-up §2.3 and §2.5, the dual gate), for callers that
 * want one launch per step less.  Sequence b's workgroup starts the copies of its
 * first context chunks, computes z_b = w . h_b while they are in flight, and
 * scans only if the probe fired.  Arguments, layouts and outputs are those of the
 * two calls (h [B][hidden] of dtype h_dtype, w [hidden] float, z_out [B] float or
 * NULL, fire_out [B] uint8; ids, cu_len, match_end, n_match, cand, cand_len,
 * copy_gate as in ssd_kgram_retrieve).  z_b may differ from ssd_probe_score's in
 * the last bits (another summation order); fire_b is then decided on this z_b.
 * Errors: the union of the two calls' (INVALID_ARG).
 */
ssd_status_t ssd_probe_kgram_retrieve(const void* h, ssd_dtype_t h_dtype, const float* w,
                                      int32_t hidden, float tau, float* z_out, uint8_t* fire_out,
                                      const int32_t* ids, const int32_t* cu_len, int32_t B,
                                      int32_t kappa, int32_t W, int32_t D, int32_t* match_end,
                                      int32_t* n_match, int32_t* cand, int32_t* cand_len,
                                      uint8_t* copy_gate, hipStream_t stream);

/*
 * Packed bf16 weights.  The projection of the verification pass (paper §3.3: all
 * candidates are checked in one target pass, ending in the LM head) streams the
 * whole N x K weight matrix once per pass; the bf16 kernels read it in a layout
 * where every wave's weight fragments for one 64-wide k-slab form one contiguous
 * 8 KB run.  Rearranging is a pure permutation (plus zero rows up to a multiple
 * of 256 tile rows), done once per model:
 *   w       [rows][K] bf16, row-major, 16-byte aligned (row n = weights of
 *           output n; for the LM head, token n)
 *   packed  ssd_pack_weight_bytes(rows, K) bytes, 16-byte aligned, caller-owned;
 *           16-byte chunk c = (((t * K/64 + s) * 4 + w) * 8 + 4a + j) * 64 + 32h + l
 *           holds tile row 64w + 32a + l of tile t, columns 64s + 16j + 8h .. +7;
 *           tile row r of tile t is row 256t + r (zeros for rows past the end)
 * ssd_pack_gate_up packs the gate and up projections of an MLP, w_gate and w_up
 * [inter][K] each, into one buffer of ssd_pack_gate_up_bytes(inter, K) bytes with
 * the same chunk order, where tile row 64w + 32a + l of tile t is feature
 * 128t + 32w + l of w_gate (a = 0) or of w_up (a = 1): the kernel then finds a
 * feature's gate and up weights in the same lane.
 * The _bytes queries return 0 for sizes < 1, K % 256 != 0 or K > 2^20.
 * Errors: INVALID_ARG (nulls, sizes < 1, misaligned pointers), UNSUPPORTED
 *   (K % 256 != 0 or K > 2^20), WORKSPACE (packed_bytes too small).
 */
size_t ssd_pack_weight_bytes(int32_t rows, int32_t K);
ssd_status_t ssd_pack_weight(const void* w, int32_t rows, int32_t K, void* packed,
                             size_t packed_bytes, hipStream_t stream);
size_t ssd_pack_gate_up_bytes(int32_t inter, int32_t K);
ssd_status_t ssd_pack_gate_up(const void* w_gate, const void* w_up, int32_t inter, int32_t K,
                              void* packed, size_t packed_bytes, hipStream_t stream);

/* Bytes of scratch that ssd_blocktri_verify needs for these sizes (0 on bad sizes). */
size_t ssd_verify_workspace_bytes(int32_t B, int32_t max_n, int32_t W, int32_t D, int32_t Hq,
                                  int32_t Hkv, int32_t d, int32_t V, ssd_dtype_t dtype);

/*
 * One verification pass.  Paper §3.3 "Parallel Verification with
 * Block-Triangular Attention": candidates follow the anchor; a token of
 * candidate w attends to the whole prefix and to candidate w's tokens up to
 * and including itself, never to another candidate; all candidates are checked
 * in one target pass.  Write-up §3.1: decoding at T = 0, so each row's
 * verdict is the argmax of its logits.
 * Attention (per query head h, key/value head h / (Hq/Hkv), scores scale*q.k):
 *   q        [B][R][Hq][d]          queries (post positional encoding)
 *   k_pre, v_pre [cu_len[B]][Hkv][d] prefix cache (entry n_b-1 is the anchor)
 *   k_cand, v_cand [B][W*D][Hkv][d] candidate keys/values
 *   cand_len [B][W], copy_gate [B]  from ssd_kgram_retrieve; sequences whose gate
 *                                   is closed are skipped entirely
 *   attn_out [B][R][Hq*d]           head-major concatenation; rows that are not
 *                                   real (gate closed, w >= M, j >= L_w) are zeros
 * LM head + argmax:
 *   lm_head  fp32: [V][Hq*d]        transposed projection (row v = weights of token v)
 *            SSD_BF16: that matrix as written by ssd_pack_weight
 *            SSD_BF16_ROWS: that matrix itself, bf16 row-major
 *   argmax_out [B][R] int32         lowest index among equal maxima (NaN logits
 *                                   never win); -1 on rows that are not real and
 *                                   on rows whose logits are all NaN
 *   logits_out [B][R][V] float or NULL (debug output; written for every row)
 * dtype: SSD_F32 (all float), SSD_BF16 (all bf16, fp32 accumulation) or SSD_BF16_ROWS
 *   (as SSD_BF16 with a row-major LM head).
 * max_n: host-side upper bound on the context lengths (every cu_len[b+1] -
 * cu_len[b] <= max_n), used to size the launch; results do not depend on it.
 * workspace: device scratch of at least ssd_verify_workspace_bytes(...) bytes;
 *   its contents on entry do not matter.
 * lm_begin, lm_end: optional events (may be NULL) recorded on `stream`
 *   immediately before and after the LM-head contraction kernel, for timing.
 * q, k_pre, v_pre, k_cand, v_cand, lm_head and attn_out must be 16-byte aligned.
 * Errors: INVALID_ARG (nulls, sizes < 1, Hq % Hkv != 0, scale not finite > 0,
 *   W/D above limits, misaligned pointers), UNSUPPORTED (bf16 with d != 128 or Hq*d % 256 != 0, or
 *   beyond the bf16 kernels' 32-bit byte offsets: (max_n + 64)*Hkv*d*2 or
 *   B*R*Hq*d*2 not below 0x7ffffff0; fp32 with d not in {64, 128}; B*R*Hq not
 *   below 2^31), WORKSPACE.
 */
ssd_status_t ssd_blocktri_verify(const void* q, const void* k_pre, const void* v_pre,
                                 const int32_t* cu_len, int32_t max_n, const void* k_cand,
                                 const void* v_cand, const int32_t* cand_len,
                                 const uint8_t* copy_gate, const void* lm_head, int32_t B,
                                 int32_t W, int32_t D, int32_t Hq, int32_t Hkv, int32_t d,
                                 int32_t V, ssd_dtype_t dtype, float scale, void* attn_out,
                                 int32_t* argmax_out, float* logits_out, void* workspace,
                                 size_t workspace_bytes, hipEvent_t lm_begin, hipEvent_t lm_end,
                                 hipStream_t stream);

/*
 * ssd_blocktri_verify without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It computes exactly what ssd_blocktri_verify
 * computes (same arguments and outputs; no timing events) and allocates nothing:
 * its scratch is a device array of SSD_NOALLOC_SCRATCH_BYTES (64 MiB) inside the
 * library, one per GPU, held from the first call on that GPU until the process
 * ends.  The current device must be the device of `stream` and of the buffers.
 * Every call on a GPU shares that GPU's scratch, so calls that overlap on one GPU
 * (on different streams, or from several threads) race; calls on one stream are
 * ordered and safe.  Nothing in the scratch needs to be zero on entry.
 * Errors: as ssd_blocktri_verify; WORKSPACE when ssd_verify_workspace_bytes(...)
 *   of the call exceeds SSD_NOALLOC_SCRATCH_BYTES; HIP when the scratch's device
 *   address cannot be obtained.
 */
#define SSD_NOALLOC_SCRATCH_BYTES (64ull << 20)
ssd_status_t ssd_blocktri_verify_noalloc(const void* q, const void* k_pre, const void* v_pre,
                                         const int32_t* cu_len, int32_t max_n, const void* k_cand,
                                         const void* v_cand, const int32_t* cand_len,
                                         const uint8_t* copy_gate, const void* lm_head, int32_t B,
                                         int32_t W, int32_t D, int32_t Hq, int32_t Hkv, int32_t d,
                                         int32_t V, ssd_dtype_t dtype, float scale, void* attn_out,
                                         int32_t* argmax_out, float* logits_out, hipStream_t stream);

/*
 * Longest accepted continuation at T = 0.  Paper §3.3: the longest validated
 * continuation is kept; greedy verification stops at the first disagreement.
 *   pred(w, -1) = argmax[b][0]; pred(w, j) = argmax[b][1 + w*D + j]
 *   a_w = largest k <= L_w with cand[w][j] == pred(w, j-1) for all j < k
 *   best_w = argmax_w a_w (lowest w on ties), best_len = a_{best_w},
 *   next_token = pred(best_w, best_len - 1) (the target's token after the
 *   accepted ones; argmax[b][0] when best_len = 0).
 *   Closed gate: accept_len = 0, best_w = -1, best_len = 0, next_token = -1.
 *   cand [B][W][D], cand_len [B][W], copy_gate [B], argmax [B][R] (inputs)
 *   accept_len [B][W], best_w [B], best_len [B], next_token [B] (int32 outputs)
 * Errors: INVALID_ARG for nulls, B < 1, W or D outside [1, limit].
 */
ssd_status_t ssd_accept_longest(const int32_t* cand, const int32_t* cand_len,
                                const uint8_t* copy_gate, const int32_t* argmax, int32_t B,
                                int32_t W, int32_t D, int32_t* accept_len, int32_t* best_w,
                                int32_t* best_len, int32_t* next_token, hipStream_t stream);

/*
 * One verification pass followed by the accept, in the launches of the
 * verification alone: exactly ssd_blocktri_verify (no logits output) and then
 * ssd_accept_longest on its argmax_out (paper §3.3 "Parallel Verification with
 * Block-Triangular Attention" and the longest-validated-continuation rule; write-up
 * §3.1), for callers that want the step's fixed launch cost lower.  The accept
 * runs in the launch after the LM head that turns its per-row results into
 * argmax_out (both dtypes).  Arguments and outputs are those of the two calls: cand [B][W][D]
 * int32 (from ssd_kgram_retrieve), accept_len [B][W], best_w, best_len,
 * next_token [B] int32; workspace of ssd_verify_workspace_bytes(...) bytes.
 * Errors: those of ssd_blocktri_verify, and INVALID_ARG for null cand or accept
 *   outputs.
 */
ssd_status_t ssd_blocktri_verify_accept(const void* q, const void* k_pre, const void* v_pre,
                                        const int32_t* cu_len, int32_t max_n, const void* k_cand,
                                        const void* v_cand, const int32_t* cand,
                                        const int32_t* cand_len, const uint8_t* copy_gate,
                                        const void* lm_head, int32_t B, int32_t W, int32_t D,
                                        int32_t Hq, int32_t Hkv, int32_t d, int32_t V,
                                        ssd_dtype_t dtype, float scale, void* attn_out,
                                        int32_t* argmax_out, int32_t* accept_len, int32_t* best_w,
                                        int32_t* best_len, int32_t* next_token, void* workspace,
                                        size_t workspace_bytes, hipEvent_t lm_begin,
                                        hipEvent_t lm_end, hipStream_t stream);

/*
 * Commit of the accepted draft into the target's KV cache.  Paper §3.3: the
 * longest validated continuation extends the context, and greedy decoding adds
 * the target's token after it (the next anchor, whose K/V the caller computes
 * in its next pass).  The verification pass already holds the accepted tokens'
 * keys and values.  For every sequence b with best_w[b] >= 0, rows
 * (best_w, 0..best_len-1) of k_cand / v_cand are copied, in order, to cache
 * rows cache_off[b] .. cache_off[b] + best_len[b] - 1.
 *   k_cand, v_cand [B][W*D][Hkv][d] (the verify inputs; dtype as given)
 *   cand [B][W][D] int32; best_w, best_len, next_token [B] int32 (the
 *   ssd_accept_longest outputs)
 *   k_cache, v_cache [cache_rows][Hkv][d], same dtype: the caller's cache
 *   cache_off [B] int64: first cache row written for sequence b (typically
 *   where that sequence's context ends)
 *   tokens_out [B][D+1] int32 (output): the accepted tokens then next_token,
 *   padded with -1
 *   n_tokens_out [B] int32 (output): best_len + 1; 0 for a closed gate; -1 when
 *   best_w / best_len are out of range or the rows do not fit
 *   (cache_off < 0 or cache_off + best_len > cache_rows).  Nothing is written
 *   to the cache in the last two cases.
 * Errors: INVALID_ARG (nulls, B < 1, W or D outside [1, limit], Hkv or d < 1,
 *   cache_rows < 1, unknown dtype), UNSUPPORTED (Hkv*d*element size not a
 *   multiple of 16 bytes).
 */
ssd_status_t ssd_commit_accepted(const void* k_cand, const void* v_cand, const int32_t* cand,
                                 const int32_t* best_w, const int32_t* best_len,
                                 const int32_t* next_token, int32_t B, int32_t W, int32_t D,
                                 int32_t Hkv, int32_t d, ssd_dtype_t dtype, void* k_cache,
                                 void* v_cache, int64_t cache_rows, const int64_t* cache_off,
                                 int32_t* tokens_out, int32_t* n_tokens_out, hipStream_t stream);

/*
 * Verification pass at temperature T > 0 (bf16 only).  The pages give no rule
 * for copy candidates at T > 0; they require that verification by the target
 * keeps speculative decoding's guarantee (paper §3.3 "Overall Framework", §2
 * "Speculative Decoding"; lossless acceptance as on the VIA-SD page "Draft-Verify
 * and Lossy Acceptance").  Each candidate is a point-mass draft: its token is
 * accepted with the target probability left after the tokens already rejected at
 * the same node of the candidates' trie, and the next token is drawn from the
 * target distribution without the rejected children (recursive rejection
 * sampling; every emitted token then follows the target's law).
 * Attention is as in ssd_blocktri_verify.  Then, per real row g = b*R + r (the
 * LM head's epilogue; logits are never written):
 *   - the trie: a node is identified by the row of its distribution (the anchor
 *     row for the root; row (w, j-1) for the node after j tokens, w the lowest
 *     candidate with those tokens); its children are the distinct next tokens of
 *     its candidates, ordered by lowest candidate.
 *   n_children [B*R] int32 (out): children of the node at row g, 0 for rows that
 *                                 are no node
 *   children, child_w [B*R][W] int32 (out): token and lowest candidate of child k,
 *                                 k < n_children[g]
 *   child_logit [B*R][W] float (out): logits[g][children[g][k]] / T; -inf for a
 *                                 token outside [0, V)
 *   lse [B*R] float (out): log-sum-exp over the vocabulary of logits[g] / T; -inf
 *                          on rows that are not real
 *   resample [B*R] int32 (out): the residual draw: argmax over the tokens x that
 *                          are not children of row g of logits[g][x] / T + G(g, x),
 *                          lowest x on ties; -1 on rows that are not real
 * G(g, x) = -ln(-ln u), u = (floor(w / 512) + 1/2) / 2^23 with w word x%4 of
 * Philox4x32-10(counter (x/4, g, 0, 0), key (seed low, seed high)).
 *   cand [B][W][D] int32: the retrieval's candidates (ssd_kgram_retrieve)
 *   temperature: finite, > 0, with a finite reciprocal
 * Other arguments, workspace and events as for ssd_blocktri_verify.
 * Errors: as ssd_blocktri_verify; INVALID_ARG for a bad temperature or a null
 *   output; UNSUPPORTED for SSD_F32 and SSD_BF16_ROWS (the sampling epilogue reads
 *   the packed LM head only).
 */
ssd_status_t ssd_blocktri_verify_sample(
    const void* q, const void* k_pre, const void* v_pre, const int32_t* cu_len, int32_t max_n,
    const void* k_cand, const void* v_cand, const int32_t* cand, const int32_t* cand_len,
    const uint8_t* copy_gate, const void* lm_head, int32_t B, int32_t W, int32_t D, int32_t Hq,
    int32_t Hkv, int32_t d, int32_t V, ssd_dtype_t dtype, float scale, float temperature,
    uint64_t seed, void* attn_out, int32_t* n_children, int32_t* children, int32_t* child_w,
    float* child_logit, float* lse, int32_t* resample, void* workspace, size_t workspace_bytes,
    hipEvent_t lm_begin, hipEvent_t lm_end, hipStream_t stream);

/*
 * Acceptance at T > 0: the walk over the trie written by
 * ssd_blocktri_verify_sample (same seed).  From the root, child k of the node at
 * row g is accepted when u < r, with u from word 0 of Philox4x32-10(counter
 * (k, g, 1, 0), key (seed low, seed high)) as above and
 * r = p / max(1 - tried, p), p = exp(child_logit - lse[g]), tried = the p of the
 * children rejected before it (r = 0 when p = 0).  An accepted child moves the
 * walk to row 1 + child_w*D + j; when no child is accepted the walk ends with
 * next_token = resample[g].
 *   best_w [B] int32: lowest candidate of the accepted path (0 when nothing is
 *                     accepted; -1 for a closed gate)
 *   best_len [B] int32: accepted tokens (0 for a closed gate)
 *   next_token [B] int32: the token drawn after them (-1 for a closed gate)
 * Errors: INVALID_ARG (nulls, B < 1, W or D outside [1, limit]).
 */
ssd_status_t ssd_accept_sample(const int32_t* n_children, const int32_t* child_w,
                               const float* child_logit, const float* lse, const int32_t* resample,
                               const uint8_t* copy_gate, int32_t B, int32_t W, int32_t D,
                               uint64_t seed, int32_t* best_w, int32_t* best_len,
                               int32_t* next_token, hipStream_t stream);

/*
 * Verification pass as a full target forward (bf16).  Paper §3.3 "Parallel
 * Verification with Block-Triangular Attention": the anchor and all W
 * candidates go through one target forward, candidate tokens seeing the prefix
 * and their own earlier tokens.  The layer is the Llama-family pre-norm decoder
 * layer of the paper's targets (§4.1):
 *   h = RMSNorm(x) * attn_norm;  q, k, v = W_qkv h;  RoPE(q), RoPE(k);
 *   x += W_o BlockTriAttention(q, k, v);  h = RMSNorm(x) * mlp_norm;
 *   x += W_down (silu(W_gate h) * (W_up h));
 * after the layers h = RMSNorm(x) * final_norm feeds the LM head and argmax.
 * RMSNorm(x) = x / sqrt(mean(x^2) + eps).  Row tokens: the anchor (the last
 * context token) at row 0, candidate token j of w at row 1 + w*D + j; their
 * positions n - 1 and n + j.  RoPE turns the adjacent pair (2i, 2i+1) of every
 * q and k head by pos * rope_base^(-2i/d).  The prefix caches hold every
 * context token's key (after RoPE) and value, the anchor's included.  The
 * residual stream is fp32; the activations between steps (h, q, k, v, the
 * attention output, the MLP activation) are bf16.  Only real rows are computed.
 * Weights, all bf16, [out][in] (the projections packed by ssd_pack_weight):
 *   embed [V][hid] and final_norm [hid] row-major; lm_head [V][hid] packed;
 *   per layer (ssd_layer_t, an array of n_layers on the host): attn_norm,
 *   mlp_norm [hid]; wqkv [(Hq + 2 Hkv) d][hid] packed (q heads, then k heads,
 *   then v heads); wo [hid][Hq d] packed; w_gate_up: the gate and up
 *   projections [inter][hid] each, packed by ssd_pack_gate_up; w_down
 *   [hid][inter] packed; k_cache, v_cache [cu_len[B]][Hkv][d] row-major.
 *   ids, cu_len, cand [B][W][D], cand_len, copy_gate: as for retrieval / verify.
 *   argmax_out [B][R] int32: as ssd_blocktri_verify (-1 on rows that are not real)
 *   x_out [B][R][hid] float or NULL, 16-byte aligned: the final residual stream
 *         (0 on rows that are not real)
 *   workspace: ssd_verify_forward_workspace_bytes(...) bytes, 16-byte aligned.
 *   begin, end: optional events recorded around the whole forward.
 * hid = Hq*d.  Errors: INVALID_ARG (nulls, sizes < 1, n_layers < 0, Hq % Hkv,
 *   limits, rope_base <= 1 or eps not finite > 0, misaligned x_out), UNSUPPORTED (d != 128,
 *   hid % 256, inter % 256, hid > 8192, or (max_n + 64)*Hkv*d*2 or
 *   B*R*max(hid, inter)*2 not below 0x7ffffff0), WORKSPACE.
 */
typedef struct {
  const void* attn_norm;
  const void* wqkv;
  const void* wo;
  const void* mlp_norm;
  const void* w_gate_up;
  const void* w_down;
  const void* k_cache;
  const void* v_cache;
} ssd_layer_t;

size_t ssd_verify_forward_workspace_bytes(int32_t B, int32_t max_n, int32_t W, int32_t D,
                                          int32_t Hq, int32_t Hkv, int32_t d, int32_t inter,
                                          int32_t V);
ssd_status_t ssd_verify_forward(const int32_t* ids, const int32_t* cu_len, int32_t max_n,
                                const int32_t* cand, const int32_t* cand_len,
                                const uint8_t* copy_gate, const void* embed,
                                const ssd_layer_t* layers, int32_t n_layers, const void* final_norm,
                                const void* lm_head, int32_t B, int32_t W, int32_t D, int32_t Hq,
                                int32_t Hkv, int32_t d, int32_t inter, int32_t V, float rope_base,
                                float eps, int32_t* argmax_out, float* x_out, void* workspace,
                                size_t workspace_bytes, hipEvent_t begin, hipEvent_t end,
                                hipStream_t stream);

/*
 * Offline probe calibration, step 1: copy-mode labels.  Paper §3.2 "Problem
 * Formulation": a position is a copy-mode instance when it lies inside a
 * verbatim run of at least n_train tokens that also occurs earlier in the same
 * context.  Computed as: labels[i] = 1 exactly when some n_train-window
 * containing i (inside i's context) also starts at an earlier position of that
 * context (the earlier occurrence may overlap it).
 *   ids      [total_n] int32: the contexts, concatenated
 *   cu_len   [B+1] int32: context b is ids[cu_len[b] .. cu_len[b+1]); the caller
 *            guarantees cu_len[B] == total_n
 *   labels   [total_n] uint8 (output): 1 = copy-mode, 0 = not
 *   workspace at least ssd_copy_labels_workspace_bytes(total_n) bytes of device
 *            memory, 8-byte aligned; its contents on entry do not matter
 * Errors: INVALID_ARG (nulls, B < 1, total_n outside [1, 2^30), n_train outside
 *   [1, SSD_MAX_NTRAIN]), WORKSPACE.
 */
size_t ssd_copy_labels_workspace_bytes(int64_t total_n);
ssd_status_t ssd_copy_labels(const int32_t* ids, const int32_t* cu_len, int32_t B,
                             int64_t total_n, int32_t n_train, uint8_t* labels, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Offline probe calibration, step 2: probe logits of every position at every
 * layer (paper §3.2: a probe per layer, scored on the layer's hidden states;
 * write-up §2.3: bias-free linear probe).
 *   z[l][i] = sum_k w[l][k] * h[l][i][k]   (fp32 fused multiply-adds)
 *   h  [L][N][hidden], dtype h_dtype
 *   w  [L][hidden] float
 *   z_out [L][N] float (output)
 * Errors: INVALID_ARG (nulls, L outside [1, SSD_MAX_CALIB_L], N outside
 *   [1, 2^36), hidden < 1, unknown dtype), UNSUPPORTED (hidden >
 *   SSD_MAX_PROBE_HIDDEN).
 */
ssd_status_t ssd_probe_logits(const void* h, ssd_dtype_t h_dtype, const float* w, int32_t L,
                              int64_t N, int32_t hidden, float* z_out, hipStream_t stream);

/*
 * Offline probe calibration, step 3: threshold and layer.  Paper §3.2 "Layer
 * and Threshold Selection": per layer the decision threshold maximising F1 on
 * the labelled set, and the layer with the highest F1; §4.3.3 reports the ROC AUC.
 * Per layer l, over the thresholds t in {z[l][i]} with copy predicted when
 * z >= t: the t with the highest F1 = 2TP / (2TP + FP + FN) (compared exactly as
 * integer fractions; a tie goes to the higher t), and 2U, the Mann-Whitney
 * statistic doubled (equal scores count one half each).  Then the layer with the
 * highest F1 (the lower layer on ties) and tau = sigmoid(its t).
 *   z       [L][N] float: scores (finite; -0 and +0 are one score)
 *   labels  [N] uint8: nonzero = copy-mode (the same positions for every layer)
 *   thr_out [L] float: the chosen t per layer; +inf when no t gives TP > 0
 *   counts_out [L][4] int32: TP, FP, FN at that t, and the positives P
 *   u2_out  [L] int64: 2U;  auc_out [L] float: 2U / (2 P (N - P)), NaN when
 *           P = 0 or P = N
 *   best_layer [1] int32, tau_out [1] float: the layer choice and
 *           sigmoid(thr_out[best_layer]) (1 for t = +inf)
 *   workspace at least ssd_calibrate_workspace_bytes(L, N) bytes, 8-byte aligned
 * Errors: INVALID_ARG (nulls, L outside [1, SSD_MAX_CALIB_L], N outside
 *   [1, SSD_MAX_CALIB_N]), WORKSPACE.
 */
size_t ssd_calibrate_workspace_bytes(int32_t L, int64_t N);
ssd_status_t ssd_calibrate(const float* z, const uint8_t* labels, int32_t L, int64_t N,
                           float* thr_out, int32_t* counts_out, int64_t* u2_out, float* auc_out,
                           int32_t* best_layer, float* tau_out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SWITCHSD_H */
