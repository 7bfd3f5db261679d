// C ABI of the copy-speculation path: argument validation, launch planning and
// dispatch.  No allocation, no synchronisation; the only global state is the
// device scratch of ssd_blocktri_verify_noalloc (below).
#include <cmath>
#include <mutex>

#include "switchsd.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool valid_dtype(ssd_dtype_t t) { return t == SSD_F32 || t == SSD_BF16; }
// the verification calls also take bf16 with a row-major LM head
bool valid_verify_dtype(ssd_dtype_t t) { return valid_dtype(t) || t == SSD_BF16_ROWS; }

ssd_status_t from_hip(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

// The bf16 kernels address one sequence's keys (with a 64-key block of slack past
// the last one) and the whole row matrix fed to a GEMM with 32-bit byte offsets.
bool fits_byte_offsets(long long B, long long max_n, long long R, long long Hkv, long long d,
                       long long widest) {
  constexpr long long kLimit = 0x7ffffff0;  // the kernels' out-of-range offset
  return (max_n + 64) * Hkv * d * 2 < kLimit && B * R * widest * 2 < kLimit;
}

// shape checks shared by the workspace query and the verify call
ssd_status_t check_verify_shape(int32_t B, int32_t max_n, int32_t W, int32_t D, int32_t Hq,
                                int32_t Hkv, int32_t d, int32_t V, ssd_dtype_t dt) {
  if (B < 1 || max_n < 1 || W < 1 || D < 1 || Hq < 1 || Hkv < 1 || d < 1 || V < 1)
    return SSD_ERR_INVALID_ARG;
  if (W > SSD_MAX_W || D > SSD_MAX_D || Hq % Hkv != 0 || !valid_verify_dtype(dt)) return SSD_ERR_INVALID_ARG;
  const long long R = 1 + static_cast<long long>(W) * D;
  if (static_cast<long long>(B) * R * Hq * d > (1ll << 40)) return SSD_ERR_INVALID_ARG;
  if (static_cast<long long>(B) * R * Hq >= (1ll << 31)) return SSD_ERR_UNSUPPORTED;
  if (dt != SSD_F32) {
    if (d != 128 || (static_cast<long long>(Hq) * d) % 256 != 0) return SSD_ERR_UNSUPPORTED;
    if (!fits_byte_offsets(B, max_n, R, Hkv, d, static_cast<long long>(Hq) * d))
      return SSD_ERR_UNSUPPORTED;
  } else {
    if (d != 64 && d != 128) return SSD_ERR_UNSUPPORTED;
  }
  return SSD_OK;
}

struct VerifyLayout {
  ssd::AttnPlan attn;
  ssd::LmPlan lm;
  size_t attn_bytes, lm_bytes;
};

VerifyLayout verify_layout(int32_t B, int32_t max_n, int32_t W, int32_t D, int32_t Hq, int32_t Hkv,
                           int32_t d, int32_t V, bool bf16) {
  VerifyLayout L;
  const int R = 1 + W * D;
  L.attn = ssd::attn_plan(B, max_n, R, Hq, Hkv, bf16);
  L.lm = ssd::lm_plan(B * R, V, bf16);
  L.attn_bytes = align_up(ssd::attn_workspace_bytes(L.attn, B, R, Hq, d));
  L.lm_bytes = align_up(ssd::lm_workspace_bytes(L.lm, B * R));
  return L;
}

}  // namespace

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char* ssd_status_string(int status) {
  switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARG: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

ssd_status_t ssd_probe_score(const void* h, ssd_dtype_t h_dtype, const float* w, int32_t B,
                             int32_t hidden, float tau, float* z_out, uint8_t* fire_out,
                             hipStream_t stream) {
  if (!h || !w || !fire_out || B < 1 || hidden < 1 || !valid_dtype(h_dtype))
    return SSD_ERR_INVALID_ARG;
  if (!(tau > 0.f && tau < 1.f)) return SSD_ERR_INVALID_ARG;
  const double t = static_cast<double>(tau);
  const float thr = static_cast<float>(std::log(t / (1.0 - t)));
  return from_hip(ssd::launch_probe(h, h_dtype == SSD_BF16, w, B, hidden, thr, z_out, fire_out, stream));
}

ssd_status_t ssd_kgram_retrieve(const int32_t* ids, const int32_t* cu_len, int32_t B,
                                int32_t kappa, int32_t W, int32_t D, const uint8_t* fire,
                                int32_t* match_end, int32_t* n_match, int32_t* cand,
                                int32_t* cand_len, uint8_t* copy_gate, hipStream_t stream) {
  if (!ids || !cu_len || !match_end || !n_match || !cand || !cand_len || !copy_gate)
    return SSD_ERR_INVALID_ARG;
  if (B < 1 || kappa < 1 || kappa > SSD_MAX_KAPPA || W < 1 || W > SSD_MAX_W || D < 1 || D > SSD_MAX_D)
    return SSD_ERR_INVALID_ARG;
  return from_hip(ssd::launch_kgram(ids, cu_len, B, kappa, W, D, fire, match_end, n_match, cand,
                                    cand_len, copy_gate, stream));
}

ssd_status_t ssd_probe_kgram_retrieve(const void* h, ssd_dtype_t h_dtype, const float* w,
                                      int32_t hidden, float tau, float* z_out, uint8_t* fire_out,
                                      const int32_t* ids, const int32_t* cu_len, int32_t B,
                                      int32_t kappa, int32_t W, int32_t D, int32_t* match_end,
                                      int32_t* n_match, int32_t* cand, int32_t* cand_len,
                                      uint8_t* copy_gate, hipStream_t stream) {
  if (!h || !w || !fire_out || hidden < 1 || !valid_dtype(h_dtype)) return SSD_ERR_INVALID_ARG;
  if (!(tau > 0.f && tau < 1.f)) return SSD_ERR_INVALID_ARG;
  if (!ids || !cu_len || !match_end || !n_match || !cand || !cand_len || !copy_gate)
    return SSD_ERR_INVALID_ARG;
  if (B < 1 || kappa < 1 || kappa > SSD_MAX_KAPPA || W < 1 || W > SSD_MAX_W || D < 1 || D > SSD_MAX_D)
    return SSD_ERR_INVALID_ARG;
  const double t = static_cast<double>(tau);
  ssd::KgProbe pr;
  pr.h = h;
  pr.bf16 = h_dtype == SSD_BF16;
  pr.w = w;
  pr.hidden = hidden;
  pr.thr = static_cast<float>(std::log(t / (1.0 - t)));
  pr.z_out = z_out;
  pr.fire_out = fire_out;
  return from_hip(ssd::launch_kgram(ids, cu_len, B, kappa, W, D, nullptr, match_end, n_match, cand,
                                    cand_len, copy_gate, stream, &pr));
}

size_t ssd_pack_weight_bytes(int32_t rows, int32_t K) {
  if (rows < 1 || K < 1 || K % ssd::lm_k_align() != 0 || K > (1 << 20)) return 0;
  return ssd::packed_weight_bytes(rows, K, false);
}

size_t ssd_pack_gate_up_bytes(int32_t inter, int32_t K) {
  if (inter < 1 || K < 1 || K % ssd::lm_k_align() != 0 || K > (1 << 20)) return 0;
  return ssd::packed_weight_bytes(inter, K, true);
}

namespace {
bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// The verification kernels read q, K, V and the LM-head weights and write the
// attention output in 16-byte pieces.
bool verify_aligned(const void* q, const void* k_pre, const void* v_pre, const void* k_cand,
                    const void* v_cand, const void* lm_head, const void* attn_out) {
  return aligned16(q) && aligned16(k_pre) && aligned16(v_pre) && aligned16(k_cand) &&
         aligned16(v_cand) && aligned16(lm_head) && aligned16(attn_out);
}

ssd_status_t pack(const void* w, const void* w2, int32_t rows, int32_t K, void* packed,
                  size_t packed_bytes, hipStream_t stream) {
  if (!w || !packed || rows < 1 || K < 1) return SSD_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(w2) || !aligned16(packed)) return SSD_ERR_INVALID_ARG;
  if (K % ssd::lm_k_align() != 0 || K > (1 << 20)) return SSD_ERR_UNSUPPORTED;
  if (packed_bytes < ssd::packed_weight_bytes(rows, K, w2 != nullptr)) return SSD_ERR_WORKSPACE;
  return from_hip(ssd::launch_pack_weight(w, w2, rows, K, packed, stream));
}
}  // namespace

ssd_status_t ssd_pack_weight(const void* w, int32_t rows, int32_t K, void* packed,
                             size_t packed_bytes, hipStream_t stream) {
  return pack(w, nullptr, rows, K, packed, packed_bytes, stream);
}

ssd_status_t ssd_pack_gate_up(const void* w_gate, const void* w_up, int32_t inter, int32_t K,
                              void* packed, size_t packed_bytes, hipStream_t stream) {
  if (!w_up) return SSD_ERR_INVALID_ARG;
  return pack(w_gate, w_up, inter, K, packed, packed_bytes, stream);
}

size_t ssd_verify_workspace_bytes(int32_t B, int32_t max_n, int32_t W, int32_t D, int32_t Hq,
                                  int32_t Hkv, int32_t d, int32_t V, ssd_dtype_t dtype) {
  if (check_verify_shape(B, max_n, W, D, Hq, Hkv, d, V, dtype) != SSD_OK) return 0;
  const VerifyLayout L = verify_layout(B, max_n, W, D, Hq, Hkv, d, V, dtype != SSD_F32);
  return L.attn_bytes + L.lm_bytes;
}

}  // extern "C"

namespace {
// ssd_blocktri_verify and its no-allocation variant; the workspace (or the scratch)
// is resolved by `get_ws` once the layout is known: it returns the buffer, or null
// with *err set.
template <typename GetWs>
ssd_status_t verify_impl(const void* q, const void* k_pre, const void* v_pre, const int32_t* cu_len,
                         int32_t max_n, const void* k_cand, const void* v_cand,
                         const int32_t* cand_len, const uint8_t* copy_gate, const void* lm_head,
                         int32_t B, int32_t W, int32_t D, int32_t Hq, int32_t Hkv, int32_t d,
                         int32_t V, ssd_dtype_t dtype, float scale, void* attn_out,
                         int32_t* argmax_out, float* logits_out, GetWs get_ws, hipEvent_t lm_begin,
                         hipEvent_t lm_end, hipStream_t stream, const ssd::AcceptArgs* acc = nullptr) {
  if (!q || !k_pre || !v_pre || !cu_len || !k_cand || !v_cand || !cand_len || !copy_gate ||
      !lm_head || !attn_out || !argmax_out)
    return SSD_ERR_INVALID_ARG;
  if (!(std::isfinite(scale) && scale > 0.f)) return SSD_ERR_INVALID_ARG;
  if (!verify_aligned(q, k_pre, v_pre, k_cand, v_cand, lm_head, attn_out)) return SSD_ERR_INVALID_ARG;
  const ssd_status_t st = check_verify_shape(B, max_n, W, D, Hq, Hkv, d, V, dtype);
  if (st != SSD_OK) return st;
  const bool bf16 = dtype != SSD_F32, rows_layout = dtype == SSD_BF16_ROWS;
  const VerifyLayout L = verify_layout(B, max_n, W, D, Hq, Hkv, d, V, bf16);
  ssd_status_t ws_err = SSD_OK;
  void* workspace = get_ws(L.attn_bytes + L.lm_bytes, &ws_err);
  if (!workspace) return ws_err;
  float* ws_attn = static_cast<float*>(workspace);
  void* ws_lm = static_cast<char*>(workspace) + L.attn_bytes;
  const int R = 1 + W * D;
  // the row compaction runs as one more workgroup of the attention launch
  const ssd::LmWsView cv = ssd::lm_ws_view(ws_lm, B * R);
  hipError_t e = ssd::launch_attention(q, k_pre, v_pre, cu_len, k_cand, v_cand, cand_len, copy_gate,
                                       B, W, D, Hq, Hkv, d, bf16, scale, L.attn, attn_out, ws_attn,
                                       stream, &cv);
  if (e != hipSuccess) return SSD_ERR_HIP;
  e = ssd::launch_lmhead(attn_out, lm_head, B * R, Hq * d, V, bf16, L.lm, logits_out, ws_lm,
                         lm_begin, lm_end, stream, nullptr, rows_layout);
  if (e != hipSuccess) return SSD_ERR_HIP;
  // one launch turns the LM head's per-row keys into argmax_out and accepts
  return from_hip(ssd::launch_argmax_finish(ws_lm, B, R, argmax_out, acc, stream));
}

// The no-allocation variant's scratch: one array per GPU (each device that loads
// the library holds its own copy until the process ends).  In host code the name
// `scratch` is only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
__device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (null and *err set on failure).
void* scratch_of_current_device(ssd_status_t* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    *err = SSD_ERR_HIP;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = SSD_ERR_UNSUPPORTED;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      *err = SSD_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

ssd_status_t ssd_blocktri_verify(const void* q, const void* k_pre, const void* v_pre,
                                 const int32_t* cu_len, int32_t max_n, const void* k_cand,
                                 const void* v_cand, const int32_t* cand_len,
                                 const uint8_t* copy_gate, const void* lm_head, int32_t B,
                                 int32_t W, int32_t D, int32_t Hq, int32_t Hkv, int32_t d,
                                 int32_t V, ssd_dtype_t dtype, float scale, void* attn_out,
                                 int32_t* argmax_out, float* logits_out, void* workspace,
                                 size_t workspace_bytes, hipEvent_t lm_begin, hipEvent_t lm_end,
                                 hipStream_t stream) {
  auto get_ws = [&](size_t need, ssd_status_t* err) -> void* {
    if (!workspace || workspace_bytes < need) {
      *err = SSD_ERR_WORKSPACE;
      return nullptr;
    }
    return workspace;
  };
  return verify_impl(q, k_pre, v_pre, cu_len, max_n, k_cand, v_cand, cand_len, copy_gate, lm_head,
                     B, W, D, Hq, Hkv, d, V, dtype, scale, attn_out, argmax_out, logits_out, get_ws,
                     lm_begin, lm_end, stream);
}

ssd_status_t ssd_blocktri_verify_noalloc(const void* q, const void* k_pre, const void* v_pre,
                                         const int32_t* cu_len, int32_t max_n, const void* k_cand,
                                         const void* v_cand, const int32_t* cand_len,
                                         const uint8_t* copy_gate, const void* lm_head, int32_t B,
                                         int32_t W, int32_t D, int32_t Hq, int32_t Hkv, int32_t d,
                                         int32_t V, ssd_dtype_t dtype, float scale, void* attn_out,
                                         int32_t* argmax_out, float* logits_out, hipStream_t stream) {
  auto get_ws = [&](size_t need, ssd_status_t* err) -> void* {
    if (need > SSD_NOALLOC_SCRATCH_BYTES) {
      *err = SSD_ERR_WORKSPACE;
      return nullptr;
    }
    return scratch_of_current_device(err);
  };
  return verify_impl(q, k_pre, v_pre, cu_len, max_n, k_cand, v_cand, cand_len, copy_gate, lm_head,
                     B, W, D, Hq, Hkv, d, V, dtype, scale, attn_out, argmax_out, logits_out, get_ws,
                     nullptr, nullptr, stream);
}

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
                                        hipEvent_t lm_end, hipStream_t stream) {
  if (!cand || !accept_len || !best_w || !best_len || !next_token) return SSD_ERR_INVALID_ARG;
  auto get_ws = [&](size_t need, ssd_status_t* err) -> void* {
    if (!workspace || workspace_bytes < need) {
      *err = SSD_ERR_WORKSPACE;
      return nullptr;
    }
    return workspace;
  };
  ssd::AcceptArgs acc;
  acc.cand = cand;
  acc.cand_len = cand_len;
  acc.copy_gate = copy_gate;
  acc.W = W;
  acc.D = D;
  acc.accept_len = accept_len;
  acc.best_w = best_w;
  acc.best_len = best_len;
  acc.next_token = next_token;
  return verify_impl(q, k_pre, v_pre, cu_len, max_n, k_cand, v_cand, cand_len, copy_gate, lm_head,
                     B, W, D, Hq, Hkv, d, V, dtype, scale, attn_out, argmax_out, nullptr, get_ws,
                     lm_begin, lm_end, stream, &acc);
}

ssd_status_t ssd_blocktri_verify_sample(
    const void* q, const void* k_pre, const void* v_pre, const int32_t* cu_len, int32_t max_n,
    const void* k_cand, const void* v_cand, const int32_t* cand, const int32_t* cand_len,
    const uint8_t* copy_gate, const void* lm_head, int32_t B, int32_t W, int32_t D, int32_t Hq,
    int32_t Hkv, int32_t d, int32_t V, ssd_dtype_t dtype, float scale, float temperature,
    uint64_t seed, void* attn_out, int32_t* n_children, int32_t* children, int32_t* child_w,
    float* child_logit, float* lse, int32_t* resample, void* workspace, size_t workspace_bytes,
    hipEvent_t lm_begin, hipEvent_t lm_end, hipStream_t stream) {
  if (!q || !k_pre || !v_pre || !cu_len || !k_cand || !v_cand || !cand || !cand_len ||
      !copy_gate || !lm_head || !attn_out || !n_children || !children || !child_w ||
      !child_logit || !lse || !resample)
    return SSD_ERR_INVALID_ARG;
  if (!(std::isfinite(scale) && scale > 0.f)) return SSD_ERR_INVALID_ARG;
  if (!(std::isfinite(temperature) && temperature > 0.f)) return SSD_ERR_INVALID_ARG;
  if (!verify_aligned(q, k_pre, v_pre, k_cand, v_cand, lm_head, attn_out)) return SSD_ERR_INVALID_ARG;
  const ssd_status_t st = check_verify_shape(B, max_n, W, D, Hq, Hkv, d, V, dtype);
  if (st != SSD_OK) return st;
  if (dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
  const float inv_t = 1.0f / temperature;
  if (!std::isfinite(inv_t)) return SSD_ERR_INVALID_ARG;
  const VerifyLayout L = verify_layout(B, max_n, W, D, Hq, Hkv, d, V, true);
  if (!workspace || workspace_bytes < L.attn_bytes + L.lm_bytes) return SSD_ERR_WORKSPACE;
  float* ws_attn = static_cast<float*>(workspace);
  void* ws_lm = static_cast<char*>(workspace) + L.attn_bytes;
  const int R = 1 + W * D;
  const ssd::LmWsView cv = ssd::lm_ws_view(ws_lm, B * R);  // compaction beside the attention
  hipError_t e = ssd::launch_attention(q, k_pre, v_pre, cu_len, k_cand, v_cand, cand_len, copy_gate,
                                       B, W, D, Hq, Hkv, d, true, scale, L.attn, attn_out, ws_attn,
                                       stream, &cv);
  if (e != hipSuccess) return SSD_ERR_HIP;
  e = ssd::launch_trie(cand, cand_len, copy_gate, B, W, D, n_children, children, child_w,
                       child_logit, stream);
  if (e != hipSuccess) return SSD_ERR_HIP;
  ssd::SampleArgs sa;
  sa.inv_t = inv_t;
  sa.k0 = static_cast<uint32_t>(seed & 0xffffffffu);
  sa.k1 = static_cast<uint32_t>(seed >> 32);
  sa.W = W;
  sa.n_children = n_children;
  sa.children = children;
  sa.child_logit = child_logit;
  e = ssd::launch_lmhead(attn_out, lm_head, B * R, Hq * d, V, true, L.lm, nullptr, ws_lm, lm_begin,
                         lm_end, stream, &sa);
  if (e != hipSuccess) return SSD_ERR_HIP;
  return from_hip(ssd::launch_sample_reduce(ws_lm, L.lm, B * R, lse, resample, stream));
}

ssd_status_t ssd_accept_sample(const int32_t* n_children, const int32_t* child_w,
                               const float* child_logit, const float* lse, const int32_t* resample,
                               const uint8_t* copy_gate, int32_t B, int32_t W, int32_t D,
                               uint64_t seed, int32_t* best_w, int32_t* best_len,
                               int32_t* next_token, hipStream_t stream) {
  if (!n_children || !child_w || !child_logit || !lse || !resample || !copy_gate || !best_w ||
      !best_len || !next_token)
    return SSD_ERR_INVALID_ARG;
  if (B < 1 || W < 1 || W > SSD_MAX_W || D < 1 || D > SSD_MAX_D) return SSD_ERR_INVALID_ARG;
  return from_hip(ssd::launch_accept_sample(n_children, child_w, child_logit, lse, resample,
                                            copy_gate, B, W, D, seed, best_w, best_len, next_token,
                                            stream));
}

namespace {
ssd_status_t check_forward_shape(int32_t B, int32_t max_n, int32_t W, int32_t D, int32_t Hq,
                                 int32_t Hkv, int32_t d, int32_t inter, int32_t V) {
  if (B < 1 || max_n < 1 || W < 1 || D < 1 || Hq < 1 || Hkv < 1 || d < 1 || inter < 1 || V < 1)
    return SSD_ERR_INVALID_ARG;
  if (W > SSD_MAX_W || D > SSD_MAX_D || Hq % Hkv != 0) return SSD_ERR_INVALID_ARG;
  const long long hid = static_cast<long long>(Hq) * d;
  if (static_cast<long long>(B) * (1 + W * D) * (hid > inter ? hid : inter) > (1ll << 34))
    return SSD_ERR_INVALID_ARG;
  if (d != 128 || hid % 256 != 0 || inter % 256 != 0 || hid > 8192) return SSD_ERR_UNSUPPORTED;
  if (!fits_byte_offsets(B, max_n, 1 + W * D, Hkv, d, hid > inter ? hid : inter))
    return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}
}  // namespace

size_t ssd_verify_forward_workspace_bytes(int32_t B, int32_t max_n, int32_t W, int32_t D,
                                          int32_t Hq, int32_t Hkv, int32_t d, int32_t inter,
                                          int32_t V) {
  if (check_forward_shape(B, max_n, W, D, Hq, Hkv, d, inter, V) != SSD_OK) return 0;
  return ssd::fwd_layout(B, max_n, W, D, Hq, Hkv, d, inter, V).bytes;
}

ssd_status_t ssd_verify_forward(const int32_t* ids, const int32_t* cu_len, int32_t max_n,
                                const int32_t* cand, const int32_t* cand_len,
                                const uint8_t* copy_gate, const void* embed,
                                const ssd_layer_t* layers, int32_t n_layers, const void* final_norm,
                                const void* lm_head, int32_t B, int32_t W, int32_t D, int32_t Hq,
                                int32_t Hkv, int32_t d, int32_t inter, int32_t V, float rope_base,
                                float eps, int32_t* argmax_out, float* x_out, void* workspace,
                                size_t workspace_bytes, hipEvent_t begin, hipEvent_t end,
                                hipStream_t stream) {
  if (!ids || !cu_len || !cand || !cand_len || !copy_gate || !embed || !final_norm || !lm_head ||
      !argmax_out || n_layers < 0 || (n_layers > 0 && !layers))
    return SSD_ERR_INVALID_ARG;
  if (!(std::isfinite(rope_base) && rope_base > 1.f) || !(std::isfinite(eps) && eps > 0.f))
    return SSD_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(x_out) % 16 != 0) return SSD_ERR_INVALID_ARG;  // float4 rows
  for (int l = 0; l < n_layers; ++l) {
    const ssd_layer_t& L = layers[l];
    if (!L.attn_norm || !L.wqkv || !L.wo || !L.mlp_norm || !L.w_gate_up || !L.w_down ||
        !L.k_cache || !L.v_cache)
      return SSD_ERR_INVALID_ARG;
  }
  const ssd_status_t st = check_forward_shape(B, max_n, W, D, Hq, Hkv, d, inter, V);
  if (st != SSD_OK) return st;
  const ssd::FwdLayout L = ssd::fwd_layout(B, max_n, W, D, Hq, Hkv, d, inter, V);
  if (!workspace || workspace_bytes < L.bytes || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return SSD_ERR_WORKSPACE;
  static_assert(sizeof(ssd_layer_t) == sizeof(ssd::FwdLayer), "layer descriptors match");
  return from_hip(ssd::launch_forward(ids, cu_len, cand, cand_len, copy_gate, embed,
                                      reinterpret_cast<const ssd::FwdLayer*>(layers), n_layers,
                                      final_norm, lm_head, B, W, D, Hq, Hkv, d, inter, V, rope_base,
                                      eps, L, workspace, argmax_out, x_out, begin, end, stream));
}

ssd_status_t ssd_accept_longest(const int32_t* cand, const int32_t* cand_len,
                                const uint8_t* copy_gate, const int32_t* argmax, int32_t B,
                                int32_t W, int32_t D, int32_t* accept_len, int32_t* best_w,
                                int32_t* best_len, int32_t* next_token, hipStream_t stream) {
  if (!cand || !cand_len || !copy_gate || !argmax || !accept_len || !best_w || !best_len || !next_token)
    return SSD_ERR_INVALID_ARG;
  if (B < 1 || W < 1 || W > SSD_MAX_W || D < 1 || D > SSD_MAX_D) return SSD_ERR_INVALID_ARG;
  return from_hip(ssd::launch_accept(cand, cand_len, copy_gate, argmax, B, W, D, accept_len, best_w,
                                     best_len, next_token, stream));
}

ssd_status_t ssd_commit_accepted(const void* k_cand, const void* v_cand, const int32_t* cand,
                                 const int32_t* best_w, const int32_t* best_len,
                                 const int32_t* next_token, int32_t B, int32_t W, int32_t D,
                                 int32_t Hkv, int32_t d, ssd_dtype_t dtype, void* k_cache,
                                 void* v_cache, int64_t cache_rows, const int64_t* cache_off,
                                 int32_t* tokens_out, int32_t* n_tokens_out, hipStream_t stream) {
  if (!k_cand || !v_cand || !cand || !best_w || !best_len || !next_token || !k_cache || !v_cache ||
      !cache_off || !tokens_out || !n_tokens_out)
    return SSD_ERR_INVALID_ARG;
  if (B < 1 || W < 1 || W > SSD_MAX_W || D < 1 || D > SSD_MAX_D || Hkv < 1 || d < 1 ||
      cache_rows < 1 || !valid_dtype(dtype))
    return SSD_ERR_INVALID_ARG;
  const long long row_bytes = static_cast<long long>(Hkv) * d * (dtype == SSD_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0 || row_bytes > (1ll << 30)) return SSD_ERR_UNSUPPORTED;
  return from_hip(ssd::launch_commit(k_cand, v_cand, cand, best_w, best_len, next_token, B, W, D,
                                     static_cast<int>(row_bytes), k_cache, v_cache, cache_rows,
                                     reinterpret_cast<const long long*>(cache_off), tokens_out,
                                     n_tokens_out, stream));
}

size_t ssd_copy_labels_workspace_bytes(int64_t total_n) {
  if (total_n < 1 || total_n >= (1ll << 30)) return 0;
  return ssd::labels_workspace_bytes(total_n);
}

ssd_status_t ssd_copy_labels(const int32_t* ids, const int32_t* cu_len, int32_t B,
                             int64_t total_n, int32_t n_train, uint8_t* labels, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!ids || !cu_len || !labels || B < 1 || total_n < 1 || total_n >= (1ll << 30) ||
      n_train < 1 || n_train > SSD_MAX_NTRAIN)
    return SSD_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < ssd::labels_workspace_bytes(total_n)) return SSD_ERR_WORKSPACE;
  return from_hip(ssd::launch_copy_labels(ids, cu_len, B, static_cast<int>(total_n), n_train, labels,
                                          workspace, stream));
}

ssd_status_t ssd_probe_logits(const void* h, ssd_dtype_t h_dtype, const float* w, int32_t L,
                              int64_t N, int32_t hidden, float* z_out, hipStream_t stream) {
  if (!h || !w || !z_out || L < 1 || L > SSD_MAX_CALIB_L || N < 1 || N >= (1ll << 36) ||
      hidden < 1 || !valid_dtype(h_dtype))
    return SSD_ERR_INVALID_ARG;
  if (hidden > SSD_MAX_PROBE_HIDDEN) return SSD_ERR_UNSUPPORTED;
  return from_hip(ssd::launch_probe_logits(h, h_dtype == SSD_BF16, w, L, N, hidden, z_out, stream));
}

size_t ssd_calibrate_workspace_bytes(int32_t L, int64_t N) {
  if (L < 1 || L > SSD_MAX_CALIB_L || N < 1 || N > SSD_MAX_CALIB_N) return 0;
  return ssd::calibrate_workspace_bytes(L, N);
}

ssd_status_t ssd_calibrate(const float* z, const uint8_t* labels, int32_t L, int64_t N,
                           float* thr_out, int32_t* counts_out, int64_t* u2_out, float* auc_out,
                           int32_t* best_layer, float* tau_out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (!z || !labels || !thr_out || !counts_out || !u2_out || !auc_out || !best_layer || !tau_out ||
      L < 1 || L > SSD_MAX_CALIB_L || N < 1 || N > SSD_MAX_CALIB_N)
    return SSD_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < ssd::calibrate_workspace_bytes(L, N)) return SSD_ERR_WORKSPACE;
  return from_hip(ssd::launch_calibrate(z, labels, L, static_cast<int>(N), thr_out, counts_out,
                                        reinterpret_cast<long long*>(u2_out), auc_out, best_layer,
                                        tau_out, workspace, stream));
}

}  // extern "C"
