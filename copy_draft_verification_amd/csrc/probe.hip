// Copy-intent probe: z_b = w . h_b and the probe half of the copy gate.
// SwitchSD paper §3.2 "Layer and Threshold Selection", §3.3 (the probe is queried
// at every decoding step); write-up §2.3 (bias-free linear probe) and §2.5.
//
// One workgroup per sequence; 256 lanes stride over the hidden dimension in
// chunks of 8, then a tree reduction in fp32.
#include "common.h"
#include "kernels.h"

namespace ssd {

// Each thread accumulates 8 consecutive k per chunk (one 16-byte load of a bf16
// row, two of an fp32 row, two of w); all of a thread's chunks are issued before
// any of them is used, so the step costs one memory latency, not one per chunk.
constexpr int kPrThreads = 256;
constexpr int kPrUnroll = 4;   // chunks in flight per thread (hidden <= 8192 in one pass)

template <typename T>
__global__ __launch_bounds__(kPrThreads) void probe_kernel(const T* __restrict__ h,
                                                           const float* __restrict__ w, int hidden,
                                                           float thr, float* __restrict__ z_out,
                                                           uint8_t* __restrict__ fire_out) {
  const int b = blockIdx.x;
  const T* hb = h + static_cast<size_t>(b) * hidden;
  float acc = 0.f;
  if ((hidden & 7) == 0) {
    const int nch = hidden >> 3;
    for (int c0 = 0; c0 < nch; c0 += kPrThreads * kPrUnroll) {
      Chunk8<T> hv[kPrUnroll];
      Chunk8<float> wv[kPrUnroll];
#pragma unroll
      for (int u = 0; u < kPrUnroll; ++u) {
        const int c = c0 + u * kPrThreads + threadIdx.x;
        if (c < nch) {
          hv[u].load(hb + 8 * c);
          wv[u].load(w + 8 * c);
        }
      }
#pragma unroll
      for (int u = 0; u < kPrUnroll; ++u) {
        const int c = c0 + u * kPrThreads + threadIdx.x;
        if (c < nch)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc += wv[u].at(e) * hv[u].at(e);
      }
    }
  } else {
    for (int k = threadIdx.x; k < hidden; k += kPrThreads) acc += w[k] * load_f32(hb, k);
  }
  __shared__ float part[kPrThreads / kWave];
  acc = wave_sum(acc);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float z = 0.f;
    for (int i = 0; i < kPrThreads / kWave; ++i) z += part[i];
    if (z_out) z_out[b] = z;
    fire_out[b] = z >= thr ? 1 : 0;
  }
}

hipError_t launch_probe(const void* h, bool bf16, const float* w, int B, int hidden, float thr,
                        float* z_out, uint8_t* fire_out, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(probe_kernel<uint16_t>, dim3(B), dim3(kPrThreads), 0, s,
                       static_cast<const uint16_t*>(h), w, hidden, thr, z_out, fire_out);
  else
    hipLaunchKernelGGL(probe_kernel<float>, dim3(B), dim3(kPrThreads), 0, s,
                       static_cast<const float*>(h), w, hidden, thr, z_out, fire_out);
  return hipGetLastError();
}

}  // namespace ssd
