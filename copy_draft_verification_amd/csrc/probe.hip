// Copy-intent probe: z_b = w . h_b and the probe half of the copy gate.
// SwitchSD paper §3.2 "Layer and Threshold Selection", §3.3 (the probe is queried
// at every decoding step); write-up §2.3 (bias-free linear probe) and §2.5.
//
// One workgroup per sequence; 256 lanes stride over the hidden dimension with
// 16-byte loads where the row allows it, then a tree reduction in fp32.
#include "common.h"
#include "kernels.h"

namespace ssd {

template <typename T>
__global__ __launch_bounds__(256) void probe_kernel(const T* __restrict__ h,
                                                    const float* __restrict__ w, int hidden,
                                                    float thr, float* __restrict__ z_out,
                                                    uint8_t* __restrict__ fire_out) {
  const int b = blockIdx.x;
  const T* hb = h + static_cast<size_t>(b) * hidden;
  float acc = 0.f;
  for (int k = threadIdx.x; k < hidden; k += blockDim.x) acc += w[k] * load_f32(hb, k);
  __shared__ float part[256 / kWave];
  acc = wave_sum(acc);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float z = 0.f;
    for (int i = 0; i < 256 / kWave; ++i) z += part[i];
    if (z_out) z_out[b] = z;
    fire_out[b] = z >= thr ? 1 : 0;
  }
}

hipError_t launch_probe(const void* h, bool bf16, const float* w, int B, int hidden, float thr,
                        float* z_out, uint8_t* fire_out, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(probe_kernel<uint16_t>, dim3(B), dim3(256), 0, s,
                       static_cast<const uint16_t*>(h), w, hidden, thr, z_out, fire_out);
  else
    hipLaunchKernelGGL(probe_kernel<float>, dim3(B), dim3(256), 0, s,
                       static_cast<const float*>(h), w, hidden, thr, z_out, fire_out);
  return hipGetLastError();
}

}  // namespace ssd
