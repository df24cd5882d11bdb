// sv_debug.hip — element-wise access to the device primitives, so that tests
// can hold the kernels' Philox blocks, accept uniforms, Gumbel noise and
// wave-wide reductions against their definitions directly.
#include "../../include/spec_verify.h"
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {
namespace {

__global__ void philox_kernel(const uint32_t* ctr, const uint32_t* key, uint32_t* out, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const Words4 w = philox10(ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3], key[2 * i], key[2 * i + 1]);
  for (int k = 0; k < 4; ++k) out[4 * i + k] = w.w[k];
}

__global__ void noise_kernel(const uint32_t* words, float* gumbel_out, float* uniform_out, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (gumbel_out) gumbel_out[i] = gumbel(words[i]);
  if (uniform_out) uniform_out[i] = uniform_accept(words[i]);
}

// One wave per 64 inputs; every lane writes the wave-wide maximum it holds.
__global__ void wave_max_kernel(const float* in, float* out, int32_t nwaves) {
  const int w = blockIdx.x * (blockDim.x / 64) + (int)(threadIdx.x >> 6);
  if (w >= nwaves) return;  // whole waves exit together
  const int i = w * 64 + (int)(threadIdx.x & 63);
  out[i] = wave_max(in[i]);
}

}  // namespace
}  // namespace sv

extern "C" {

sv_status_t sv_debug_philox(const uint32_t* ctr, const uint32_t* key, uint32_t* out, int32_t n, void* stream) {
  if (!ctr || !key || !out) return SV_ERR_NULL_ARG;
  if (n < 0) return SV_ERR_BAD_SHAPE;
  if (n == 0) return SV_OK;
  hipLaunchKernelGGL(sv::philox_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, ctr, key, out, n);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status_t sv_debug_wave_max(const float* in, float* out, int32_t nwaves, void* stream) {
  if (!in || !out) return SV_ERR_NULL_ARG;
  if (nwaves < 0) return SV_ERR_BAD_SHAPE;
  if (nwaves == 0) return SV_OK;
  hipLaunchKernelGGL(sv::wave_max_kernel, dim3((nwaves + 3) / 4), dim3(256), 0, (hipStream_t)stream, in, out, nwaves);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status_t sv_debug_noise(const uint32_t* words, float* gumbel_out, float* uniform_out, int32_t n, void* stream) {
  if (!words) return SV_ERR_NULL_ARG;
  if (n < 0) return SV_ERR_BAD_SHAPE;
  if (n == 0) return SV_OK;
  hipLaunchKernelGGL(sv::noise_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, words, gumbel_out,
                     uniform_out, n);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"
