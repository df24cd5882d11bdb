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

// A plain streaming read of nvec 16-byte words, folded with XOR so that
// nothing is optimized away; lane 0 of each wave writes its wave's fold to
// out[4 * block + wave]. Workgroup b reads the contiguous range [b per,
// (b + 1) per) (per: a multiple of 2048 words), eight nontemporal loads in
// flight per lane; a contiguous range per workgroup streams faster on MI355X
// than a grid-wide stride. The read-bandwidth yardstick the verify kernels
// are compared with.
__global__ __launch_bounds__(256) void read_stream_kernel(const uint8_t* p, size_t nvec, size_t per, uint32_t* out) {
  const size_t start = (size_t)blockIdx.x * per;
  const size_t end = start < nvec ? (start + per < nvec ? start + per : nvec) : start;
  uint32_t acc = 0u;
  size_t base = start;
  for (; base + 256 * 8 <= end; base += 256 * 8) {
    u32x4 q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = load_vec_stream(p + (base + k * 256 + threadIdx.x) * 16);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= q[k][0] ^ q[k][1] ^ q[k][2] ^ q[k][3];
  }
  for (size_t v = base + threadIdx.x; v < end; v += 256) {
    const u32x4 q = load_vec_stream(p + v * 16);
    acc ^= q[0] ^ q[1] ^ q[2] ^ q[3];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

}  // namespace
}  // namespace sv

extern "C" {

sv_status_t sv_debug_read_stream(const void* src, size_t bytes, uint32_t* out, int32_t nblocks, void* stream) {
  if (!src || !out) return SV_ERR_NULL_ARG;
  if (nblocks < 1 || bytes % 16 != 0) return SV_ERR_BAD_SHAPE;
  if ((uintptr_t)src % 16 != 0) return SV_ERR_BAD_ARG;
  const size_t nvec = bytes / 16, chunk = 256 * 8;
  const size_t per = ((nvec + (size_t)nblocks - 1) / (size_t)nblocks + chunk - 1) / chunk * chunk;
  hipLaunchKernelGGL(sv::read_stream_kernel, dim3((unsigned)nblocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint8_t*)src, nvec, per, out);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

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
