// Calibration kernels for the measurement harness (not part of the method): what
// the device actually sustains for the two resources the scan's rooflines use.
//   * a streaming copy (16-byte vectors, grid-stride): achievable HBM read + write
//     bandwidth, and the reference kernel that HBM byte counters are scaled by;
//   * independent chains of fp32 FMAs, or of v_exp_f32, per lane: the VALU and
//     transcendental issue rates on gfx950.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ssm_calib.h"

namespace {

__global__ __launch_bounds__(256) void calib_copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                                         int64_t n4) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride)
    dst[i] = src[i];
}

constexpr int kChains = 8;   // independent dependency chains per lane

// kind 0: x = x * a + b (v_fma_f32); kind 1: x = exp2(x * c) (v_mul_f32 then
// v_exp_f32; the multiply keeps the argument bounded).  The chains' results are
// stored, so nothing is dead code.
template <int KIND>
__global__ __launch_bounds__(256) void calib_alu_kernel(float* __restrict__ out, int iters, float a, float b) {
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = 0.25f + 0.01f * c + 1e-7f * threadIdx.x;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (KIND == 0)
        x[c] = __builtin_fmaf(x[c], a, b);
      else
        x[c] = __builtin_amdgcn_exp2f(x[c] * a);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

ssm_status ssm_calib_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) ||
      (reinterpret_cast<uintptr_t>(dst) & 15u))
    return SSM_ERR_INVALID_ARG;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + bytes && d0 < s0 + bytes) return SSM_ERR_INVALID_ARG;
  if (bytes == 0) return SSM_OK;
  const int64_t n4 = static_cast<int64_t>(bytes / 16);
  const int64_t want = (n4 + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(calib_copy_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const float4*>(src), static_cast<float4*>(dst), n4);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int64_t ssm_calib_alu_ops(int64_t blocks, int iters) {
  return blocks * 256 * static_cast<int64_t>(iters) * kChains;
}

ssm_status ssm_calib_alu(int kind, float* out, int64_t blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || blocks > 0x7fffffff || iters <= 0 || (kind != 0 && kind != 1))
    return SSM_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(calib_alu_kernel<0>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, out, iters,
                       0.999f, 1e-3f);
  else
    hipLaunchKernelGGL(calib_alu_kernel<1>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, out, iters,
                       -0.5f, 0.0f);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"
