// Causal depthwise conv1d (+ optional SiLU) along L, the branch of the Mamba
// block in front of the selective scan (dileepadev "Mamba Architecture", SSM
// block internals; vanos001 "The Mamba Block" and its model card's d_conv = 4):
//
//   out[b,d,t] = act( sum_{k<K} w[d,k] * x[b,d,t-K+1+k] + bias[d] ),  x = 0 before t = 0
//
// A standalone streaming kernel (the scan can also apply it to its input on the
// fly; see scan_chunked.hip).  HBM-bound: each thread reads 8 consecutive tokens
// of one channel as one vector and the 3 before them (cache hits: the previous
// thread's vector), and writes 8 outputs.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssm {
namespace {

constexpr int kTok = 8;   // tokens per thread

template <typename ACT, bool VEC>
__global__ __launch_bounds__(256) void causal_conv1d_kernel(const void* __restrict__ x, const float* __restrict__ w,
                                                            const float* __restrict__ bias, void* __restrict__ out,
                                                            int64_t rows, int64_t L, int D, int K, int act) {
  const int64_t groups = (L + kTok - 1) / kTok;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= rows * groups) return;
  const int64_t row = g / groups;
  const int64_t t0 = (g - row * groups) * kTok;
  const int d = static_cast<int>(row % D);
  const int64_t base = row * L;
  // taps aligned to the window x[t-3 .. t]: w4[4-K+k] = w[d,k], the rest zero
  float w4[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w4[k] = (k >= 4 - K) ? w[d * K + k - (4 - K)] : 0.0f;
  const float b = bias ? bias[d] : 0.0f;
  float xx[kTok + 3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int64_t t = t0 - 3 + k;
    xx[k] = t >= 0 ? load_act<ACT>(x, base + t) : 0.0f;
  }
  if (VEC) {
    float v[kTok];
    load_act8<ACT>(x, base + t0, v);
#pragma unroll
    for (int j = 0; j < kTok; ++j) xx[3 + j] = v[j];
  } else {
#pragma unroll
    for (int j = 0; j < kTok; ++j) xx[3 + j] = t0 + j < L ? load_act<ACT>(x, base + t0 + j) : 0.0f;
  }
  float o[kTok];
#pragma unroll
  for (int j = 0; j < kTok; ++j) {
    float s = b;
#pragma unroll
    for (int k = 0; k < 4; ++k) s = __builtin_fmaf(w4[k], xx[j + k], s);
    o[j] = act ? s * __builtin_amdgcn_rcpf(1.0f + exp2_hw(-s * kLog2e)) : s;
  }
  if (VEC) {
    store_act8<ACT>(out, base + t0, o);
  } else {
#pragma unroll
    for (int j = 0; j < kTok; ++j)
      if (t0 + j < L) store_act<ACT>(out, base + t0 + j, o[j]);
  }
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

template <typename ACT>
hipError_t launch_typed(const ConvArgs& a, hipStream_t s) {
  const int64_t rows = a.batch * a.D;
  const int64_t threads = rows * ((a.L + kTok - 1) / kTok);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256)), block(256);
  const bool vec = a.L % kTok == 0 && aligned16(a.x) && aligned16(a.out);
  if (vec)
    hipLaunchKernelGGL((causal_conv1d_kernel<ACT, true>), grid, block, 0, s, a.x, a.w, a.bias, a.out, rows, a.L,
                       static_cast<int>(a.D), a.K, a.silu);
  else
    hipLaunchKernelGGL((causal_conv1d_kernel<ACT, false>), grid, block, 0, s, a.x, a.w, a.bias, a.out, rows, a.L,
                       static_cast<int>(a.D), a.K, a.silu);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_causal_conv1d(const ConvArgs& a, Dt dt, hipStream_t s) {
  return dt == Dt::F32 ? launch_typed<ActF32>(a, s) : launch_typed<ActBF16>(a, s);
}

}  // namespace ssm
