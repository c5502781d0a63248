// Recurrent decode step: one token per sequence, state [S][D][N] float32 read,
// updated and written back (in place allowed).  The O(1)-state generation mode
// of the slide deck's introduction and the lecture notes' §5: per token, one
// D x N state update and a readout, no cache that grows with the context.
//
// The step is HBM-bound (8 bytes of state traffic per element against ~6 flops),
// so the layout is chosen for streaming: N/4 lanes per (s, d) channel, each lane
// owning a float4 of state, so a wave moves 1 KB of contiguous state per access.
// The readout sum over n is a reduction across those N/4 lanes.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssm {
namespace {

template <typename ACT>
__device__ __forceinline__ float4 load_act4(const void* p, int64_t i);  // i multiple of 4
template <>
__device__ __forceinline__ float4 load_act4<ActF32>(const void* p, int64_t i) {
  return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
}
template <>
__device__ __forceinline__ float4 load_act4<ActBF16>(const void* p, int64_t i) {
  const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
  return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
}

// LPC = N / 4 lanes per channel (1, 2, 4, 8 or 16).
template <typename ACT, bool GATE, int LPC>
__global__ __launch_bounds__(256) void state_update_vec_kernel(StepArgs p) {
  constexpr int N = 4 * LPC;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t ch = g / LPC;
  const int q = static_cast<int>(g % LPC);
  const int64_t nch = p.batch * p.D;
  const bool valid = ch < nch;
  const int64_t chc = valid ? ch : 0;    // lanes past the end compute on channel 0, store nothing
  const int64_t s = chc / p.D;
  const int64_t d = chc - s * p.D;

  const float4 h0 = *reinterpret_cast<const float4*>(p.state_in + chc * N + 4 * q);
  const float4 a4 = *reinterpret_cast<const float4*>(p.A + d * N + 4 * q);
  const float4 b4 = load_act4<ACT>(p.Bm, s * N + 4 * q);
  const float4 c4 = load_act4<ACT>(p.Cm, s * N + 4 * q);
  const float u = load_act<ACT>(p.u, chc);
  float dl = load_act<ACT>(p.delta, chc) + (p.bias ? p.bias[d] : 0.0f);
  if (p.softplus) dl = softplus_f(dl);
  const float du = dl * u;

  float4 h;
  h.x = __builtin_fmaf(exp2_hw(dl * (a4.x * kLog2e)), h0.x, du * b4.x);
  h.y = __builtin_fmaf(exp2_hw(dl * (a4.y * kLog2e)), h0.y, du * b4.y);
  h.z = __builtin_fmaf(exp2_hw(dl * (a4.z * kLog2e)), h0.z, du * b4.z);
  h.w = __builtin_fmaf(exp2_hw(dl * (a4.w * kLog2e)), h0.w, du * b4.w);
  float y = c4.x * h.x;
  y = __builtin_fmaf(c4.y, h.y, y);
  y = __builtin_fmaf(c4.z, h.z, y);
  y = __builtin_fmaf(c4.w, h.w, y);
#pragma unroll
  for (int off = LPC / 2; off > 0; off >>= 1) y += __shfl_xor(y, off, LPC);

  if (valid) {
    *reinterpret_cast<float4*>(p.state_out + ch * N + 4 * q) = h;
    if (q == 0) {
      y = __builtin_fmaf(p.Dskip ? p.Dskip[d] : 0.0f, u, y);
      if (GATE) y *= silu_f(load_act<ACT>(p.z, ch));
      store_act<ACT>(p.y, ch, y);
    }
  }
}

// Any N: one thread per channel, loop over the state.
template <typename ACT, bool GATE>
__global__ __launch_bounds__(256) void state_update_generic_kernel(StepArgs p) {
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (ch >= p.batch * p.D) return;
  const int64_t s = ch / p.D;
  const int64_t d = ch - s * p.D;
  const int N = p.N;
  const float u = load_act<ACT>(p.u, ch);
  float dl = load_act<ACT>(p.delta, ch) + (p.bias ? p.bias[d] : 0.0f);
  if (p.softplus) dl = softplus_f(dl);
  const float du = dl * u;
  float y = 0.0f;
  for (int n = 0; n < N; ++n) {
    const float a = exp2_hw(dl * (p.A[d * N + n] * kLog2e));
    const float h = __builtin_fmaf(a, p.state_in[ch * N + n], du * load_act<ACT>(p.Bm, s * N + n));
    p.state_out[ch * N + n] = h;
    y = __builtin_fmaf(load_act<ACT>(p.Cm, s * N + n), h, y);
  }
  y = __builtin_fmaf(p.Dskip ? p.Dskip[d] : 0.0f, u, y);
  if (GATE) y *= silu_f(load_act<ACT>(p.z, ch));
  store_act<ACT>(p.y, ch, y);
}

bool aligned(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <typename ACT, bool GATE>
hipError_t launch_typed(const StepArgs& a, hipStream_t s) {
  const int64_t nch = a.batch * a.D;
  const int N = a.N;
  const unsigned bc_align = ACT::kBytes * 4;
  const bool vec = (N == 4 || N == 8 || N == 16 || N == 32 || N == 64) && aligned(a.state_in, 16) &&
                   aligned(a.state_out, 16) && aligned(a.A, 16) && aligned(a.Bm, bc_align) &&
                   aligned(a.Cm, bc_align);
  if (vec) {
    const int lpc = N / 4;
    const int64_t threads = nch * lpc;
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256)), block(256);
    switch (lpc) {
      case 1: hipLaunchKernelGGL((state_update_vec_kernel<ACT, GATE, 1>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((state_update_vec_kernel<ACT, GATE, 2>), grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL((state_update_vec_kernel<ACT, GATE, 4>), grid, block, 0, s, a); break;
      case 8: hipLaunchKernelGGL((state_update_vec_kernel<ACT, GATE, 8>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((state_update_vec_kernel<ACT, GATE, 16>), grid, block, 0, s, a); break;
    }
  } else {
    const dim3 grid(static_cast<unsigned>((nch + 255) / 256)), block(256);
    hipLaunchKernelGGL((state_update_generic_kernel<ACT, GATE>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_update(const StepArgs& a, Dt dt, hipStream_t s) {
  const bool gate = a.z != nullptr;
  if (dt == Dt::F32)
    return gate ? launch_typed<ActF32, true>(a, s) : launch_typed<ActF32, false>(a, s);
  return gate ? launch_typed<ActBF16, true>(a, s) : launch_typed<ActBF16, false>(a, s);
}

}  // namespace ssm
