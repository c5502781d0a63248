// Sequential selective scan: one thread per (batch, channel), stepping through
// time with the N-dimensional state in registers.  This is the plain recurrence
// of the interview-prep page's "Selective scan pseudo-code" (decay exp(Delta*A),
// input Delta*B*u, readout C.h after the update) with the skip term and gate.
// It is the reference the chunked kernel is checked against on the GPU, and the
// path for shapes the chunked kernel does not take.  Throughput is limited by the
// small number of channels; the chunked kernel is the fast path.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssm {
namespace {

template <typename ACT, bool GATE, int NB>
__global__ __launch_bounds__(64) void scan_sequential_kernel(ScanArgs p) {
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (ch >= p.batch * p.D) return;
  const int64_t b = ch / p.D;
  const int64_t d = ch - b * p.D;
  const int N = p.N;

  float a2[NB];   // A[d, n] * log2(e), so that exp(Delta*A) = 2^(Delta*a2)
  float h[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    a2[n] = (n < N) ? p.A[d * N + n] * kLog2e : 0.0f;
    h[n] = (n < N && p.h0) ? p.h0[ch * N + n] : 0.0f;
  }
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float dsk = p.Dskip ? p.Dskip[d] : 0.0f;
  const int64_t row = ch * p.L;                // u / delta / z / y offset of this channel
  const int64_t bc_row = b * p.L * N;          // B / C offset of this batch row ([L][N] within it)
  // saved chunk states: entry c is the state entering 512-token chunk c
  const int64_t nck = (p.L + kSaveChunk - 1) / kSaveChunk;
  float* cst = p.chunk_states ? p.chunk_states + ch * nck * N : nullptr;
  if (cst) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
      if (n < N) cst[n] = h[n];
  }

  for (int64_t t = 0; t < p.L; ++t) {
    const float u = load_act<ACT>(p.u, row + t);
    float dl = load_act<ACT>(p.delta, row + t) + bias;
    if (p.softplus) dl = softplus_f(dl);
    const float du = dl * u;
    float y = 0.0f;
    const int64_t bo = bc_row + t * N;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      if (n < N) {
        const float a = exp2_hw(dl * a2[n]);
        h[n] = __builtin_fmaf(a, h[n], du * load_act<ACT>(p.Bm, bo + n));
        y = __builtin_fmaf(load_act<ACT>(p.Cm, bo + n), h[n], y);
      }
    }
    y = __builtin_fmaf(dsk, u, y);
    if (GATE) y *= silu_f(load_act<ACT>(p.z, row + t));
    store_act<ACT>(p.y, row + t, y);
    if (cst && (t + 1) % kSaveChunk == 0 && t + 1 < p.L) {
      float* o = cst + ((t + 1) / kSaveChunk) * N;
#pragma unroll
      for (int n = 0; n < NB; ++n)
        if (n < N) o[n] = h[n];
    }
  }
  if (p.final_state) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
      if (n < N) p.final_state[ch * N + n] = h[n];
  }
}

template <typename ACT, bool GATE>
hipError_t launch_nb(const ScanArgs& a, hipStream_t s) {
  const int64_t channels = a.batch * a.D;
  const dim3 grid(static_cast<unsigned>((channels + 63) / 64));
  const dim3 block(64);
  if (a.N <= 4)
    hipLaunchKernelGGL((scan_sequential_kernel<ACT, GATE, 4>), grid, block, 0, s, a);
  else if (a.N <= 8)
    hipLaunchKernelGGL((scan_sequential_kernel<ACT, GATE, 8>), grid, block, 0, s, a);
  else if (a.N <= 16)
    hipLaunchKernelGGL((scan_sequential_kernel<ACT, GATE, 16>), grid, block, 0, s, a);
  else if (a.N <= 32)
    hipLaunchKernelGGL((scan_sequential_kernel<ACT, GATE, 32>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((scan_sequential_kernel<ACT, GATE, 64>), grid, block, 0, s, a);
  return hipGetLastError();
}

__global__ void copy_state_kernel(float* dst, const float* src, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

}  // namespace

hipError_t launch_scan_sequential(const ScanArgs& a, Dt dt, hipStream_t s) {
  const bool gate = a.z != nullptr;
  if (dt == Dt::F32) return gate ? launch_nb<ActF32, true>(a, s) : launch_nb<ActF32, false>(a, s);
  return gate ? launch_nb<ActBF16, true>(a, s) : launch_nb<ActBF16, false>(a, s);
}

hipError_t launch_copy_state(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0 || dst == src) return hipSuccess;
  hipLaunchKernelGGL(copy_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, dst, src,
                     n);
  return hipGetLastError();
}

}  // namespace ssm
