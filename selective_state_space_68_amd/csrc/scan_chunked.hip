// Chunked selective scan for gfx950.
//
// The recurrence h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t u_t is a linear
// recurrence, so it can be evaluated as a prefix scan over (decay, input) pairs
// under the associative operator (a1, b1) then (a2, b2) = (a2 a1, a2 b1 + b2)
// (the slide deck's "Parallel scan" section; the lecture notes' §4.1).  The
// kernel is fused end to end, as the pages' hardware-aware scan is: inputs are
// read from HBM once, the (L, D, N) states never leave registers, and only y and
// the final state are written.
//
// Work decomposition (one wave = one (batch b, channel d) pair):
//   * a chunk is 64 * KPL consecutive tokens; lane i owns tokens [i*KPL, (i+1)*KPL)
//     of it, so u / delta / z / y move as coalesced 16-byte vectors along L;
//   * per token, once for all N states: Delta = softplus(delta + bias), Delta*u,
//     the skip term D*u and, at the end, the SiLU(z) gate;
//   * per state n (a runtime loop; A[d, n] is wave-uniform and sits in an SGPR):
//       pass 1  each lane folds its KPL tokens sequentially into a local end state
//               (lane 0 starts from the carry of the previous chunk) and keeps the
//               per-token decay a_j and input b_j in registers;
//               the lane's aggregate decay is one exp2 of A * (sum of its Deltas);
//       scan    a 64-lane inclusive DPP scan of the (aggregate decay, end state)
//               pairs turns each lane's end state into the true state;
//       pass 2  each lane replays its KPL tokens from the true state of the lane
//               before it and accumulates y_t += C_t,n h_t,n;
//     the carry for the next chunk is lane 63's end state;
//   * a workgroup holds W waves = W channels of the same batch row.  B and C are
//     shared by all channels of a row, so each (chunk, block of NB states) tile of
//     B and C is staged once per workgroup in LDS, transposed so that a lane reads
//     its KPL values of one state with 128-bit, conflict-free LDS reads.
// No MFMA: the readout is a per-token dot product over n, not a shared-operand
// contraction.  The kernel is bound by HBM bandwidth and the VALU/transcendental
// rate (one exp per element).
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssm {
namespace {

constexpr int kNB = 4;   // states per staged B/C tile
constexpr int kW = 4;    // waves (channels) per workgroup

template <typename ACT, int KPL>
struct TokenIO;

template <int KPL>
struct TokenIO<ActF32, KPL> {
  static __device__ __forceinline__ void load(const void* base, int64_t off, float (&v)[KPL]) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int q = 0; q < KPL / 4; ++q) {
      const float4 x = p[q];
      v[4 * q + 0] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
  }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float (&v)[KPL]) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
#pragma unroll
    for (int q = 0; q < KPL / 4; ++q)
      p[q] = make_float4(v[4 * q + 0], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
};

template <int KPL>
struct TokenIO<ActBF16, KPL> {
  static __device__ __forceinline__ void load(const void* base, int64_t off, float (&v)[KPL]) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int q = 0; q < KPL / 8; ++q) {
      const uint4 x = p[q];
      v[8 * q + 0] = bf16_lo(x.x); v[8 * q + 1] = bf16_hi(x.x);
      v[8 * q + 2] = bf16_lo(x.y); v[8 * q + 3] = bf16_hi(x.y);
      v[8 * q + 4] = bf16_lo(x.z); v[8 * q + 5] = bf16_hi(x.z);
      v[8 * q + 6] = bf16_lo(x.w); v[8 * q + 7] = bf16_hi(x.w);
    }
  }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float (&v)[KPL]) {
    uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off);
#pragma unroll
    for (int q = 0; q < KPL / 8; ++q) {
      uint4 x;
      x.x = pack_bf16x2(v[8 * q + 0], v[8 * q + 1]);
      x.y = pack_bf16x2(v[8 * q + 2], v[8 * q + 3]);
      x.z = pack_bf16x2(v[8 * q + 4], v[8 * q + 5]);
      x.w = pack_bf16x2(v[8 * q + 6], v[8 * q + 7]);
      p[q] = x;
    }
  }
};

// Loads the lane's KPL tokens starting at token index `t` of the channel whose
// series starts at element `row`; tokens at or past L read as zero.
template <typename ACT, int KPL, bool VEC>
__device__ __forceinline__ void load_lane(const void* base, int64_t row, int64_t t, int64_t L,
                                          float (&v)[KPL]) {
  if (VEC && t + KPL <= L) {
    TokenIO<ACT, KPL>::load(base, row + t, v);
  } else {
#pragma unroll
    for (int j = 0; j < KPL; ++j) v[j] = (t + j < L) ? load_act<ACT>(base, row + t + j) : 0.0f;
  }
}

template <typename ACT, int KPL, bool VEC>
__device__ __forceinline__ void store_lane(void* base, int64_t row, int64_t t, int64_t L,
                                           const float (&v)[KPL]) {
  if (VEC && t + KPL <= L) {
    TokenIO<ACT, KPL>::store(base, row + t, v);
  } else {
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (t + j < L) store_act<ACT>(base, row + t + j, v[j]);
  }
}

// Four consecutive states [n, n+4) of one token row of B or C; past N or L reads 0.
template <typename ACT, bool VEC>
__device__ __forceinline__ float4 load_bc4(const void* base, int64_t rowoff, int n, int N, bool tok_ok) {
  if (!tok_ok) return make_float4(0.f, 0.f, 0.f, 0.f);
  if (VEC && n + 4 <= N) {
    if constexpr (ACT::kBytes == 4) {
      return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + rowoff + n);
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + rowoff + n);
      return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
    }
  }
  float4 r;
  r.x = (n + 0 < N) ? load_act<ACT>(base, rowoff + n + 0) : 0.f;
  r.y = (n + 1 < N) ? load_act<ACT>(base, rowoff + n + 1) : 0.f;
  r.z = (n + 2 < N) ? load_act<ACT>(base, rowoff + n + 2) : 0.f;
  r.w = (n + 3 < N) ? load_act<ACT>(base, rowoff + n + 3) : 0.f;
  return r;
}

// Stage one matrix (B or C) tile: tokens [t0, t0 + 64*KPL), states [n0, n0 + kNB).
// LDS element (state nl, token 64-block lane i, token j within the lane) lives at
//   nl * CH + (j / 4) * 256 + i * 4 + (j % 4)
// so that lane i reads tokens 4q..4q+3 of state nl as one float4 at float4 index
//   nl * CH/4 + q * 64 + i           (64 consecutive float4 per read: conflict-free).
template <typename ACT, int KPL, bool VEC>
__device__ __forceinline__ void stage_tile(float4* __restrict__ dst, const void* src, int64_t b,
                                           int64_t t0, int n0, int64_t L, int N) {
  constexpr int CH = 64 * KPL;
  constexpr int QUADS = 64 * (KPL / 4);            // (lane block, token quad) pairs
  constexpr int THREADS = 64 * kW;
  for (int qd = threadIdx.x; qd < QUADS; qd += THREADS) {
    const int i = qd & 63;
    const int jq = qd >> 6;
    const int64_t tt = t0 + static_cast<int64_t>(i) * KPL + jq * 4;
    float4 r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t t = tt + k;
      r[k] = load_bc4<ACT, VEC>(src, (b * L + (t < L ? t : 0)) * N, n0, N, t < L);
    }
    // transpose 4 tokens x 4 states -> one float4 of 4 tokens per state
    dst[0 * (CH / 4) + jq * 64 + i] = make_float4(r[0].x, r[1].x, r[2].x, r[3].x);
    dst[1 * (CH / 4) + jq * 64 + i] = make_float4(r[0].y, r[1].y, r[2].y, r[3].y);
    dst[2 * (CH / 4) + jq * 64 + i] = make_float4(r[0].z, r[1].z, r[2].z, r[3].z);
    dst[3 * (CH / 4) + jq * 64 + i] = make_float4(r[0].w, r[1].w, r[2].w, r[3].w);
  }
}

template <typename ACT, bool GATE, int KPL, bool VEC>
__global__ __launch_bounds__(64 * kW) void scan_chunked_kernel(ScanArgs p, int n_dblk) {
  constexpr int CH = 64 * KPL;
  static_assert(kNB == 4, "tile transpose assumes 4 states per tile");
  __shared__ float4 sB[kNB * CH / 4];
  __shared__ float4 sC[kNB * CH / 4];

  const int lane = threadIdx.x & 63;
  const int w = uniform_int(threadIdx.x >> 6);
  const int blk = blockIdx.x;
  const int64_t b = blk / n_dblk;
  const int64_t d = static_cast<int64_t>(blk % n_dblk) * kW + w;
  const bool valid = d < p.D;                       // wave-uniform
  const int N = p.N;
  const int64_t L = p.L;
  const int64_t row = (b * p.D + (valid ? d : 0)) * L;
  const float bias = (valid && p.bias) ? p.bias[d] : 0.0f;
  const float dsk = (valid && p.Dskip) ? p.Dskip[d] : 0.0f;

  // carry[n] lives in lane n of this register (N <= 64).
  float carry_v = 0.0f;

  const int64_t nchunks = (L + CH - 1) / CH;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t tl = c * CH + static_cast<int64_t>(lane) * KPL;   // first token of this lane
    float dl[KPL], du[KPL], yv[KPL], zv[KPL];
    float sdl = 0.0f;
    if (valid) {
      float uv[KPL];
      load_lane<ACT, KPL, VEC>(p.u, row, tl, L, uv);
      load_lane<ACT, KPL, VEC>(p.delta, row, tl, L, dl);
      if (GATE) load_lane<ACT, KPL, VEC>(p.z, row, tl, L, zv);
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        float x = dl[j] + bias;
        if (p.softplus) x = softplus_f(x);
        dl[j] = (tl + j < L) ? x : 0.0f;            // padding tokens: identity step
        du[j] = dl[j] * uv[j];
        yv[j] = dsk * uv[j];
        sdl += dl[j];
      }
    }

    for (int n0 = 0; n0 < N; n0 += kNB) {
      __syncthreads();                                // previous tile fully consumed
      stage_tile<ACT, KPL, VEC>(sB, p.Bm, b, c * CH, n0, L, N);
      stage_tile<ACT, KPL, VEC>(sC, p.Cm, b, c * CH, n0, L, N);
      __syncthreads();
      if (!valid) continue;
      const int nn = (N - n0 < kNB) ? (N - n0) : kNB;
      for (int nl = 0; nl < nn; ++nl) {
        const int n = n0 + nl;
        const float a2 = p.A[d * N + n] * kLog2e;     // wave-uniform
        const float carry = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, carry_v), n));
        float av[KPL], bv[KPL];
        float h = (lane == 0) ? carry : 0.0f;
        const float4* bq = sB + nl * (CH / 4) + lane;
#pragma unroll
        for (int q = 0; q < KPL / 4; ++q) {
          const float4 bb = bq[q * 64];
          const float bs[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 4 * q + r;
            av[j] = exp2_hw(dl[j] * a2);
            bv[j] = du[j] * bs[r];
            h = __builtin_fmaf(av[j], h, bv[j]);
          }
        }
        float P = exp2_hw(a2 * sdl);                  // this lane's aggregate decay
        wave_scan_pairs(P, h);                        // h: true state after this lane
        const float hin = wave_shift_up(h, carry);    // true state before this lane
        const float cnew = wave_lane63(h);
        carry_v = (lane == n) ? cnew : carry_v;
        float hh = hin;
        const float4* cq = sC + nl * (CH / 4) + lane;
#pragma unroll
        for (int q = 0; q < KPL / 4; ++q) {
          const float4 cc = cq[q * 64];
          const float cs[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 4 * q + r;
            hh = __builtin_fmaf(av[j], hh, bv[j]);
            yv[j] = __builtin_fmaf(cs[r], hh, yv[j]);
          }
        }
      }
    }

    if (valid) {
      if (GATE) {
#pragma unroll
        for (int j = 0; j < KPL; ++j) yv[j] *= silu_f(zv[j]);
      }
      store_lane<ACT, KPL, VEC>(p.y, row, tl, L, yv);
    }
  }
  if (valid && p.final_state && lane < N) p.final_state[(b * p.D + d) * N + lane] = carry_v;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

template <typename ACT, bool GATE, int KPL>
hipError_t launch_kpl(const ScanArgs& a, hipStream_t s) {
  const int n_dblk = static_cast<int>((a.D + kW - 1) / kW);
  const int64_t blocks = a.batch * n_dblk;
  const bool vec = (a.L % 8 == 0) && (a.N % 4 == 0) && aligned16(a.u) && aligned16(a.delta) &&
                   aligned16(a.y) && aligned16(a.Bm) && aligned16(a.Cm) &&
                   (a.z == nullptr || aligned16(a.z));
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kW);
  if (vec)
    hipLaunchKernelGGL((scan_chunked_kernel<ACT, GATE, KPL, true>), grid, block, 0, s, a, n_dblk);
  else
    hipLaunchKernelGGL((scan_chunked_kernel<ACT, GATE, KPL, false>), grid, block, 0, s, a, n_dblk);
  return hipGetLastError();
}

template <typename ACT, bool GATE>
hipError_t launch_gate(const ScanArgs& a, int kpl, hipStream_t s) {
  if (kpl == 8) return launch_kpl<ACT, GATE, 8>(a, s);
  return launch_kpl<ACT, GATE, 16>(a, s);
}

}  // namespace

bool chunked_supported(const ScanArgs& a, Dt, int tokens_per_lane) {
  if (!(tokens_per_lane == 0 || tokens_per_lane == 8 || tokens_per_lane == 16)) return false;
  if (a.N < 1 || a.N > 64) return false;
  const int64_t n_dblk = (a.D + kW - 1) / kW;
  return a.batch * n_dblk <= 0x7fffffff && n_dblk <= 0x7fffffff;
}

hipError_t launch_scan_chunked(const ScanArgs& a, Dt dt, int tokens_per_lane, hipStream_t s) {
  if (!chunked_supported(a, dt, tokens_per_lane)) return hipErrorInvalidValue;
  const int kpl = tokens_per_lane == 0 ? 16 : tokens_per_lane;
  const bool gate = a.z != nullptr;
  if (dt == Dt::F32)
    return gate ? launch_gate<ActF32, true>(a, kpl, s) : launch_gate<ActF32, false>(a, kpl, s);
  return gate ? launch_gate<ActBF16, true>(a, kpl, s) : launch_gate<ActBF16, false>(a, kpl, s);
}

}  // namespace ssm
