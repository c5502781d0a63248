// Backward pass of the selective scan for gfx950, by recomputation.
//
// The gradient of the state h_t is the reverse-time recurrence
//     lam_t = g_t C_t + abar_{t+1} lam_{t+1},  g_t = dy_t * SiLU(z_t)
// (lam past the last token is the final state's cotangent), the same linear
// recurrence run backwards, so it scans with the same associative operator as the
// forward pass (the slide deck's "Parallel scan" section).  The forward states are
// recomputed from the saved inputs rather than stored, as the pages' hardware-aware
// design does (the slide deck on Mamba's fused kernel; the "Hardware-Aware Parallel
// Scan" sections of the dileepadev and vanos001 pages).  Every parameter gradient is a sum over
// t of lam_t (or g_t) times one step's partial derivative:
//     dC[b,t,n]  = sum_d g_t h_t                  dB[b,t,n] = sum_d lam_t Delta_t u_t
//     du_t       = D g_t + Delta_t sum_n lam_t B_t
//     dDelta_t   = u_t sum_n lam_t B_t + sum_n A_n abar_t lam_t h_{t-1}
//     dA[d,n]    = sum_{b,t} abar_t lam_t h_{t-1} Delta_t
//     dz_t       = dy_t ytilde_t SiLU'(z_t)       (ytilde: the output before the gate)
//     draw_t     = dDelta_t sigmoid(raw_t)        (softplus' = sigmoid)
//     dh0        = abar_0 lam_0
//
// Work decomposition: chunks of CH = 64 * KPL tokens are independent once each
// chunk knows the state entering it and the adjoint entering it from the right,
// so the work is split over (batch row, chunk, channel) with no sequential loop
// over chunks:
//   1. summary: per (b, chunk, d, n), the chunk's forward aggregate F (its end
//      state from a zero start) and reverse aggregate X (the adjoint it sends to
//      the previous chunk from a zero start), and its decay P = exp(A sum Delta);
//   2. combine: per (b, d, n), a sequential pass over the chunks turns F into the
//      state entering each chunk and X into the adjoint entering each chunk;
//   3. main: per (b, chunk, d), recompute the states inside the chunk from its
//      entering state (fold, wave scan, replay), run the adjoint recurrence from
//      its entering adjoint (reverse fold, reverse wave scan, reverse replay) and
//      accumulate every gradient;
//   4. finalize: fixed-order sums of the per-(b, chunk) partials of dA, dD and the
//      delta bias; dB and dC from float32 to the activation dtype.
//
// A workgroup of kBW waves owns one (batch row, chunk) pair and a slice of
// kBW * rounds channels: it stages the chunk's B and C once in LDS (float32,
// permuted so that each lane's tokens are contiguous), and each wave runs one
// channel per round.  dB and dC are sums over channels: the waves add their
// terms into a float32 LDS accumulator with LDS atomics, and the workgroup adds
// the accumulator to a float32 copy in memory with one global atomic per element
// at its end, so the reduction over D happens on chip.  The LDS and global
// atomics make dB and dC the only outputs whose last bits depend on the order of
// the additions; every other output is a fixed-order computation.
#include <utility>

#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_common.hpp"

namespace ssm {
namespace {

constexpr int kBW = 8;                // waves per workgroup (channels per round)

struct BwdLayout {
  int64_t nchunks;                    // chunks of 64 * KPL tokens
  int64_t nslices;                    // channel slices of kBW * rounds
  int rounds;
  int kpl;
  float* F;                           // [batch][nchunks][D][N]: F, then the entering state
  float* X;                           // [batch][nchunks][D][N]: X, then the entering adjoint
  float* P;                           // [batch][nchunks][D][N]: chunk decay, then dA partials
  float* dBC;                         // [batch][2][N][L] float32 dB (0) and dC (1)
  float* dDp;                         // [batch][nchunks][D] dD partials
  float* dbp;                         // [batch][nchunks][D] delta-bias partials
};

// KPL tokens per lane for a state count: the main kernel holds a chunk's B and C
// and the dB/dC accumulator for all N states in LDS, 2 * N * 64 * KPL floats each.
int bwd_kpl(int N) { return N <= 16 ? 8 : 4; }
// States a main-kernel instantiation holds in LDS (LDSACC) or in the tile alone.
template <int KPL, bool LDSACC>
struct BwdCap {
  static constexpr int CH = 64 * KPL;
  static constexpr int NMAX = (LDSACC ? 16384 : 32768) / (2 * CH);
};

int64_t align64(int64_t n) { return (n + 63) / 64 * 64; }

BwdLayout bwd_layout(int64_t batch, int64_t L, int64_t D, int N, float* ws) {
  BwdLayout g{};
  g.kpl = bwd_kpl(N);
  const int64_t CH = 64 * g.kpl;
  g.nchunks = (L + CH - 1) / CH;
  const int64_t tasks = batch * g.nchunks * D;
  // About 512 workgroups (two per CU) where the shape allows, at most 16 rounds.
  int64_t r = (tasks + kBW * 512 - 1) / (kBW * 512);
  const int64_t rmax = (D + kBW - 1) / kBW;
  r = r < 1 ? 1 : (r > 16 ? 16 : r);
  r = r > rmax ? rmax : r;
  g.rounds = static_cast<int>(r);
  g.nslices = (D + kBW * r - 1) / (kBW * r);
  const int64_t st = align64(batch * g.nchunks * D * N);
  const int64_t bc = align64(batch * 2 * N * L);
  const int64_t pp = align64(batch * g.nchunks * D);
  if (ws) {
    g.F = ws;
    g.X = g.F + st;
    g.P = g.X + st;
    g.dBC = g.P + st;
    g.dDp = g.dBC + bc;
    g.dbp = g.dDp + pp;
  }
  return g;
}

size_t bwd_ws_floats(int64_t batch, int64_t L, int64_t D, int N) {
  const BwdLayout g = bwd_layout(batch, L, D, N, nullptr);
  return static_cast<size_t>(3 * align64(batch * g.nchunks * D * N) + align64(batch * 2 * N * L) +
                             2 * align64(batch * g.nchunks * D));
}

// ---- cross-lane helpers -------------------------------------------------------

// Reverse (suffix) scan across the 64 lanes of (a, b) pairs: on return lane i's b
// is mu_i = b_i + a_i mu_{i+1} with mu_64 = carry, i.e. the composition of lanes
// 63 .. i applied to the carry.  Within each row of 16 lanes, Kogge-Stone steps
// with row_shl 1, 2, 4, 8 (in-place DPP as in the forward scan; a lane whose
// source is past its row's end is not written, which is combining with the
// identity).  Then the three row boundaries are resolved from lanes 48, 32, 16
// read as scalars: row r's lanes apply their row suffix to mu of the first lane
// of row r + 1.  Pure VALU, no memory access.
__device__ __forceinline__ void wave_rscan_pairs(float& a, float& b, float carry) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(b), "+v"(a));
  auto rl = [](float v, int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); };
  const float m2 = __builtin_fmaf(rl(a, 48), carry, rl(b, 48));
  const float m1 = __builtin_fmaf(rl(a, 32), m2, rl(b, 32));
  const float m0 = __builtin_fmaf(rl(a, 16), m1, rl(b, 16));
  const int row = (threadIdx.x & 63) >> 4;
  const float m = row == 3 ? carry : (row == 2 ? m2 : (row == 1 ? m1 : m0));
  b = __builtin_fmaf(a, m, b);
}

// Value of lane i+1 in lane i; lane 63 receives `last`.
__device__ __forceinline__ float wave_shift_down(float v, float last) {
  return dpp_mov<0x130, 0xf, false>(last, v);
}

// Sum over the 64 lanes (wave-uniform result): row reductions with row_shr
// (bound_ctrl zero fills), then the row broadcasts 15 and 31 into lane 63.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0x111, 0xf, true>(0.0f, v);
  v += dpp_mov<0x112, 0xf, true>(0.0f, v);
  v += dpp_mov<0x114, 0xf, true>(0.0f, v);
  v += dpp_mov<0x118, 0xf, true>(0.0f, v);
  v += dpp_mov<0x142, 0xa, false>(0.0f, v);
  v += dpp_mov<0x143, 0xc, false>(0.0f, v);
  return wave_lane63(v);
}

__device__ __forceinline__ float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// ---- memory helpers -------------------------------------------------------------

// Four consecutive activations from element offset i (vector: 16- or 8-byte
// aligned load).
template <typename ACT>
__device__ __forceinline__ void load4(const void* p, int64_t i, float (&x)[4]);
template <>
__device__ __forceinline__ void load4<ActF32>(const void* p, int64_t i, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <>
__device__ __forceinline__ void load4<ActBF16>(const void* p, int64_t i, float (&x)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
}

// KPL consecutive tokens of one channel starting at token t of the row at element
// offset `row`; tokens at or past L read as 0.
template <typename ACT, int KPL>
__device__ __forceinline__ void load_tokens(const void* src, int64_t row, int64_t t, int64_t L, bool vec,
                                            float (&v)[KPL]) {
  if constexpr (KPL == 8) {
    if (vec && t + KPL <= L) {
      using IO = TokenIO<ACT, KPL>;
      typename IO::raw_t r[IO::kVec];
      IO::load_raw(src, row + t, r);
      IO::unpack(r, v);
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < KPL; ++j) v[j] = t + j < L ? load_act<ACT>(src, row + t + j) : 0.0f;
}

template <typename ACT, int KPL>
__device__ __forceinline__ void store_tokens(void* dst, int64_t row, int64_t t, int64_t L, bool vec,
                                             const float (&v)[KPL]) {
  if constexpr (KPL == 8) {
    if (vec && t + KPL <= L) {
      TokenIO<ACT, KPL>::store(dst, row + t, v);
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < KPL; ++j)
    if (t + j < L) store_act<ACT>(dst, row + t + j, v[j]);
}

// Stages chunk [t0, t0 + CH) of B (states 0..N-1) then C into LDS as float32:
// float4 f of block m*N + n (tokens 4f .. 4f+3 of the chunk) goes to slot
// (f % (KPL/4)) * 64 + f / (KPL/4), so lane i finds its KPL tokens as KPL/4
// float4 at q * 64 + i.  Tokens past L are zero.
template <typename ACT, int KPL>
__device__ __forceinline__ void load_tile(float4* tile, const BwdArgs& p, int64_t b, int64_t t0, bool vec) {
  constexpr int CH = 64 * KPL, F4 = CH / 4, Q = KPL / 4;
  const int N = p.N;
  const int64_t L = p.L;
  const int total = 2 * N * F4;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int mn = e / F4, f = e % F4;
    const int m = mn / N, n = mn % N;
    const void* src = m ? p.Cm : p.Bm;
    const int64_t off = (b * N + n) * L;
    const int64_t t = t0 + 4 * f;
    float x[4];
    if (vec && t + 4 <= L) {
      load4<ACT>(src, off + t, x);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = t + r < L ? load_act<ACT>(src, off + t + r) : 0.0f;
    }
    tile[mn * F4 + (f % Q) * 64 + f / Q] = make_float4(x[0], x[1], x[2], x[3]);
  }
}

// Per-token values of one channel's chunk shared by the summary and main kernels:
// Delta (zero on tokens past L, which makes them identity steps), Delta*u and the
// gate-scaled output gradient g (zero past L).
template <typename ACT, int KPL>
struct TokenState {
  float u[KPL], dl[KPL], du[KPL], g[KPL];
  float sdl;

  // Returns the raw delta + bias in `raw` (for the softplus derivative) and, with
  // a gate, the factor dy * SiLU'(z) in `dzf`.
  template <bool FULL>
  __device__ __forceinline__ void load(const BwdArgs& p, int64_t row, int64_t t, bool vec, float bias,
                                       float (&sg)[KPL], float (&dzf)[KPL]) {
    const int64_t L = p.L;
    float dy[KPL];
    load_tokens<ACT, KPL>(p.u, row, t, L, vec, u);
    load_tokens<ACT, KPL>(p.delta, row, t, L, vec, dl);
    load_tokens<ACT, KPL>(p.dy, row, t, L, vec, dy);
    if (p.z) {
      float z[KPL];
      load_tokens<ACT, KPL>(p.z, row, t, L, vec, z);
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const float s = __builtin_amdgcn_rcpf(1.0f + exp2_hw(-z[j] * kLog2e));
        g[j] = dy[j] * z[j] * s;
        if constexpr (FULL) dzf[j] = dy[j] * s * __builtin_fmaf(z[j], 1.0f - s, 1.0f);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPL; ++j) g[j] = dy[j];
    }
    sdl = 0.0f;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const float raw = dl[j] + bias;
      float d = raw;
      if (p.softplus) {
        d = softplus_f(raw);
        if constexpr (FULL) sg[j] = __builtin_amdgcn_rcpf(1.0f + exp2_hw(-raw * kLog2e));
      }
      d = t + j < L ? d : 0.0f;
      dl[j] = d;
      du[j] = d * u[j];
      sdl += d;
    }
  }
};

// ---- 1. chunk summaries -----------------------------------------------------------
template <typename ACT, int KPL>
__global__ __launch_bounds__(64 * kBW) void bwd_summary_kernel(BwdArgs p, BwdLayout g, int vec_flag) {
  constexpr int CH = 64 * KPL, F4 = CH / 4, Q = KPL / 4;
  constexpr int NMAX = KPL == 8 ? 16 : 64;
  __shared__ float4 s_tile[2 * NMAX * F4];
  const bool vec = vec_flag != 0;
  const int lane = threadIdx.x & 63;
  const int w = uniform_int(threadIdx.x >> 6);
  const int64_t nbc = p.batch * g.nchunks;
  // Workgroups of one (batch row, chunk) pair are nbc apart, so they share an XCD
  // (and its L2) whenever nbc is a multiple of the 8 XCDs.
  const int64_t bc = blockIdx.x % nbc, slice = blockIdx.x / nbc;
  const int64_t b = bc % p.batch, c = bc / p.batch;
  const int N = p.N;
  const int64_t L = p.L, D = p.D;
  const int64_t t0 = c * CH;
  load_tile<ACT, KPL>(s_tile, p, b, t0, vec);
  if (slice == 0) {
    // this chunk's part of the float32 dB/dC sums starts at zero
    for (int e = threadIdx.x; e < 2 * N * CH; e += blockDim.x) {
      const int64_t t = t0 + e % CH;
      if (t < L) g.dBC[(b * 2 * N + e / CH) * L + t] = 0.0f;
    }
  }
  __syncthreads();

  const int64_t tl = t0 + static_cast<int64_t>(lane) * KPL;
  const int64_t dg = static_cast<int64_t>(kBW) * g.rounds;
  for (int r = 0; r < g.rounds; ++r) {
    const int64_t d = slice * dg + r * kBW + w;
    if (d >= D) break;
    const int64_t row = (b * D + d) * L;
    TokenState<ACT, KPL> ts;
    float unused0[KPL], unused1[KPL];
    ts.template load<false>(p, row, tl, vec, p.bias ? p.bias[d] : 0.0f, unused0, unused1);
    const float stot = wave_sum(ts.sdl);
    const float a2_v = lane < N ? p.A[d * N + lane] * kLog2e : 0.0f;
    float Fv = 0.0f, Xv = 0.0f;
    for (int n = 0; n < N; ++n) {
      const float a2 = lane_value(a2_v, n);
      const float4* sB = s_tile + n * F4;
      const float4* sC = s_tile + (N + n) * F4;
      float av[KPL], cv[KPL];
      float h = 0.0f;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float4 bb = sB[q * 64 + lane], cc = sC[q * 64 + lane];
        const float bs[4] = {bb.x, bb.y, bb.z, bb.w}, cs[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = 4 * q + k;
          av[j] = exp2_hw(ts.dl[j] * a2);
          cv[j] = cs[k];
          h = __builtin_fmaf(av[j], h, ts.du[j] * bs[k]);
        }
      }
      float x = 0.0f;
#pragma unroll
      for (int j = KPL - 1; j >= 0; --j) x = av[j] * __builtin_fmaf(ts.g[j], cv[j], x);
      float P1 = exp2_hw(a2 * ts.sdl);
      float P2 = P1;
      wave_scan_pairs(P1, h);
      wave_rscan_pairs(P2, x, 0.0f);
      const float fn = wave_lane63(h), xn = lane_value(x, 0);
      Fv = lane == n ? fn : Fv;
      Xv = lane == n ? xn : Xv;
    }
    if (lane < N) {
      const int64_t off = ((b * g.nchunks + c) * D + d) * N + lane;
      g.F[off] = Fv;
      g.X[off] = Xv;
      g.P[off] = exp2_hw(a2_v * stot);
    }
  }
}

// ---- 2. sequential combine over chunks --------------------------------------------
__global__ void bwd_combine_kernel(BwdArgs p, BwdLayout g) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int N = p.N;
  const int64_t D = p.D;
  if (i >= p.batch * D * N) return;
  const int64_t n = i % N, d = (i / N) % D, b = i / (N * D);
  const int64_t stride = D * N;
  const int64_t base = b * g.nchunks * stride + d * N + n;
  float h = p.h0 ? p.h0[i] : 0.0f;
  for (int64_t c = 0; c < g.nchunks; ++c) {
    const int64_t o = base + c * stride;
    const float f = g.F[o];
    g.F[o] = h;                                      // state entering chunk c
    h = __builtin_fmaf(g.P[o], h, f);
  }
  float mu = p.dfinal ? p.dfinal[i] : 0.0f;
  for (int64_t c = g.nchunks - 1; c >= 0; --c) {
    const int64_t o = base + c * stride;
    const float x = g.X[o];
    g.X[o] = mu;                                     // adjoint entering chunk c from the right
    mu = __builtin_fmaf(g.P[o], mu, x);
  }
  if (p.dh0) p.dh0[i] = mu;
}

// ---- 3. the gradients -----------------------------------------------------------------
template <typename ACT, int KPL, bool LDSACC>
__global__ __launch_bounds__(64 * kBW) void bwd_main_kernel(BwdArgs p, BwdLayout g, int vec_flag) {
  constexpr int CH = 64 * KPL, F4 = CH / 4, Q = KPL / 4;
  constexpr int NMAX = BwdCap<KPL, LDSACC>::NMAX;
  __shared__ float4 s_tile[2 * NMAX * F4];
  __shared__ float s_acc[LDSACC ? 2 * NMAX * CH : 1];
  const bool vec = vec_flag != 0;
  const int lane = threadIdx.x & 63;
  const bool lane0 = lane == 0;
  const int w = uniform_int(threadIdx.x >> 6);
  const int64_t nbc = p.batch * g.nchunks;
  const int64_t bc = blockIdx.x % nbc, slice = blockIdx.x / nbc;
  const int64_t b = bc % p.batch, c = bc / p.batch;
  const int N = p.N;
  const int64_t L = p.L, D = p.D;
  const int64_t t0 = c * CH;
  load_tile<ACT, KPL>(s_tile, p, b, t0, vec);
  if constexpr (LDSACC) {
    for (int e = threadIdx.x; e < 2 * N * CH; e += blockDim.x) s_acc[e] = 0.0f;
  }
  __syncthreads();

  // dB (m = 0) or dC (m = 1) term of state n, token j of this lane
  auto acc_add = [&](int m, int n, int j, float v) __attribute__((always_inline)) {
    if constexpr (LDSACC) {
      __hip_atomic_fetch_add(&s_acc[((m * N + n) * KPL + j) * 64 + lane], v, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      const int64_t t = t0 + static_cast<int64_t>(lane) * KPL + j;
      if (t < L) unsafeAtomicAdd(&g.dBC[(b * 2 * N + m * N + n) * L + t], v);
    }
  };

  const int64_t tl = t0 + static_cast<int64_t>(lane) * KPL;
  const int64_t dg = static_cast<int64_t>(kBW) * g.rounds;
  for (int r = 0; r < g.rounds; ++r) {
    const int64_t d = slice * dg + r * kBW + w;
    if (d >= D) break;
    const int64_t row = (b * D + d) * L;
    const int64_t soff = ((b * g.nchunks + c) * D + d) * N;
    const float dsk = p.Dskip ? p.Dskip[d] : 0.0f;
    TokenState<ACT, KPL> ts;
    float sg[KPL], dzf[KPL];
    ts.template load<true>(p, row, tl, vec, p.bias ? p.bias[d] : 0.0f, sg, dzf);
    const float A_v = lane < N ? p.A[d * N + lane] : 0.0f;
    const float a2_v = A_v * kLog2e;
    const float hs_v = lane < N ? g.F[soff + lane] : 0.0f;
    const float mu_v = lane < N ? g.X[soff + lane] : 0.0f;
    float s1[KPL], s2[KPL], yt[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      s1[j] = 0.0f;
      s2[j] = 0.0f;
      yt[j] = dsk * ts.u[j];
    }
    float dA_v = 0.0f;
    for (int n = 0; n < N; ++n) {
      const float a2 = lane_value(a2_v, n), An = lane_value(A_v, n);
      const float hst = lane_value(hs_v, n), mue = lane_value(mu_v, n);
      const float4* sB = s_tile + n * F4;
      const float4* sC = s_tile + (N + n) * F4;
      float av[KPL], bv[KPL], hv[KPL], bs[KPL], cs[KPL];
      // forward recomputation: fold, scan, replay (h_j kept per token)
      float h = lane0 ? hst : 0.0f;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float4 bb = sB[q * 64 + lane], cc = sC[q * 64 + lane];
        bs[4 * q + 0] = bb.x; bs[4 * q + 1] = bb.y; bs[4 * q + 2] = bb.z; bs[4 * q + 3] = bb.w;
        cs[4 * q + 0] = cc.x; cs[4 * q + 1] = cc.y; cs[4 * q + 2] = cc.z; cs[4 * q + 3] = cc.w;
      }
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        av[j] = exp2_hw(ts.dl[j] * a2);
        bv[j] = ts.du[j] * bs[j];
        h = __builtin_fmaf(av[j], h, bv[j]);
      }
      float P1 = exp2_hw(a2 * ts.sdl);
      float P2 = P1;
      wave_scan_pairs(P1, h);
      const float hin = wave_shift_up(h, hst);
      float hh = hin;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        hh = __builtin_fmaf(av[j], hh, bv[j]);
        hv[j] = hh;
        yt[j] = __builtin_fmaf(cs[j], hh, yt[j]);
        acc_add(1, n, j, ts.g[j] * hh);
      }
      // adjoint: reverse fold, reverse scan, reverse replay
      float x = 0.0f;
#pragma unroll
      for (int j = KPL - 1; j >= 0; --j) x = av[j] * __builtin_fmaf(ts.g[j], cs[j], x);
      wave_rscan_pairs(P2, x, mue);
      float mu = wave_shift_down(x, mue);            // adjoint entering this lane's last token
      float dal = 0.0f;
#pragma unroll
      for (int j = KPL - 1; j >= 0; --j) {
        const float lam = __builtin_fmaf(ts.g[j], cs[j], mu);
        s1[j] = __builtin_fmaf(lam, bs[j], s1[j]);
        acc_add(0, n, j, lam * ts.du[j]);
        mu = av[j] * lam;
        const float t = mu * (j > 0 ? hv[j - 1] : hin);
        s2[j] = __builtin_fmaf(t, An, s2[j]);
        dal = __builtin_fmaf(t, ts.dl[j], dal);
      }
      const float dan = wave_sum(dal);
      dA_v = lane == n ? dan : dA_v;
    }
    // per-token gradients
    float o_du[KPL], o_dd[KPL];
    float dDl = 0.0f, dbl = 0.0f;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      o_du[j] = __builtin_fmaf(dsk, ts.g[j], ts.dl[j] * s1[j]);
      float dd = __builtin_fmaf(ts.u[j], s1[j], s2[j]);
      if (p.softplus) dd *= sg[j];
      o_dd[j] = dd;
      dDl = __builtin_fmaf(ts.g[j], ts.u[j], dDl);
      dbl += tl + j < L ? dd : 0.0f;
    }
    store_tokens<ACT, KPL>(p.du, row, tl, L, vec, o_du);
    store_tokens<ACT, KPL>(p.ddelta, row, tl, L, vec, o_dd);
    if (p.dz) {
#pragma unroll
      for (int j = 0; j < KPL; ++j) o_du[j] = yt[j] * dzf[j];
      store_tokens<ACT, KPL>(p.dz, row, tl, L, vec, o_du);
    }
    const float dDs = wave_sum(dDl), dbs = wave_sum(dbl);
    if (lane < N) g.P[soff + lane] = dA_v;
    if (lane0) {
      g.dDp[(b * g.nchunks + c) * D + d] = dDs;
      g.dbp[(b * g.nchunks + c) * D + d] = dbs;
    }
  }
  if constexpr (LDSACC) {
    __syncthreads();
    for (int e = threadIdx.x; e < 2 * N * CH; e += blockDim.x) {
      const int mn = e / CH, tt = e % CH;
      const int64_t t = t0 + tt;
      if (t < L) unsafeAtomicAdd(&g.dBC[(b * 2 * N + mn) * L + t], s_acc[(mn * KPL + tt % KPL) * 64 + tt / KPL]);
    }
  }
}

// ---- 4. fixed-order sums and dtype conversion ---------------------------------------
__global__ void bwd_param_sums_kernel(BwdArgs p, BwdLayout g) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t D = p.D, DN = D * p.N, parts = p.batch * g.nchunks;
  if (i < DN) {
    float s = 0.0f;
    for (int64_t k = 0; k < parts; ++k) s += g.P[k * DN + i];
    p.dA[i] = s;
  } else if (i < DN + D) {
    const int64_t d = i - DN;
    float s = 0.0f;
    for (int64_t k = 0; k < parts; ++k) s += g.dDp[k * D + d];
    if (p.dD) p.dD[d] = s;
  } else if (i < DN + 2 * D) {
    const int64_t d = i - DN - D;
    float s = 0.0f;
    for (int64_t k = 0; k < parts; ++k) s += g.dbp[k * D + d];
    if (p.dbias) p.dbias[d] = s;
  }
}

template <typename ACT>
__global__ void bwd_bc_out_kernel(BwdArgs p, BwdLayout g) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t L = p.L, NL = p.N * L;
  if (i >= p.batch * 2 * NL) return;
  const int64_t b = i / (2 * NL), rem = i % (2 * NL);
  const int m = static_cast<int>(rem / NL);
  store_act<ACT>(m ? p.dC : p.dB, b * NL + rem % NL, g.dBC[i]);
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

template <typename ACT, int KPL, bool LDSACC>
hipError_t launch_bwd_typed(const BwdArgs& a, const BwdLayout& g, hipStream_t s) {
  const bool vec = (a.L % 8 == 0) && aligned16(a.u) && aligned16(a.delta) && aligned16(a.dy) &&
                   (a.z == nullptr || aligned16(a.z)) && aligned16(a.du) && aligned16(a.ddelta) &&
                   (a.dz == nullptr || aligned16(a.dz)) && aligned16(a.Bm) && aligned16(a.Cm);
  const int64_t blocks = a.batch * g.nchunks * g.nslices;
  hipLaunchKernelGGL((bwd_summary_kernel<ACT, KPL>), dim3(static_cast<unsigned>(blocks)), dim3(64 * kBW), 0, s,
                     a, g, vec ? 1 : 0);
  const int64_t nc = a.batch * a.D * a.N;
  hipLaunchKernelGGL(bwd_combine_kernel, dim3(static_cast<unsigned>((nc + 255) / 256)), dim3(256), 0, s, a, g);
  hipLaunchKernelGGL((bwd_main_kernel<ACT, KPL, LDSACC>), dim3(static_cast<unsigned>(blocks)), dim3(64 * kBW), 0,
                     s, a, g, vec ? 1 : 0);
  const int64_t np = a.D * a.N + 2 * a.D;
  hipLaunchKernelGGL(bwd_param_sums_kernel, dim3(static_cast<unsigned>((np + 255) / 256)), dim3(256), 0, s, a, g);
  const int64_t nbc = a.batch * 2 * a.N * a.L;
  hipLaunchKernelGGL((bwd_bc_out_kernel<ACT>), dim3(static_cast<unsigned>((nbc + 255) / 256)), dim3(256), 0, s, a,
                     g);
  return hipGetLastError();
}

template <typename ACT>
hipError_t launch_bwd_act(const BwdArgs& a, const BwdLayout& g, hipStream_t s) {
  if (g.kpl == 8) return launch_bwd_typed<ACT, 8, true>(a, g, s);
  if (a.N <= BwdCap<4, true>::NMAX) return launch_bwd_typed<ACT, 4, true>(a, g, s);
  return launch_bwd_typed<ACT, 4, false>(a, g, s);
}

}  // namespace

size_t scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t D, int N) {
  if (batch <= 0 || L <= 0 || D <= 0) return 0;
  return bwd_ws_floats(batch, L, D, N) * sizeof(float);
}

bool scan_bwd_grid_ok(int64_t batch, int64_t L, int64_t D, int N) {
  if (batch <= 0 || L <= 0 || D <= 0) return true;
  const BwdLayout g = bwd_layout(batch, L, D, N, nullptr);
  return batch * g.nchunks * g.nslices <= 0x7fffffff && batch * 2 * N * L / 256 < 0x7fffffff &&
         batch * D * N / 256 < 0x7fffffff;
}

hipError_t launch_scan_bwd(const BwdArgs& a, Dt dt, void* ws, hipStream_t s) {
  const BwdLayout g = bwd_layout(a.batch, a.L, a.D, a.N, static_cast<float*>(ws));
  if (dt == Dt::F32) return launch_bwd_act<ActF32>(a, g, s);
  return launch_bwd_act<ActBF16>(a, g, s);
}

}  // namespace ssm
