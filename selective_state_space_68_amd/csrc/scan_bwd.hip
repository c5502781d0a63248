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
//      the previous chunk from a zero start), and its decay P = exp(A sum Delta)
//      (at N = 16 with enough channels, from one token-sequential forward walk:
//      bwd_summary_tokseq_kernel);
//   2. combine: per (b, d, n), a sequential pass over the chunks turns F into the
//      state entering each chunk and X into the adjoint entering each chunk;
//   3. main: per (b, chunk, d), recompute the states inside the chunk from its
//      entering state (fold, wave scan, replay), run the adjoint recurrence from
//      its entering adjoint (reverse fold, reverse wave scan, reverse replay) and
//      accumulate every gradient;
//   4. finalize: fixed-order sums of the per-(b, chunk) partials of dA, dD and the
//      delta bias; dB and dC from float32 to the activation dtype.
//
// With the forward pass's saved chunk states (the state entering every 512-token
// chunk, written by the forward kernels' SAVE builds) and enough channels to fill
// the chip without splitting the sequence, steps 1 and 2 go: the main kernel's SEQ
// build walks each workgroup's chunks from the last to the first, takes the
// entering state from the saved states and the entering adjoint from the chunk it
// processed before, and so reads every input once.
//
// A workgroup of kW waves owns one (batch row, chunk) pair and a slice of
// kW * rounds channels (about one workgroup per CU): it stages the chunk's B and C
// once in LDS (float32, permuted so that each lane's tokens are contiguous), and
// each wave runs one channel per round.  dB and dC are sums over channels.  The
// main kernel's waves step through the states in pairs together: each wave writes
// its channel's dB and dC terms for the pair to its own LDS slot, and after a
// barrier every thread adds the kW slots' values of the entries it owns, in wave
// order, to the workgroup's region of the workspace (its slice's partial for this
// batch row and chunk, read and rewritten once per round); the finalize kernel
// adds the slices in slice order.  Every output is formed in a fixed order, so
// the results are bitwise reproducible.  (LDS float atomics, the obvious alternative,
// measured 7x slower on gfx950 than this whole kernel.)
#include <utility>

#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_common.hpp"

namespace ssm {
namespace {

struct BwdLayout {
  int kpl;                            // tokens per lane: chunks of 64 * kpl tokens
  int waves;                          // waves per workgroup
  int rounds;                         // channels per wave
  int64_t nchunks;
  int64_t nslices;                    // channel slices of waves * rounds
  float* F;                           // [batch][nchunks][D][N]: F, then the entering state
  float* X;                           // [batch][nchunks][D][N]: X, then the entering adjoint
  float* P;                           // [batch][nchunks][D][N]: chunk decay, then dA partials
  float* part;                        // [nslices][batch][2][N][L] per-slice dB (0) and dC (1) sums
  float* dDp;                         // [batch][nchunks][D] dD partials
  float* dbp;                         // [batch][nchunks][D] delta-bias partials
};

// Up to 16 states (the models' state size is 16): 8 tokens per lane and 8 waves
// per workgroup.  More states: 4 tokens per lane and 4 waves, so that a chunk's B
// and C for up to 64 states (2 * 64 * 256 floats, 128 KB) and the waves' slots
// still fit in LDS.
constexpr int kWFast = 8, kWGen = 4;
constexpr int kNMaxFast = 16, kNMaxGen = 64;
bool bwd_fast(int N) { return N <= kNMaxFast; }

int64_t align64(int64_t n) { return (n + 63) / 64 * 64; }

BwdLayout bwd_layout(int64_t batch, int64_t L, int64_t D, int N, float* ws) {
  BwdLayout g{};
  g.kpl = bwd_fast(N) ? 8 : 4;
  g.waves = bwd_fast(N) ? kWFast : kWGen;
  const int64_t CH = 64 * g.kpl, W = g.waves;
  g.nchunks = (L + CH - 1) / CH;
  const int64_t tasks = batch * g.nchunks * D;
  // About one workgroup per CU (256; the main kernel runs one per CU) where the
  // shape allows: more rounds amortise the tile load and the partial-sum write over
  // more channels.  (Measured against a target of 512: 2-8 % faster from
  // 2 x 2048 x 512 to 2 x 4096 x 1536, 1 % slower at 200 channels; against a cap
  // of 16 rounds: 2 % faster on the 1.4B and 131k shapes.)
  constexpr int64_t kTargetGroups = 256;
  int64_t r = (tasks + W * kTargetGroups - 1) / (W * kTargetGroups);
  const int64_t rmax = (D + W - 1) / W;
  r = r < 1 ? 1 : r;
  r = r > rmax ? rmax : r;
  g.rounds = static_cast<int>(r);
  g.nslices = (D + W * r - 1) / (W * r);
  const int64_t st = align64(batch * g.nchunks * D * N);
  const int64_t pt = align64(g.nslices * batch * 2 * N * L);
  const int64_t pp = align64(batch * g.nchunks * D);
  if (ws) {
    g.F = ws;
    g.X = g.F + st;
    g.P = g.X + st;
    g.part = g.P + st;
    g.dDp = g.part + pt;
    g.dbp = g.dDp + pp;
  }
  return g;
}

// The chunk walk (bwd_main_kernel's SEQ build, from saved forward states): a
// workgroup per (batch row, slice of 8 * rounds channels), with the rounds chosen
// for about 256 workgroups.  Workspace: the carried adjoints (batch * D * N), the
// per-chunk dA partials, the per-slice dB/dC partials and the per-chunk dD and bias
// partials.
BwdLayout bwd_layout_seq(int64_t batch, int64_t L, int64_t D, int N, float* ws) {
  BwdLayout g{};
  g.kpl = 8;
  g.waves = kWFast;
  const int64_t CH = 64 * g.kpl, W = g.waves;
  g.nchunks = (L + CH - 1) / CH;
  constexpr int64_t kTargetGroups = 256;
  int64_t r = (batch * D + W * kTargetGroups - 1) / (W * kTargetGroups);
  const int64_t rmax = (D + W - 1) / W;
  r = r < 1 ? 1 : (r > rmax ? rmax : r);
  g.rounds = static_cast<int>(r);
  g.nslices = (D + W * r - 1) / (W * r);
  const int64_t cs = align64(batch * D * N), pp = align64(batch * g.nchunks * D * N);
  const int64_t pt = align64(g.nslices * batch * 2 * N * L), pd = align64(batch * g.nchunks * D);
  if (ws) {
    g.F = nullptr;
    g.X = ws;
    g.P = g.X + cs;
    g.part = g.P + pp;
    g.dDp = g.part + pt;
    g.dbp = g.dDp + pd;
  }
  return g;
}

size_t bwd_seq_ws_floats(int64_t batch, int64_t L, int64_t D, int N) {
  const BwdLayout g = bwd_layout_seq(batch, L, D, N, nullptr);
  return static_cast<size_t>(align64(batch * D * N) + align64(batch * g.nchunks * D * N) +
                             align64(g.nslices * batch * 2 * N * L) + 2 * align64(batch * g.nchunks * D));
}

// The chunk walk replaces the summary where the channels alone give every CU at
// least 8 rounds of work (from 16384 channels); with fewer, the chunk-parallel
// decomposition keeps the chip full.
bool bwd_seq_suits(int64_t batch, int64_t D, int N) { return bwd_fast(N) && batch * D >= 16384; }

size_t bwd_ws_floats(int64_t batch, int64_t L, int64_t D, int N) {
  const BwdLayout g = bwd_layout(batch, L, D, N, nullptr);
  return static_cast<size_t>(3 * align64(batch * g.nchunks * D * N) + align64(g.nslices * batch * 2 * N * L) +
                             2 * align64(batch * g.nchunks * D));
}

// ---- cross-lane helpers -------------------------------------------------------

// Two reverse (suffix) scans across the 64 lanes of (a, b) pairs, interleaved (no
// wait states between the DPP steps): on return lane i's b
// is mu_i = b_i + a_i mu_{i+1} with mu_64 = carry, i.e. the composition of lanes
// 63 .. i applied to the carry.  Within each row of 16 lanes, Kogge-Stone steps
// with row_shl 1, 2, 4, 8 (in-place DPP as in the forward scan; a lane whose
// source is past its row's end is not written, which is combining with the
// identity).  Then the three row boundaries are resolved from lanes 48, 32, 16
// read as scalars: row r's lanes apply their row suffix to mu of the first lane
// of row r + 1.  Pure VALU, no memory access.
__device__ __forceinline__ void wave_rscan_pairs2(float& a0, float& b0, float carry0, float& a1, float& b1,
                                                  float carry1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %3 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %3, %3 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %3 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %3, %3 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %3 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %3, %3 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %3 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %3, %3 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(b0), "+v"(a0), "+v"(b1), "+v"(a1));
  auto rl = [](float v, int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); };
  const float m2a = __builtin_fmaf(rl(a0, 48), carry0, rl(b0, 48));
  const float m2b = __builtin_fmaf(rl(a1, 48), carry1, rl(b1, 48));
  const float m1a = __builtin_fmaf(rl(a0, 32), m2a, rl(b0, 32));
  const float m1b = __builtin_fmaf(rl(a1, 32), m2b, rl(b1, 32));
  float m0a = __builtin_fmaf(rl(a0, 16), m1a, rl(b0, 16));
  float m0b = __builtin_fmaf(rl(a1, 16), m1b, rl(b1, 16));
  float xa1 = m1a, xa2 = m2a, xb1 = m1b, xb2 = m2b;
  asm volatile("" : "+v"(m0a), "+v"(xa1), "+v"(xa2), "+v"(m0b), "+v"(xb1), "+v"(xb2));
  const int row = (threadIdx.x & 63) >> 4;
  const float ma = row == 3 ? carry0 : (row == 2 ? xa2 : (row == 1 ? xa1 : m0a));
  const float mb = row == 3 ? carry1 : (row == 2 ? xb2 : (row == 1 ? xb1 : m0b));
  b0 = __builtin_fmaf(a0, ma, b0);
  b1 = __builtin_fmaf(a1, mb, b1);
}

// Value of lane i+1 in lane i; lane 63 receives `last`.
__device__ __forceinline__ float wave_shift_down(float v, float last) {
  return dpp_mov<0x130, 0xf, false>(last, v);
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
// offset `row`; tokens at or past L read as 0 (element by element).
template <typename ACT, int KPL>
__device__ __forceinline__ void load_tokens(const void* src, int64_t row, int64_t t, int64_t L, float (&v)[KPL]) {
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

// Stages chunk [t0, t0 + 64*KPL) of B (states 0..NP-1) then C into LDS as float32,
// block m*NP + n for matrix m and state n (states N..NP-1, and tokens past L, are
// zero).  Float4 f of a block (tokens 4f .. 4f+3 of the chunk) goes to slot
// (f % (KPL/4)) * 64 + f / (KPL/4), so lane i finds its KPL tokens as KPL/4
// float4 at q * 64 + i.  B and C are [batch][L][N]: a thread loads 4 consecutive
// states of one token (one 16- or 8-byte vector when N % 4 == 0) and scatters them
// into their blocks; consecutive threads take consecutive tokens.
template <typename ACT, int KPL>
__device__ __forceinline__ void load_tile(float4* tile, const BwdArgs& p, int64_t b, int64_t t0, int NP, bool vec) {
  constexpr int CH = 64 * KPL, F4 = CH / 4, Q = KPL / 4;
  const int N = p.N;
  const int64_t L = p.L;
  const int G = (NP + 3) / 4;                        // groups of 4 states per token
  const int total = 2 * G * CH;
  const bool v4 = vec && (N % 4 == 0);
  float* tf = reinterpret_cast<float*>(tile);
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int tk = e % CH, mg = e / CH;
    const int m = mg / G, n0 = 4 * (mg % G);
    const void* src = m ? p.Cm : p.Bm;
    const int64_t t = t0 + tk;
    float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (t < L) {
      const int64_t off = (b * L + t) * N + n0;
      if (v4) {
        load4<ACT>(src, off, x);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = n0 + r < N ? load_act<ACT>(src, off + r) : 0.0f;
      }
    }
    const int f = tk >> 2;
    const int slot = ((f % Q) * 64 + f / Q) * 4 + (tk & 3);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n0 + r < NP) tf[(m * NP + n0 + r) * (4 * F4) + slot] = x[r];
  }
}

// One channel's per-token inputs for its KPL tokens of the chunk.  The vector path
// (8 tokens per lane, L % 8 == 0, 16-byte aligned rows) loads them as raw 16-byte
// vectors ahead of use: fetch() issues the loads, get() unpacks them.  In float32
// only u and delta are fetched ahead; dy and z are loaded in get().  (Before the
// main kernel's LDS accumulator freed about 40 registers, the four float32 vectors
// held across a round made it spill 18 registers and two spilled 10, 6 % faster on
// the 130M-shaped backward; with the accumulator, four measured the same as two.)
// A lane whose
// tokens start at or past L loads the row's last tokens instead (the start is
// clamped) and its values are masked by the caller.
template <typename ACT, int KPL>
struct TokenLoader {
  static constexpr bool kVecOk = KPL == 8;
  using IO = TokenIO<ACT, 8>;
  typename IO::raw_t ru[IO::kVec], rd[IO::kVec], ry[IO::kVec], rz[IO::kVec];

  __device__ __forceinline__ void fetch(const BwdArgs& p, int64_t row, int64_t t) {
    if constexpr (kVecOk) {
      const int64_t tc = t + KPL <= p.L ? t : p.L - KPL;
      IO::load_raw(p.u, row + tc, ru);
      IO::load_raw(p.delta, row + tc, rd);
      if constexpr (ACT::kBytes == 2) {
        IO::load_raw(p.dy, row + tc, ry);
        if (p.z) IO::load_raw(p.z, row + tc, rz);
      }
    }
  }
  // u, raw delta, dy, z (z only with a gate)
  __device__ __forceinline__ void get(const BwdArgs& p, int64_t row, int64_t t, bool vec, float (&u)[KPL],
                                      float (&dl)[KPL], float (&dy)[KPL], float (&z)[KPL]) {
    if constexpr (kVecOk) {
      if (vec) {
        if constexpr (ACT::kBytes == 4) {           // float32: dy and z loaded here, not prefetched
          const int64_t tc = t + KPL <= p.L ? t : p.L - KPL;
          IO::load_raw(p.dy, row + tc, ry);
          if (p.z) IO::load_raw(p.z, row + tc, rz);
        }
        IO::unpack(ru, u);
        IO::unpack(rd, dl);
        IO::unpack(ry, dy);
        if (p.z) IO::unpack(rz, z);
        return;
      }
    }
    load_tokens<ACT, KPL>(p.u, row, t, p.L, u);
    load_tokens<ACT, KPL>(p.delta, row, t, p.L, dl);
    load_tokens<ACT, KPL>(p.dy, row, t, p.L, dy);
    if (p.z) load_tokens<ACT, KPL>(p.z, row, t, p.L, z);
  }
};

// Per-token values of one channel's chunk: Delta (zero on tokens past L or for a
// wave past the last channel, which makes them identity steps), Delta*u, the
// gate-scaled output gradient g (zero likewise), and for the main kernel the
// softplus derivative sigmoid(raw) and the gate factor dy * SiLU'(z).
template <int KPL, bool FULL>
struct TokenState {
  float u[KPL], dl[KPL], du[KPL], g[KPL];
  float sg[FULL ? KPL : 1], dzf[FULL ? KPL : 1];
  float sdl;

  __device__ __forceinline__ void set(const BwdArgs& p, int64_t t, bool live, float bias, const float (&dy)[KPL],
                                      const float (&z)[KPL]) {
    const int64_t L = p.L;
    if (p.z) {
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const float s = __builtin_amdgcn_rcpf(1.0f + exp2_hw(-z[j] * kLog2e));
        g[j] = dy[j] * z[j] * s;
        if constexpr (FULL) dzf[j] = dy[j] * s * __builtin_fmaf(z[j], 1.0f - s, 1.0f);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        g[j] = dy[j];
        if constexpr (FULL) dzf[j] = 0.0f;
      }
    }
    sdl = 0.0f;
    // Branch-free in the softplus flag (selects, with sg = 1 without it): a branch per
    // token here left values in scratch memory in the main kernel.
    const bool sp = p.softplus != 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const float raw = dl[j] + bias;
      float d = sp ? softplus_f(raw) : raw;
      if constexpr (FULL) sg[j] = sp ? __builtin_amdgcn_rcpf(1.0f + exp2_hw(-raw * kLog2e)) : 1.0f;
      const bool ok = live && t + j < L;
      d = ok ? d : 0.0f;
      g[j] = ok ? g[j] : 0.0f;
      dl[j] = d;
      du[j] = d * u[j];
      sdl += d;
    }
  }
};

// ---- 1. chunk summaries -----------------------------------------------------------
// One wave per channel per round; the states two at a time.  NT: the most states
// the instantiation holds in LDS.
template <typename ACT, int KPL, int kW, int NT>
__global__ __launch_bounds__(64 * kW) void bwd_summary_kernel(BwdArgs p, BwdLayout g, int vec_flag) {
  constexpr int CH = 64 * KPL, F4 = CH / 4, Q = KPL / 4;
  __shared__ float4 s_tile[2 * NT * F4];
  const bool vec = vec_flag != 0;
  const int lane = threadIdx.x & 63;
  const int w = uniform_int(threadIdx.x >> 6);
  const int64_t nbc = p.batch * g.nchunks;
  // Workgroups of one (batch row, chunk) pair are nbc apart, so they share an XCD
  // (and its L2) whenever nbc is a multiple of the 8 XCDs.
  const int64_t bc = blockIdx.x % nbc, slice = blockIdx.x / nbc;
  const int64_t b = bc % p.batch, c = bc / p.batch;
  const int N = p.N;
  const int NP = (N + 1) & ~1;
  const int64_t L = p.L, D = p.D;
  const int64_t t0 = c * CH;
  load_tile<ACT, KPL>(s_tile, p, b, t0, NP, vec);
  __syncthreads();

  const int64_t tl = t0 + static_cast<int64_t>(lane) * KPL;
  const int64_t dg = static_cast<int64_t>(kW) * g.rounds;
  for (int r = 0; r < g.rounds; ++r) {
    const int64_t d = slice * dg + r * kW + w;
    if (d >= D) break;
    const int64_t row = (b * D + d) * L;
    TokenLoader<ACT, KPL> ld;
    TokenState<KPL, false> ts;
    float dy[KPL], z[KPL];
    if (vec) ld.fetch(p, row, tl);
    ld.get(p, row, tl, vec, ts.u, ts.dl, dy, z);
    ts.set(p, tl, true, p.bias ? p.bias[d] : 0.0f, dy, z);
    const float stot = wave_sum(ts.sdl);
    const float a2_v = lane < N ? p.A[d * N + lane] * kLog2e : 0.0f;
    float Fv = 0.0f, Xv = 0.0f;
    // two states at a time (the second may be the zero padding state N when N is
    // odd: zero A, B and C, nothing stored)
    for (int n0 = 0; n0 < NP; n0 += 2) {
      const int n1 = n0 + 1;
      const float a20 = lane_value(a2_v, n0), a21 = lane_value(a2_v, n1);
      const float4* sB0 = s_tile + n0 * F4;
      const float4* sB1 = s_tile + n1 * F4;
      const float4* sC0 = s_tile + (NP + n0) * F4;
      const float4* sC1 = s_tile + (NP + n1) * F4;
      float av0[KPL], av1[KPL], cv0[KPL], cv1[KPL];
      float h0 = 0.0f, h1 = 0.0f;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float4 x0 = sB0[q * 64 + lane], x1 = sB1[q * 64 + lane];
        const float4 y0 = sC0[q * 64 + lane], y1 = sC1[q * 64 + lane];
        const float b0[4] = {x0.x, x0.y, x0.z, x0.w}, b1[4] = {x1.x, x1.y, x1.z, x1.w};
        const float c0[4] = {y0.x, y0.y, y0.z, y0.w}, c1[4] = {y1.x, y1.y, y1.z, y1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = 4 * q + k;
          av0[j] = exp2_hw(ts.dl[j] * a20);
          av1[j] = exp2_hw(ts.dl[j] * a21);
          cv0[j] = c0[k];
          cv1[j] = c1[k];
          h0 = __builtin_fmaf(av0[j], h0, ts.du[j] * b0[k]);
          h1 = __builtin_fmaf(av1[j], h1, ts.du[j] * b1[k]);
        }
      }
      float x0 = 0.0f, x1 = 0.0f;
#pragma unroll
      for (int j = KPL - 1; j >= 0; --j) {
        x0 = av0[j] * __builtin_fmaf(ts.g[j], cv0[j], x0);
        x1 = av1[j] * __builtin_fmaf(ts.g[j], cv1[j], x1);
      }
      float P0 = exp2_hw(a20 * ts.sdl), P1 = exp2_hw(a21 * ts.sdl);
      float R0 = P0, R1 = P1;
      wave_scan_pairs2(P0, h0, P1, h1);
      wave_rscan_pairs2(R0, x0, 0.0f, R1, x1, 0.0f);
      const float f0 = wave_lane63(h0), f1 = wave_lane63(h1);
      const float y0 = lane_value(x0, 0), y1 = lane_value(x1, 0);
      Fv = lane == n0 ? f0 : (lane == n1 ? f1 : Fv);
      Xv = lane == n0 ? y0 : (lane == n1 ? y1 : Xv);
    }
    if (lane < N) {
      const int64_t off = ((b * g.nchunks + c) * D + d) * N + lane;
      g.F[off] = Fv;
      g.X[off] = Xv;
      g.P[off] = exp2_hw(a2_v * stot);
    }
  }
}

// ---- 1b. chunk summaries, token-sequential (N = 16, many channels) ----------------
// The same F, X and P as bwd_summary_kernel, from one forward walk over the chunk:
// a lane owns 4 states of one channel (a wave 16 channels), as in the forward
// token-sequential scan.  X, the adjoint a chunk sends left from a zero start,
// nests as x = a_t (g_t C_t + x) from the chunk's end; unrolled it is
// X = sum_t (prod_{s <= t} a_s) g_t C_t over the chunk, which the forward walk
// accumulates with the running decay product (re-anchored at every 32-token block
// to exp2(A * sum of the Deltas before it), so its rounding spans 32 products),
// sharing each token's exp with the state fold.  About 8 issue slots per element
// against the two folds and two wave scans of bwd_summary_kernel.
//   SUB = 1: the workgroup's 4 waves take 4 channel groups of one chunk and are
//            independent (own LDS slice, no barrier).
//   SUB = 4: for fewer channels, the 4 waves take the 4 quarter-chunks (128 tokens)
//            of one channel group, each from a zero start, and wave 0 joins them in
//            order: P = P1 P2 P3 P4, F folds the quarters' F left to right with their
//            decays, and X = X1 + P1 X2 + P1 P2 X3 + P1 P2 P3 X4 (a quarter past L
//            has Delta = g = 0: P = 1, F = X = 0).
constexpr int kSumWaves = 4;
constexpr int64_t kSumTokseqMinWaves = 4096;      // one wave per (chunk, channel group) from here
constexpr int64_t kSumSplitMinWaves = 1024;       // quarter-chunk waves from here (measured)

// Eight consecutive activations of one channel (cached: in bfloat16 a block's 8
// tokens of a channel are half of a cache line whose other half the next block reads).
template <typename ACT>
__device__ __forceinline__ void load8_cached(const void* base, int64_t off, float (&v)[8]) {
  if constexpr (ACT::kBytes == 4) {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 x = q[0], y = q[1];
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else {
    const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x); v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
    v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z); v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
  }
}

template <typename ACT, bool GATE, int SUB>
__global__ __launch_bounds__(64 * kSumWaves) void bwd_summary_tokseq_kernel(BwdArgs p, BwdLayout g) {
  static_assert(SUB == 1 || SUB == kSumWaves, "one channel group per wave, or one per workgroup");
  constexpr int NS = 16, QL = 4, CPW = 16, T = 32, CH = 512, SCH = CH / SUB;
  __shared__ float4 s_bc[kSumWaves][2][T][NS / 4];   // B, C [token][state group], groups XOR-swizzled by piece
  __shared__ float4 s_tok[kSumWaves][CPW][T + 1];    // (Delta, Delta*u, g, -) per channel and token
  const int lane = threadIdx.x & 63;
  const int w = uniform_int(threadIdx.x >> 6);
  const int64_t L = p.L, D = p.D;
  const int64_t nbc = p.batch * g.nchunks;
  // (workgroups of one (batch row, chunk) pair are nbc apart: one XCD when nbc % 8 == 0)
  const int64_t bc = blockIdx.x % nbc;
  const int64_t b = bc % p.batch, c = bc / p.batch;
  const int64_t ngrp = (D + CPW - 1) / CPW;
  const int64_t grp = SUB == 1 ? static_cast<int64_t>(blockIdx.x / nbc) * kSumWaves + w
                               : static_cast<int64_t>(blockIdx.x / nbc);
  const int sub = SUB == 1 ? 0 : w;                  // this wave's part of the chunk
  const int64_t gcl = grp < ngrp ? grp : ngrp - 1;
  const int ch = lane / QL, q = lane % QL;
  const int64_t d_own = gcl * CPW + ch;
  const bool store_ok = grp < ngrp && d_own < D;
  const int64_t d = d_own < D ? d_own : D - 1;
  const int64_t row = (b * D + d) * L;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  float a2[4], h[4], X[4], Dc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a2[j] = p.A[d * NS + 4 * q + j] * kLog2e;
    h[j] = 0.0f;
    X[j] = 0.0f;
  }
  float cum = 0.0f;                                   // sum of Delta over the wave's part so far (the channel's)
  const int64_t bc_row = b * L * NS;
  float* bc_w = reinterpret_cast<float*>(s_bc[w]);
  float4* tok_w = s_tok[w][ch];

  float ru[8], rd[8], ry[8], rz[8], rb[8], rc[8];
  auto fetch = [&](int64_t t0) __attribute__((always_inline)) {
    int64_t tp = t0 + 8 * q;
    tp = tp + 8 <= L ? tp : L - 8;
    load8_cached<ACT>(p.u, row + tp, ru);
    load8_cached<ACT>(p.delta, row + tp, rd);
    load8_cached<ACT>(p.dy, row + tp, ry);
    if constexpr (GATE) load8_cached<ACT>(p.z, row + tp, rz);
    // B and C piece of this lane ([L][N]): token lane / 2 of the block, states 8 (lane % 2) ..
    int64_t t = t0 + lane / 2;
    t = t < L ? t : L - 1;
    load8_cached<ACT>(p.Bm, bc_row + t * NS + 8 * (lane % 2), rb);
    load8_cached<ACT>(p.Cm, bc_row + t * NS + 8 * (lane % 2), rc);
  };

  const int64_t tc0 = c * CH + sub * SCH;
  fetch(tc0);
  for (int blk = 0; blk < SCH / T; ++blk) {
    const int64_t t0 = tc0 + blk * T;
    const bool pvalid = t0 + 8 * q < L;              // L % 8 == 0: a piece is all in or all out
    // ---- per-token work of this lane's piece; the block's B and C
    float sp = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float raw = rd[k] + bias;
      float dl = p.softplus ? softplus_f(raw) : raw;
      float gk = ry[k];
      if constexpr (GATE) gk *= silu_f(rz[k]);
      dl = pvalid ? dl : 0.0f;
      gk = pvalid ? gk : 0.0f;
      sp += dl;
      tok_w[8 * q + k] = make_float4(dl, dl * ru[k], gk, 0.0f);
    }
    {
      // token t, state groups 2h and 2h + 1, each at its swizzled slot (group g of
      // token t sits at g ^ (t / 8))
      const int t = lane / 2, h2 = 2 * (lane % 2), sw = (t / 8) & 3;
      float4* brow = reinterpret_cast<float4*>(bc_w + (0 * T + t) * NS);
      float4* crow = reinterpret_cast<float4*>(bc_w + (1 * T + t) * NS);
#pragma unroll
      for (int g4 = 0; g4 < 2; ++g4) {
        brow[(h2 + g4) ^ sw] = make_float4(rb[4 * g4], rb[4 * g4 + 1], rb[4 * g4 + 2], rb[4 * g4 + 3]);
        crow[(h2 + g4) ^ sw] = make_float4(rc[4 * g4], rc[4 * g4 + 1], rc[4 * g4 + 2], rc[4 * g4 + 3]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    fetch(t0 + T < tc0 + SCH ? t0 + T : t0);         // next block (the last one reloads itself, unused)

    // ---- the forward walk: F (the state), X (decay-weighted g C) over the block
#pragma unroll
    for (int j = 0; j < 4; ++j) Dc[j] = exp2_hw(a2[j] * cum);
#pragma unroll
    for (int tb = 0; tb < T / 8; ++tb) {
      const int gsw = q ^ tb;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int t = 8 * tb + k;
        const float4 tv = tok_w[t];
        const float4 bb = reinterpret_cast<const float4*>(bc_w + (0 * T + t) * NS)[gsw];
        const float4 cc = reinterpret_cast<const float4*>(bc_w + (1 * T + t) * NS)[gsw];
        const float bs[4] = {bb.x, bb.y, bb.z, bb.w}, cs[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = exp2_hw(tv.x * a2[j]);
          h[j] = __builtin_fmaf(a, h[j], tv.y * bs[j]);
          Dc[j] *= a;
          X[j] = __builtin_fmaf(Dc[j], tv.z * cs[j], X[j]);
        }
      }
    }
    // the channel's sum of Delta over the block (its 4 pieces)
    sp += dpp_mov<0xB1, 0xf, false>(0.0f, sp);       // quad_perm [1, 0, 3, 2]
    sp += dpp_mov<0x4E, 0xf, false>(0.0f, sp);       // quad_perm [2, 3, 0, 1]
    cum += sp;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  const int64_t off = ((b * g.nchunks + c) * D + d) * NS + 4 * q;
  if constexpr (SUB == 1) {
    if (store_ok) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        g.F[off + j] = h[j];
        g.X[off + j] = X[j];
        g.P[off + j] = exp2_hw(a2[j] * cum);
      }
    }
  } else {
    // each wave's (F, X, sum of Delta) per lane into its own LDS slice (its token
    // values are no longer needed), then wave 0 joins the parts in token order
    float4* part_w = &s_tok[w][0][0];
    part_w[3 * lane + 0] = make_float4(h[0], h[1], h[2], h[3]);
    part_w[3 * lane + 1] = make_float4(X[0], X[1], X[2], X[3]);
    part_w[3 * lane + 2] = make_float4(cum, 0.0f, 0.0f, 0.0f);
    __syncthreads();
    if (w == 0 && store_ok) {
      float F[4] = {0.0f, 0.0f, 0.0f, 0.0f}, Xs[4] = {0.0f, 0.0f, 0.0f, 0.0f}, Dp[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      float ctot = 0.0f;
#pragma unroll
      for (int k = 0; k < SUB; ++k) {
        const float4* part_k = &s_tok[k][0][0];
        const float4 hv = part_k[3 * lane + 0], xv = part_k[3 * lane + 1];
        const float ck = part_k[3 * lane + 2].x;
        const float hs[4] = {hv.x, hv.y, hv.z, hv.w}, xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float Pk = exp2_hw(a2[j] * ck);
          F[j] = __builtin_fmaf(Pk, F[j], hs[j]);
          Xs[j] = __builtin_fmaf(Dp[j], xs[j], Xs[j]);
          Dp[j] *= Pk;
        }
        ctot += ck;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        g.F[off + j] = F[j];
        g.X[off + j] = Xs[j];
        g.P[off + j] = exp2_hw(a2[j] * ctot);
      }
    }
  }
}

// ---- 2. sequential combine over chunks --------------------------------------------
constexpr int kAhead = 8;   // loads issued ahead in the sequential combine and sums

// sum_{k < count} src[k * stride], added in k order (so bitwise the plain loop's
// result), with the loads issued kAhead at a time (each behind a uniform branch,
// so the group has no wait between its loads).
__device__ __forceinline__ float ordered_sum(const float* src, int64_t stride, int64_t count) {
  float s = 0.0f;
  for (int64_t k0 = 0; k0 < count; k0 += kAhead) {
    float v[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
      if (k0 + j < count) v[j] = src[(k0 + j) * stride];
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
      if (k0 + j < count) s += v[j];
  }
  return s;
}

__global__ void bwd_combine_kernel(BwdArgs p, BwdLayout g) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int N = p.N;
  const int64_t D = p.D;
  if (i >= p.batch * D * N) return;
  const int64_t n = i % N, d = (i / N) % D, b = i / (N * D);
  const int64_t stride = D * N;
  const int64_t base = b * g.nchunks * stride + d * N + n;
  const int64_t nch = g.nchunks;
  // The chunks' values are loaded kAhead at a time before any of them is replaced,
  // so each group costs one memory round trip instead of one per chunk.
  float h = p.h0 ? p.h0[i] : 0.0f;
  for (int64_t c0 = 0; c0 < nch; c0 += kAhead) {
    float f[kAhead], dec[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      if (c0 + j < nch) {
        const int64_t o = base + (c0 + j) * stride;
        f[j] = g.F[o];
        dec[j] = g.P[o];
      }
    }
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      if (c0 + j < nch) {
        g.F[base + (c0 + j) * stride] = h;           // state entering chunk c0 + j
        h = __builtin_fmaf(dec[j], h, f[j]);
      }
    }
  }
  float mu = p.dfinal ? p.dfinal[i] : 0.0f;
  for (int64_t c0 = nch - 1; c0 >= 0; c0 -= kAhead) {
    float x[kAhead], dec[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      if (c0 - j >= 0) {
        const int64_t o = base + (c0 - j) * stride;
        x[j] = g.X[o];
        dec[j] = g.P[o];
      }
    }
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      if (c0 - j >= 0) {
        g.X[base + (c0 - j) * stride] = mu;          // adjoint entering chunk c0 - j from the right
        mu = __builtin_fmaf(dec[j], mu, x[j]);
      }
    }
  }
  if (p.dh0) p.dh0[i] = mu;
}

// ---- 3. the gradients -----------------------------------------------------------------
// NT: the most states the instantiation holds in LDS (even).  The workgroup's dB/dC
// sums over its channels (its slice's partial for this batch row and chunk) are
// formed in a fixed order: per pair, every wave writes its channel's terms to its
// own LDS slot, and after a barrier each thread adds the waves' values of the
// entries it owns (the same entries in every round, so no two threads touch one).
//   ACC (when it fits in LDS: N <= 16 at 8 tokens per lane): the running sums stay
//     in an LDS accumulator across all rounds and are written to the workspace once,
//     at the end.  The slots then hold one matrix at a time (dC after the forward
//     replay, dB after the reverse replay), two more barriers per pair, so that tile
//     (64 KB), slots (32 KB) and accumulator (64 KB) fit in the CU's 160 KB.
//   otherwise: the running sums live in the workspace region; a thread loads a
//     pair's entries before computing the pair and writes them back after adding
//     the waves' terms, so the loads have a pair's compute time to arrive from L2.
//
// SEQ (with the forward pass's saved chunk states, p.chunk_states): a workgroup owns
// one batch row and a channel slice and walks the chunks from the last to the
// first.  The state entering each chunk comes from the saved states and the
// adjoint entering it from the right is the one the workgroup's previous chunk sent
// left (kept per channel in the workspace, g.X, by the lane that reads it next), so
// no summary or combine pass is needed and every input is read once.
template <typename ACT, int KPL, int kW, int NT, bool SEQ = false>
__global__ __launch_bounds__(64 * kW) void bwd_main_kernel(BwdArgs p, BwdLayout g, int vec_flag) {
  constexpr int CH = 64 * KPL, F4 = CH / 4, Q = KPL / 4;
  constexpr int kThreads = 64 * kW;
  constexpr int RED4 = 4 * F4;                      // float4 per pair: 2 states x (dB, dC) x chunk
  static_assert(NT % 2 == 0, "states are processed in pairs");
  static_assert(RED4 % kThreads == 0, "every thread owns whole float4 entries");
  constexpr int RPT = RED4 / kThreads;               // entries per thread per pair
  constexpr int kTileBytes = 2 * NT * F4 * 16, kAccBytes = (NT / 2) * RED4 * 16;
  constexpr bool ACC = kTileBytes + kAccBytes + kW * 2 * F4 * 16 <= 160 * 1024;
  constexpr int SLOT4 = ACC ? 2 * F4 : RED4;         // float4 per wave slot: one matrix (ACC) or both
  constexpr int H2 = 4 * F4;                         // ACC: float2 per (pair, matrix): 2 states x chunk
  static_assert(!ACC || H2 % kThreads == 0, "every thread owns whole float2 entries");
  constexpr int RPT2 = H2 / kThreads;                // ACC: float2 entries per thread per (pair, matrix)
  __shared__ float4 s_tile[2 * NT * F4];
  __shared__ float4 s_red[kW * SLOT4];              // per wave: its channel's terms for the current pair
  __shared__ float2 s_acc[ACC ? (NT / 2) * 2 * H2 : 2];   // ACC: [pair][matrix][state in pair][chunk] sums
  const bool vec = vec_flag != 0;
  const int lane = threadIdx.x & 63;
  const bool lane0 = lane == 0;
  const int w = uniform_int(threadIdx.x >> 6);
  static_assert(!SEQ || ACC, "the chunk walk keeps its sums in the LDS accumulator");
  const int64_t nbc = SEQ ? p.batch : p.batch * g.nchunks;
  const int64_t bc = blockIdx.x % nbc, slice = blockIdx.x / nbc;
  const int64_t b = bc % p.batch;
  int64_t c = SEQ ? g.nchunks - 1 : bc / p.batch;   // SEQ: from the last chunk to the first
  const int N = p.N;
  const int NP = (N + 1) & ~1;
  const int64_t L = p.L, D = p.D;
  int64_t t0 = c * CH;
  load_tile<ACT, KPL>(s_tile, p, b, t0, NP, vec);

  // Entry x (< RED4) of a pair: block x / F4 = 2 * (state within the pair) +
  // matrix, slot x % F4 (lane slot % 64 and vector slot / 64 of the permuted
  // layout).  Thread threadIdx.x owns entries threadIdx.x + k * kThreads.
  float* part = g.part + (slice * p.batch + b) * 2 * N * L;
  auto entry = [&](int pp, int x, int& n, int& m, int64_t& t) __attribute__((always_inline)) {
    const int blk = x / F4, slot = x % F4;
    n = 2 * pp + (blk >> 1);
    m = blk & 1;
    t = t0 + static_cast<int64_t>(slot % 64) * KPL + 4 * (slot / 64);
  };
  __syncthreads();

  int64_t tl = t0 + static_cast<int64_t>(lane) * KPL;
  const int64_t dg = static_cast<int64_t>(kW) * g.rounds;
  auto chan = [&](int r) __attribute__((always_inline)) -> int64_t {
    const int64_t d = slice * dg + r * kW + w;
    return d < D ? d : D - 1;
  };
  // ACC: accumulator entry e of (pair pp, matrix m) is float2 e of the two states'
  // blocks of the chunk (state in pair e / (2 F4), then the permuted slot layout)
  auto acc_sum = [&](int pp, int m) __attribute__((always_inline)) {
    const float2* red2 = reinterpret_cast<const float2*>(s_red);
    float2* acc2 = s_acc + (pp * 2 + m) * H2;
#pragma unroll
    for (int k = 0; k < RPT2; ++k) {
      const int e = threadIdx.x + k * kThreads;
      float2 sum = red2[e];
#pragma unroll
      for (int ww = 1; ww < kW; ++ww) {
        const float2 v = red2[ww * H2 + e];
        sum.x += v.x;
        sum.y += v.y;
      }
      float2 a = acc2[e];
      a.x += sum.x;
      a.y += sum.y;
      acc2[e] = a;
    }
  };
  TokenLoader<ACT, KPL> ld;
  if (vec) ld.fetch(p, (b * D + chan(0)) * L, tl);
  for (int64_t ci = 0; ci < (SEQ ? g.nchunks : 1); ++ci) {
  if constexpr (SEQ) {
    if (ci > 0) {
      // every wave is past the previous chunk's last tile read (its last pair's
      // final barrier), so the next tile can be staged
      c = g.nchunks - 1 - ci;
      t0 = c * CH;
      tl = t0 + static_cast<int64_t>(lane) * KPL;
      load_tile<ACT, KPL>(s_tile, p, b, t0, NP, vec);
      __syncthreads();
    }
  }
  if constexpr (ACC) {
    for (int e = threadIdx.x; e < (NT / 2) * 2 * H2; e += kThreads) s_acc[e] = make_float2(0.0f, 0.0f);
  }
  for (int r = 0; r < g.rounds; ++r) {
    // A wave past the last channel runs the last channel with zero g and Delta*u:
    // it takes part in the barriers and adds only zeros.
    const bool valid = slice * dg + r * kW + w < D;
    const int64_t d = chan(r);
    const int64_t row = (b * D + d) * L;
    const int64_t soff = ((b * g.nchunks + c) * D + d) * N;
    const float dsk = p.Dskip ? p.Dskip[d] : 0.0f;
    TokenState<KPL, true> ts;
    {
      float dy[KPL], z[KPL];
      ld.get(p, row, tl, vec, ts.u, ts.dl, dy, z);
      ts.set(p, tl, valid, p.bias ? p.bias[d] : 0.0f, dy, z);
    }
    if (vec && r + 1 < g.rounds) {
      ld.fetch(p, (b * D + chan(r + 1)) * L, tl);   // next round's inputs
    } else if (SEQ && vec && c > 0) {
      ld.fetch(p, (b * D + chan(0)) * L, (c - 1) * CH + static_cast<int64_t>(lane) * KPL);   // next chunk's
    }
    const float A_v = lane < N ? p.A[d * N + lane] : 0.0f;
    const float a2_v = A_v * kLog2e;
    float hs_v = 0.0f, mu_v = 0.0f;
    if constexpr (SEQ) {
      // the saved state entering chunk c; the adjoint entering it from the right:
      // the final state's cotangent for the last chunk, else what chunk c + 1 sent
      // (a wave past the last channel takes zeros: it reads nothing another wave writes)
      const int64_t cidx = (b * D + d) * N + lane;
      if (lane < N && valid) {
        hs_v = p.chunk_states[((b * D + d) * g.nchunks + c) * N + lane];
        mu_v = c == g.nchunks - 1 ? (p.dfinal ? p.dfinal[cidx] : 0.0f) : g.X[cidx];
      }
    } else {
      hs_v = lane < N ? g.F[soff + lane] : 0.0f;
      mu_v = lane < N ? g.X[soff + lane] : 0.0f;
    }
    float mu_out_v = 0.0f;                            // SEQ: lane n, the adjoint this chunk sends left
    float s1[KPL], s2[KPL], yt[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      s1[j] = 0.0f;
      s2[j] = 0.0f;
      yt[j] = dsk * ts.u[j];
    }
    float dA_v = 0.0f;

    // States n0 = 2 pp and n1 = n0 + 1 (n1 may be the zero padding state N when N
    // is odd: zero B, C, A and carries, so it contributes nothing).
    auto pair = [&](int pp) __attribute__((always_inline)) {
      const int n0 = 2 * pp, n1 = n0 + 1;
      const float a20 = lane_value(a2_v, n0), a21 = lane_value(a2_v, n1);
      const float A0 = lane_value(A_v, n0), A1 = lane_value(A_v, n1);
      const float hs0 = lane_value(hs_v, n0), hs1 = lane_value(hs_v, n1);
      const float me0 = lane_value(mu_v, n0), me1 = lane_value(mu_v, n1);
      const float4* sB0 = s_tile + n0 * F4;
      const float4* sB1 = s_tile + n1 * F4;
      const float4* sC0 = s_tile + (NP + n0) * F4;
      const float4* sC1 = s_tile + (NP + n1) * F4;
      float4* slot = s_red + w * SLOT4;                // this wave's dB/dC terms for the pair
      // B and C are read from LDS again in each phase instead of being held in
      // registers across the pair (the compiler barrier keeps it from reusing them).
      auto reload = []() __attribute__((always_inline)) { asm volatile("" ::: "memory"); };
      if constexpr (!ACC) barrier_lds();             // the previous pair's sums have read the slots
      // this thread's accumulated entries of the pair (none yet in the first round)
      float4 prev[ACC ? 1 : RPT];
      float* dst[ACC ? 1 : RPT];
      bool whole[ACC ? 1 : RPT];
      if constexpr (!ACC) {
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
          int n, m;
          int64_t t;
          entry(pp, threadIdx.x + k * kThreads, n, m, t);
          dst[k] = n < N ? part + (m * N + n) * L + t : nullptr;
          whole[k] = n < N && t + 4 <= L && L % 4 == 0;
          prev[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          if (r > 0 && whole[k]) prev[k] = *reinterpret_cast<const float4*>(dst[k]);
        }
      }
      // slot blocks: ACC, one matrix at a time: 0 = state n0, 1 = state n1;
      // otherwise 2 * (state in pair) + matrix
      constexpr int kC0 = ACC ? 0 : 1, kC1 = ACC ? 1 : 3, kB0 = 0, kB1 = ACC ? 1 : 2;

      // forward recomputation: fold, scan, replay (h_j kept per token; the input
      // terms Delta u B from the fold are kept for the replay, which reads only C)
      float av0[KPL], av1[KPL], hv0[KPL], hv1[KPL];
      float h0 = lane0 ? hs0 : 0.0f, h1 = lane0 ? hs1 : 0.0f;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float4 x0 = sB0[q * 64 + lane], x1 = sB1[q * 64 + lane];
        const float b0[4] = {x0.x, x0.y, x0.z, x0.w}, b1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = 4 * q + k;
          av0[j] = exp2_hw(ts.dl[j] * a20);
          av1[j] = exp2_hw(ts.dl[j] * a21);
          hv0[j] = ts.du[j] * b0[k];
          hv1[j] = ts.du[j] * b1[k];
          h0 = __builtin_fmaf(av0[j], h0, hv0[j]);
          h1 = __builtin_fmaf(av1[j], h1, hv1[j]);
        }
      }
      float P0 = exp2_hw(a20 * ts.sdl), P1 = exp2_hw(a21 * ts.sdl);
      float R0 = P0, R1 = P1;
      wave_scan_pairs2(P0, h0, P1, h1);
      const float hin0 = wave_shift_up(h0, hs0), hin1 = wave_shift_up(h1, hs1);
      // ACC: the previous pair's dB sums have read the slots (placed after the fold
      // and scan, which do not touch them, so the waves' skew is absorbed there)
      if constexpr (ACC) barrier_lds();
      reload();
      {
        float hh0 = hin0, hh1 = hin1;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          const float4 y0 = sC0[q * 64 + lane], y1 = sC1[q * 64 + lane];
          const float c0[4] = {y0.x, y0.y, y0.z, y0.w}, c1[4] = {y1.x, y1.y, y1.z, y1.w};
          float t0[4], t1[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int j = 4 * q + k;
            hh0 = __builtin_fmaf(av0[j], hh0, hv0[j]);   // hv: the input term, then the state
            hh1 = __builtin_fmaf(av1[j], hh1, hv1[j]);
            hv0[j] = hh0;
            hv1[j] = hh1;
            yt[j] = __builtin_fmaf(c0[k], hh0, yt[j]);
            yt[j] = __builtin_fmaf(c1[k], hh1, yt[j]);
            t0[k] = ts.g[j] * hh0;                     // dC terms
            t1[k] = ts.g[j] * hh1;
          }
          slot[kC0 * F4 + q * 64 + lane] = make_float4(t0[0], t0[1], t0[2], t0[3]);
          slot[kC1 * F4 + q * 64 + lane] = make_float4(t1[0], t1[1], t1[2], t1[3]);
        }
      }
      if constexpr (ACC) {
        barrier_lds();                               // every wave's dC terms are in its slot
        acc_sum(pp, 1);
      }
      // adjoint: reverse fold, reverse scan, reverse replay
      reload();
      float x0 = 0.0f, x1 = 0.0f;
#pragma unroll
      for (int q = Q - 1; q >= 0; --q) {
        const float4 y0 = sC0[q * 64 + lane], y1 = sC1[q * 64 + lane];
        const float c0[4] = {y0.x, y0.y, y0.z, y0.w}, c1[4] = {y1.x, y1.y, y1.z, y1.w};
#pragma unroll
        for (int k = 3; k >= 0; --k) {
          const int j = 4 * q + k;
          x0 = av0[j] * __builtin_fmaf(ts.g[j], c0[k], x0);
          x1 = av1[j] * __builtin_fmaf(ts.g[j], c1[k], x1);
        }
      }
      wave_rscan_pairs2(R0, x0, me0, R1, x1, me1);
      float mu0 = wave_shift_down(x0, me0), mu1 = wave_shift_down(x1, me1);
      float dal0 = 0.0f, dal1 = 0.0f;
      if constexpr (ACC) barrier_lds();              // every thread has added the dC terms
      reload();
#pragma unroll
      for (int q = Q - 1; q >= 0; --q) {
        const float4 x0v = sB0[q * 64 + lane], x1v = sB1[q * 64 + lane];
        const float4 y0 = sC0[q * 64 + lane], y1 = sC1[q * 64 + lane];
        const float b0[4] = {x0v.x, x0v.y, x0v.z, x0v.w}, b1[4] = {x1v.x, x1v.y, x1v.z, x1v.w};
        const float c0[4] = {y0.x, y0.y, y0.z, y0.w}, c1[4] = {y1.x, y1.y, y1.z, y1.w};
        float t0[4], t1[4];
#pragma unroll
        for (int k = 3; k >= 0; --k) {
          const int j = 4 * q + k;
          const float lam0 = __builtin_fmaf(ts.g[j], c0[k], mu0);
          const float lam1 = __builtin_fmaf(ts.g[j], c1[k], mu1);
          s1[j] = __builtin_fmaf(lam0, b0[k], s1[j]);
          s1[j] = __builtin_fmaf(lam1, b1[k], s1[j]);
          t0[k] = lam0 * ts.du[j];                     // dB terms
          t1[k] = lam1 * ts.du[j];
          mu0 = av0[j] * lam0;
          mu1 = av1[j] * lam1;
          const float e0 = mu0 * (j > 0 ? hv0[j - 1] : hin0);
          const float e1 = mu1 * (j > 0 ? hv1[j - 1] : hin1);
          s2[j] = __builtin_fmaf(e0, A0, s2[j]);
          s2[j] = __builtin_fmaf(e1, A1, s2[j]);
          dal0 = __builtin_fmaf(e0, ts.dl[j], dal0);
          dal1 = __builtin_fmaf(e1, ts.dl[j], dal1);
        }
        slot[kB0 * F4 + q * 64 + lane] = make_float4(t0[0], t0[1], t0[2], t0[3]);
        slot[kB1 * F4 + q * 64 + lane] = make_float4(t1[0], t1[1], t1[2], t1[3]);
      }
      if constexpr (SEQ) {
        // lane 0's adjoint after its first token is what this chunk sends to the one before
        const float o0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mu0), 0));
        const float o1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mu1), 0));
        mu_out_v = lane == n0 ? o0 : (lane == n1 ? o1 : mu_out_v);
      }
      const float dan0 = wave_sum(dal0), dan1 = wave_sum(dal1);
      dA_v = lane == n0 ? dan0 : (lane == n1 ? dan1 : dA_v);

      barrier_lds();                                 // every wave's terms are in its slot
      if constexpr (ACC) {
        acc_sum(pp, 0);
      } else {
        // the fixed-order sum over the waves' slots of the entries this thread owns
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
          const int x = threadIdx.x + k * kThreads;
          float4 sum = s_red[x];
#pragma unroll
          for (int ww = 1; ww < kW; ++ww) {
            const float4 v = s_red[ww * RED4 + x];
            sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
          }
          if (whole[k]) {
            sum.x += prev[k].x; sum.y += prev[k].y; sum.z += prev[k].z; sum.w += prev[k].w;
            *reinterpret_cast<float4*>(dst[k]) = sum;
          } else if (dst[k]) {
            int n, m;
            int64_t t;
            entry(pp, x, n, m, t);
            const float sv[4] = {sum.x, sum.y, sum.z, sum.w};
            for (int rr = 0; rr < 4; ++rr)
              if (t + rr < L) dst[k][rr] = (r > 0 ? dst[k][rr] : 0.0f) + sv[rr];
          }
        }
      }
    };
    for (int pp = 0; pp < NP / 2; ++pp) pair(pp);

    // per-token gradients
    float o_du[KPL], o_dd[KPL];
    float dDl = 0.0f, dbl = 0.0f;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      o_du[j] = __builtin_fmaf(dsk, ts.g[j], ts.dl[j] * s1[j]);
      const float dd = __builtin_fmaf(ts.u[j], s1[j], s2[j]) * ts.sg[j];   // (sg = 1 without the softplus)
      o_dd[j] = dd;
      dDl = __builtin_fmaf(ts.g[j], ts.u[j], dDl);
      dbl += tl + j < L ? dd : 0.0f;
    }
    const float dDs = wave_sum(dDl), dbs = wave_sum(dbl);
    if (valid) {
      store_tokens<ACT, KPL>(p.du, row, tl, L, vec, o_du);
      store_tokens<ACT, KPL>(p.ddelta, row, tl, L, vec, o_dd);
      if (p.dz) {
#pragma unroll
        for (int j = 0; j < KPL; ++j) o_du[j] = yt[j] * ts.dzf[j];
        store_tokens<ACT, KPL>(p.dz, row, tl, L, vec, o_du);
      }
      if (lane < N) g.P[soff + lane] = dA_v;
      if (lane0) {
        g.dDp[(b * g.nchunks + c) * D + d] = dDs;
        g.dbp[(b * g.nchunks + c) * D + d] = dbs;
      }
      if constexpr (SEQ) {
        // the adjoint sent to chunk c - 1 (read back by this lane for it), or past
        // the first token the gradient of the initial state
        if (lane < N) {
          if (c > 0)
            g.X[(b * D + d) * N + lane] = mu_out_v;
          else if (p.dh0)
            p.dh0[(b * D + d) * N + lane] = mu_out_v;
        }
      }
    }
  }
  if constexpr (ACC) {
    // the workgroup's sums, written once: float2 e of (pair pp, matrix m) holds
    // tokens t, t + 1 of state 2 pp + e / (2 F4) (the slot layout of the terms)
    for (int pp = 0; pp < NP / 2; ++pp) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int k = 0; k < RPT2; ++k) {
          const int e = threadIdx.x + k * kThreads;
          const int n = 2 * pp + e / (2 * F4);
          const int f2 = e % (2 * F4), sl = f2 >> 1;
          const int64_t t = t0 + static_cast<int64_t>(sl % 64) * KPL + 4 * (sl / 64) + 2 * (f2 & 1);
          if (n >= N || t >= L) continue;
          float* dp = part + (m * N + n) * L + t;
          const float2 v = s_acc[(pp * 2 + m) * H2 + e];
          if (t + 2 <= L && L % 2 == 0) {
            *reinterpret_cast<float2*>(dp) = v;
          } else {
            dp[0] = v.x;
            if (t + 1 < L) dp[1] = v.y;
          }
        }
      }
    }
  }
  }  // chunks (SEQ: from the last to the first)
}

// ---- 4. fixed-order sums and dtype conversion ---------------------------------------
__global__ void bwd_param_sums_kernel(BwdArgs p, BwdLayout g) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t D = p.D, DN = D * p.N, parts = p.batch * g.nchunks;
  if (i < DN) {
    p.dA[i] = ordered_sum(g.P + i, DN, parts);
  } else if (i < DN + D) {
    const int64_t d = i - DN;
    if (p.dD) p.dD[d] = ordered_sum(g.dDp + d, D, parts);
  } else if (i < DN + 2 * D) {
    const int64_t d = i - DN - D;
    if (p.dbias) p.dbias[d] = ordered_sum(g.dbp + d, D, parts);
  }
}

// dB, dC = the sum over channel slices (in slice order) of the per-slice partials
// ([slice][batch][matrix][N][L]), stored in the B/C layout [batch][L][N].
template <typename ACT>
__global__ void bwd_bc_out_kernel(BwdArgs p, BwdLayout g) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t L = p.L, NL = p.N * L, per = p.batch * 2 * NL;
  if (i >= per) return;
  const float s = ordered_sum(g.part + i, per, g.nslices);
  const int64_t b = i / (2 * NL), rem = i % (2 * NL);
  const int m = static_cast<int>(rem / NL);
  const int64_t n = (rem % NL) / L, t = rem % L;
  store_act<ACT>(m ? p.dC : p.dB, (b * L + t) * p.N + n, s);
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

// The token-sequential summary: N = 16 (512-token chunks) and the vector path.
// Returns the parts per chunk (1 or 4) that give enough waves to fill the chip, or 0
// for the chunked summary (measured thresholds).
int bwd_summary_tokseq_parts(const BwdArgs& a, const BwdLayout& g, bool vec) {
  if (a.N != 16 || g.kpl != 8 || !vec) return 0;
  const int64_t waves = a.batch * g.nchunks * ((a.D + 15) / 16);
  if (waves >= kSumTokseqMinWaves) return 1;
  if (waves * kSumWaves >= kSumSplitMinWaves) return kSumWaves;
  return 0;
}

template <typename ACT, int KPL, int kW, int NT>
hipError_t launch_bwd_typed(const BwdArgs& a, const BwdLayout& g, hipStream_t s) {
  const bool vec = (a.L % 8 == 0) && aligned16(a.u) && aligned16(a.delta) && aligned16(a.dy) &&
                   (a.z == nullptr || aligned16(a.z)) && aligned16(a.du) && aligned16(a.ddelta) &&
                   (a.dz == nullptr || aligned16(a.dz)) && aligned16(a.Bm) && aligned16(a.Cm);
  const int64_t blocks = a.batch * g.nchunks * g.nslices;
  const int parts = bwd_summary_tokseq_parts(a, g, vec);
  if (parts == 1) {
    const int64_t sblocks = a.batch * g.nchunks * ((a.D + 16 * kSumWaves - 1) / (16 * kSumWaves));
    if (a.z)
      hipLaunchKernelGGL((bwd_summary_tokseq_kernel<ACT, true, 1>), dim3(static_cast<unsigned>(sblocks)),
                         dim3(64 * kSumWaves), 0, s, a, g);
    else
      hipLaunchKernelGGL((bwd_summary_tokseq_kernel<ACT, false, 1>), dim3(static_cast<unsigned>(sblocks)),
                         dim3(64 * kSumWaves), 0, s, a, g);
  } else if (parts == kSumWaves) {
    const int64_t sblocks = a.batch * g.nchunks * ((a.D + 15) / 16);
    if (a.z)
      hipLaunchKernelGGL((bwd_summary_tokseq_kernel<ACT, true, kSumWaves>), dim3(static_cast<unsigned>(sblocks)),
                         dim3(64 * kSumWaves), 0, s, a, g);
    else
      hipLaunchKernelGGL((bwd_summary_tokseq_kernel<ACT, false, kSumWaves>), dim3(static_cast<unsigned>(sblocks)),
                         dim3(64 * kSumWaves), 0, s, a, g);
  } else {
    hipLaunchKernelGGL((bwd_summary_kernel<ACT, KPL, kW, NT>), dim3(static_cast<unsigned>(blocks)), dim3(64 * kW), 0,
                       s, a, g, vec ? 1 : 0);
  }
  const int64_t nc = a.batch * a.D * a.N;
  hipLaunchKernelGGL(bwd_combine_kernel, dim3(static_cast<unsigned>((nc + 255) / 256)), dim3(256), 0, s, a, g);
  hipLaunchKernelGGL((bwd_main_kernel<ACT, KPL, kW, NT>), dim3(static_cast<unsigned>(blocks)), dim3(64 * kW), 0,
                     s, a, g, vec ? 1 : 0);
  const int64_t np = a.D * a.N + 2 * a.D;
  hipLaunchKernelGGL(bwd_param_sums_kernel, dim3(static_cast<unsigned>((np + 255) / 256)), dim3(256), 0, s, a, g);
  const int64_t nbc = a.batch * 2 * a.N * a.L;
  hipLaunchKernelGGL((bwd_bc_out_kernel<ACT>), dim3(static_cast<unsigned>((nbc + 255) / 256)), dim3(256), 0, s, a,
                     g);
  return hipGetLastError();
}

template <typename ACT>
hipError_t launch_bwd_seq(const BwdArgs& a, const BwdLayout& g, hipStream_t s) {
  const bool vec = (a.L % 8 == 0) && aligned16(a.u) && aligned16(a.delta) && aligned16(a.dy) &&
                   (a.z == nullptr || aligned16(a.z)) && aligned16(a.du) && aligned16(a.ddelta) &&
                   (a.dz == nullptr || aligned16(a.dz)) && aligned16(a.Bm) && aligned16(a.Cm);
  const int64_t blocks = a.batch * g.nslices;
  hipLaunchKernelGGL((bwd_main_kernel<ACT, 8, kWFast, kNMaxFast, true>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * kWFast), 0, s, a, g, vec ? 1 : 0);
  const int64_t np = a.D * a.N + 2 * a.D;
  hipLaunchKernelGGL(bwd_param_sums_kernel, dim3(static_cast<unsigned>((np + 255) / 256)), dim3(256), 0, s, a, g);
  const int64_t nbc = a.batch * 2 * a.N * a.L;
  hipLaunchKernelGGL((bwd_bc_out_kernel<ACT>), dim3(static_cast<unsigned>((nbc + 255) / 256)), dim3(256), 0, s, a,
                     g);
  return hipGetLastError();
}

template <typename ACT>
hipError_t launch_bwd_act(const BwdArgs& a, const BwdLayout& g, hipStream_t s) {
  if (bwd_fast(a.N)) return launch_bwd_typed<ACT, 8, kWFast, kNMaxFast>(a, g, s);
  return launch_bwd_typed<ACT, 4, kWGen, kNMaxGen>(a, g, s);
}

}  // namespace

size_t scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t D, int N, bool saved) {
  if (batch <= 0 || L <= 0 || D <= 0) return 0;
  if (saved && bwd_seq_suits(batch, D, N)) return bwd_seq_ws_floats(batch, L, D, N) * sizeof(float);
  return bwd_ws_floats(batch, L, D, N) * sizeof(float);
}

bool scan_bwd_grid_ok(int64_t batch, int64_t L, int64_t D, int N) {
  if (batch <= 0 || L <= 0 || D <= 0) return true;
  const BwdLayout g = bwd_layout(batch, L, D, N, nullptr);
  return batch * g.nchunks * g.nslices <= 0x7fffffff && batch * 2 * N * L / 256 < 0x7fffffff &&
         batch * D * N / 256 < 0x7fffffff;
}

hipError_t launch_scan_bwd(const BwdArgs& a, Dt dt, void* ws, hipStream_t s) {
  if (a.chunk_states && bwd_seq_suits(a.batch, a.D, a.N)) {
    const BwdLayout g = bwd_layout_seq(a.batch, a.L, a.D, a.N, static_cast<float*>(ws));
    if (dt == Dt::F32) return launch_bwd_seq<ActF32>(a, g, s);
    return launch_bwd_seq<ActBF16>(a, g, s);
  }
  const BwdLayout g = bwd_layout(a.batch, a.L, a.D, a.N, static_cast<float*>(ws));
  if (dt == Dt::F32) return launch_bwd_act<ActF32>(a, g, s);
  return launch_bwd_act<ActBF16>(a, g, s);
}

}  // namespace ssm
