// Chunked selective scan for gfx950.
//
// The recurrence h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t u_t is a linear
// recurrence, so it can be evaluated as a prefix scan over (decay, input) pairs
// under the associative operator (a1, b1) then (a2, b2) = (a2 a1, a2 b1 + b2)
// (the slide deck's "Parallel scan" section; the lecture notes' §4.1).  The
// kernel is fused end to end, as the pages' hardware-aware scan is: every input
// is read from HBM once, the (L, D, N) states never leave registers, and only y
// and the final state are written.
//
// Work decomposition (one wave = one (batch b, channel d) pair):
//   * a chunk is 64 * KPL consecutive tokens; lane i owns tokens [i*KPL, (i+1)*KPL)
//     of it, so u / delta / z / y move as coalesced 16-byte vectors along L;
//   * per token, once for all N states: Delta = softplus(delta + bias), Delta*u,
//     the skip term D*u and, at the end, the SiLU(z) gate;
//   * per state n (A[d, n] is wave-uniform and comes from lane n of a register):
//       pass 1  each lane folds its KPL tokens sequentially into a local end state
//               (lane 0 starts from the carry of the previous chunk) and keeps the
//               per-token decay a_j and input b_j in registers; the lane's
//               aggregate decay is one exp2 of A * (sum of its Deltas);
//       scan    a 64-lane inclusive DPP scan of (aggregate decay, end state) pairs
//               turns each lane's end state into the true state;
//       pass 2  each lane replays its KPL tokens from the true state of the lane
//               before it and accumulates y_t += C_t,n h_t,n;
//     the carry for the next chunk is lane 63's end state.
//
// Data movement (kW waves = kW channels of one batch row per workgroup):
//   * B and C are shared by all channels of a row and stored [batch][L][N] (the
//     pages' order), so a token's states are one contiguous run.  Each step of the
//     kernel covers kNB states of one chunk: the workgroup loads the next step's
//     B/C tile into registers (one 16-byte vector of kNB states per token and
//     matrix; the L2 serves the other steps' states of the same lines) while it
//     computes on the current one, and at the end of the step writes it, as
//     float32 and permuted into the order the lanes read it, to the other of two
//     LDS buffers; one barrier per step publishes it;
//   * a wave loads its next chunk's u and delta and this chunk's z into registers
//     during the current chunk, each as early as its registers are free, and stores
//     the previous chunk's y at its first step.  The barriers order LDS only; a load
//     is waited for where its value is first used.
// No MFMA: the readout is a per-token dot product over n, not a shared-operand
// contraction.  The kernel is bound by HBM bandwidth and by the VALU and
// transcendental rate (one exp per element).
#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_common.hpp"

namespace ssm {
namespace {

constexpr int kNBGeneric = 4;        // states per step (per staged B/C tile), any N
constexpr int64_t kSplitMaxChannels = 10 * 256;   // the split build: one 10-channel workgroup per CU

// ---- the scan ----------------------------------------------------------------
// kNB states per step.  NBLK > 0: N == kNB * NBLK, fixed at compile time; the steps of a chunk are
// unrolled, the last chunk is peeled, and the per-state values sit in scalar
// registers.  The steady state then has no branch around any load, so the
// compiler's tracking of outstanding loads stays exact and it never waits for a
// load before its value is needed.  NBLK = 0: any N, steps in a runtime loop.
//
// ZOH: the full zero-order-hold input term (e^{Delta A} - 1)/A * B * u instead of
// Delta * B * u: u * B times zoh_factor (about six VALU operations more per element
// than the simplified term; 1/A is per state, computed once per channel).
//
// AP: the build with the arithmetic-progression decay path (scan_two), used when the
// caller allows it (SSM_SCAN_AP); rows that are not such progressions still take
// the general path in it.  A separate build so that the default one keeps its
// registers and schedule.
//
// SAVE: the build that also writes the saved chunk states (p.chunk_states), for the
// backward pass; 8 tokens per lane, so a chunk is one 512-token saved entry.  A
// separate build, so that the default ones keep their registers.
//
// SPLIT: a workgroup of kW waves owns kW - 2 channels.  Waves 0 .. kW-5 run one
// channel each; the last four run two channels, two waves per channel, each wave
// taking half of every step's states (the first wave states n0 .. n0+3 of the
// step, the second n0+4 .. n0+7).  The states of a channel are independent until
// the readout sums over them, so the second wave adds its partial readout to the
// first one's through LDS once per chunk, and the first wave applies the gate and
// stores y.  With one workgroup per CU and waves dealt to the four SIMDs in turn,
// every SIMD holds two whole channels and one half: at 10 channels per CU (2560
// channels on 256 CUs) that is 2.5 channels' work per SIMD where 12-channel groups
// put 3 on some SIMDs and leave CUs idle.  (A split channel's readout is summed as
// two halves, so its y can differ from a whole channel's in the last bit: results
// are deterministic, but a channel's rounding depends on its slot in the group.)
template <typename ACT, bool GATE, int KPL, bool VEC, int NBLK, int kNB, int kW, bool CONV, bool ZOH, bool AP = false,
          bool SAVE = false, bool SPLIT = false>
__global__ __launch_bounds__(64 * kW) void scan_chunked_kernel(ScanArgs p, int n_dblk) {
  constexpr int kThreads = 64 * kW;
  static_assert(KPL >= 3, "the fused conv takes its 3 earlier tokens from the previous lane");
  // states processed two at a time where the registers allow it (8 or 12 tokens per lane)
  constexpr bool PAIR = KPL <= 12;
  // The arithmetic-progression build exists for bfloat16 12-wave N == 16 vector-load
  // kernels only: its running powers take about 40 more registers, which the
  // one-workgroup-per-CU 12-wave launch has to spare; in the 8- and 16-wave groups,
  // the scalar-load kernels and float32 they would cost occupancy or spill.
  constexpr bool kAP = AP;
  static_assert(!AP || (ACT::kBytes == 2 && kW == 12 && VEC && NBLK > 0 && PAIR && !ZOH && !CONV),
                "no arithmetic-progression build for this configuration");
  static_assert(!SPLIT || (kW == 12 && (KPL == 12 || KPL == 8) && VEC && NBLK > 0 && kNB == 8 && PAIR && !SAVE &&
                          !ZOH && !CONV),
                "no split build for this configuration");
  using IO = TokenIO<ACT, KPL>;
  using raw_t = typename IO::raw_t;
  constexpr int CH = 64 * KPL;
  constexpr int BLK4 = CH / 4;                       // float4 per (state, matrix) block
  // ROWS (float32, N == 16, vector path, 8 tokens per lane): B and C are staged a
  // whole chunk at a time, all 16 states of a token together (each B/C line is
  // fetched once per chunk); otherwise one step's kNB states at a time.
  constexpr bool ROWS = ACT::kBytes == 4 && VEC && NBLK > 0 && kNB * NBLK == 16 && KPL == 8;
  constexpr int TILE4 = (ROWS ? 16 : kNB) * 2 * BLK4;  // float4 per LDS buffer
  __shared__ float4 s_tile[2][TILE4];
  // SPLIT: the second wave's partial readout of the last chunk, per split channel
  __shared__ float4 s_y[SPLIT ? 2 * 16 * KPL : 1];

  const int lane = threadIdx.x & 63;
  const bool lane0 = lane == 0;
  const int w = uniform_int(threadIdx.x >> 6);
  // Consecutive workgroups go to different XCDs (round robin over 8); taking the
  // batch row as blk % batch keeps one row per XCD when batch divides 8, so each
  // XCD's L2 holds only that row's B and C.
  const int blk = blockIdx.x;
  const int64_t b = blk % p.batch;
  constexpr int kChan = SPLIT ? kW - 2 : kW;          // channels per workgroup
  constexpr int kWhole = SPLIT ? kW - 4 : kW;         // waves that run a whole channel
  const bool split = SPLIT && w >= kWhole;            // wave-uniform
  const int half = split ? ((w - kWhole) & 1) : 0;    // 1: the second half of each step's states
  const int64_t d_own = static_cast<int64_t>(blk / p.batch) * kChan + (split ? kWhole + (w - kWhole) / 2 : w);
  const bool valid = d_own < p.D;                    // wave-uniform
  // A wave past the last channel runs the same code on the last channel (so no
  // branch depends on it) and stores nothing.
  const int64_t d = valid ? d_own : p.D - 1;
  const int N = p.N;
  const int64_t L = p.L;
  const int64_t row = (b * p.D + d) * L;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  // (SPLIT: the skip term is added once, by the first wave of a channel)
  const float dsk = (p.Dskip && !(SPLIT && half)) ? p.Dskip[d] : 0.0f;
  // A[d, n] * log2(e) in lane n (read once, so the state loop never issues a
  // vector load of A).
  const float a2_v = lane < N ? p.A[d * N + lane] * kLog2e : 0.0f;
  // 1/A[d, n] in lane n (full zero-order hold only; inf at A == 0, never selected
  // there by zoh_factor)
  const float ra_v = (ZOH && lane < N) ? 1.0f / p.A[d * N + lane] : 0.0f;
  // carry of state n lives in lane n; it starts as the initial state (zero if none)
  float carry_v = (lane < N && p.h0) ? p.h0[(b * p.D + d) * N + lane] : 0.0f;
  // AP build: is this channel's A row a non-increasing arithmetic progression,
  // A[d, n] == A[d, 0] + n b exactly with b <= 0 (wave-uniform)?  Then its decays
  // come from multiply chains (scan_two).  With b <= 0 the ratio exp(Delta b) is at
  // most 1, so a chain neither overflows nor loses a value the direct exp would keep
  // (when exp(Delta A[n0]) underflows, the later states' decays are smaller still).
  bool ap_row = false;
  float ap_b2 = 0.0f;
  if constexpr (kAP) {
    const float a_v = lane < N ? p.A[d * N + lane] : 0.0f;
    const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a_v), 0));
    const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a_v), 1));
    const float bstep = a1 - a0;
    const bool off = lane < N && __builtin_fmaf(static_cast<float>(lane), bstep, a0) != a_v;
    ap_row = bstep <= 0.0f && __ballot(off) == 0;
    ap_b2 = bstep * kLog2e;
  }

  const int nblk = NBLK > 0 ? NBLK : (N + kNB - 1) / kNB;
  const int64_t nchunks = (L + CH - 1) / CH;
  // Saved chunk states (8 tokens per lane: a chunk is one 512-token saved entry):
  // entry c is the state entering chunk c; entry 0 is the initial state.
  static_assert(!SAVE || (CH == kSaveChunk && !AP), "the saving build has 512-token chunks");
  float* cst = nullptr;
  if constexpr (SAVE) {
    if (valid) cst = p.chunk_states + (b * p.D + d) * nchunks * N;
    if (cst && lane < N) cst[lane] = carry_v;
  }
  const int64_t nsteps = nchunks * nblk;

  float dl[KPL], du[KPL], yv[KPL];
  float sdl = 0.0f;
  // Fused causal conv1d + SiLU on the input (CONV): per-channel taps aligned to
  // the window x[t-3 .. t] (cw4[4-K+k] = w[d,k], the rest zero) and the last
  // three inputs of the previous chunk (zero before the sequence starts).
  float cw4[4] = {0.f, 0.f, 0.f, 0.f}, cbias = 0.0f, cvc[3] = {0.f, 0.f, 0.f};
  if constexpr (CONV) {
#pragma unroll
    for (int k = 0; k < 4; ++k) cw4[k] = (k >= 4 - p.conv_k) ? p.conv_w[d * p.conv_k + k - (4 - p.conv_k)] : 0.0f;
    cbias = p.conv_b ? p.conv_b[d] : 0.0f;
  }
  int nv = KPL;                                      // valid tokens of this lane in its chunk
  raw_t u_raw[IO::kVec], d_raw[IO::kVec];            // next chunk's u and delta
  raw_t z_raw[IO::kVec];                             // this chunk's z

  // Vector path: load this lane's KPL values of chunk c.  The start is clamped
  // into the row (the vector path needs L >= KPL), so a lane past the end loads
  // real data that it never uses and the load needs no branch.
  auto prefetch_act = [&](const void* src, int64_t c, raw_t (&dst)[IO::kVec]) __attribute__((always_inline)) {
    if constexpr (VEC) {
      int64_t tl = c * CH + static_cast<int64_t>(lane) * KPL;
      tl = tl + KPL <= L ? tl : L - KPL;
      IO::load_raw(src, row + tl, dst);
    }
  };

  // Per-token work of chunk c, once for all N states.
  auto prologue = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t tl = c * CH + static_cast<int64_t>(lane) * KPL;
    const int64_t rem = L - tl;
    nv = rem >= KPL ? KPL : (rem > 0 ? static_cast<int>(rem) : 0);
    float uv[KPL];
    if (VEC && nv == KPL) {
      IO::unpack(u_raw, uv);
      IO::unpack(d_raw, dl);
    } else if (CONV && VEC && KPL == 8) {
      // The vector path has L % 8 == 0, so at 8 tokens per lane a lane's tokens
      // are all in the row or all past it: this lane is past the end.  (With the
      // fused conv, element loads here, merged with the vector path, made the
      // compiler keep the prefetched vectors in scratch memory.)
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        uv[j] = 0.0f;
        dl[j] = 0.0f;
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const bool ok = j < nv;
        uv[j] = ok ? load_act<ACT>(p.u, row + tl + j) : 0.0f;
        dl[j] = ok ? load_act<ACT>(p.delta, row + tl + j) : 0.0f;
      }
    }
    if constexpr (CONV) {
      // uv holds x: u = SiLU(conv(x)).  The 3 inputs before this lane's first
      // token are the previous lane's last three (lane 0: the previous chunk's).
      // A sliding window of three scalars (an indexed window array was left in
      // scratch memory by the compiler); taps applied oldest first.
      float xm3 = wave_shift_up(uv[KPL - 3], cvc[0]);
      float xm2 = wave_shift_up(uv[KPL - 2], cvc[1]);
      float xm1 = wave_shift_up(uv[KPL - 1], cvc[2]);
#pragma unroll
      for (int k = 0; k < 3; ++k) cvc[k] = wave_lane63(uv[KPL - 3 + k]);
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const float x0 = uv[j];
        float sc = __builtin_fmaf(cw4[0], xm3, cbias);
        sc = __builtin_fmaf(cw4[1], xm2, sc);
        sc = __builtin_fmaf(cw4[2], xm1, sc);
        sc = __builtin_fmaf(cw4[3], x0, sc);
        xm3 = xm2;
        xm2 = xm1;
        xm1 = x0;
        uv[j] = sc * __builtin_amdgcn_rcpf(1.0f + exp2_hw(-sc * kLog2e));
      }
      if (p.u_out && valid) {
        if (VEC && nv == KPL) {
          IO::store(p.u_out, row + tl, uv);
        } else {
#pragma unroll
          for (int j = 0; j < KPL; ++j)
            if (j < nv) store_act<ACT>(p.u_out, row + tl + j, uv[j]);
        }
      }
    }
    if (p.softplus) {
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        dl[j] = ACT::kBytes == 2 ? softplus_bf16act(dl[j] + bias) : softplus_f(dl[j] + bias);
    } else {
#pragma unroll
      for (int j = 0; j < KPL; ++j) dl[j] = dl[j] + bias;
    }
    if (nv < KPL) {                                  // padding tokens: identity step
#pragma unroll
      for (int j = 0; j < KPL; ++j) dl[j] = j < nv ? dl[j] : 0.0f;
    }
    sdl = 0.0f;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      du[j] = ZOH ? uv[j] : dl[j] * uv[j];              // (ZOH: u itself; the term needs e^{Delta A} first)
      yv[j] = dsk * uv[j];
      sdl += dl[j];
    }
  };

  auto epilogue = [&](int64_t c) __attribute__((always_inline)) {
    if constexpr (SPLIT) {
      if (half) return;                              // its partial readout went to LDS
      if (split) {                                   // add the second wave's partial
        const float4* src = s_y + ((w - kWhole) / 2) * 16 * KPL;
#pragma unroll
        for (int q = 0; q < KPL / 4; ++q) {
          const float4 v = src[q * 64 + lane];
          yv[4 * q] += v.x;
          yv[4 * q + 1] += v.y;
          yv[4 * q + 2] += v.z;
          yv[4 * q + 3] += v.w;
        }
      }
    }
    const int64_t tl = c * CH + static_cast<int64_t>(lane) * KPL;
    if (GATE) {
      float zv[KPL];
      if (VEC && nv == KPL) {
        IO::unpack(z_raw, zv);
      } else if (CONV && VEC && KPL == 8) {         // past the end (as in the prologue)
#pragma unroll
        for (int j = 0; j < KPL; ++j) zv[j] = 0.0f;
      } else {
#pragma unroll
        for (int j = 0; j < KPL; ++j) zv[j] = j < nv ? load_act<ACT>(p.z, row + tl + j) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < KPL; ++j) yv[j] *= silu_f(zv[j]);
    }
    if (valid) {
      if (VEC && nv == KPL) {
        IO::store(p.y, row + tl, yv);
      } else {
#pragma unroll
        for (int j = 0; j < KPL; ++j)
          if (j < nv) store_act<ACT>(p.y, row + tl + j, yv[j]);
      }
    }
  };

  // Input term of token j for a state with B value bj, decay avj = 2^yj and 1/A = ra.
  auto input_term = [&](float avj, float yj, int j, float bj, float ra) __attribute__((always_inline)) -> float {
    if constexpr (ZOH) {
      return (du[j] * bj) * zoh_factor(yj, avj, ra, dl[j]);
    } else {
      return du[j] * bj;
    }
  };

  // One state over the current chunk: its B and C blocks are sB, sC in LDS,
  // a2 = A[d, n] * log2(e) and `carry` (the state before the chunk) are
  // wave-uniform.  Returns the state after the chunk (lane 63's).
  auto scan_one = [&](const float4* __restrict__ sB, const float4* __restrict__ sC, float a2, float ra,
                      float carry) __attribute__((always_inline)) -> float {
    float av[KPL], bv[KPL];
    float h = lane0 ? carry : 0.0f;
#pragma unroll
    for (int q = 0; q < KPL / 4; ++q) {
      const float4 bb = sB[q * 64 + lane];
      const float bs[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * q + r;
        const float yj = dl[j] * a2;
        av[j] = exp2_hw(yj);
        bv[j] = input_term(av[j], yj, j, bs[r], ra);
        h = __builtin_fmaf(av[j], h, bv[j]);
      }
    }
    float P = exp2_hw(a2 * sdl);                     // this lane's decay over its tokens
    wave_scan_pairs(P, h);                           // h: true state after this lane
    const float hin = wave_shift_up(h, carry);       // true state before this lane
    const float cnew = wave_lane63(h);
    float hh = hin;
#pragma unroll
    for (int q = 0; q < KPL / 4; ++q) {
      const float4 cc = sC[q * 64 + lane];
      const float cs[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * q + r;
        hh = __builtin_fmaf(av[j], hh, bv[j]);
        yv[j] = __builtin_fmaf(cs[r], hh, yv[j]);
      }
    }
    return cnew;
  };

  // Two states at once, interleaved instruction by instruction: two independent
  // dependency chains in every phase, and one DPP scan sequence with no wait states.
  //
  // `apm` (a compile-time tag) selects where the decays come from.  General: one
  // exp2 per token and state.  Arithmetic-progression rows (A[d, n] = A[d, 0] + n b,
  // the S4D-real and HiPPO-style rows of the pages): exp(Delta A[n+1]) =
  // exp(Delta A[n]) exp(Delta b), so the caller passes the running powers `apc` (the
  // decays of the pair's first state), the step ratios `apr` = exp(Delta b) per token,
  // and the lane's aggregate decay and its ratio; this pair takes two multiplies per
  // token instead of two exponentials, and advances the powers by two states.
  auto scan_two = [&](auto apm, const float4* __restrict__ sB0, const float4* __restrict__ sC0, float a20,
                      float ra0, float carry0, const float4* __restrict__ sB1, const float4* __restrict__ sC1,
                      float a21, float ra1, float carry1, float& out0, float& out1, float (&apc)[KPL],
                      const float (&apr)[KPL], float& apP, float apR) __attribute__((always_inline)) {
    constexpr bool APM = decltype(apm)::value;
    float av0[KPL], bv0[KPL], av1[KPL], bv1[KPL];
    float h0 = lane0 ? carry0 : 0.0f;
    float h1 = lane0 ? carry1 : 0.0f;
#pragma unroll
    for (int q = 0; q < KPL / 4; ++q) {
      const float4 b0 = sB0[q * 64 + lane];
      const float4 b1 = sB1[q * 64 + lane];
      const float bs0[4] = {b0.x, b0.y, b0.z, b0.w};
      const float bs1[4] = {b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * q + r;
        float y0 = 0.0f, y1 = 0.0f;
        if constexpr (APM) {
          av0[j] = apc[j];
          av1[j] = apc[j] * apr[j];
          apc[j] = av1[j] * apr[j];
        } else {
          y0 = dl[j] * a20;
          y1 = dl[j] * a21;
          av0[j] = exp2_hw(y0);
          av1[j] = exp2_hw(y1);
        }
        bv0[j] = input_term(av0[j], y0, j, bs0[r], ra0);
        bv1[j] = input_term(av1[j], y1, j, bs1[r], ra1);
        h0 = __builtin_fmaf(av0[j], h0, bv0[j]);
        h1 = __builtin_fmaf(av1[j], h1, bv1[j]);
      }
    }
    float P0, P1;
    if constexpr (APM) {
      P0 = apP;
      P1 = apP * apR;
      apP = P1 * apR;
    } else {
      P0 = exp2_hw(a20 * sdl);
      P1 = exp2_hw(a21 * sdl);
    }
    wave_scan_pairs2(P0, h0, P1, h1);
    float hh0 = wave_shift_up(h0, carry0);
    float hh1 = wave_shift_up(h1, carry1);
    out0 = wave_lane63(h0);
    out1 = wave_lane63(h1);
#pragma unroll
    for (int q = 0; q < KPL / 4; ++q) {
      const float4 c0 = sC0[q * 64 + lane];
      const float4 c1 = sC1[q * 64 + lane];
      const float cs0[4] = {c0.x, c0.y, c0.z, c0.w};
      const float cs1[4] = {c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * q + r;
        hh0 = __builtin_fmaf(av0[j], hh0, bv0[j]);
        hh1 = __builtin_fmaf(av1[j], hh1, bv1[j]);
        yv[j] = __builtin_fmaf(cs0[r], hh0, yv[j]);
        yv[j] = __builtin_fmaf(cs1[r], hh1, yv[j]);
      }
    }
  };

  // Generic state loop: A*log2(e) and the carry of state n live in lane n of a
  // register and are read with readlane.
  auto scan_state = [&](const float4* sB, const float4* sC, int n) __attribute__((always_inline)) {
    const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a2_v), n));
    const float carry = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, carry_v), n));
    const float ra = ZOH ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ra_v), n)) : 0.0f;
    const float cnew = scan_one(sB, sC, a2, ra, carry);
    carry_v = (lane == n) ? cnew : carry_v;
  };

  // Tile of step k = (chunk c = k / nblk, states n0 = (k % nblk) * kNB ...): B and C
  // are [batch][L][N], so one token's nn = min(kNB, N - n0) states of the step are
  // contiguous in memory.  A tile element is (matrix m, token tk of the chunk): one
  // 16-byte vector (4 float32 or 8 bfloat16 states) when N == 16 on the vector path,
  // else element loads.  Element e = m * CH + tk; a wave's 64 elements share m.
  // In LDS the tile is float32 blocks (2 * state + matrix) of the chunk's CH tokens:
  // float4 f of a block holds tokens 4f .. 4f+3 and sits at the slot lane f / (KPL/4)
  // reads as its vector f % (KPL/4), so the state loop's LDS reads are contiguous.
  // store_tile scatters each element's states into their blocks.
  //
  // Pipeline: tile j is loaded into register set j % 2 during step j - 2 and
  // written (as float32, permuted) to LDS buffer j % 2 at the end of step j - 1,
  // so each load has a whole step to arrive before its value is needed.
  //
  // ROWS: tile j is instead piece s of chunk cc, j = cc * NBLK + s + 1 - NBLK: the
  // PIECE = CH / NBLK tokens from s * PIECE, all 16 states, element e = m * CH +
  // g * PIECE + tq holding states 4g .. 4g+3 of token tq of the piece (a wave's
  // elements share m and g, and its loads hit the L1 lines the other groups' waves
  // fetch).  Piece s of chunk cc is written to LDS buffer cc % 2 at the end of step
  // (cc - 1) * NBLK + s: after chunk cc - 2 has finished with that buffer, and the
  // whole chunk is in place by the barrier that ends chunk cc - 1.
  using SR = StateRun<ACT, kNB>;
  using traw_t = typename SR::raw_t;
  constexpr int TILER = 2 * CH;                              // elements per tile
  constexpr int TPT = (TILER + kThreads - 1) / kThreads;     // elements per thread
  static_assert(TPT <= 3, "tile share per thread held in three registers");
  static_assert(CH % 64 == 0, "a wave's tile elements share one matrix");
  // vector loads of a token's states: N == 16 (compile-time) on the aligned path
  constexpr bool BCVEC = VEC && NBLK > 0 && kNB * NBLK == 16;
  traw_t tr[2][TPT];
  int tile_nn[2] = {0, 0};                                   // states in each staged tile
  int tile_pc[2] = {0, 0};                                   // ROWS: piece | chunk parity << 8
  const int64_t bc_row = b * L * N;                          // this batch row of B and C
  constexpr int PIECE = ROWS ? CH / NBLK : CH;
  static_assert(!ROWS || PIECE % 64 == 0, "a wave's piece elements share one state group");
  auto load_rows = [&](int64_t j, int set) __attribute__((always_inline)) {
    int64_t cc = (j - 1 + NBLK) / NBLK;
    const int sp = static_cast<int>((j - 1 + NBLK) % NBLK);
    cc = cc < nchunks ? cc : nchunks - 1;                   // past the last chunk: never stored
    tile_pc[set] = sp | static_cast<int>((cc & 1) << 8);
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      int eb = w * 64 + i * kThreads;
      eb = eb < TILER ? eb : TILER - 64;
      const void* src = (eb / CH) ? p.Cm : p.Bm;
      const int g = (eb % CH) / PIECE;
      int64_t t = cc * CH + sp * PIECE + (eb % PIECE) + lane;
      t = t < L ? t : L - 1;                                 // padding tokens: identity steps (Delta = 0)
      tr[set][i] = SR::load_vec(src, bc_row + t * N + 4 * g);
    }
  };
  auto store_rows = [&](int set) __attribute__((always_inline)) {
    float* dst = reinterpret_cast<float*>(s_tile[tile_pc[set] >> 8]);
    const int sp = tile_pc[set] & 0xff;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int eb = w * 64 + i * kThreads;
      if (eb < TILER) {
        const int m = eb / CH, g = (eb % CH) / PIECE, tk = sp * PIECE + eb % PIECE + lane, f = tk >> 2;
        const int slot = ((f % (KPL / 4)) * 64 + f / (KPL / 4)) * 4 + (tk & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[(2 * (4 * g + j) + m) * (4 * BLK4) + slot] = SR::get(tr[set][i], j);
      }
    }
  };
  auto load_tile = [&](int64_t k, int set) __attribute__((always_inline)) {
    if constexpr (ROWS) {
      load_rows(k, set);
      return;
    }
    const int64_t c = k / nblk;
    const int n0 = static_cast<int>(k % nblk) * kNB;
    const int nn = NBLK > 0 ? kNB : ((N - n0 < kNB) ? (N - n0) : kNB);
    tile_nn[set] = nn;
    const int64_t tok0 = c * CH;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      // this wave's first element, clamped into the tile (the surplus is never stored)
      int eb = w * 64 + i * kThreads;
      eb = eb < TILER ? eb : TILER - 64;
      const void* src = (eb / CH) ? p.Cm : p.Bm;
      // Unconditional load, clamped into the row: a token past L reloads the row's
      // last token.  Those padding tokens have Delta = 0, so they are identity steps
      // whatever finite B and C they see, and their y is never stored.
      int64_t t = tok0 + (eb % CH) + lane;
      t = t < L ? t : L - 1;
      const int64_t off = bc_row + t * N + n0;
      if constexpr (BCVEC) {
        tr[set][i] = SR::load_vec(src, off);
      } else {
        tr[set][i] = SR::load_elems(src, off, nn);
      }
    }
  };
  auto store_tile = [&](int set) __attribute__((always_inline)) {
    if constexpr (ROWS) {
      store_rows(set);
      return;
    }
    float* dst = reinterpret_cast<float*>(s_tile[set]);
    const int nn = tile_nn[set];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int eb = w * 64 + i * kThreads;
      if (eb < TILER) {
        const int m = eb / CH, tk = eb % CH + lane, f = tk >> 2;
        const int slot = ((f % (KPL / 4)) * 64 + f / (KPL / 4)) * 4 + (tk & 3);
#pragma unroll
        for (int j = 0; j < kNB; ++j)
          if (NBLK > 0 || j < nn) dst[(2 * j + m) * (4 * BLK4) + slot] = SR::get(tr[set][i], j);
      }
    }
  };

  // A chunk's HBM traffic: at step 0 the previous chunk's y is stored and this chunk's
  // z loaded (its registers were just read by the previous chunk's epilogue, and it is
  // used by this chunk's, so it has the whole chunk to arrive).  The next chunk's u and
  // delta: with two steps per chunk (bfloat16, N = 16) at step 0 as well, right after
  // the prologue has read this chunk's, two steps before their use; with more steps
  // per chunk spread over steps 1 and 2.  Measured on the 131072-token bfloat16
  // workload (two steps): z at step 0 instead of the last step 1560 -> 1539 us, then
  // u and delta at step 0 instead of step 1 1534 -> 1517 us.  On the float32 130M
  // workload (four steps) z at step 0 measured the same, and u and delta at step 0
  // 5 % slower than at steps 1 and 2.
  const int st_u = nblk > 2 ? 1 : 0;
  const int st_d = nblk > 2 ? 2 : 0;
  const int st_z = 0;

  // Per-state wave-uniform values when the state count is fixed at compile time
  // (NBLK > 0): A*log2(e) and the carry of state n in scalar registers, indexed
  // by compile-time n once the steps are unrolled.
  constexpr int NS = NBLK > 0 ? kNB * NBLK : 1;
  float a2s[NS], cs[NS], ras[NS];
  // SPLIT: slot n (n % 8 < 4) of the second wave of a channel holds state n + 4.
  auto slot_state = [&](int n) __attribute__((always_inline)) -> int {
    return (SPLIT && (n % 8) < 4) ? n + 4 * half : n;
  };
  if constexpr (NBLK > 0) {
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      const int sn = slot_state(n);
      a2s[n] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a2_v), sn));
      ras[n] = ZOH ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ra_v), sn)) : 0.0f;
      cs[n] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, carry_v), sn));
    }
  }

  // The states of step nb of the current chunk, from the tile `cur`.
  auto states = [&](const float4* cur, int nb) __attribute__((always_inline)) {
    const int n0 = nb * kNB;
    if constexpr (NBLK > 0) {
      constexpr int nn = kNB;                          // N == kNB * NBLK: every step is full
      const float4* t = cur;
      if constexpr (PAIR) {
        float apc[KPL], apr[KPL], apP = 0.0f, apR = 0.0f;
        auto pairs = [&](auto apm) __attribute__((always_inline)) {
#pragma unroll
          for (int nl = 0; nl < nn; nl += 2) {
            // SPLIT: a split wave runs the step's first two pairs only, on the tile
            // `cur` offset by 4 half states, with its states' scalars in slots
            // n0 .. n0 + 3 (the second wave loaded them there)
            if constexpr (SPLIT) {
              if (nl >= nn / 2 && split) break;
            }
            const int n = n0 + nl;
            scan_two(apm, t + nl * 2 * BLK4, t + (nl * 2 + 1) * BLK4, a2s[n], ras[n], cs[n],
                     t + (nl * 2 + 2) * BLK4, t + (nl * 2 + 3) * BLK4, a2s[n + 1], ras[n + 1], cs[n + 1], cs[n],
                     cs[n + 1], apc, apr, apP, apR);
          }
        };
        if (kAP && ap_row) {
          // the step's first state exactly, then the chain over its kNB states (the
          // ratio recomputed per step: nothing extra stays live across steps)
#pragma unroll
          for (int j = 0; j < KPL; ++j) {
            apc[j] = exp2_hw(dl[j] * a2s[n0]);
            apr[j] = exp2_hw(dl[j] * ap_b2);
          }
          apP = exp2_hw(a2s[n0] * sdl);
          apR = exp2_hw(ap_b2 * sdl);
          pairs(std::true_type{});
        } else {
          pairs(std::false_type{});
        }
      } else {
#pragma unroll
        for (int nl = 0; nl < nn; ++nl) {
          const int n = n0 + nl;
          cs[n] = scan_one(t + nl * 2 * BLK4, t + (nl * 2 + 1) * BLK4, a2s[n], ras[n], cs[n]);
        }
      }
    } else {
      const int nn = (N - n0 < kNB) ? (N - n0) : kNB;
      for (int nl = 0; nl < nn; ++nl) scan_state(cur + nl * 2 * BLK4, cur + (nl * 2 + 1) * BLK4, n0 + nl);
    }
  };

  // Step k (state block nb of chunk c) computes on LDS buffer k % 2.  It loads
  // tile k + 2 into register set k % 2 (unless `tail`), prefetches the next
  // chunk's u and delta (unless `last_chunk`) and this chunk's z, and at its end
  // writes tile k + 1 (register set (k + 1) % 2) to LDS buffer (k + 1) % 2.
  auto step = [&](int64_t k, int64_t c, int nb, int par, bool last_chunk, bool tail2, bool tail1) __attribute__((always_inline)) {
    if (nb == 0) {
      if (c > 0) epilogue(c - 1);                    // z of c-1 loaded during chunk c-1
      prologue(c);                                   // u, delta of c prefetched during c-1
    }
    if (!tail2) load_tile(k + 2, par);
    if (!last_chunk && nb == st_u) prefetch_act(p.u, c + 1, u_raw);
    if (!last_chunk && nb == st_d) prefetch_act(p.delta, c + 1, d_raw);
    if (GATE && nb == st_z) prefetch_act(p.z, c, z_raw);
    // (a wave past the last channel skips the state loop; keeping the loop in
    // its own block also keeps the compiler from scheduling it into the
    // surrounding per-token code, which costs registers)
    if (valid) {
      if constexpr (ROWS) {
        states(s_tile[c & 1] + nb * kNB * 2 * BLK4, nb);
      } else if constexpr (2 * TILE4 * 16 > 65536) {
        // Buffers past the 64 KB reach of an LDS read's immediate offset (48 KB
        // each at 12 tokens per lane): the buffer's offset goes through a scalar
        // register the compiler cannot see into, so each step forms one base
        // address and every read of the tile is an immediate offset from it.  With
        // the constant folded in, every read of the second buffer's upper blocks
        // needed an address instruction of its own (32 VALU per step).  Where the
        // tiles fit in 64 KB the constant is better (measured 1.3 % slower
        // opaque).
        int toff = par * TILE4 + (SPLIT ? half * kNB * BLK4 : 0);   // (SPLIT: the second wave's states)
        asm volatile("" : "+s"(toff));
        states(&s_tile[0][0] + toff, nb);
      } else {
        states(s_tile[par] + (SPLIT ? half * kNB * BLK4 : 0), nb);   // (SPLIT: the second wave's states)
      }
    }
    if constexpr (SPLIT) {
      // the second wave's partial readout of this chunk, for the first wave's
      // epilogue after the barrier (which reads it before the next chunk's last step)
      if (half && nb == nblk - 1) {
        float4* dst = s_y + ((w - kWhole) / 2) * 16 * KPL;
#pragma unroll
        for (int q = 0; q < KPL / 4; ++q)
          dst[q * 64 + lane] = make_float4(yv[4 * q], yv[4 * q + 1], yv[4 * q + 2], yv[4 * q + 3]);
      }
    }
    if (!tail1) store_tile(par ^ 1);
    // ROWS: the steps of chunk c all read buffer c % 2, and the pieces of chunk c + 1
    // go to the other buffer, which chunk c - 1 finished reading before the barrier
    // that ended it.  So only the chunk's last step needs the barrier: it publishes
    // chunk c + 1 and frees buffer c % 2 for the pieces of chunk c + 2.  Otherwise each
    // step's tile is its own buffer, written during the step before: a barrier per step.
    if (!ROWS || nb == nblk - 1) barrier_lds();
  };

  prefetch_act(p.u, 0, u_raw);
  prefetch_act(p.delta, 0, d_raw);
  if constexpr (ROWS) {
    // the whole first chunk (tiles 1 - NBLK .. 0), then the next chunk's first piece
#pragma unroll
    for (int j = 1 - NBLK; j <= 0; ++j) {
      load_tile(j, 0);
      store_tile(0);
    }
    load_tile(1, 1);
  } else {
    load_tile(0, 0);
    if (nsteps > 1) load_tile(1, 1);
    store_tile(0);
  }
  barrier_lds();
  // the state entering chunk c (after the steps of chunk c - 1) to the saved entry c
  auto save_chunk = [&](int64_t c) __attribute__((always_inline)) {
    if constexpr (SAVE) {
      if (cst) {
        float v = carry_v;
        if constexpr (NBLK > 0) {
#pragma unroll
          for (int n = 0; n < NS; ++n) v = lane == n ? cs[n] : v;
        }
        if (lane < N) cst[c * N + lane] = v;
      }
    }
  };
  if constexpr (NBLK > 0) {
    static_assert(NBLK % 2 == 0, "steps are unrolled in pairs");
    for (int64_t c = 0; c + 1 < nchunks; ++c) {
      static_for<NBLK>([&](auto nbc) __attribute__((always_inline)) {
        constexpr int nb = decltype(nbc)::value;
        step(c * NBLK + nb, c, nb, nb & 1, false, false, false);
      });
      save_chunk(c + 1);
    }
    const int64_t c = nchunks - 1;
    static_for<NBLK>([&](auto nbc) __attribute__((always_inline)) {
      constexpr int nb = decltype(nbc)::value;
      const int64_t k = c * NBLK + nb;
      // (ROWS: the last chunk's steps would stage the chunk after it, which is none)
      step(k, c, nb, nb & 1, true, ROWS || k + 2 >= nsteps, ROWS || k + 1 >= nsteps);
    });
  } else {
    for (int64_t k = 0; k < nsteps; k += 2) {
      const int64_t c0 = k / nblk, c1 = (k + 1) / nblk;
      step(k, c0, static_cast<int>(k % nblk), 0, c0 + 1 >= nchunks, k + 2 >= nsteps, k + 1 >= nsteps);
      if constexpr (SAVE) {
        if ((k + 1) % nblk == 0 && c0 + 1 < nchunks) save_chunk(c0 + 1);
      }
      if (k + 1 < nsteps) {
        step(k + 1, c1, static_cast<int>((k + 1) % nblk), 1, c1 + 1 >= nchunks, k + 3 >= nsteps, k + 2 >= nsteps);
        if constexpr (SAVE) {
          if ((k + 2) % nblk == 0 && c1 + 1 < nchunks) save_chunk(c1 + 1);
        }
      }
    }
  }
  if constexpr (NBLK > 0) {
    // carries back into lane n for the final-state store (SPLIT: a split wave's
    // slots n % 8 < 4, holding states slot_state(n))
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      if (SPLIT && split && (n % 8) >= 4) continue;
      carry_v = lane == slot_state(n) ? cs[n] : carry_v;
    }
  }
  epilogue(nchunks - 1);
  // (SPLIT: each wave of a channel stores the states it ran, n % 8 < 4 the first)
  const bool own = !split || (((lane >> 2) & 1) == half);
  if (valid && p.final_state && lane < N && own) p.final_state[(b * p.D + d) * N + lane] = carry_v;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

// Vector path: 16-byte vectors of u, delta, z, y (and the fused conv's u_out) along
// L (L % 8 == 0 keeps every row start 16-byte aligned in both dtypes), and of a
// token's states of B and C (N == 16 keeps every token's row 16-byte aligned).
bool vec_path(const ScanArgs& a, int kpl) {
  return (a.L % 8 == 0) && a.L >= kpl && aligned16(a.u) && aligned16(a.delta) && aligned16(a.y) &&
         (a.z == nullptr || aligned16(a.z)) && (a.u_out == nullptr || aligned16(a.u_out)) && aligned16(a.Bm) &&
         aligned16(a.Cm);
}

template <typename ACT, bool GATE, int KPL, int W, bool CONV, bool ZOH>
hipError_t launch_w(const ScanArgs& a, hipStream_t s) {
  const int n_dblk = static_cast<int>((a.D + W - 1) / W);
  const int64_t blocks = a.batch * n_dblk;
  const bool vec = vec_path(a, KPL);
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * W);
  const bool n16 = a.N == 16;
  // N == 16, bfloat16, 8 tokens per lane: 8 states per step (two steps per
  // chunk, half the barriers; measured 2 % faster).  float32 measured no faster
  // that way, and at 16 tokens per lane the larger tile's registers would spill.
  constexpr int N16_STEPS = (ACT::kBytes == 2 && KPL <= 12) ? 2 : 4;
  if constexpr (KPL == 8 && !CONV && !ZOH) {
    if (a.chunk_states) {   // (the host sends only N == 16 vector-path shapes here)
      if (!(vec && n16)) return hipErrorInvalidValue;
      hipLaunchKernelGGL(
          (scan_chunked_kernel<ACT, GATE, KPL, true, N16_STEPS, 16 / N16_STEPS, W, CONV, ZOH, false, true>), grid,
          block, 0, s, a, n_dblk);
      return hipGetLastError();
    }
  }
  if constexpr (ACT::kBytes == 2 && W == 12 && (KPL == 8 || KPL == 12) && !CONV && !ZOH) {
    // Up to 10 channels per CU: 10-channel workgroups with the last two channels
    // split over two waves each (SPLIT), one workgroup per CU; at 8 tokens per lane
    // also in the arithmetic-progression build.
    if (vec && n16 && a.batch * a.D <= kSplitMaxChannels) {
      const int n_split = static_cast<int>((a.D + W - 3) / (W - 2));
      const dim3 sgrid(static_cast<unsigned>(a.batch * n_split));
      if (KPL == 8 && a.ap)
        hipLaunchKernelGGL(
            (scan_chunked_kernel<ACT, GATE, KPL, true, N16_STEPS, 16 / N16_STEPS, W, CONV, ZOH, KPL == 8, false, true>),
            sgrid, block, 0, s, a, n_split);
      else
        hipLaunchKernelGGL(
            (scan_chunked_kernel<ACT, GATE, KPL, true, N16_STEPS, 16 / N16_STEPS, W, CONV, ZOH, false, false, true>),
            sgrid, block, 0, s, a, n_split);
      return hipGetLastError();
    }
  }
  if constexpr (ACT::kBytes == 2 && W == 12 && KPL == 8 && !CONV && !ZOH) {
    if (vec && n16 && a.ap) {
      hipLaunchKernelGGL((scan_chunked_kernel<ACT, GATE, KPL, true, N16_STEPS, 16 / N16_STEPS, W, CONV, ZOH, true>),
                         grid, block, 0, s, a, n_dblk);
      return hipGetLastError();
    }
  }
  if (vec && n16)
    hipLaunchKernelGGL((scan_chunked_kernel<ACT, GATE, KPL, true, N16_STEPS, 16 / N16_STEPS, W, CONV, ZOH>), grid, block,
                       0, s, a, n_dblk);
  else if (vec)
    hipLaunchKernelGGL((scan_chunked_kernel<ACT, GATE, KPL, true, 0, kNBGeneric, W, CONV, ZOH>), grid, block, 0, s, a,
                       n_dblk);
  else if (n16)
    hipLaunchKernelGGL((scan_chunked_kernel<ACT, GATE, KPL, false, N16_STEPS, 16 / N16_STEPS, W, CONV, ZOH>), grid, block,
                       0, s, a, n_dblk);
  else
    hipLaunchKernelGGL((scan_chunked_kernel<ACT, GATE, KPL, false, 0, kNBGeneric, W, CONV, ZOH>), grid, block, 0, s, a,
                       n_dblk);
  return hipGetLastError();
}

template <typename ACT, bool GATE, int KPL, bool CONV, bool ZOH>
hipError_t launch_kpl(const ScanArgs& a, hipStream_t s) {
  // Waves per workgroup, from measurement on gfx950 (256 CUs).  Workgroup sizes
  // are multiples of 4 waves: a 6-wave group puts two waves on two of the four
  // SIMDs, and ran 50 % slower.
  //  * 12 waves (3 per SIMD, one workgroup per CU) leaves the most registers per
  //    wave.  It is the choice when one round of 12-wave groups covers every
  //    channel (at most 12 * 256), as on the 130M- and 131k-shaped workloads.
  //  * bfloat16, 8 tokens per lane, fits 128 registers, so two 8-wave groups share
  //    a CU: 4 waves per SIMD, and each barrier waits for 8 waves, not 16.  Above
  //    12 * 256 channels that is 7 % faster than one 16-wave group and 6-20 %
  //    faster than 12 waves (1.4B-shaped workload: 307 against 329 us).  The
  //    scalar-load kernel for N = 16 needs more registers and keeps 12 waves.
  //  * float32 needs more than 128 registers unless the launch bound of a 16-wave
  //    group forces it under; 16 waves (4 per SIMD) win once there are channels
  //    for three rounds of them (8 % faster at 12288 channels, 14 % slower at 6144).
  constexpr int64_t kCUs = 256;
  if constexpr (KPL == 8) {
    const int64_t ch = a.batch * a.D;
    if constexpr (ACT::kBytes == 2) {
      if (ch > 12 * kCUs && (a.N != 16 || vec_path(a, KPL))) return launch_w<ACT, GATE, KPL, 8, CONV, ZOH>(a, s);
    } else {
      if (ch >= 16 * kCUs * 3) return launch_w<ACT, GATE, KPL, 16, CONV, ZOH>(a, s);
    }
  }
  return launch_w<ACT, GATE, KPL, 12, CONV, ZOH>(a, s);
}

template <typename ACT, bool GATE>
hipError_t launch_gate(const ScanArgs& a, int kpl, hipStream_t s) {
  const bool conv = a.conv_w != nullptr;
  if (a.zoh) return launch_kpl<ACT, GATE, 8, false, true>(a, s);   // (8 tokens per lane, no conv: see chunked_supported)
  if (kpl == 8) return conv ? launch_kpl<ACT, GATE, 8, true, false>(a, s) : launch_kpl<ACT, GATE, 8, false, false>(a, s);
  if (kpl == 12) return launch_kpl<ACT, GATE, 12, false, false>(a, s);   // (no conv: see chunked_supported)
  return conv ? launch_kpl<ACT, GATE, 16, true, false>(a, s) : launch_kpl<ACT, GATE, 16, false, false>(a, s);
}

// Default tokens per lane, from measurement on gfx950: 8, where the registers
// leave room to run two states at once, beats 16 (half the wave-scan overhead
// per element, one state at a time) for both activation types.  12 still runs
// two states at once in the 12-wave launch (bfloat16, N == 16, 168 registers) and
// spends a third less on the wave scan per element: 2.7 % faster on a 131072-token
// sequence (1869 against 1920 us).  Its 768-token chunks pad a short sequence
// (2048 tokens: 12.5 % padding), so it is the default from 32768 tokens, and not
// with the arithmetic-progression path, whose build is for 8 (in the split form,
// 131072 x 2560: 1466 us against the general path's 1565 us at 12).
int resolve_kpl(const ScanArgs& a, int tokens_per_lane, Dt dt) {
  if (tokens_per_lane != 0) return tokens_per_lane;
  const bool twelve = dt == Dt::BF16 && a.N == 16 && !a.zoh && a.conv_w == nullptr && !a.ap && a.L >= 32768 &&
                      a.batch * a.D <= 12 * 256 && vec_path(a, 12);
  return twelve ? 12 : 8;
}

}  // namespace

bool chunked_save_supported(const ScanArgs& a) {
  return a.N == 16 && a.zoh == 0 && a.conv_w == nullptr && vec_path(a, 8);
}

bool chunked_supported(const ScanArgs& a, Dt, int tokens_per_lane) {
  if (!(tokens_per_lane == 0 || tokens_per_lane == 8 || tokens_per_lane == 12 || tokens_per_lane == 16)) return false;
  if (a.N < 1 || a.N > 64) return false;
  // the full zero-order hold is built for the default 8 tokens per lane without the fused conv
  if (a.zoh && (a.conv_w != nullptr || tokens_per_lane == 16 || tokens_per_lane == 12)) return false;
  // 12 tokens per lane is built without the fused conv
  if (a.conv_w != nullptr && tokens_per_lane == 12) return false;
  const int64_t n_dblk = (a.D + 8 - 1) / 8;                  // the most workgroups any launch uses (8 waves each)
  return a.batch * n_dblk <= 0x7fffffff;
}

hipError_t launch_scan_chunked(const ScanArgs& a, Dt dt, int tokens_per_lane, hipStream_t s) {
  if (!chunked_supported(a, dt, tokens_per_lane)) return hipErrorInvalidValue;
  const int kpl = resolve_kpl(a, tokens_per_lane, dt);
  const bool gate = a.z != nullptr;
  if (dt == Dt::F32)
    return gate ? launch_gate<ActF32, true>(a, kpl, s) : launch_gate<ActF32, false>(a, kpl, s);
  return gate ? launch_gate<ActBF16, true>(a, kpl, s) : launch_gate<ActBF16, false>(a, kpl, s);
}

}  // namespace ssm
