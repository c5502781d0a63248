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
//   * B and C are shared by all channels of a row and stored [batch][N][L], so a
//     state's values over a chunk are one contiguous run.  Each step of the
//     kernel covers kNB states of one chunk: the workgroup loads the next step's
//     B/C tile into registers (coalesced 16- or 8-byte vectors along L) while it
//     computes on the current one, and at the end of the step writes it, as
//     float32 and permuted into the order the lanes read it, to the other of two
//     LDS buffers; one barrier per step publishes it;
//   * a wave loads its next chunk's u and delta and this chunk's z into registers
//     during the current chunk, and stores the previous chunk's y at its first
//     step, one kind of traffic per step, so a chunk's HBM traffic is spread over
//     its steps instead of arriving as one burst per chunk.  The barriers order
//     LDS only; a load is waited for where its value is first used.
// No MFMA: the readout is a per-token dot product over n, not a shared-operand
// contraction.  The kernel is bound by HBM bandwidth and by the VALU and
// transcendental rate (one exp per element).
#include <utility>

#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_common.hpp"

namespace ssm {
namespace {

constexpr int kNBGeneric = 4;        // states per step (per staged B/C tile), any N

// ---- the scan ----------------------------------------------------------------
// kNB states per step.  NBLK > 0: N == kNB * NBLK, fixed at compile time; the steps of a chunk are
// unrolled, the last chunk is peeled, and the per-state values sit in scalar
// registers.  The steady state then has no branch around any load, so the
// compiler's tracking of outstanding loads stays exact and it never waits for a
// load before its value is needed.  NBLK = 0: any N, steps in a runtime loop.
//
// ZOH: the full zero-order-hold input term (e^{Delta A} - 1)/A * B * u instead of
// Delta * B * u: with w = u * B / A it is a*w - w, one FMA and one multiply more per
// element than the simplified term (1/A is per state, computed once per channel).
template <typename ACT, bool GATE, int KPL, bool VEC, int NBLK, int kNB, int kW, bool CONV, bool ZOH>
__global__ __launch_bounds__(64 * kW) void scan_chunked_kernel(ScanArgs p, int n_dblk) {
  constexpr int kThreads = 64 * kW;
  static_assert(KPL >= 3, "the fused conv takes its 3 earlier tokens from the previous lane");
  // states processed two at a time where the registers allow it (8 tokens per lane)
  constexpr bool PAIR = KPL <= 8;
  using IO = TokenIO<ACT, KPL>;
  using raw_t = typename IO::raw_t;
  constexpr int CH = 64 * KPL;
  constexpr int BLK4 = CH / 4;                       // float4 per (state, matrix) block
  constexpr int TILE4 = kNB * 2 * BLK4;              // float4 per step tile
  __shared__ float4 s_tile[2][TILE4];

  const int lane = threadIdx.x & 63;
  const bool lane0 = lane == 0;
  const int w = uniform_int(threadIdx.x >> 6);
  // Consecutive workgroups go to different XCDs (round robin over 8); taking the
  // batch row as blk % batch keeps one row per XCD when batch divides 8, so each
  // XCD's L2 holds only that row's B and C.
  const int blk = blockIdx.x;
  const int64_t b = blk % p.batch;
  const int64_t d_own = static_cast<int64_t>(blk / p.batch) * kW + w;
  const bool valid = d_own < p.D;                    // wave-uniform
  // A wave past the last channel runs the same code on the last channel (so no
  // branch depends on it) and stores nothing.
  const int64_t d = valid ? d_own : p.D - 1;
  const int N = p.N;
  const int64_t L = p.L;
  const int64_t row = (b * p.D + d) * L;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float dsk = p.Dskip ? p.Dskip[d] : 0.0f;
  // A[d, n] * log2(e) in lane n (read once, so the state loop never issues a
  // vector load of A).
  const float a2_v = lane < N ? p.A[d * N + lane] * kLog2e : 0.0f;
  // 1/A[d, n] in lane n (full zero-order hold only)
  const float ra_v = (ZOH && lane < N) ? 1.0f / p.A[d * N + lane] : 0.0f;
  // carry of state n lives in lane n; it starts as the initial state (zero if none)
  float carry_v = (lane < N && p.h0) ? p.h0[(b * p.D + d) * N + lane] : 0.0f;

  const int nblk = NBLK > 0 ? NBLK : (N + kNB - 1) / kNB;
  const int64_t nchunks = (L + CH - 1) / CH;
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
      for (int j = 0; j < KPL; ++j) dl[j] = softplus_f(dl[j] + bias);
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

  // Input term of token j for a state with B value bj and 1/A = ra.
  auto input_term = [&](float avj, float duj, float bj, float ra) __attribute__((always_inline)) -> float {
    if constexpr (ZOH) {
      const float w = (duj * ra) * bj;
      return __builtin_fmaf(avj, w, -w);
    } else {
      return duj * bj;
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
        av[j] = exp2_hw(dl[j] * a2);
        bv[j] = input_term(av[j], du[j], bs[r], ra);
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
  auto scan_two = [&](const float4* __restrict__ sB0, const float4* __restrict__ sC0, float a20, float ra0,
                      float carry0, const float4* __restrict__ sB1, const float4* __restrict__ sC1, float a21,
                      float ra1, float carry1, float& out0, float& out1) __attribute__((always_inline)) {
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
        av0[j] = exp2_hw(dl[j] * a20);
        av1[j] = exp2_hw(dl[j] * a21);
        bv0[j] = input_term(av0[j], du[j], bs0[r], ra0);
        bv1[j] = input_term(av1[j], du[j], bs1[r], ra1);
        h0 = __builtin_fmaf(av0[j], h0, bv0[j]);
        h1 = __builtin_fmaf(av1[j], h1, bv1[j]);
      }
    }
    float P0 = exp2_hw(a20 * sdl);
    float P1 = exp2_hw(a21 * sdl);
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

  // Tile of step k = (chunk c = k / nblk, states n0 = (k % nblk) * kNB ...): for
  // each of its nn = min(kNB, N - n0) states, B's then C's CH values of the
  // chunk, which are contiguous in memory.  Float4 f of a block (2 * state +
  // matrix) holds tokens 4f .. 4f+3; in LDS it goes to the slot lane f / (KPL/4)
  // reads as its vector f % (KPL/4), so the state loop's LDS reads are
  // contiguous.  Threads move one 16-byte vector (kTok tokens) each per element:
  // element e of the tile covers float4 (e % BLKR) * kOut ... of block e / BLKR.
  // A block is a multiple of 64 elements, so a wave's block (state, matrix) is
  // wave-uniform and only the token offset is per lane.
  //
  // Pipeline: tile j is loaded into register set j % 2 during step j - 2 and
  // written (as float32, permuted) to LDS buffer j % 2 at the end of step j - 1,
  // so each load has a whole step to arrive before its value is needed.
  using TIO = TileIO<ACT>;
  using traw_t = typename TIO::raw_t;
  constexpr int BLKR = BLK4 / TIO::kOut;                     // 16-byte elements per block
  constexpr int TILER = kNB * 2 * BLKR;                      // elements per tile
  constexpr int TPT = (TILER + kThreads - 1) / kThreads;     // elements per thread
  static_assert(TPT <= 3, "tile share per thread held in three registers");
  static_assert(BLKR % 64 == 0, "a tile block spans whole waves");
  traw_t tr[2][TPT];
  int tile_nr[2] = {0, 0};                                   // elements in each staged tile
  const int64_t bc_row = b * N * L;                          // this batch row of B and C
  auto load_tile = [&](int64_t k, int set) __attribute__((always_inline)) {
    const int64_t c = k / nblk;
    const int n0 = static_cast<int>(k % nblk) * kNB;
    const int nr = ((N - n0 < kNB) ? (N - n0) : kNB) * 2 * BLKR;
    tile_nr[set] = nr;
    const int64_t tok0 = c * CH;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      // this wave's first element, clamped into the tile (the surplus is never stored)
      int eb = w * 64 + i * kThreads;
      eb = eb < nr ? eb : nr - 64;
      const int blkk = eb / BLKR;
      const void* src = (blkk & 1) ? p.Cm : p.Bm;
      const int64_t srow = bc_row + static_cast<int64_t>(n0 + (blkk >> 1)) * L;
      const int64_t t = tok0 + TIO::kTok * (eb % BLKR + lane);
      if constexpr (VEC) {
        // Unconditional load, clamped into the row: a lane past L reloads the
        // row's last tokens.  Those padding tokens have Delta = 0, so they are
        // identity steps whatever finite B and C they see, and their y is never
        // stored.
        tr[set][i] = TIO::load(src, srow + (t < L ? t : L - TIO::kTok));
      } else {
        float x[TIO::kTok];
#pragma unroll
        for (int r = 0; r < TIO::kTok; ++r) x[r] = t + r < L ? load_act<ACT>(src, srow + t + r) : 0.0f;
        if constexpr (ACT::kBytes == 4) {
          tr[set][i] = make_float4(x[0], x[1], x[2], x[3]);
        } else {
          tr[set][i] = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                  pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
        }
      }
    }
  };
  auto store_tile = [&](int set) __attribute__((always_inline)) {
    float4* dst = s_tile[set];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int eb = w * 64 + i * kThreads;
      if (eb < tile_nr[set]) {
        const int blkk = eb / BLKR;
#pragma unroll
        for (int j = 0; j < TIO::kOut; ++j) {
          const int f = (eb % BLKR + lane) * TIO::kOut + j;
          dst[blkk * BLK4 + (f % (KPL / 4)) * 64 + f / (KPL / 4)] = TIO::out(tr[set][i], j);
        }
      }
    }
  };

  // HBM traffic is spread over a chunk's steps, one kind per step: y of the
  // previous chunk is stored at step 0, the next chunk's u is loaded at step 1,
  // its delta at step 2 and this chunk's z at step 3.
  const int st_u = nblk > 1 ? 1 : 0;
  const int st_d = nblk > 2 ? 2 : st_u;
  const int st_z = nblk > 3 ? 3 : st_d;

  // Per-state wave-uniform values when the state count is fixed at compile time
  // (NBLK > 0): A*log2(e) and the carry of state n in scalar registers, indexed
  // by compile-time n once the steps are unrolled.
  constexpr int NS = NBLK > 0 ? kNB * NBLK : 1;
  float a2s[NS], cs[NS], ras[NS];
  if constexpr (NBLK > 0) {
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      a2s[n] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a2_v), n));
      ras[n] = ZOH ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ra_v), n)) : 0.0f;
      cs[n] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, carry_v), n));
    }
  }

  // The states of step nb of the current chunk, from the tile `cur`.
  auto states = [&](const float4* cur, int nb) __attribute__((always_inline)) {
    const int n0 = nb * kNB;
    if constexpr (NBLK > 0) {
      constexpr int nn = kNB;                          // N == kNB * NBLK: every step is full
      const float4* t = cur;
      if constexpr (PAIR) {
#pragma unroll
        for (int nl = 0; nl < nn; nl += 2) {
          const int n = n0 + nl;
          scan_two(t + nl * 2 * BLK4, t + (nl * 2 + 1) * BLK4, a2s[n], ras[n], cs[n],
                   t + (nl * 2 + 2) * BLK4, t + (nl * 2 + 3) * BLK4, a2s[n + 1], ras[n + 1], cs[n + 1], cs[n],
                   cs[n + 1]);
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
    if (valid) states(s_tile[par], nb);
    if (!tail1) store_tile(par ^ 1);
    barrier_lds();
  };

  prefetch_act(p.u, 0, u_raw);
  prefetch_act(p.delta, 0, d_raw);
  load_tile(0, 0);
  if (nsteps > 1) load_tile(1, 1);
  store_tile(0);
  barrier_lds();
  if constexpr (NBLK > 0) {
    static_assert(NBLK % 2 == 0, "steps are unrolled in pairs");
    for (int64_t c = 0; c + 1 < nchunks; ++c) {
      static_for<NBLK>([&](auto nbc) __attribute__((always_inline)) {
        constexpr int nb = decltype(nbc)::value;
        step(c * NBLK + nb, c, nb, nb & 1, false, false, false);
      });
    }
    const int64_t c = nchunks - 1;
    static_for<NBLK>([&](auto nbc) __attribute__((always_inline)) {
      constexpr int nb = decltype(nbc)::value;
      const int64_t k = c * NBLK + nb;
      step(k, c, nb, nb & 1, true, k + 2 >= nsteps, k + 1 >= nsteps);
    });
  } else {
    for (int64_t k = 0; k < nsteps; k += 2) {
      const int64_t c0 = k / nblk, c1 = (k + 1) / nblk;
      step(k, c0, static_cast<int>(k % nblk), 0, c0 + 1 >= nchunks, k + 2 >= nsteps, k + 1 >= nsteps);
      if (k + 1 < nsteps)
        step(k + 1, c1, static_cast<int>((k + 1) % nblk), 1, c1 + 1 >= nchunks, k + 3 >= nsteps, k + 2 >= nsteps);
    }
  }
  if constexpr (NBLK > 0) {
    // carries back into lane n for the final-state store
#pragma unroll
    for (int n = 0; n < NS; ++n) carry_v = lane == n ? cs[n] : carry_v;
  }
  epilogue(nchunks - 1);
  if (valid && p.final_state && lane < N) p.final_state[(b * p.D + d) * N + lane] = carry_v;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

// Vector path: 16-byte vectors of u, delta, z, y along L, and of B and C (L % 8
// == 0 keeps every row start 16-byte aligned in both dtypes).
bool vec_path(const ScanArgs& a, int kpl) {
  return (a.L % 8 == 0) && a.L >= kpl && aligned16(a.u) && aligned16(a.delta) && aligned16(a.y) &&
         (a.z == nullptr || aligned16(a.z)) && aligned16(a.Bm) && aligned16(a.Cm);
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
  constexpr int N16_STEPS = (ACT::kBytes == 2 && KPL <= 8) ? 2 : 4;
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
  return conv ? launch_kpl<ACT, GATE, 16, true, false>(a, s) : launch_kpl<ACT, GATE, 16, false, false>(a, s);
}

// Default tokens per lane, from measurement on gfx950: 8, where the registers
// leave room to run two states at once, beats 16 (half the wave-scan overhead
// per element, one state at a time) for both activation types.
int resolve_kpl(int tokens_per_lane, Dt) {
  return tokens_per_lane != 0 ? tokens_per_lane : 8;
}

}  // namespace

bool chunked_supported(const ScanArgs& a, Dt, int tokens_per_lane) {
  if (!(tokens_per_lane == 0 || tokens_per_lane == 8 || tokens_per_lane == 16)) return false;
  if (a.N < 1 || a.N > 64) return false;
  // the full zero-order hold is built for the default 8 tokens per lane without the fused conv
  if (a.zoh && (a.conv_w != nullptr || tokens_per_lane == 16)) return false;
  const int64_t n_dblk = (a.D + 8 - 1) / 8;                  // the most workgroups any launch uses (8 waves each)
  return a.batch * n_dblk <= 0x7fffffff;
}

hipError_t launch_scan_chunked(const ScanArgs& a, Dt dt, int tokens_per_lane, hipStream_t s) {
  if (!chunked_supported(a, dt, tokens_per_lane)) return hipErrorInvalidValue;
  const int kpl = resolve_kpl(tokens_per_lane, dt);
  const bool gate = a.z != nullptr;
  if (dt == Dt::F32)
    return gate ? launch_gate<ActF32, true>(a, kpl, s) : launch_gate<ActF32, false>(a, kpl, s);
  return gate ? launch_gate<ActBF16, true>(a, kpl, s) : launch_gate<ActBF16, false>(a, kpl, s);
}

}  // namespace ssm
