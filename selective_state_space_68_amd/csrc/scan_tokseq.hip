// Token-sequential selective scan for gfx950, for workloads with many channels.
//
// The chunked kernel owns tokens per lane and pays for that with a wave scan, a
// replay of every token and a per-lane aggregate decay, about 2.75 of its ~11.6
// VALU issue slots per element.  When batch * D is large there are enough
// (channel, state) pairs to give every lane its own states and walk the sequence
// in order, as the recurrence is written (the slide deck's selective-SSM listing;
// the prep page's sequential pseudo-code):
//
//   * a lane owns SPL consecutive states of one channel, 16 / SPL lanes (an aligned
//     group) own a channel, and a wave owns 64 * SPL / 16 channels of one batch row;
//   * per token a lane computes exp(Delta A), the state update and its part of the
//     readout for its SPL states, and the group adds the parts with DPP (two
//     quad_perm steps, plus a half-row mirror for 8-lane groups);
//   * the per-token work (softplus, Delta * u, D * u, the SiLU gate) runs once per
//     (token, channel): each lane does it for one 8-token piece of its channel in
//     a block of 8 * 16 / SPL tokens and leaves (Delta, Delta * u) in LDS, and the
//     readout of its piece's tokens ends up in the same lane for the output;
//   * B and C ([batch][L][N], so a block's B is one contiguous run of T * 16
//     values) are staged in LDS as float32 [token][state], so a lane reads its
//     SPL states of one token as one vector.
//
// Every wave uses its own LDS slice and never waits for another: a workgroup is
// kTsWaves independent waves.  Loads of the next block are issued when the current
// block's inputs have been written to LDS, so they have the whole block to arrive.
// VALU issue per element: SPL x (multiply, exp, multiply, FMA) and the readout
// FMA, plus the group reduction and the per-token work spread over 16 states.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_common.hpp"

namespace ssm {
namespace {

constexpr int kTsWaves = 4;          // independent waves per workgroup
constexpr int kTsN = 16;             // states per channel the kernel is built for

// Eight consecutive B or C values: states 8h .. 8h+7 of one token (a 16- or 32-byte
// load, cached: every channel group of the batch row reads the same tile).
template <typename ACT>
struct Piece8;
template <>
struct Piece8<ActF32> {
  float4 r[2];
  __device__ __forceinline__ void load(const void* base, int64_t off) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    r[0] = p[0];
    r[1] = p[1];
  }
  __device__ __forceinline__ float get(int k) const {
    const float4& v = r[k >> 2];
    const int e = k & 3;
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
  }
};
template <>
struct Piece8<ActBF16> {
  uint4 r;
  __device__ __forceinline__ void load(const void* base, int64_t off) {
    r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  }
  __device__ __forceinline__ float get(int k) const {
    const uint32_t w = (k >> 1) == 0 ? r.x : ((k >> 1) == 1 ? r.y : ((k >> 1) == 2 ? r.z : r.w));
    return (k & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};

// Eight consecutive activations of one channel, cached (temporal) loads and stores.
// In bfloat16 a channel's block is 64 bytes, half a cache line, and the other half
// is the next block's: non-temporal accesses lost the line in between and fetched
// every line twice (1.69x the algorithmic HBM reads, 3 % slower).
template <typename ACT>
struct ActIO8;
template <>
struct ActIO8<ActF32> {
  using raw_t = float4;
  static constexpr int kVec = 2;
  static __device__ __forceinline__ void load_raw(const void* base, int64_t off, raw_t (&r)[2]) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    r[0] = p[0]; r[1] = p[1];
  }
  static __device__ __forceinline__ void unpack(const raw_t (&r)[2], float (&v)[8]) { TokenIO<ActF32, 8>::unpack(r, v); }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float (&v)[8]) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]); p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};
template <>
struct ActIO8<ActBF16> {
  using raw_t = uint4;
  static constexpr int kVec = 1;
  static __device__ __forceinline__ void load_raw(const void* base, int64_t off, raw_t (&r)[1]) {
    r[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  }
  static __device__ __forceinline__ void unpack(const raw_t (&r)[1], float (&v)[8]) { TokenIO<ActBF16, 8>::unpack(r, v); }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float (&v)[8]) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) =
        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  }
};

// ZOH: the full zero-order-hold input term (e^{Delta A} - 1)/A * B * u = u B times
// zoh_factor: the lanes keep (Delta, u) instead of (Delta, Delta u) in LDS, and 1/A
// per state.
//
// CONV: the scan input is u = SiLU(causal conv1d(x)) with the taps of p.conv_w,
// computed in the per-token work: a lane's piece needs the 3 inputs before it, from
// the previous lane of its group (quad_perm [3, 0, 1, 2]) or, for the block's first
// piece, from the previous block's last piece, carried (zero before the sequence).
//
// AP: the build with the arithmetic-progression decay path, used when the caller
// allows it (SSM_SCAN_AP); a separate build so that the default one keeps its
// registers and schedule.
//
// SAVE: the build that also writes the saved chunk states (p.chunk_states) every
// 512 tokens, for the backward pass; a separate build, so that the default ones keep
// their registers.
template <typename ACT, bool GATE, int SPL, bool ZOH, bool CONV, bool AP = false, bool SAVE = false, bool PF2 = false>
__global__ __launch_bounds__(64 * kTsWaves) void scan_tokseq_kernel(ScanArgs p) {
  constexpr int QL = kTsN / SPL;           // lanes per channel (an aligned group)
  constexpr int CPW = 64 / QL;             // channels per wave
  constexpr int T = 8 * QL;                // tokens per block: one 8-token piece per lane of a group
  constexpr int DUS = 2 * T + 4;           // row stride (floats) of a channel's (Delta, Delta*u) pairs
  constexpr int BCP = QL / 4;              // B (and C) pieces per lane per block
  static_assert(SPL == 2 || SPL == 4, "4 or 8 lanes per channel");
  static_assert(!AP || (ACT::kBytes == 2 && SPL == 4 && !ZOH && !CONV),
                "no arithmetic-progression build for this configuration");
  using IO = ActIO8<ACT>;
  using raw_t = typename IO::raw_t;
  // [wave][matrix][token][16 states]; the float4 group of states g of token t sits
  // at group g ^ ((t / 8) % 4), so the lanes writing one token row of different
  // pieces fall in different banks
  __shared__ float4 s_bc[kTsWaves][2][T][kTsN / 4];
  __shared__ __attribute__((aligned(16))) float s_du[kTsWaves][CPW * DUS];

  const int lane = threadIdx.x & 63;
  const int w = uniform_int(threadIdx.x >> 6);
  const int64_t L = p.L, D = p.D;
  const int64_t ngrp = (D + CPW - 1) / CPW;
  // Consecutive workgroups go to different XCDs; the batch row is blockIdx % batch
  // so that one row's B and C stay in one XCD's L2 when the batch size divides 8.
  const int64_t b = blockIdx.x % p.batch;
  const int64_t grp = static_cast<int64_t>(blockIdx.x / p.batch) * kTsWaves + w;
  // A wave past the last channel group runs the last group and stores nothing; a
  // lane past the last channel runs the last channel and stores nothing.
  const int64_t gcl = grp < ngrp ? grp : ngrp - 1;
  const int ch = lane / QL, q = lane % QL;           // channel in the wave; state group and token piece
  const int64_t d_own = gcl * CPW + ch;
  const bool store_ok = grp < ngrp && d_own < D;
  const int64_t d = d_own < D ? d_own : D - 1;
  const int64_t row = (b * D + d) * L;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float dsk = p.Dskip ? p.Dskip[d] : 0.0f;
  float a2[SPL], ra[SPL], h[SPL];
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const int64_t sidx = d * kTsN + SPL * q + j;
    a2[j] = p.A[sidx] * kLog2e;
    ra[j] = ZOH ? 1.0f / p.A[sidx] : 0.0f;   // (inf at A == 0, never selected there by zoh_factor)
    h[j] = p.h0 ? p.h0[(b * D + d) * kTsN + SPL * q + j] : 0.0f;
  }
  // AP build, non-increasing arithmetic-progression A rows (A[d, n] == A[d, 0] + n b
  // exactly with b <= 0, for every channel of the wave; wave-uniform): a lane's
  // decays exp(Delta A) over its SPL consecutive states are its first state's times
  // powers of exp(Delta b) <= 1, two exponentials per token instead of SPL (built for
  // bfloat16, 4 states per lane and the simplified input term; at 2 states per lane
  // it would save nothing).
  float ap_b2 = 0.0f;
  bool ap_wave = false;
  if constexpr (AP) {
    const float a0 = p.A[d * kTsN], bstep = p.A[d * kTsN + 1] - a0;
    bool off = false;
#pragma unroll
    for (int j = 0; j < SPL; ++j)
      off = off || __builtin_fmaf(static_cast<float>(SPL * q + j), bstep, a0) != p.A[d * kTsN + SPL * q + j];
    ap_wave = __ballot(off || !(bstep <= 0.0f)) == 0;
    ap_b2 = bstep * kLog2e;
  }
  static_assert(!CONV || SPL == 4, "the fused conv is built for 4 states per lane");
  // conv taps aligned to the window x[t-3 .. t] (cw4[4-K+k] = w[d, k], the rest zero)
  float cw4[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cbias = 0.0f, carry[3] = {0.0f, 0.0f, 0.0f};
  if constexpr (CONV) {
#pragma unroll
    for (int k = 0; k < 4; ++k) cw4[k] = (k >= 4 - p.conv_k) ? p.conv_w[d * p.conv_k + k - (4 - p.conv_k)] : 0.0f;
    cbias = p.conv_b ? p.conv_b[d] : 0.0f;
  }
  const int64_t bc_row = b * L * kTsN;               // B, C of this batch row ([L][N])
  float* du_w = s_du[w];
  float* bc_w = reinterpret_cast<float*>(s_bc[w]);

  // Block inputs in registers: this lane's piece (tokens 8q .. 8q+7 of the block) of
  // u, delta and z, and its BCP pieces of B and C (piece v = lane + 64k: token v / 2
  // of the block, states 8 (v % 2) ..).  Pieces past L (L % 8 == 0: an activation
  // piece is all in or all out) reload the row's last piece or token; their Delta
  // is set to 0.
  // PF2: two sets, alternating by block, so block k's loads are issued while block
  // k - 2 computes, two blocks ahead of their use instead of one.  The second set
  // takes about 24 more registers, so the host picks this build only where the launch
  // has at most 2 waves per SIMD and the registers cost no occupancy.
  struct BlockRegs {
    raw_t u[IO::kVec], d[IO::kVec], z[IO::kVec];
    Piece8<ACT> bp[BCP], cp[BCP];
  };
  auto fetch = [&](int64_t t0, BlockRegs& rg) __attribute__((always_inline)) {
    int64_t tp = t0 + 8 * q;
    tp = tp + 8 <= L ? tp : L - 8;
    IO::load_raw(p.u, row + tp, rg.u);
    IO::load_raw(p.delta, row + tp, rg.d);
    if constexpr (GATE) IO::load_raw(p.z, row + tp, rg.z);
#pragma unroll
    for (int k = 0; k < BCP; ++k) {
      const int v = lane + 64 * k;
      int64_t t = t0 + v / 2;
      t = t < L ? t : L - 1;
      rg.bp[k].load(p.Bm, bc_row + t * kTsN + 8 * (v % 2));
      rg.cp[k].load(p.Cm, bc_row + t * kTsN + 8 * (v % 2));
    }
  };

  const int64_t nblk = (L + T - 1) / T;
  // saved chunk states: entry c is the state entering 512-token chunk c (T divides 512)
  static_assert(kSaveChunk % T == 0, "a block never straddles a saved chunk");
  float* cst = nullptr;
  if constexpr (SAVE) {
    if (store_ok) cst = p.chunk_states + (b * D + d) * ((L + kSaveChunk - 1) / kSaveChunk) * kTsN;
  }
  if (SAVE && cst) {
#pragma unroll
    for (int j = 0; j < SPL; ++j) cst[SPL * q + j] = h[j];
  }
  constexpr int kAhead = PF2 ? 2 : 1;                 // blocks between a set's load and its use
  BlockRegs rg0, rg1;
  auto block = [&](int64_t blk, BlockRegs& rg) __attribute__((always_inline)) {
    const int64_t t0 = blk * T;
    const bool pvalid = t0 + 8 * q < L;
    // ---- per-token work of this lane's piece; (Delta, Delta*u) and the B/C tile to LDS
    float uv[8], dl[8], ysk[8], gt[8] = {};
    IO::unpack(rg.u, uv);
    IO::unpack(rg.d, dl);
    if constexpr (CONV) {
      // uv holds x: u = SiLU(conv(x)), accumulated oldest tap first
      float xx[11];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float prev = dpp_mov<0x93, 0xf, false>(0.0f, uv[5 + k]);   // quad_perm [3, 0, 1, 2]
        const float last = dpp_mov<0xFF, 0xf, false>(0.0f, uv[5 + k]);   // quad_perm [3, 3, 3, 3]
        xx[k] = q == 0 ? carry[k] : prev;
        carry[k] = last;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) xx[3 + j] = uv[j];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float sc = cbias;
#pragma unroll
        for (int k = 0; k < 4; ++k) sc = __builtin_fmaf(cw4[k], xx[j + k], sc);
        uv[j] = sc * __builtin_amdgcn_rcpf(1.0f + exp2_hw(-sc * kLog2e));
      }
      if (p.u_out && store_ok && pvalid) IO::store(p.u_out, row + t0 + 8 * q, uv);
    }
    if constexpr (GATE) {
      float zv[8];
      IO::unpack(rg.z, zv);
#pragma unroll
      for (int k = 0; k < 8; ++k) gt[k] = silu_f(zv[k]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float x = dl[k] + bias;
      dl[k] = p.softplus ? softplus_f(x) : x;   // (the bfloat16 form measured 2 % slower here)
      dl[k] = pvalid ? dl[k] : 0.0f;                 // padding tokens: identity steps
      ysk[k] = dsk * uv[k];
    }
    float4* dst = reinterpret_cast<float4*>(du_w + ch * DUS + 16 * q);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      dst[k] = ZOH ? make_float4(dl[2 * k], uv[2 * k], dl[2 * k + 1], uv[2 * k + 1])
                   : make_float4(dl[2 * k], dl[2 * k] * uv[2 * k], dl[2 * k + 1], dl[2 * k + 1] * uv[2 * k + 1]);
#pragma unroll
    for (int k = 0; k < BCP; ++k) {
      // token t of the block, state groups 2h and 2h + 1, each at its swizzled slot
      const int v = lane + 64 * k, t = v / 2, h2 = 2 * (v % 2), sw = (t / 8) & 3;
      float4* brow = reinterpret_cast<float4*>(bc_w + (0 * T + t) * kTsN);
      float4* crow = reinterpret_cast<float4*>(bc_w + (1 * T + t) * kTsN);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        brow[(h2 + g) ^ sw] = make_float4(rg.bp[k].get(4 * g), rg.bp[k].get(4 * g + 1), rg.bp[k].get(4 * g + 2),
                                          rg.bp[k].get(4 * g + 3));
        crow[(h2 + g) ^ sw] = make_float4(rg.cp[k].get(4 * g), rg.cp[k].get(4 * g + 1), rg.cp[k].get(4 * g + 2),
                                          rg.cp[k].get(4 * g + 3));
      }
    }
    // the wave's own LDS writes before its reads (one wave's LDS operations are
    // performed in order; this keeps the compiler from moving reads above writes)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    fetch(t0 + kAhead * T < L ? t0 + kAhead * T : t0, rg);   // block blk + kAhead into this set (past the end: this block, unused)

    // ---- the recurrence, token by token; lane q keeps the readout of tokens 8q .. 8q+7
    float rsel[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) rsel[k] = 0.0f;
    const float* du_c = du_w + ch * DUS;
    const int qg = SPL == 4 ? q : q >> 1;           // this lane's float4 group of states
    // (fully unrolled: the compiler then pipelines the LDS reads across pieces, 2-5 %
    // faster at the 2-3 waves per SIMD this kernel runs with)
    auto walk = [&](auto apm) __attribute__((always_inline)) {
      constexpr bool APM = decltype(apm)::value;
#pragma unroll
      for (int tb = 0; tb < T / 8; ++tb) {             // 8-token piece tb (its per-token work was lane tb's)
        const int gsw = qg ^ (tb & 3);
        const float* brow = bc_w + (0 * T + 8 * tb) * kTsN;
        const float* crow = bc_w + (1 * T + 8 * tb) * kTsN;
        const bool mine = q == tb;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float2 dd = *reinterpret_cast<const float2*>(du_c + 2 * (8 * tb + k));
          float bs[SPL], cs[SPL];
          if constexpr (SPL == 4) {
            const float4 bb = reinterpret_cast<const float4*>(brow + k * kTsN)[gsw];
            const float4 cc = reinterpret_cast<const float4*>(crow + k * kTsN)[gsw];
            bs[0] = bb.x; bs[1] = bb.y; bs[2] = bb.z; bs[3] = bb.w;
            cs[0] = cc.x; cs[1] = cc.y; cs[2] = cc.z; cs[3] = cc.w;
          } else {
            const float2 bb = reinterpret_cast<const float2*>(brow + k * kTsN)[2 * gsw + (q & 1)];
            const float2 cc = reinterpret_cast<const float2*>(crow + k * kTsN)[2 * gsw + (q & 1)];
            bs[0] = bb.x; bs[1] = bb.y;
            cs[0] = cc.x; cs[1] = cc.y;
          }
          float r = 0.0f;
          float apc = 0.0f, apr = 0.0f;
          if constexpr (APM) {
            apc = exp2_hw(dd.x * a2[0]);
            apr = exp2_hw(dd.x * ap_b2);
          }
#pragma unroll
          for (int j = 0; j < SPL; ++j) {
            const float yj = dd.x * a2[j];
            float a;
            if constexpr (APM) {
              a = apc;
              apc *= apr;
            } else {
              a = exp2_hw(yj);
            }
            float term;
            if constexpr (ZOH) {
              term = (dd.y * bs[j]) * zoh_factor(yj, a, ra[j], dd.x);
            } else {
              term = dd.y * bs[j];
            }
            h[j] = __builtin_fmaf(a, h[j], term);
            r = __builtin_fmaf(cs[j], h[j], r);
          }
          r += dpp_mov<0xB1, 0xf, false>(0.0f, r);     // quad_perm [1, 0, 3, 2]
          r += dpp_mov<0x4E, 0xf, false>(0.0f, r);     // quad_perm [2, 3, 0, 1]
          if constexpr (SPL == 2) r += dpp_mov<0x141, 0xf, false>(0.0f, r);   // row_half_mirror
          rsel[k] = mine ? r : rsel[k];
        }
      }
    };
    if (ap_wave)
      walk(std::true_type{});
    else
      walk(std::false_type{});
    // ---- the outputs of this lane's piece
    if (store_ok && pvalid) {
      float yv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        yv[k] = rsel[k] + ysk[k];
        if constexpr (GATE) yv[k] *= gt[k];
      }
      IO::store(p.y, row + t0 + 8 * q, yv);
    }
    // the state after this block, when it ends a saved 512-token chunk
    if (SAVE && cst && (t0 + T) % kSaveChunk == 0 && t0 + T < L) {
#pragma unroll
      for (int j = 0; j < SPL; ++j) cst[((t0 + T) / kSaveChunk) * kTsN + SPL * q + j] = h[j];
    }
    // reads of this block's LDS before the next block's writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  fetch(0, rg0);
  if constexpr (PF2) {
    fetch(T < L ? T : 0, rg1);                       // (one block only: block 0 again, unused)
    for (int64_t blk = 0; blk < nblk; blk += 2) {
      block(blk, rg0);
      if (blk + 1 < nblk) block(blk + 1, rg1);
    }
  } else {
    for (int64_t blk = 0; blk < nblk; ++blk) block(blk, rg0);
  }
  if (store_ok && p.final_state) {
#pragma unroll
    for (int j = 0; j < SPL; ++j) p.final_state[(b * D + d) * kTsN + SPL * q + j] = h[j];
  }
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

template <typename ACT, bool GATE, int SPL, bool ZOH, bool CONV = false, bool AP = false, bool SAVE = false>
hipError_t launch_spl(const ScanArgs& a, hipStream_t s) {
  constexpr int CPW = 64 * SPL / kTsN;
  const int64_t ngrp = (a.D + CPW - 1) / CPW;
  const int64_t blocks = a.batch * ((ngrp + kTsWaves - 1) / kTsWaves);
  // Two block loads in flight per wave (PF2) where the launch has at most 2 waves per
  // SIMD (1024 SIMDs), so its extra registers cost no occupancy.  Measured at the
  // 1.4B shape (2 waves per SIMD), same box: fused conv 317.5 -> 307.8 us, ZOH 456.2
  // -> 452.9 us, the plain scan 282.8 -> 282.3 us.
  if (blocks * kTsWaves <= 2 * 1024)
    hipLaunchKernelGGL((scan_tokseq_kernel<ACT, GATE, SPL, ZOH, CONV, AP, SAVE, true>),
                       dim3(static_cast<unsigned>(blocks)), dim3(64 * kTsWaves), 0, s, a);
  else
    hipLaunchKernelGGL((scan_tokseq_kernel<ACT, GATE, SPL, ZOH, CONV, AP, SAVE, false>),
                       dim3(static_cast<unsigned>(blocks)), dim3(64 * kTsWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool tokseq_supported(const ScanArgs& a) {
  if (a.N != kTsN || (a.conv_w != nullptr && (a.zoh || a.conv_k < 1 || a.conv_k > 4))) return false;
  if (a.u_out != nullptr && !aligned16(a.u_out)) return false;
  if (a.L < 8 || a.L % 8 != 0) return false;
  if (!aligned16(a.u) || !aligned16(a.delta) || !aligned16(a.y) || !aligned16(a.Bm) || !aligned16(a.Cm)) return false;
  if (a.z != nullptr && !aligned16(a.z)) return false;
  const int64_t ngrp = (a.D + 8 - 1) / 8;            // the smallest channel group (SPL = 2)
  return a.batch * ((ngrp + kTsWaves - 1) / kTsWaves) <= 0x7fffffff;
}

// Measured on gfx950 (256 CUs), N = 16, 2048 tokens, against the chunked kernel.
// The kernel has no split of the sequence, so it needs channels: at 4 states per
// lane a SIMD gets batch * D / 16384 waves.
//  * 32768 channels (2 waves per SIMD): bfloat16 8 % faster (279 against 302 us on
//    the 1.4B-shaped workload), float32 18 % faster;
//  * 49152 and 65536 channels: bfloat16 13-15 % and float32 16 % faster;
//  * 24576 channels (1.5 waves per SIMD, unevenly spread) and 16384: bfloat16
//    17-22 % slower, float32 even.  Two states per lane measured slower throughout.
bool tokseq_preferred(const ScanArgs& a, Dt) {
  return tokseq_supported(a) && a.batch * a.D >= 32768;
}

hipError_t launch_scan_tokseq(const ScanArgs& a, Dt dt, int states_per_lane, hipStream_t s) {
  if (!tokseq_supported(a)) return hipErrorInvalidValue;
  const bool gate = a.z != nullptr;
  // (the full zero-order hold and the fused conv are built for 4 states per lane,
  // the automatic choice)
  const int spl = (states_per_lane == 2 && !a.zoh && a.conv_w == nullptr) ? 2 : 4;
  if (a.chunk_states) {   // saving the chunk states (simplified input term, no conv: checked by the host)
    if (a.zoh || a.conv_w != nullptr) return hipErrorInvalidValue;
    if (dt == Dt::F32)
      return gate ? launch_spl<ActF32, true, 4, false, false, false, true>(a, s)
                  : launch_spl<ActF32, false, 4, false, false, false, true>(a, s);
    return gate ? launch_spl<ActBF16, true, 4, false, false, false, true>(a, s)
                : launch_spl<ActBF16, false, 4, false, false, false, true>(a, s);
  }
  if (a.conv_w != nullptr) {
    if (dt == Dt::F32)
      return gate ? launch_spl<ActF32, true, 4, false, true>(a, s) : launch_spl<ActF32, false, 4, false, true>(a, s);
    return gate ? launch_spl<ActBF16, true, 4, false, true>(a, s) : launch_spl<ActBF16, false, 4, false, true>(a, s);
  }
  if (dt == Dt::F32) {
    if (a.zoh) return gate ? launch_spl<ActF32, true, 4, true>(a, s) : launch_spl<ActF32, false, 4, true>(a, s);
    if (spl == 4) return gate ? launch_spl<ActF32, true, 4, false>(a, s) : launch_spl<ActF32, false, 4, false>(a, s);
    return gate ? launch_spl<ActF32, true, 2, false>(a, s) : launch_spl<ActF32, false, 2, false>(a, s);
  }
  if (a.zoh) return gate ? launch_spl<ActBF16, true, 4, true>(a, s) : launch_spl<ActBF16, false, 4, true>(a, s);
  if (spl == 4 && a.ap)
    return gate ? launch_spl<ActBF16, true, 4, false, false, true>(a, s)
                : launch_spl<ActBF16, false, 4, false, false, true>(a, s);
  if (spl == 4) return gate ? launch_spl<ActBF16, true, 4, false>(a, s) : launch_spl<ActBF16, false, 4, false>(a, s);
  return gate ? launch_spl<ActBF16, true, 2, false>(a, s) : launch_spl<ActBF16, false, 2, false>(a, s);
}

}  // namespace ssm
