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
//   * B and C are shared by all channels of a row.  A small pre-pass packs them
//     (as float32) into a workspace laid out exactly like the LDS tiles: per
//     (b, chunk, state, B|C) a 4*CH-byte block in the order the lanes read it.
//     Each step of the kernel covers kNB states of one chunk; the workgroup loads
//     the next step's tile into registers while it computes on the current one
//     and writes it to the other of two LDS buffers, and one barrier per step
//     publishes it;
//   * a wave loads its next chunk's u and delta into registers and this chunk's z
//     into LDS during the current chunk, and stores the previous chunk's y at its
//     first step, one kind of traffic per step: every barrier waits for the wave's
//     outstanding memory operations, so a chunk's HBM traffic is spread over its
//     steps instead of arriving as one burst per chunk.
// No MFMA: the readout is a per-token dot product over n, not a shared-operand
// contraction.  The kernel is bound by HBM bandwidth and by the VALU and
// transcendental rate (one exp per element).
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ssm {
namespace {

constexpr int kNB = 4;               // states per step (per staged B/C tile)
constexpr int kW = 12;               // waves (channels) per workgroup
constexpr int kThreads = 64 * kW;

typedef __attribute__((address_space(3))) void lds_void;

// Direct global->LDS copy: lane l moves 16 bytes from gsrc (per lane) to
// lds_base + 16*l (lds_base must be wave-uniform).
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)(lds_base), 16, 0, 0);
}

template <typename ACT, int KPL>
struct TokenIO;

template <int KPL>
struct TokenIO<ActF32, KPL> {
  static constexpr int kVec = KPL / 4;                 // 16-byte vectors per lane
  using raw_t = float4;
  static __device__ __forceinline__ void load_raw(const void* base, int64_t off, raw_t (&r)[kVec]) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int q = 0; q < kVec; ++q) r[q] = p[q];
  }
  static __device__ __forceinline__ void unpack(const raw_t (&r)[kVec], float (&v)[KPL]) {
#pragma unroll
    for (int q = 0; q < kVec; ++q) {
      v[4 * q + 0] = r[q].x; v[4 * q + 1] = r[q].y; v[4 * q + 2] = r[q].z; v[4 * q + 3] = r[q].w;
    }
  }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float (&v)[KPL]) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
#pragma unroll
    for (int q = 0; q < kVec; ++q)
      p[q] = make_float4(v[4 * q + 0], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
};

template <int KPL>
struct TokenIO<ActBF16, KPL> {
  static constexpr int kVec = KPL / 8;
  using raw_t = uint4;
  static __device__ __forceinline__ void load_raw(const void* base, int64_t off, raw_t (&r)[kVec]) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int q = 0; q < kVec; ++q) r[q] = p[q];
  }
  static __device__ __forceinline__ void unpack(const raw_t (&r)[kVec], float (&v)[KPL]) {
#pragma unroll
    for (int q = 0; q < kVec; ++q) {
      v[8 * q + 0] = bf16_lo(r[q].x); v[8 * q + 1] = bf16_hi(r[q].x);
      v[8 * q + 2] = bf16_lo(r[q].y); v[8 * q + 3] = bf16_hi(r[q].y);
      v[8 * q + 4] = bf16_lo(r[q].z); v[8 * q + 5] = bf16_hi(r[q].z);
      v[8 * q + 6] = bf16_lo(r[q].w); v[8 * q + 7] = bf16_hi(r[q].w);
    }
  }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float (&v)[KPL]) {
    uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off);
#pragma unroll
    for (int q = 0; q < kVec; ++q) {
      uint4 x;
      x.x = pack_bf16x2(v[8 * q + 0], v[8 * q + 1]);
      x.y = pack_bf16x2(v[8 * q + 2], v[8 * q + 3]);
      x.z = pack_bf16x2(v[8 * q + 4], v[8 * q + 5]);
      x.w = pack_bf16x2(v[8 * q + 6], v[8 * q + 7]);
      p[q] = x;
    }
  }
};

// ---- B/C packing pre-pass --------------------------------------------------
// Workspace layout, float32: [b][chunk][n][m = B, C][q][i][r] with token
// t = chunk*CH + i*KPL + 4q + r (zero past L).  One block [q][i][r] is 4*CH
// bytes; a step tile (kNB states x {B, C}) is kNB*2 consecutive blocks.
// One thread per (b, token quad, matrix, group of 4 states): it reads 4 states of
// 4 consecutive token rows (four threads cover a quad's rows, so a wave reads one
// contiguous span when N == 16) and writes one float4 of 4 tokens per state.
template <typename ACT, int KPL>
__global__ __launch_bounds__(64) void pack_bc_kernel(const void* __restrict__ Bm, const void* __restrict__ Cm,
                                                     float4* __restrict__ ws, int64_t batch, int64_t L, int N,
                                                     int64_t nchunks, int vec4) {
  constexpr int CH = 64 * KPL;
  const int nsq = (N + 3) / 4;                           // state groups
  const int64_t quads = nchunks * (CH / 4);              // token quads per batch row (padded)
  const int64_t total = batch * quads * 2 * nsq;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int sq = static_cast<int>(g % nsq);
    const int m = static_cast<int>((g / nsq) % 2);
    const int64_t gq = (g / (2 * nsq)) % quads;          // token quad within the batch row
    const int64_t b = g / (2 * nsq * quads);
    const int64_t t0 = gq * 4;
    const int64_t c = t0 / CH;
    const int tc = static_cast<int>(t0 - c * CH);        // token within the chunk
    const int i = tc / KPL;
    const int q = (tc % KPL) / 4;
    const int n0 = sq * 4;
    const void* src = m == 0 ? Bm : Cm;
    const int64_t stride = 2 * (CH / 4);                 // float4 between consecutive states
    float4* dst = ws + ((b * nchunks + c) * N * 2 + m) * (CH / 4) + q * 64 + i + n0 * stride;
    float4 r4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = t0 + r;
      const int64_t o = (b * L + (t < L ? t : 0)) * N + n0;
      float4 x;
      if (vec4) {                                        // N % 4 == 0 and 4-state aligned rows
        if constexpr (ACT::kBytes == 4) {
          x = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + o);
        } else {
          const uint2 w2 = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + o);
          x = make_float4(bf16_lo(w2.x), bf16_hi(w2.x), bf16_lo(w2.y), bf16_hi(w2.y));
        }
      } else {
        x.x = n0 + 0 < N ? load_act<ACT>(src, o + 0) : 0.f;
        x.y = n0 + 1 < N ? load_act<ACT>(src, o + 1) : 0.f;
        x.z = n0 + 2 < N ? load_act<ACT>(src, o + 2) : 0.f;
        x.w = n0 + 3 < N ? load_act<ACT>(src, o + 3) : 0.f;
      }
      r4[r] = t < L ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    dst[0] = make_float4(r4[0].x, r4[1].x, r4[2].x, r4[3].x);
    if (n0 + 1 < N) dst[stride] = make_float4(r4[0].y, r4[1].y, r4[2].y, r4[3].y);
    if (n0 + 2 < N) dst[2 * stride] = make_float4(r4[0].z, r4[1].z, r4[2].z, r4[3].z);
    if (n0 + 3 < N) dst[3 * stride] = make_float4(r4[0].w, r4[1].w, r4[2].w, r4[3].w);
  }
}

// ---- the scan ----------------------------------------------------------------
// NBLK > 0: N == 4 * NBLK, fixed at compile time; the steps of a chunk are
// unrolled (so every prefetch register is consumed before it is refilled within
// one loop iteration, and the compiler's wait tracking stays exact) and the
// per-state values sit in scalar registers.  NBLK = 0: any N, steps in a runtime
// loop.
template <typename ACT, bool GATE, int KPL, bool VEC, int NBLK>
__global__ __launch_bounds__(kThreads) void scan_chunked_kernel(ScanArgs p, int n_dblk) {
  // states processed two at a time where the registers allow it (8 tokens per lane)
  constexpr bool PAIR = KPL <= 8;
  using IO = TokenIO<ACT, KPL>;
  using raw_t = typename IO::raw_t;
  constexpr int CH = 64 * KPL;
  constexpr int BLK4 = CH / 4;                       // float4 per (state, matrix) block
  constexpr int TILE4 = kNB * 2 * BLK4;              // float4 per step tile
  constexpr int ZBYTES = KPL * ACT::kBytes * 64;     // z of one chunk for one wave
  // Two distinct objects, so the compiler can tell the buffer being read from the
  // one being filled (a DMA into one never forces a wait before reading the other).
  __shared__ float4 s_tile0[TILE4];
  __shared__ float4 s_tile1[TILE4];
  __shared__ float4 s_z[(GATE && VEC) ? kW * ZBYTES / 16 : 1];

  const int lane = threadIdx.x & 63;
  const bool lane0 = lane == 0;
  const int w = uniform_int(threadIdx.x >> 6);
  // Consecutive workgroups go to different XCDs (round robin over 8); taking the
  // batch row as blk % batch keeps one row per XCD when batch divides 8, so each
  // XCD's L2 holds only that row's packed B/C tiles.
  const int blk = blockIdx.x;
  const int64_t b = blk % p.batch;
  const int64_t d = static_cast<int64_t>(blk / p.batch) * kW + w;
  const bool valid = d < p.D;                        // wave-uniform
  const int N = p.N;
  const int64_t L = p.L;
  const int64_t row = (b * p.D + (valid ? d : 0)) * L;
  const float bias = (valid && p.bias) ? p.bias[d] : 0.0f;
  const float dsk = (valid && p.Dskip) ? p.Dskip[d] : 0.0f;
  // A[d, n] * log2(e) in lane n (read once, before any store, so the state loop
  // never issues a vector load of A).
  const float a2_v = (valid && lane < N) ? p.A[d * N + lane] * kLog2e : 0.0f;
  float carry_v = 0.0f;                              // carry of state n lives in lane n

  const int nblk = NBLK > 0 ? NBLK : (N + kNB - 1) / kNB;
  const int64_t nchunks = (L + CH - 1) / CH;
  const int64_t nsteps = nchunks * nblk;
  const float4* ws = reinterpret_cast<const float4*>(p.workspace) + b * nchunks * N * 2 * BLK4;

  float dl[KPL], du[KPL], yv[KPL];
  float sdl = 0.0f;
  int nv = KPL;                                      // valid tokens of this lane in its chunk
  raw_t u_raw[IO::kVec], d_raw[IO::kVec];            // next chunk's u and delta

  // Issue the loads of chunk c's u (or delta) for full lanes of the vector path.
  auto prefetch_act = [&](const void* src, int64_t c, raw_t (&dst)[IO::kVec]) {
    const int64_t tl = c * CH + static_cast<int64_t>(lane) * KPL;
    if (VEC && tl + KPL <= L) IO::load_raw(src, row + tl, dst);
  };
  // Copy chunk c's z for this wave into LDS: DMA q moves this lane's 16-byte
  // vector q to s_z + w*ZBYTES + q*1024 + 16*lane.  Vectors at or past L read a
  // valid address (their values are never used).
  auto prefetch_z = [&](int64_t c) {
    if constexpr (GATE && VEC) {
      const int64_t tl = c * CH + static_cast<int64_t>(lane) * KPL;
#pragma unroll
      for (int q = 0; q < IO::kVec; ++q) {
        const int64_t t = tl + q * (16 / ACT::kBytes);
        const int64_t off = (t < L ? row + t : 0) * ACT::kBytes;
        dma16(static_cast<const char*>(p.z) + off, reinterpret_cast<char*>(s_z) + w * ZBYTES + q * 1024);
      }
    }
  };

  // Per-token work of chunk c, once for all N states.
  auto prologue = [&](int64_t c) {
    const int64_t tl = c * CH + static_cast<int64_t>(lane) * KPL;
    const int64_t rem = L - tl;
    nv = rem >= KPL ? KPL : (rem > 0 ? static_cast<int>(rem) : 0);
    float uv[KPL];
    if (VEC && nv == KPL) {
      IO::unpack(u_raw, uv);
      IO::unpack(d_raw, dl);
    } else {
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const bool ok = j < nv;
        uv[j] = ok ? load_act<ACT>(p.u, row + tl + j) : 0.0f;
        dl[j] = ok ? load_act<ACT>(p.delta, row + tl + j) : 0.0f;
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
      du[j] = dl[j] * uv[j];
      yv[j] = dsk * uv[j];
      sdl += dl[j];
    }
  };

  auto epilogue = [&](int64_t c) {
    const int64_t tl = c * CH + static_cast<int64_t>(lane) * KPL;
    if (GATE) {
      float zv[KPL];
      if (VEC) {
        raw_t zr[IO::kVec];
        const raw_t* zs = reinterpret_cast<const raw_t*>(reinterpret_cast<const char*>(s_z) + w * ZBYTES);
#pragma unroll
        for (int q = 0; q < IO::kVec; ++q) zr[q] = zs[q * 64 + lane];
        IO::unpack(zr, zv);
      } else {
#pragma unroll
        for (int j = 0; j < KPL; ++j) zv[j] = j < nv ? load_act<ACT>(p.z, row + tl + j) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < KPL; ++j) yv[j] *= silu_f(zv[j]);
    }
    if (VEC && nv == KPL) {
      IO::store(p.y, row + tl, yv);
    } else {
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        if (j < nv) store_act<ACT>(p.y, row + tl + j, yv[j]);
    }
  };

  // One state over the current chunk: its B and C blocks are sB, sC in LDS,
  // a2 = A[d, n] * log2(e) and `carry` (the state before the chunk) are
  // wave-uniform.  Returns the state after the chunk (lane 63's).
  auto scan_one = [&](const float4* __restrict__ sB, const float4* __restrict__ sC, float a2,
                      float carry) -> float {
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
        bv[j] = du[j] * bs[r];
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
  auto scan_two = [&](const float4* __restrict__ sB0, const float4* __restrict__ sC0, float a20, float carry0,
                      const float4* __restrict__ sB1, const float4* __restrict__ sC1, float a21, float carry1,
                      float& out0, float& out1) {
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
        bv0[j] = du[j] * bs0[r];
        bv1[j] = du[j] * bs1[r];
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
  auto scan_state = [&](const float4* sB, const float4* sC, int n) {
    const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a2_v), n));
    const float carry = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, carry_v), n));
    const float cnew = scan_one(sB, sC, a2, carry);
    carry_v = (lane == n) ? cnew : carry_v;
  };

  // Tile of step k = (chunk k / nblk, states n0 = (k % nblk) * kNB ...) is the
  // contiguous run of float4 at ws + (c * N + n0) * 2 * BLK4 covering min(kNB,
  // N - n0) states.  Thread t moves float4 t, t + kThreads, ...: loaded into
  // registers at the start of a step, written to LDS at its end (a plain vector
  // load plus an LDS store is far cheaper to issue than a direct global->LDS copy).
  constexpr int TPT = (TILE4 + kThreads - 1) / kThreads;    // tile float4 per thread
  static_assert(TPT <= 3, "tile share per thread held in three registers");
  float4 tr0 = make_float4(0.f, 0.f, 0.f, 0.f), tr1 = tr0, tr2 = tr0;
  int tile_n4 = 0;                                           // float4 in the prefetched tile
  const int e0 = threadIdx.x, e1 = threadIdx.x + kThreads, e2 = threadIdx.x + 2 * kThreads;
  auto load_tile = [&](int64_t k) {
    const int64_t c = k / nblk;
    const int n0 = static_cast<int>(k % nblk) * kNB;
    tile_n4 = ((N - n0 < kNB) ? (N - n0) : kNB) * 2 * BLK4;
    const float4* src = ws + (c * N + n0) * 2 * BLK4;
    // Unconditional loads (indices clamped into the tile; the surplus values are
    // never stored) so the compiler cannot sink them to their use after the
    // state loop, which would expose their latency at the end of every step.
    tr0 = src[e0 < tile_n4 ? e0 : tile_n4 - 1];
    if (TPT > 1) tr1 = src[e1 < tile_n4 ? e1 : tile_n4 - 1];
    if (TPT > 2) tr2 = src[e2 < tile_n4 ? e2 : tile_n4 - 1];
    asm volatile("" ::: "memory");                 // compiler-only fence: keep the loads here
  };
  auto store_tile = [&](float4* dst) {
    if (e0 < tile_n4) dst[e0] = tr0;
    if (TPT > 1 && e1 < tile_n4) dst[e1] = tr1;
    if (TPT > 2 && e2 < tile_n4) dst[e2] = tr2;
  };

  // Every barrier first waits for all of this wave's outstanding memory
  // operations (the copies into LDS must have landed before any wave reads the
  // tile, and they are tracked by the same counter as the HBM loads, with no
  // ordering between the two kinds).  So a load issued in a step lands within that
  // step, and a chunk's HBM traffic is spread over its steps, one kind per step:
  // y of the previous chunk is stored at step 0, the next chunk's u is loaded at
  // step 1, its delta at step 2 and this chunk's z at step 3.
  const int st_u = nblk > 1 ? 1 : 0;
  const int st_d = nblk > 2 ? 2 : st_u;
  const int st_z = nblk > 3 ? 3 : st_d;

  // Per-state wave-uniform values when the state count is fixed at compile time
  // (NBLK > 0): A*log2(e) and the carry of state n in scalar registers, indexed
  // by compile-time n once the steps are unrolled.
  constexpr int NS = NBLK > 0 ? 4 * NBLK : 1;
  float a2s[NS], cs[NS];
  if constexpr (NBLK > 0) {
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      a2s[n] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a2_v), n));
      cs[n] = 0.0f;
    }
  }

  // The states of step nb of the current chunk, from the tile `cur`.
  auto states = [&](const float4* cur, int nb) {
    const int n0 = nb * kNB;
    if constexpr (NBLK > 0) {
      constexpr int nn = kNB;                          // N == 4 * NBLK: every step is full
      const float4* t = cur;
      if constexpr (PAIR) {
#pragma unroll
        for (int nl = 0; nl < kNB; nl += 2) {
          const int n = n0 + nl;
          if (nl + 1 < nn) {
            scan_two(t + nl * 2 * BLK4, t + (nl * 2 + 1) * BLK4, a2s[n], cs[n],
                     t + (nl * 2 + 2) * BLK4, t + (nl * 2 + 3) * BLK4, a2s[n + 1], cs[n + 1], cs[n], cs[n + 1]);
          } else if (nl < nn) {
            cs[n] = scan_one(t + nl * 2 * BLK4, t + (nl * 2 + 1) * BLK4, a2s[n], cs[n]);
          }
        }
      } else {
#pragma unroll
        for (int nl = 0; nl < kNB; ++nl) {
          const int n = n0 + nl;
          if (nl < nn) cs[n] = scan_one(t + nl * 2 * BLK4, t + (nl * 2 + 1) * BLK4, a2s[n], cs[n]);
        }
      }
    } else {
      const int nn = (N - n0 < kNB) ? (N - n0) : kNB;
      for (int nl = 0; nl < nn; ++nl) scan_state(cur + nl * 2 * BLK4, cur + (nl * 2 + 1) * BLK4, n0 + nl);
    }
  };

  // Step k (state block nb of chunk c) computes on `cur` while the next step's
  // tile lands in `nxt`.
  auto step = [&](int64_t k, int64_t c, int nb, const float4* cur, float4* nxt) {
    if (valid && nb == 0) {
      if (c > 0) epilogue(c - 1);                    // z of c-1 landed during chunk c-1
      prologue(c);                                   // u, delta of c prefetched during c-1
    }
    if (k + 1 < nsteps) load_tile(k + 1);
    __builtin_amdgcn_sched_barrier(0);               // issue the tile loads now, not at their use
    if (valid) {
      if (c + 1 < nchunks && nb == st_u) prefetch_act(p.u, c + 1, u_raw);
      if (c + 1 < nchunks && nb == st_d) prefetch_act(p.delta, c + 1, d_raw);
      if (nb == st_z) prefetch_z(c);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (valid) states(cur, nb);
    if (k + 1 < nsteps) store_tile(nxt);
    __syncthreads();                                 // publishes the tile; waits for all loads
  };

  if (valid) {
    prefetch_act(p.u, 0, u_raw);
    prefetch_act(p.delta, 0, d_raw);
  }
  load_tile(0);
  store_tile(s_tile0);
  __syncthreads();
  if constexpr (NBLK > 0 && NBLK % 2 == 0) {
    for (int64_t c = 0; c < nchunks; ++c) {
#pragma unroll
      for (int nb = 0; nb < NBLK; nb += 2) {
        step(c * NBLK + nb, c, nb, s_tile0, s_tile1);
        step(c * NBLK + nb + 1, c, nb + 1, s_tile1, s_tile0);
      }
    }
  } else {
    for (int64_t k = 0; k < nsteps; k += 2) {
      step(k, k / nblk, static_cast<int>(k % nblk), s_tile0, s_tile1);
      if (k + 1 < nsteps) step(k + 1, (k + 1) / nblk, static_cast<int>((k + 1) % nblk), s_tile1, s_tile0);
    }
  }
  if constexpr (NBLK > 0) {
    // carries back into lane n for the final-state store
#pragma unroll
    for (int n = 0; n < NS; ++n) carry_v = lane == n ? cs[n] : carry_v;
  }
  if (valid) {
    epilogue(nchunks - 1);
    if (p.final_state && lane < N) p.final_state[(b * p.D + d) * N + lane] = carry_v;
  }
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

template <typename ACT, bool GATE, int KPL>
hipError_t launch_kpl(const ScanArgs& a, hipStream_t s) {
  constexpr int CH = 64 * KPL;
  const int64_t nchunks = (a.L + CH - 1) / CH;
  const int64_t pack_threads = a.batch * nchunks * (CH / 4) * 2 * ((a.N + 3) / 4);
  const int pack_blocks = static_cast<int>(std::min<int64_t>((pack_threads + 63) / 64, 1 << 20));
  const int vec4 = (a.N % 4 == 0) && (reinterpret_cast<uintptr_t>(a.Bm) % (4 * ACT::kBytes) == 0) &&
                   (reinterpret_cast<uintptr_t>(a.Cm) % (4 * ACT::kBytes) == 0);
  hipLaunchKernelGGL((pack_bc_kernel<ACT, KPL>), dim3(pack_blocks), dim3(64), 0, s, a.Bm, a.Cm,
                     reinterpret_cast<float4*>(a.workspace), a.batch, a.L, a.N, nchunks, vec4);
  const int n_dblk = static_cast<int>((a.D + kW - 1) / kW);
  const int64_t blocks = a.batch * n_dblk;
  const bool vec = (a.L % 8 == 0) && aligned16(a.u) && aligned16(a.delta) && aligned16(a.y) &&
                   (a.z == nullptr || aligned16(a.z));
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  const bool n16 = a.N == 16;
  if (vec && n16)
    hipLaunchKernelGGL((scan_chunked_kernel<ACT, GATE, KPL, true, 4>), grid, block, 0, s, a, n_dblk);
  else if (vec)
    hipLaunchKernelGGL((scan_chunked_kernel<ACT, GATE, KPL, true, 0>), grid, block, 0, s, a, n_dblk);
  else if (n16)
    hipLaunchKernelGGL((scan_chunked_kernel<ACT, GATE, KPL, false, 4>), grid, block, 0, s, a, n_dblk);
  else
    hipLaunchKernelGGL((scan_chunked_kernel<ACT, GATE, KPL, false, 0>), grid, block, 0, s, a, n_dblk);
  return hipGetLastError();
}

template <typename ACT, bool GATE>
hipError_t launch_gate(const ScanArgs& a, int kpl, hipStream_t s) {
  if (kpl == 8) return launch_kpl<ACT, GATE, 8>(a, s);
  return launch_kpl<ACT, GATE, 16>(a, s);
}

// Default tokens per lane, from measurement on gfx950: with float32 activations
// 8 tokens per lane (no register spills) beats 16; with bfloat16, 16 (half the
// wave-scan overhead per element) wins.
int resolve_kpl(int tokens_per_lane, Dt dt) {
  if (tokens_per_lane != 0) return tokens_per_lane;
  return dt == Dt::F32 ? 8 : 16;
}

}  // namespace

size_t chunked_workspace_bytes(int64_t batch, int64_t L, int64_t N, int tokens_per_lane) {
  // 0 = whichever default the launch picks: size for the larger chunk (16 tokens per lane)
  const int64_t ch = 64 * (tokens_per_lane == 0 ? 16 : tokens_per_lane);
  const int64_t nchunks = (L + ch - 1) / ch;
  return static_cast<size_t>(batch) * nchunks * N * 2 * ch * sizeof(float);
}

bool chunked_supported(const ScanArgs& a, Dt, int tokens_per_lane) {
  if (!(tokens_per_lane == 0 || tokens_per_lane == 8 || tokens_per_lane == 16)) return false;
  if (a.N < 1 || a.N > 64) return false;
  const int64_t n_dblk = (a.D + kW - 1) / kW;
  return a.batch * n_dblk <= 0x7fffffff;
}

hipError_t launch_scan_chunked(const ScanArgs& a, Dt dt, int tokens_per_lane, hipStream_t s) {
  if (!chunked_supported(a, dt, tokens_per_lane) || a.workspace == nullptr) return hipErrorInvalidValue;
  const int kpl = resolve_kpl(tokens_per_lane, dt);
  const bool gate = a.z != nullptr;
  if (dt == Dt::F32)
    return gate ? launch_gate<ActF32, true>(a, kpl, s) : launch_gate<ActF32, false>(a, kpl, s);
  return gate ? launch_gate<ActBF16, true>(a, kpl, s) : launch_gate<ActBF16, false>(a, kpl, s);
}

}  // namespace ssm
