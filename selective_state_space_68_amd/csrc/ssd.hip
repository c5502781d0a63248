// Mamba-2 SSD scan (scalar decay per head) for gfx950, on the matrix cores.
//
// Per head h the state is a P x N matrix and the recurrence is
//     H_t = a_t H_{t-1} + Delta_t x_t B_t^T,   a_t = exp(Delta_t A_h),   y_t = H_t C_t + D_h x_t
// (the slide deck's "Mamba-2" table; the interview-prep page's "Mamba-2 and State
// Space Duality").  Over a chunk of Q = 64 tokens it unrolls into the chunk-parallel
// form of the prep page's table: with cum_j = sum_{k<=j} Delta_k A_h inside the chunk,
//     Y = (C B^T o M) (Delta x)          M[j][i] = exp(cum_j - cum_i) for i <= j, else 0
//       + diag(exp(cum_j)) C H_in^T      (the state carried in from earlier chunks)
//       + D x
//     H_out = exp(cum_{Q-1}) H_in + x^T diag(exp(cum_{Q-1} - cum_i) Delta_i) B
// i.e. four small matrix products per chunk (C B^T, its masked product with x, the
// chunk's state contribution and the product with the carried state), which run
// on MFMA; only the P x N state crosses chunks, in registers.
//
// Work decomposition: one workgroup of 4 waves per (batch row, head, segment) walks
// its segment of the sequence chunk by chunk.  With one segment per sequence there
// are too few waves to hide latency (one per SIMD at the model shapes), so the
// sequence is cut into segments: a pre-pass computes each segment's end state from
// zero, a small kernel chains them into each segment's entering state (the operator
// of the forward recurrence on whole segments), and the main pass runs every
// segment from its entering state.  Within a workgroup, wave w owns head channels p in [16w, 16w+16) of the
// products with x, H and y, and rows j in [16w, 16w+16) of C B^T.  The chunk's x, B
// and C go through LDS as bfloat16 (x and B also transposed, so every MFMA operand
// is a contiguous 16-byte LDS read), and the next chunk's inputs are loaded into
// registers while the current one computes.  Inputs are bfloat16; the products
// accumulate in float32 and the state stays float32 (it is rounded to bfloat16
// only as the operand of the carried-state product).
//
// MFMA lane layouts (gfx950, checked on the device): for v_mfma_f32_16x16x32_bf16,
// lane l holds A[m = l%16][k = 8(l/16) .. +7], B[k = 8(l/16) .. +7][n = l%16] and
// D[m = 4(l/16) + e][n = l%16]; v_mfma_f32_16x16x16_bf16 the same with 4 k per lane.
// The D layout of a 16 x 16 tile equals the 16x16x16 B-operand layout, so the state
// produced by one product feeds the next without a shuffle.
#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_common.hpp"

namespace ssm {
namespace {

constexpr int kQ = 64;            // tokens per chunk
constexpr int kP = 64;            // head channels (4 waves x 16)
constexpr int kPad = 8;           // bfloat16 elements of row padding in LDS

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(const uint2& a, const uint2& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b), c,
                                                   0, 0, 0);
}

// Inclusive prefix sum over the 64 lanes (Kogge-Stone with row shifts and the row
// broadcasts; lanes whose source is outside the row add 0).
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp_mov<0x111, 0xf, true>(0.0f, v);
  v += dpp_mov<0x112, 0xf, true>(0.0f, v);
  v += dpp_mov<0x114, 0xf, true>(0.0f, v);
  v += dpp_mov<0x118, 0xf, true>(0.0f, v);
  v += dpp_mov<0x142, 0xa, false>(0.0f, v);
  v += dpp_mov<0x143, 0xc, false>(0.0f, v);
  return v;
}

__device__ __forceinline__ uint32_t bf16x2(float lo, float hi) { return pack_bf16x2(lo, hi); }
__device__ __forceinline__ float bf16_at(const uint16_t* p) { return __uint_as_float(static_cast<uint32_t>(*p) << 16); }

// One chunk's inputs in registers (prefetch): thread t moves the 16-byte pieces
// v = t + 256 k of the 64-token tiles of x (8 channels per piece: token v / 8, piece
// v % 8) and of B and C (8 states per piece), so 8 consecutive lanes read one token's
// contiguous row.
template <int NS>
struct ChunkRegs {
  static constexpr int kXV = kQ * kP / 8 / 256;     // x pieces per thread (2)
  static constexpr int kBV = kQ * NS / 8 / 256;     // B (and C) pieces per thread
  uint4 x[kXV], b[kBV], c[kBV];
  float dt;                                          // raw Delta of token `lane` (each wave loads it)
};

// STATE_ONLY: the pre-pass of the segmented form: the segment's end state from a
// zero start (x, B and Delta only; no C, no output), written to the workspace.
// Otherwise the full scan of the segment's chunks from its entering state: the
// initial state for segment 0, else the combined state in the workspace.
template <int NS, bool STATE_ONLY>
__global__ __launch_bounds__(256) void ssd_scan_kernel(SsdArgs p) {
  constexpr int RX = kQ + kPad;                     // row stride of [.][Q] arrays
  constexpr int RN = NS + kPad;                     // row stride of [.][N] arrays
  constexpr int NT = NS / 16;                       // 16-row tiles of the state
  __shared__ __attribute__((aligned(16))) uint16_t sXT[kP * RX];    // x^T [p][i]
  __shared__ __attribute__((aligned(16))) uint16_t sB[kQ * RN];     // B [i][n]
  __shared__ __attribute__((aligned(16))) uint16_t sBwT[NS * RX];   // (B diag(w))^T [n][i]
  __shared__ __attribute__((aligned(16))) uint16_t sC[kQ * RN];     // C [j][n]
  __shared__ __attribute__((aligned(16))) uint16_t sS[kQ * RX];     // (C B^T o M) Delta [j][i]
  __shared__ __attribute__((aligned(16))) uint16_t sY[kQ * RX];     // y [j][p] staging
  __shared__ float sCum[kQ], sDl[kQ], sEc[kQ];
  // [row][token] arrays written transposed (x^T, B^T) place the 8-token block b of
  // row r at block b ^ ((r / 8) % 8): the 8 rows one instruction writes for one
  // token then fall in 8 different banks, and every 8-token block stays a contiguous,
  // aligned 16-byte MFMA operand.
  auto swz = [](int r, int i) __attribute__((always_inline)) { return r * RX + (i ^ (((r >> 3) & 7) << 3)); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform_int(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t H = p.H, L = p.L;
  const int nseg = p.nseg;
  const int64_t bh = blockIdx.x / nseg;
  const int seg = static_cast<int>(blockIdx.x % nseg);
  const int64_t b = bh / H, h = bh % H;
  const float A2 = p.A[h] * kLog2e;                 // decay exponent in base 2
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
  const float dsk = p.Dskip ? p.Dskip[h] : 0.0f;
  const int64_t nchunks = (L + kQ - 1) / kQ;
  const int64_t c_begin = seg * p.seg_chunks;
  const int64_t c_end = c_begin + p.seg_chunks < nchunks ? c_begin + p.seg_chunks : nchunks;
  // [batch][H][nseg][P][N]: the pre-pass writes segment s's own end state into slot
  // s; the combine replaces it with the state entering segment s + 1, and puts the
  // initial state into the last slot (so that no workgroup of the main pass reads
  // the initial state, which the final state may overwrite in place)
  float* seg_state = p.seg_state ? p.seg_state + (bh * nseg) * kP * NS : nullptr;
  if (STATE_ONLY && seg == nseg - 1) return;         // the last segment's own state is not needed
  const int64_t xrow = H * kP;                      // elements between consecutive tokens of x / y
  const uint16_t* xg = static_cast<const uint16_t*>(p.x) + (b * L * H + h) * kP;
  const uint16_t* bg = static_cast<const uint16_t*>(p.Bm) + b * L * NS;
  const uint16_t* cg = static_cast<const uint16_t*>(p.Cm) + b * L * NS;
  const uint16_t* dtg = static_cast<const uint16_t*>(p.dt) + b * L * H + h;
  uint16_t* yg = static_cast<uint16_t*>(p.y) + (b * L * H + h) * kP;

  // State H[p][n] for p = 16w + c16, n = 16 mt + 4g + e: tile mt, element e.
  f32x4_t Hs[NT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
    const int64_t off = (16 * w + c16) * NS + 16 * mt + 4 * g;
    const float* src = nullptr;
    if (!STATE_ONLY) {
      if (nseg == 1) src = p.h0 ? p.h0 + (b * H + h) * kP * NS : nullptr;
      else src = seg_state + static_cast<int64_t>(seg == 0 ? nseg - 1 : seg - 1) * kP * NS;
    }
    if (src) {
      const float4 v = *reinterpret_cast<const float4*>(src + off);
      Hs[mt] = f32x4_t{v.x, v.y, v.z, v.w};
    } else {
      Hs[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  float log_decay = 0.0f;                           // the segment's total decay exponent (base 2)

  using CR = ChunkRegs<NS>;
  CR cr;
  // Loads of chunk c into registers; tokens past L read as zero.  No load sits
  // behind a branch (rows past L reload the last row and are then replaced by zero),
  // so the loads issued for the next chunk stay in flight during this one.
  auto fetch = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t t0 = c * kQ;
    const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < CR::kXV; ++k) {
      const int v = tid + 256 * k, i = v >> 3, q = v & 7;
      const int64_t t = t0 + i < L ? t0 + i : L - 1;
      const uint4 r = *reinterpret_cast<const uint4*>(xg + t * xrow + 8 * q);
      cr.x[k] = t0 + i < L ? r : zero;
    }
#pragma unroll
    for (int k = 0; k < CR::kBV; ++k) {
      const int v = tid + 256 * k, i = v / (NS / 8), q = v % (NS / 8);
      const int64_t t = t0 + i < L ? t0 + i : L - 1;
      const uint4 rb = *reinterpret_cast<const uint4*>(bg + t * NS + 8 * q);
      cr.b[k] = t0 + i < L ? rb : zero;
      if constexpr (!STATE_ONLY) {
        const uint4 rc = *reinterpret_cast<const uint4*>(cg + t * NS + 8 * q);
        cr.c[k] = t0 + i < L ? rc : zero;
      }
    }
    const int64_t tl = t0 + lane < L ? t0 + lane : L - 1;
    const float dv = bf16_at(dtg + tl * H);
    cr.dt = t0 + lane < L ? dv : 0.0f;
  };

  fetch(c_begin);
  for (int64_t c = c_begin; c < c_end; ++c) {
    const int64_t t0 = c * kQ;
    // ---- 1. Delta and the cumulative decay exponent (every wave, lane = token); the
    // chunk's tiles into LDS
    float dl = cr.dt + bias;
    if (p.softplus) dl = softplus_f(dl);
    dl = t0 + lane < L ? dl : 0.0f;                 // padding tokens: no decay, no input
    const float cum = wave_prefix_sum(dl * A2);     // in base-2 exponent units
    const float cum_last = wave_lane63(cum);
    // weight of token `lane` in the chunk's state contribution
    const float wgt = exp2_hw(cum_last - cum) * dl;
    if (w == 0) {
      sCum[lane] = cum;
      sDl[lane] = dl;
      sEc[lane] = exp2_hw(cum);                     // decay of the carried state up to token `lane`
    }
    {
      const uint16_t* e;
#pragma unroll
      for (int k = 0; k < CR::kXV; ++k) {
        const int v = tid + 256 * k, i = v >> 3, q = v & 7;
        e = reinterpret_cast<const uint16_t*>(&cr.x[k]);
#pragma unroll
        for (int r = 0; r < 8; ++r) sXT[swz(8 * q + r, i)] = e[r];
      }
#pragma unroll
      for (int k = 0; k < CR::kBV; ++k) {
        const int v = tid + 256 * k, i = v / (NS / 8), q = v % (NS / 8);
        if constexpr (!STATE_ONLY) {
          *reinterpret_cast<uint4*>(&sB[i * RN + 8 * q]) = cr.b[k];
          *reinterpret_cast<uint4*>(&sC[i * RN + 8 * q]) = cr.c[k];
        }
        // B^T scaled by the token weights, for the state contribution
        const float wi = __shfl(wgt, i);
        const uint32_t rw[4] = {cr.b[k].x, cr.b[k].y, cr.b[k].z, cr.b[k].w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sBwT[swz(8 * q + 2 * r, i)] = to_bf16(bf16_lo(rw[r]) * wi);
          sBwT[swz(8 * q + 2 * r + 1, i)] = to_bf16(bf16_hi(rw[r]) * wi);
        }
      }
    }
    fetch(c + 1 < c_end ? c + 1 : c);                // (the last chunk reloads itself, unused)
    log_decay += cum_last;
    barrier_lds();

    // ---- 2. S' = (C B^T o M) Delta for rows j of this wave; the chunk's state
    // contribution; the output from the carried state
    if constexpr (!STATE_ONLY) {
      f32x4_t S[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) S[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < NS / 32; ++kb) {
        const uint4 a = *reinterpret_cast<const uint4*>(&sC[(16 * w + c16) * RN + 32 * kb + 8 * g]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const uint4 bo = *reinterpret_cast<const uint4*>(&sB[(16 * nt + c16) * RN + 32 * kb + 8 * g]);
          S[nt] = mfma32(a, bo, S[nt]);
        }
      }
      // mask and scale: element (j = 16w + 4g + e, i = 16nt + c16)
      float cj[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) cj[e] = sCum[16 * w + 4 * g + e];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int i = 16 * nt + c16;
        const float ci = sCum[i], di = sDl[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * w + 4 * g + e;
          // (computed for every element, then selected: no branch per element)
          float v = S[nt][e] * exp2_hw(fminf(cj[e] - ci, 0.0f)) * di;
          asm volatile("" : "+v"(v));
          sS[j * RX + i] = to_bf16(j >= i ? v : 0.0f);
        }
      }
    }
    // the chunk's state contribution st[n][p] = sum_i B[i][n] w_i x[i][p],
    // w_i = exp(cum_last - cum_i) Delta_i (folded into the LDS copy of B^T)
    f32x4_t st[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) st[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint4 xo = *reinterpret_cast<const uint4*>(&sXT[swz(16 * w + c16, 32 * kb + 8 * g)]);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const uint4 a = *reinterpret_cast<const uint4*>(&sBwT[swz(16 * mt + c16, 32 * kb + 8 * g)]);
        st[mt] = mfma32(a, xo, st[mt]);
      }
    }
    if constexpr (STATE_ONLY) {
      const float decay = exp2_hw(cum_last);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) Hs[mt][e] = __builtin_fmaf(decay, Hs[mt][e], st[mt][e]);
      barrier_lds();                                // every wave is done with this chunk's LDS
      continue;
    }
    // output from the carried state: Yc[j][p] = sum_n C[j][n] H[p][n] (16x16x16: the
    // state tiles are the B operands as they are).  The float32 state is split into
    // two bfloat16 terms, hi + lo, so the product keeps ~16 bits of the state.
    f32x4_t Yc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) Yc[jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      float hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = __uint_as_float(static_cast<uint32_t>(to_bf16(Hs[mt][e])) << 16);
        lo[e] = Hs[mt][e] - hi[e];
      }
      const uint2 hb = make_uint2(bf16x2(hi[0], hi[1]), bf16x2(hi[2], hi[3]));
      const uint2 lb = make_uint2(bf16x2(lo[0], lo[1]), bf16x2(lo[2], lo[3]));
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const uint2 a = *reinterpret_cast<const uint2*>(&sC[(16 * jt + c16) * RN + 16 * mt + 4 * g]);
        Yc[jt] = mfma16(a, hb, Yc[jt]);
        Yc[jt] = mfma16(a, lb, Yc[jt]);
      }
    }
    barrier_lds();                                  // S' complete

    // ---- 3. Y = S' x + exp(cum_j) Yc + D x; the state update
    f32x4_t Yo[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) Yo[jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint4 xo = *reinterpret_cast<const uint4*>(&sXT[swz(16 * w + c16, 32 * kb + 8 * g)]);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const uint4 a = *reinterpret_cast<const uint4*>(&sS[(16 * jt + c16) * RX + 32 * kb + 8 * g]);
        Yo[jt] = mfma32(a, xo, Yo[jt]);
      }
    }
    const int pcol = 16 * w + c16;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const uint2 xr = *reinterpret_cast<const uint2*>(&sXT[swz(pcol, 16 * jt + 4 * g)]);
      const float xv[4] = {bf16_lo(xr.x), bf16_hi(xr.x), bf16_lo(xr.y), bf16_hi(xr.y)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * jt + 4 * g + e;
        const float v = Yo[jt][e] + sEc[j] * Yc[jt][e] + dsk * xv[e];
        sY[j * RX + pcol] = to_bf16(v);
      }
    }
    const float decay = exp2_hw(cum_last);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) Hs[mt][e] = __builtin_fmaf(decay, Hs[mt][e], st[mt][e]);
    barrier_lds();                                  // y tile complete

    // ---- 4. y rows to memory (128 contiguous bytes per token)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int v = tid + 256 * k, j = v >> 3, q = v & 7;
      if (t0 + j < L)
        *reinterpret_cast<uint4*>(yg + (t0 + j) * xrow + 8 * q) = *reinterpret_cast<const uint4*>(&sY[j * RX + 8 * q]);
    }
  }
  float* dst = nullptr;
  if (STATE_ONLY) dst = seg_state + static_cast<int64_t>(seg) * kP * NS;
  else if (seg == nseg - 1 && p.final_state) dst = p.final_state + (b * H + h) * kP * NS;
  if (dst) {
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
      *reinterpret_cast<float4*>(dst + (16 * w + c16) * NS + 16 * mt + 4 * g) =
          make_float4(Hs[mt][0], Hs[mt][1], Hs[mt][2], Hs[mt][3]);
  }
  if (STATE_ONLY && tid == 0) p.seg_decay[bh * nseg + seg] = exp2_hw(log_decay);
}

// States entering each segment: one thread per (batch, head, state entry), a
// sequential pass over the segments: H_in(s+1) = decay(s) H_in(s) + (segment s's own
// end state), with H_in(0) the initial state.  H_in(s+1) is written over slot s of
// the workspace and H_in(0) into the last slot.
__global__ void ssd_combine_kernel(SsdArgs p, int64_t PN) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= p.batch * p.H * PN) return;
  const int64_t bh = i / PN, e = i % PN;
  float hin = p.h0 ? p.h0[i] : 0.0f;
  p.seg_state[(bh * p.nseg + p.nseg - 1) * PN + e] = hin;
  for (int s = 0; s + 1 < p.nseg; ++s) {
    float* slot = p.seg_state + (bh * p.nseg + s) * PN + e;
    hin = __builtin_fmaf(p.seg_decay[bh * p.nseg + s], hin, *slot);
    *slot = hin;
  }
}

}  // namespace

bool ssd_supported(int64_t P, int64_t N) { return P == kP && (N == 64 || N == 128); }

// Segments per sequence: enough workgroups for about three per CU (the kernel is
// latency-bound at one wave per SIMD), at least 4 chunks per segment.
int ssd_segments(int64_t batch, int64_t L, int64_t H) {
  const int64_t nch = (L + kQ - 1) / kQ;
  int64_t s = (768 + batch * H - 1) / (batch * H);
  const int64_t smax = nch / 4 > 1 ? nch / 4 : 1;
  s = s < 1 ? 1 : (s > smax ? smax : s);
  return static_cast<int>(s > 64 ? 64 : s);
}

size_t ssd_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N) {
  const int s = ssd_segments(batch, L, H);
  if (s <= 1) return 0;
  return static_cast<size_t>(batch * H * s) * (P * N + 1) * sizeof(float) + 256;
}

template <int NS>
hipError_t launch_ssd_n(SsdArgs a, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t nch = (a.L + kQ - 1) / kQ;
  int nseg = ssd_segments(a.batch, a.L, a.H);
  if (!ws || ws_bytes < ssd_workspace_bytes(a.batch, a.L, a.H, kP, NS)) nseg = 1;
  a.nseg = nseg;
  a.seg_chunks = (nch + nseg - 1) / nseg;
  a.seg_state = nullptr;
  a.seg_decay = nullptr;
  const dim3 block(256);
  if (nseg > 1) {
    a.seg_state = static_cast<float*>(ws);
    a.seg_decay = a.seg_state + a.batch * a.H * nseg * kP * NS;
    hipLaunchKernelGGL((ssd_scan_kernel<NS, true>), dim3(static_cast<unsigned>(a.batch * a.H * nseg)), block, 0, s,
                       a);
    const int64_t n = a.batch * a.H * kP * NS;
    hipLaunchKernelGGL(ssd_combine_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a,
                       static_cast<int64_t>(kP * NS));
  }
  hipLaunchKernelGGL((ssd_scan_kernel<NS, false>), dim3(static_cast<unsigned>(a.batch * a.H * nseg)), block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ssd_scan(const SsdArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  if (a.N == 64) return launch_ssd_n<64>(a, ws, ws_bytes, s);
  if (a.N == 128) return launch_ssd_n<128>(a, ws, ws_bytes, s);
  return hipErrorInvalidValue;
}

}  // namespace ssm
