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
// its segment of the sequence chunk by chunk.  When the (batch row, head) pairs are
// too few to fill one resident wave of workgroups, the sequence is cut into
// segments: a pre-pass computes each segment's end state from zero, a small kernel
// chains them into each segment's entering state (the operator of the forward
// recurrence on whole segments), and the main pass runs every segment from its
// entering state.  Within a workgroup, wave w owns head channels p in [16w, 16w+16) of the
// products with x, H and y, and rows j in [16w, 16w+16) of C B^T.  The chunk's x, B
// and C go through LDS as bfloat16 (x and B also transposed, so every MFMA operand
// is a contiguous 16-byte LDS read), and the next chunk's inputs are loaded into
// registers while the current one computes.  Inputs are bfloat16; the products
// accumulate in float32 and the state stays float32 (it is split into two bfloat16
// terms, hi + lo, only as the operand of the carried-state product).
//
// MFMA lane layout (gfx950, checked on the device): for v_mfma_f32_16x16x32_bf16,
// lane l holds A[m = l%16][k = 8(l/16) .. +7], B[k = 8(l/16) .. +7][n = l%16] and
// D[m = 4(l/16) + e][n = l%16].  Only the pairing of A's and B's K slots matters, so
// the state, which a product leaves in the D layout, is used as an A operand without
// a shuffle by giving the K slots of each lane the state entries it already holds.
#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_common.hpp"

namespace ssm {
namespace {

constexpr int kQ = 64;            // tokens per chunk
constexpr int kP = 64;            // head channels (4 waves x 16)
constexpr int kPad = 8;           // bfloat16 elements of row padding in LDS

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
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

// One chunk's inputs in registers (prefetch), moved as token pairs: thread t takes
// the 16-byte piece q of tokens 2m and 2m + 1 of the 64-token tiles of x (8 channels
// per piece) and of B and C (8 states per piece), (m, q) = (v / R, v % R) for
// v = t + 256 k and R pieces per token row.  R consecutive lanes read one token's
// contiguous row, and a thread holds both tokens of every pair it writes into the
// transposed LDS copies, so those writes are 4-byte token pairs.
template <int NS>
struct ChunkRegs {
  static constexpr int kXR = kP / 8;                // 16-byte pieces per token row of x
  static constexpr int kBR = NS / 8;                // ... of B and C
  static constexpr int kXV = kQ / 2 * kXR / 256;    // x token pairs per thread (1)
  static constexpr int kBV = kQ / 2 * kBR / 256;    // B (and C) token pairs per thread (1 or 2)
  uint4 x[kXV][2], b[kBV][2], c[kBV][2];
  float dt;                                         // raw Delta of token `lane` (each wave loads it)
};

// Two bfloat16 words -> the pair of their low (HI = false) or high halves, the first
// word's in the low half of the result.
template <bool HI>
__device__ __forceinline__ uint32_t pair16(uint32_t a, uint32_t b) {
  return HI ? (a >> 16) | (b & 0xffff0000u) : (a & 0xffffu) | (b << 16);
}

// STATE_ONLY: the pre-pass of the segmented form: the segment's end state from a
// zero start (x, B and Delta only; no C, no output), written to the workspace.
// Otherwise the full scan of the segment's chunks from its entering state: the
// initial state for segment 0, else the combined state in the workspace.
//
// Operand order: every product is arranged so that the four values a lane holds of
// its output tile (four consecutive rows m of one column n) are contiguous in the
// array the next step reads: S is computed transposed (rows i of B against rows j of
// C), so a lane's four entries of a row j of S' are one 8-byte LDS write, and the
// output is computed as y^T (x^T against S'^T and H against C^T), so a lane's four
// entries of a token's row of y are one 8-byte write.
template <int NS, bool STATE_ONLY>
__global__ __launch_bounds__(256) void ssd_scan_kernel(SsdArgs p) {
  constexpr int RX = kQ + kPad;                     // row stride of [.][Q] and [.][P] arrays
  constexpr int RN = NS + kPad;                     // row stride of [.][N] arrays
  constexpr int NT = NS / 16;                       // 16-row tiles of the state
  using CR = ChunkRegs<NS>;
  __shared__ __attribute__((aligned(16))) uint16_t sXT[kP * RX];    // x^T [p][i]
  __shared__ __attribute__((aligned(16))) uint16_t sX[kQ * RX];     // x [i][p]
  __shared__ __attribute__((aligned(16))) uint16_t sB[kQ * RN];     // B [i][n]
  __shared__ __attribute__((aligned(16))) uint16_t sBwT[NS * RX];   // (B diag(w))^T [n][i]
  __shared__ __attribute__((aligned(16))) uint16_t sC[kQ * RN];     // C [j][n]
  __shared__ __attribute__((aligned(16))) uint16_t sS[kQ * RX];     // (C B^T o M) Delta [j][i]
  __shared__ __attribute__((aligned(16))) uint16_t sY[kQ * RX];     // y [j][p] staging
  __shared__ __attribute__((aligned(16))) float sCum[kQ], sDl[kQ], sEc[kQ];
  // [row][token] arrays written transposed (x^T, B^T) place the 8-token block b of
  // row r at block b ^ ((r / 8) % 8): the 8 rows one instruction writes for one
  // token pair then fall in 8 different banks, and every 8-token block stays a
  // contiguous, aligned 16-byte MFMA operand.
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
  // Byte strides between consecutive tokens (x / y rows, B / C rows, dt) and the
  // sequence bases; a chunk's loads are 32-bit offsets from its first token.
  const uint32_t xrow_b = static_cast<uint32_t>(H) * kP * 2;
  constexpr uint32_t brow_b = NS * 2;
  const uint32_t dtrow_b = static_cast<uint32_t>(H) * 2;
  const char* xg = static_cast<const char*>(p.x) + (b * L * H + h) * kP * 2;
  const char* bg = static_cast<const char*>(p.Bm) + b * L * NS * 2;
  const char* cg = static_cast<const char*>(p.Cm) + b * L * NS * 2;
  const char* dtg = static_cast<const char*>(p.dt) + (b * L * H + h) * 2;
  char* yg = static_cast<char*>(p.y) + (b * L * H + h) * kP * 2;

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

  // Per-thread byte offsets of its pieces within a chunk, and of piece q of the
  // chunk's row `lim` (the clamp: min(offset, row lim) for a piece in row i is the
  // piece in row min(i, lim)).
  uint32_t xo_off[CR::kXV][2], xq_b[CR::kXV], bo_off[CR::kBV][2], bq_b[CR::kBV];
#pragma unroll
  for (int k = 0; k < CR::kXV; ++k) {
    const int v = tid + 256 * k, m = v / CR::kXR, q = v % CR::kXR;
    xq_b[k] = 16u * q;
    xo_off[k][0] = (2 * m) * xrow_b + xq_b[k];
    xo_off[k][1] = (2 * m + 1) * xrow_b + xq_b[k];
  }
#pragma unroll
  for (int k = 0; k < CR::kBV; ++k) {
    const int v = tid + 256 * k, m = v / CR::kBR, q = v % CR::kBR;
    bq_b[k] = 16u * q;
    bo_off[k][0] = (2 * m) * brow_b + bq_b[k];
    bo_off[k][1] = (2 * m + 1) * brow_b + bq_b[k];
  }
  const uint32_t dt_off = static_cast<uint32_t>(lane) * dtrow_b;

  CR cr;
  // Loads of chunk c into registers.  Rows past L reload row L - 1 (finite values);
  // those padding tokens get Delta = 0, which zeroes their weight in every product
  // that reaches a stored output, and their own output rows are not stored.  No load
  // sits behind a branch, so the loads issued for the next chunk stay in flight
  // during this one.
  auto fetch = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t t0 = c * kQ;
    const uint32_t lim = static_cast<uint32_t>(L - 1 - t0 < kQ - 1 ? L - 1 - t0 : kQ - 1);
    const char* xc = xg + t0 * xrow_b;
    const char* bc = bg + t0 * brow_b;
    const char* cc = cg + t0 * brow_b;
#pragma unroll
    for (int k = 0; k < CR::kXV; ++k) {
      const uint32_t cap = lim * xrow_b + xq_b[k];
#pragma unroll
      for (int s = 0; s < 2; ++s)
        cr.x[k][s] = *reinterpret_cast<const uint4*>(xc + (xo_off[k][s] < cap ? xo_off[k][s] : cap));
    }
#pragma unroll
    for (int k = 0; k < CR::kBV; ++k) {
      const uint32_t cap = lim * brow_b + bq_b[k];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t o = bo_off[k][s] < cap ? bo_off[k][s] : cap;
        cr.b[k][s] = *reinterpret_cast<const uint4*>(bc + o);
        if constexpr (!STATE_ONLY) cr.c[k][s] = *reinterpret_cast<const uint4*>(cc + o);
      }
    }
    const uint32_t dcap = lim * dtrow_b;
    cr.dt = bf16_at(reinterpret_cast<const uint16_t*>(dtg + t0 * dtrow_b + (dt_off < dcap ? dt_off : dcap)));
  };

  // (a segment always has a chunk; the clamp keeps the first fetch inside the
  // sequence regardless: a chunk starting at or past L would wrap the row limit)
  fetch(c_begin < nchunks ? c_begin : nchunks - 1);
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
#pragma unroll
    for (int k = 0; k < CR::kXV; ++k) {
      const int v = tid + 256 * k, i0 = 2 * (v / CR::kXR), q = v % CR::kXR;
      if constexpr (!STATE_ONLY) {
        *reinterpret_cast<uint4*>(&sX[i0 * RX + 8 * q]) = cr.x[k][0];
        *reinterpret_cast<uint4*>(&sX[(i0 + 1) * RX + 8 * q]) = cr.x[k][1];
      }
      const uint32_t a0[4] = {cr.x[k][0].x, cr.x[k][0].y, cr.x[k][0].z, cr.x[k][0].w};
      const uint32_t a1[4] = {cr.x[k][1].x, cr.x[k][1].y, cr.x[k][1].z, cr.x[k][1].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<uint32_t*>(&sXT[swz(8 * q + 2 * r, i0)]) = pair16<false>(a0[r], a1[r]);
        *reinterpret_cast<uint32_t*>(&sXT[swz(8 * q + 2 * r + 1, i0)]) = pair16<true>(a0[r], a1[r]);
      }
    }
#pragma unroll
    for (int k = 0; k < CR::kBV; ++k) {
      const int v = tid + 256 * k, i0 = 2 * (v / CR::kBR), q = v % CR::kBR;
      if constexpr (!STATE_ONLY) {
        *reinterpret_cast<uint4*>(&sB[i0 * RN + 8 * q]) = cr.b[k][0];
        *reinterpret_cast<uint4*>(&sB[(i0 + 1) * RN + 8 * q]) = cr.b[k][1];
        *reinterpret_cast<uint4*>(&sC[i0 * RN + 8 * q]) = cr.c[k][0];
        *reinterpret_cast<uint4*>(&sC[(i0 + 1) * RN + 8 * q]) = cr.c[k][1];
      }
      // B^T scaled by the token weights, for the state contribution
      const float w0 = __shfl(wgt, i0), w1 = __shfl(wgt, i0 + 1);
      const uint32_t b0[4] = {cr.b[k][0].x, cr.b[k][0].y, cr.b[k][0].z, cr.b[k][0].w};
      const uint32_t b1[4] = {cr.b[k][1].x, cr.b[k][1].y, cr.b[k][1].z, cr.b[k][1].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<uint32_t*>(&sBwT[swz(8 * q + 2 * r, i0)]) =
            bf16x2(bf16_lo(b0[r]) * w0, bf16_lo(b1[r]) * w1);
        *reinterpret_cast<uint32_t*>(&sBwT[swz(8 * q + 2 * r + 1, i0)]) =
            bf16x2(bf16_hi(b0[r]) * w0, bf16_hi(b1[r]) * w1);
      }
    }
    fetch(c + 1 < c_end ? c + 1 : c);                // (the last chunk reloads itself, unused)
    log_decay += cum_last;
    barrier_lds();

    // this wave's channels p = 16w + c16 of x^T, as MFMA operands (state and output)
    uint4 xo[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) xo[kb] = *reinterpret_cast<const uint4*>(&sXT[swz(16 * w + c16, 32 * kb + 8 * g)]);

    // ---- 2. S' = (C B^T o M) Delta for rows j = 16w + c16 of this wave (computed as
    // tiles of S^T: rows i of B against row j of C); the chunk's state contribution;
    // the output from the carried state
    if constexpr (!STATE_ONLY) {
      const int j = 16 * w + c16;
      const float cj = sCum[j];
      uint4 cb[NS / 32];
#pragma unroll
      for (int kb = 0; kb < NS / 32; ++kb) cb[kb] = *reinterpret_cast<const uint4*>(&sC[j * RN + 32 * kb + 8 * g]);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int i0 = 16 * it + 4 * g;             // this lane's 4 consecutive i
        uint2 packed = make_uint2(0u, 0u);
        if (it <= w) {                              // tiles right of the diagonal are all zero
          f32x4_t S = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int kb = 0; kb < NS / 32; ++kb) {
            const uint4 a = *reinterpret_cast<const uint4*>(&sB[(16 * it + c16) * RN + 32 * kb + 8 * g]);
            S = mfma32(a, cb[kb], S);
          }
          const float4 ci = *reinterpret_cast<const float4*>(&sCum[i0]);
          const float4 di = *reinterpret_cast<const float4*>(&sDl[i0]);
          const float cis[4] = {ci.x, ci.y, ci.z, ci.w}, dis[4] = {di.x, di.y, di.z, di.w};
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // (computed for every element, then selected: no branch per element)
            v[e] = S[e] * exp2_hw(fminf(cj - cis[e], 0.0f)) * dis[e];
            asm volatile("" : "+v"(v[e]));
            v[e] = j >= i0 + e ? v[e] : 0.0f;
          }
          packed = make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
        }
        *reinterpret_cast<uint2*>(&sS[j * RX + i0]) = packed;
      }
    }
    // the chunk's state contribution st[n][p] = sum_i B[i][n] w_i x[i][p],
    // w_i = exp(cum_last - cum_i) Delta_i (folded into the LDS copy of B^T)
    f32x4_t st[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) st[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const uint4 a = *reinterpret_cast<const uint4*>(&sBwT[swz(16 * mt + c16, 32 * kb + 8 * g)]);
        st[mt] = mfma32(a, xo[kb], st[mt]);
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
    // output from the carried state, transposed: Yc[p][j] = sum_n H[p][n] C[j][n].
    // The float32 state is split into two bfloat16 terms, hi + lo, so the product
    // keeps ~16 bits of it.  A product's K order is free: the 8 K slots of a lane
    // hold the entries it already has of two state tiles, n = 32t + 4g + e and
    // 32t + 16 + 4g + e, against the same entries of C (two 8-byte reads); hi and lo
    // are two products sharing that C operand.
    f32x4_t Yc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) Yc[jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < NT / 2; ++t) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f32x4_t hv = Hs[2 * t + u];
        const uint32_t h01 = bf16x2(hv[0], hv[1]), h23 = bf16x2(hv[2], hv[3]);
        hw[2 * u] = h01;
        hw[2 * u + 1] = h23;
        lw[2 * u] = bf16x2(hv[0] - bf16_lo(h01), hv[1] - bf16_hi(h01));
        lw[2 * u + 1] = bf16x2(hv[2] - bf16_lo(h23), hv[3] - bf16_hi(h23));
      }
      const uint4 hq = make_uint4(hw[0], hw[1], hw[2], hw[3]), lq = make_uint4(lw[0], lw[1], lw[2], lw[3]);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const uint16_t* crow = &sC[(16 * jt + c16) * RN + 32 * t + 4 * g];
        const uint2 c0 = *reinterpret_cast<const uint2*>(crow);
        const uint2 c1 = *reinterpret_cast<const uint2*>(crow + 16);
        const uint4 cq = make_uint4(c0.x, c0.y, c1.x, c1.y);
        Yc[jt] = mfma32(hq, cq, Yc[jt]);
        Yc[jt] = mfma32(lq, cq, Yc[jt]);
      }
    }
    barrier_lds();                                  // S' complete

    // ---- 3. y^T = x^T S'^T + H C^T diag(exp(cum_j)) + D x^T; the state update.  Lane
    // (g, c16) holds y[j = 16 jt + c16][p = 16w + 4g + e].
    f32x4_t Yo[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) Yo[jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const uint4 sb = *reinterpret_cast<const uint4*>(&sS[(16 * jt + c16) * RX + 32 * kb + 8 * g]);
        Yo[jt] = mfma32(xo[kb], sb, Yo[jt]);
      }
    }
    const int p0 = 16 * w + 4 * g;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int j = 16 * jt + c16;
      const uint2 xr = *reinterpret_cast<const uint2*>(&sX[j * RX + p0]);
      const float xv[4] = {bf16_lo(xr.x), bf16_hi(xr.x), bf16_lo(xr.y), bf16_hi(xr.y)};
      const float ec = sEc[j];
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(dsk, xv[e], __builtin_fmaf(ec, Yc[jt][e], Yo[jt][e]));
      *reinterpret_cast<uint2*>(&sY[j * RX + p0]) = make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
    }
    const float decay = exp2_hw(cum_last);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) Hs[mt][e] = __builtin_fmaf(decay, Hs[mt][e], st[mt][e]);
    barrier_lds();                                  // y tile complete

    // ---- 4. y rows to memory (128 contiguous bytes per token)
    char* yc = yg + t0 * xrow_b;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int v = tid + 256 * k, j = v >> 3, q = v & 7;
      if (t0 + j < L)
        *reinterpret_cast<uint4*>(yc + j * xrow_b + 16 * q) = *reinterpret_cast<const uint4*>(&sY[j * RX + 8 * q]);
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

// (H is bounded so that a chunk's 64 token rows of x span less than 4 GB: the loads
// use 32-bit offsets from the chunk's first token)
constexpr int64_t kSsdCUs = 256;                 // compute units of the MI355X

bool ssd_supported(int64_t H, int64_t P, int64_t N) { return H <= 65536 && P == kP && (N == 64 || N == 128); }

// Segments per sequence: as many as keep the main pass's workgroups within one
// wave of what the chip holds at once (N = 64: 2 per CU; N = 128: 1), at least 4
// chunks per segment.  Measured over segment counts on ten shapes, that count was
// the fastest wherever the (batch, head) pairs fit in one wave: a second, partial
// wave of workgroups, and the pre-pass and combine that segments need, cost more
// than the parallelism gains (at 4 x 2048 x 80 heads, N = 64, one segment: 105.5 us
// against 112.6 with three).  Past one wave, N = 64 measured fastest unsegmented;
// N = 128 (4 x 2048 x 80 heads) with about 768 workgroups, 3 segments: 191 us
// against 212 unsegmented.  The count is then derived back from the segment
// length, so that no segment is empty: with ceil(chunks / s) chunks per segment,
// s segments can leave the last ones without a chunk (130 chunks in 21 segments of
// 7 use only 19).
int ssd_segments(int64_t batch, int64_t L, int64_t H, int64_t N) {
  const int64_t nch = (L + kQ - 1) / kQ;
  const int64_t resident = (N <= 64 ? 2 : 1) * kSsdCUs;
  const int64_t pairs = batch * H;
  int64_t s = pairs <= resident ? resident / pairs : (N <= 64 ? 1 : (768 + pairs - 1) / pairs);
  const int64_t smax = nch / 4 > 1 ? nch / 4 : 1;
  s = s < 1 ? 1 : (s > smax ? smax : s);
  s = s > 64 ? 64 : s;
  const int64_t per = (nch + s - 1) / s;
  return static_cast<int>((nch + per - 1) / per);
}

size_t ssd_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N) {
  const int s = ssd_segments(batch, L, H, N);
  if (s <= 1) return 0;
  return static_cast<size_t>(batch * H * s) * (P * N + 1) * sizeof(float) + 256;
}

template <int NS>
hipError_t launch_ssd_n(SsdArgs a, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t nch = (a.L + kQ - 1) / kQ;
  int nseg = ssd_segments(a.batch, a.L, a.H, NS);
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
