// Device helpers shared by the gfx950 kernels: activation load/store, the
// transcendental pieces of the scan (exp2 on the hardware unit, an accurate
// softplus, SiLU) and DPP cross-lane moves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;

// Activation storage tags.
struct ActF32 {
  using storage = float;
  static constexpr int kBytes = 4;
};
struct ActBF16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (a in the low half), round to nearest even.
// gfx950 does this in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t to_bf16(float a) {
  return static_cast<uint16_t>(pack_bf16x2(a, 0.0f) & 0xffffu);
}

template <typename ACT>
__device__ __forceinline__ float load_act(const void* p, int64_t i);
template <>
__device__ __forceinline__ float load_act<ActF32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float load_act<ActBF16>(const void* p, int64_t i) {
  return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <typename ACT>
__device__ __forceinline__ void store_act(void* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_act<ActF32>(void* p, int64_t i, float v) {
  static_cast<float*>(p)[i] = v;
}
template <>
__device__ __forceinline__ void store_act<ActBF16>(void* p, int64_t i, float v) {
  static_cast<uint16_t*>(p)[i] = to_bf16(v);
}

// Eight consecutive activations as one 32-byte (float32) or 16-byte (bfloat16)
// access; the element offset must keep the address 16-byte aligned.
template <typename ACT>
__device__ __forceinline__ void load_act8(const void* p, int64_t i, float (&v)[8]);
template <>
__device__ __forceinline__ void load_act8<ActF32>(const void* p, int64_t i, float (&v)[8]) {
  const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
  const float4 a = q[0], b = q[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load_act8<ActBF16>(const void* p, int64_t i, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
  v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
  v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}
template <typename ACT>
__device__ __forceinline__ void store_act8(void* p, int64_t i, const float (&v)[8]);
template <>
__device__ __forceinline__ void store_act8<ActF32>(void* p, int64_t i, const float (&v)[8]) {
  float4* q = reinterpret_cast<float4*>(static_cast<float*>(p) + i);
  q[0] = make_float4(v[0], v[1], v[2], v[3]);
  q[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <>
__device__ __forceinline__ void store_act8<ActBF16>(void* p, int64_t i, const float (&v)[8]) {
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + i) =
      make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLn2 = 0.69314718055994531f;

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e) with e = e^-|x| in (0, 1]: no
// overflow for large x.  log1p(e) is evaluated as ln(w) + (e - (w - 1)) with
// w = fl(1 + e): the second term is the exact rounding error of 1 + e (w - 1 is
// exact by Sterbenz), which restores the low bits of e that w lost, and the
// first-order remainder is below |rounding error| * e.  With the hardware log2
// this keeps ~1e-6 relative accuracy even where e ~ 1e-4, where a plain
// log(1 + e^x) in float32 is off by ~3e-4.
__device__ __forceinline__ float softplus_f(float x) {
  const float e = exp2_hw(-fabsf(x) * kLog2e);
  const float w = 1.0f + e;
  const float err = e - (w - 1.0f);
  return fmaxf(x, 0.0f) + __builtin_fmaf(__builtin_amdgcn_logf(w), kLn2, err);
}

// softplus for bfloat16 activations: max(x, 0) + log(1 + e^-|x|) from the hardware
// exp2 and log2, without the compensation above.  Rounding 1 + e^-|x| costs about
// 6e-8 absolute, so the relative error is about 6e-8 / e^x where x < 0 (1e-3 at
// x = -10, where Delta is 4.5e-5; Delta's own error then stays below 1e-7 absolute)
// and a few 1e-8 for x >= 0, with no overflow for large x.  Four VALU operations
// (max, the scaled argument, 1 + e, the final FMA) and two transcendentals: three
// VALU operations and two transcendentals per token fewer than the compensated
// form, within the bfloat16 bar by orders of magnitude.
__device__ __forceinline__ float softplus_bf16act(float x) {
  const float l = __builtin_amdgcn_logf(1.0f + exp2_hw(-fabsf(x) * kLog2e));
  return __builtin_fmaf(l, kLn2, fmaxf(x, 0.0f));
}

// Full zero-order hold: the factor (e^x - 1)/A = Delta * (e^x - 1)/x of the input
// term, x = Delta * A, from y = x * log2(e) (the exp2 argument), a = 2^y, ra = 1/A and
// Delta.  Away from x = 0 it is (a - 1)/A.  Near 0 that difference loses relative
// accuracy to the rounding of a (about 1e-7 / |x|), so for |x| < 0.0624 (|y| < 0.09)
// it is Delta * (1 + x/2 + x^2/6 + x^3/24), whose truncation is below 1.3e-7 there;
// at A == 0 that is Delta itself, the term's limit.  (The unselected side may be a
// NaN at A == 0; the select does not propagate it.)
__device__ __forceinline__ float zoh_factor(float y, float a, float ra, float delta) {
  constexpr float c1 = 0.34657359f;     // ln2 / 2      (powers of x = y ln2)
  constexpr float c2 = 0.08007550f;     // ln2^2 / 6
  constexpr float c3 = 0.013876027f;    // ln2^3 / 24
  const float p = __builtin_fmaf(y, __builtin_fmaf(y, __builtin_fmaf(y, c3, c2), c1), 1.0f);
  const float far = __builtin_fmaf(a, ra, -ra);
  return fabsf(y) < 0.09f ? delta * p : far;
}

// SiLU(z) = z / (1 + e^-z); e^-z = inf for very negative z gives -0.
__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + exp2_hw(-z * kLog2e));
}

// ---- DPP lane moves (gfx9 controls) ---------------------------------------
// dpp_ctrl encodings: row_shr:n = 0x110 + n, wave_shr:1 = 0x138,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143.
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ float dpp_mov(float old, float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                         CTRL, ROW_MASK, 0xf, BOUND_ZERO));
}

// Inclusive scan across the 64 lanes of a wave of (a, b) pairs under the operator
// (a1, b1) then (a2, b2) = (a2 a1, a2 b1 + b2): Kogge-Stone with the row shifts
// 1, 2, 4, 8 and the two row broadcasts (15 -> rows 1, 3; 31 -> rows 2, 3).
// On return lane i's b is the composition of lanes 0..i applied to zero (its a is
// a scratch value: the final decay product is not needed by the callers).
//
// Each step is one in-place DPP instruction per component:
//   v_fmac_f32_dpp b, b(src lane), a   ->  b = a * b_src + b
//   v_mul_f32_dpp  a, a(src lane), a   ->  a = a_src * a
// with bound_ctrl off, so a lane whose source is outside its row (or whose row
// is masked off in the broadcasts) is not written: it keeps (a, b), which is
// exactly combining with the identity (1, 0).  The compiler does not form these
// in-place DPP operations itself, hence the asm.  gfx9 needs two wait states
// between a VALU write and a DPP read of the same VGPR: one s_nop 0 between steps
// (plus the other component's instruction), s_nop 1 on entry and exit because
// the surrounding code is compiler-scheduled.  Pure VALU, no memory access.
__device__ __forceinline__ void wave_scan_pairs(float& a, float& b) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(b), "+v"(a));
}

// Two independent scans of the same kind, interleaved: each instruction's DPP
// source was written three instructions earlier, so the steps need no s_nop.
__device__ __forceinline__ void wave_scan_pairs2(float& a0, float& b0, float& a1, float& b1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %3 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %3, %3 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %3 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %3, %3 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %3 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %3, %3 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %3 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %3, %3 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %3 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %3, %3 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %3 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(b0), "+v"(a0), "+v"(b1), "+v"(a1));
}

// Value of lane i-1 in lane i; lane 0 receives `lane0`.
__device__ __forceinline__ float wave_shift_up(float v, float lane0) {
  return dpp_mov<0x138, 0xf, false>(lane0, v);
}

__device__ __forceinline__ float wave_lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

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

}  // namespace ssm
