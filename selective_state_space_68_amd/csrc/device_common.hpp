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

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// log(1 + e^x) = max(x, 0) + log1p(e^-|x|): no overflow for large x and, through
// an accurate log1p, full relative accuracy for the small steps the scan sees
// (a plain log(1 + e^x) loses ~3e-4 relative at e^x ~ 2e-4).
__device__ __forceinline__ float softplus_f(float x) {
  const float e = exp2_hw(-fabsf(x) * kLog2e);
  return fmaxf(x, 0.0f) + log1pf(e);
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

// One Kogge-Stone step of the inclusive scan of (a, b) pairs under the operator
// (a1, b1) then (a2, b2) = (a2 a1, a2 b1 + b2).  Lanes whose source lane is out
// of range (or whose row is masked off) combine with the identity (1, 0).
template <int CTRL, int ROW_MASK, bool UPDATE_A>
__device__ __forceinline__ void scan_step(float& a, float& b) {
  const float bs = dpp_mov<CTRL, ROW_MASK, false>(0.0f, b);
  if (UPDATE_A) {
    const float as = dpp_mov<CTRL, ROW_MASK, false>(1.0f, a);
    b = __builtin_fmaf(a, bs, b);
    a = a * as;
  } else {
    b = __builtin_fmaf(a, bs, b);
  }
}

// Inclusive scan across the 64 lanes of a wave.  On return b holds, in lane i,
// the composition of lanes 0..i applied to zero; `a` is left partially combined
// (its final value is not needed by the callers).
__device__ __forceinline__ void wave_scan_pairs(float& a, float& b) {
  scan_step<0x111, 0xf, true>(a, b);   // row_shr:1
  scan_step<0x112, 0xf, true>(a, b);   // row_shr:2
  scan_step<0x114, 0xf, true>(a, b);   // row_shr:4
  scan_step<0x118, 0xf, true>(a, b);   // row_shr:8
  scan_step<0x142, 0xa, true>(a, b);   // row_bcast:15 into rows 1, 3
  scan_step<0x143, 0xc, false>(a, b);  // row_bcast:31 into rows 2, 3
}

// Value of lane i-1 in lane i; lane 0 receives `lane0`.
__device__ __forceinline__ float wave_shift_up(float v, float lane0) {
  return dpp_mov<0x138, 0xf, false>(lane0, v);
}

__device__ __forceinline__ float wave_lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace ssm
