// Pieces shared by the scan kernels (forward and backward): vector I/O of per-lane
// runs of KPL consecutive tokens of one channel (TokenIO) and of the 16-byte B/C
// tile elements (TileIO), with non-temporal accesses for data read or written
// once; a compile-time loop; an LDS-only workgroup barrier.
#pragma once

#include <utility>

#include "device_common.hpp"

namespace ssm {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
// u, delta and z are read once and y is written once: non-temporal accesses
// (measured 3.5 % faster on the float32 workload, neutral on bfloat16).
__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(float4* p, float4 v) {
  const f32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t*>(p));
}
__device__ __forceinline__ void st_stream(uint4* p, uint4 v) {
  const u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
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
    for (int q = 0; q < kVec; ++q) r[q] = ld_stream(p + q);
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
      st_stream(p + q, make_float4(v[4 * q + 0], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]));
  }
};

template <int KPL>
struct TokenIO<ActBF16, KPL> {
  static constexpr int kVec = KPL / 8;
  using raw_t = uint4;
  static __device__ __forceinline__ void load_raw(const void* base, int64_t off, raw_t (&r)[kVec]) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int q = 0; q < kVec; ++q) r[q] = ld_stream(p + q);
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
      st_stream(p + q, x);
    }
  }
};

// One B/C tile element: the largest vector load of consecutive tokens of one
// state (16 bytes): 4 float32 or 8 bfloat16 tokens, converted to kOut float4.
template <typename ACT>
struct TileIO;

template <>
struct TileIO<ActF32> {
  static constexpr int kTok = 4;
  static constexpr int kOut = 1;
  using raw_t = float4;
  static __device__ __forceinline__ raw_t load(const void* base, int64_t off) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
  }
  static __device__ __forceinline__ float4 out(const raw_t& r, int) { return r; }
};

template <>
struct TileIO<ActBF16> {
  static constexpr int kTok = 8;
  static constexpr int kOut = 2;
  using raw_t = uint4;
  static __device__ __forceinline__ raw_t load(const void* base, int64_t off) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  }
  static __device__ __forceinline__ float4 out(const raw_t& r, int j) {
    const unsigned a = j == 0 ? r.x : r.z, b = j == 0 ? r.y : r.w;
    return make_float4(bf16_lo(a), bf16_hi(a), bf16_lo(b), bf16_hi(b));
  }
};

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1, as straight-line code
// (a compile-time loop the compiler cannot leave rolled).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Workgroup barrier that orders LDS only: outstanding global loads stay in
// flight across it (the compiler waits for each where its value is used).
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace
}  // namespace ssm
