// Device-side helpers for the SeKV HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "sekv_internal.h"

namespace sekv {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float32 -> bfloat16, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPer16 = 4;
  __device__ __forceinline__ static float to_f(float x) { return x; }
  __device__ __forceinline__ static float from_f(float x) { return x; }
  // 16 bytes -> 4 floats
  __device__ __forceinline__ static void load16(const float* p, float* f) {
    float4 v = *reinterpret_cast<const float4*>(p);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
  __device__ __forceinline__ static void store16(float* p, const float* f) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
};
template <> struct Elem<bf16_t> {
  static constexpr int kPer16 = 8;
  __device__ __forceinline__ static float to_f(bf16_t x) { return bf16_to_f32(x); }
  __device__ __forceinline__ static bf16_t from_f(float x) { return f32_to_bf16(x); }
  __device__ __forceinline__ static void load16(const bf16_t* p, float* f) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ __forceinline__ static void store16(bf16_t* p, const float* f) {
    uint4 v;
    v.x = (uint32_t)f32_to_bf16(f[0]) | ((uint32_t)f32_to_bf16(f[1]) << 16);
    v.y = (uint32_t)f32_to_bf16(f[2]) | ((uint32_t)f32_to_bf16(f[3]) << 16);
    v.z = (uint32_t)f32_to_bf16(f[4]) | ((uint32_t)f32_to_bf16(f[5]) << 16);
    v.w = (uint32_t)f32_to_bf16(f[6]) | ((uint32_t)f32_to_bf16(f[7]) << 16);
    *reinterpret_cast<uint4*>(p) = v;
  }
};

// ------------------------------------------------------------ lane exchange

// DPP moves inside a row of 16 lanes (all rows and banks enabled).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each 16

// Exchanges with the lane 16 or 32 apart through the gfx950 lane-swap
// instructions (VALU, no LDS round trip).  v_permlane16_swap swaps the odd
// 16-lane rows of its first operand with the even rows of its second, and
// v_permlane32_swap the upper half of the first with the lower half of the
// second; with both operands = x, the two results hold x and x of the partner
// lane, in an order that depends on the lane's side.
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// x of the lane 16 (32) apart.
__device__ __forceinline__ float xor16_get(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32_get(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Sum over aligned groups of N consecutive lanes (N = 1..64, power of two);
// every lane of a group ends with the group's sum.  After the two quad steps
// all lanes of a quad hold the same value, so a mirror inside 8 (16) lanes
// pairs each quad (octet) with the other one.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp_f<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp_f<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f<kDppMirror>(x);
  if constexpr (N >= 32) x = xor16_sum(x);
  if constexpr (N >= 64) x = xor32_sum(x);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp_f<kDppXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp_f<kDppXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_f<kDppMirror>(x));
  if constexpr (N >= 32) x = xor16_max(x);
  if constexpr (N >= 64) x = xor32_max(x);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }
__device__ __forceinline__ float wave_max(float x) { return group_max<64>(x); }

__device__ __forceinline__ double wave_sum_f64(double x) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Orders LDS traffic between lanes of one wave: no code motion across it and
// all of the wave's LDS operations issued before it complete first.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

}  // namespace sekv
