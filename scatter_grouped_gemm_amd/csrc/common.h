// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (gfx950's v_cvt_pk_bf16_f32, which the compiler
// emits for this conversion); NaN stays NaN; overflow goes to inf.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two values rounded to bf16 and packed (a in the low half): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 h2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, h2_t));
}

// UE8M0 exponent of a non-negative finite group maximum: the smallest e in
// [-126, 127] with amax <= 448 * 2^e.  448 = 1.75 * 2^8, so with
// amax = 1.m * 2^E the answer is E - 8, plus one when 1.m > 1.75.  Zero and
// subnormal maxima give e <= -134 before clamping.
__device__ __forceinline__ int ue8m0_exponent(float amax) {
  uint32_t u = __float_as_uint(amax);
  int ef = static_cast<int>(u >> 23);
  if (ef == 0) return -126;
  int e = ef - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}

// Four fp32 values times 2^-e as e4m3fn (OCP, bias 7) codes packed
// little-endian, rounded to nearest even with the sign of zero kept, by the
// hardware conversion (two values per instruction).  For |v * 2^-e| <= 448,
// which a UE8M0 exponent from ue8m0_exponent of the group maximum guarantees
// for finite groups, this is the exact RNE encoding (the conversion matches an
// integer implementation of it on every fp32 bit pattern in that range);
// larger magnitudes and NaN give the NaN code 0x7f.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, int e) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(a, -e),
                                          __builtin_amdgcn_ldexpf(b, -e), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(c, -e),
                                      __builtin_amdgcn_ldexpf(d, -e), w, true);
  return static_cast<uint32_t>(w);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// max over aligned groups of `width` lanes (width a power of two <= 64)
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ unsigned long long ballot(bool p) { return __ballot(p); }

// SiLU in fp32: g * 1 / (1 + e^-g), with e^-g as 2^(-g log2 e) and the
// reciprocal from the hardware approximations (each within about one fp32 ulp),
// so that it stays a handful of instructions.  Every kernel that computes the
// activation uses this one definition, which keeps them bit-identical.
__device__ __forceinline__ float silu_f32(float g) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace moe

// Host-side helpers
#define MOE_CHECK_LAUNCH()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return MOE_EDEVICE; \
  } while (0)
