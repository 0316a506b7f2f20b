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

// Round to nearest even; NaN stays NaN; overflow goes to inf.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
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

// e4m3fn (OCP, bias 7) of an fp32 value, round to nearest even, saturating to
// +-448, sign of zero kept.  Integer arithmetic on the fp32 encoding, so the
// result does not depend on conversion-instruction modes.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                       // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;               // >= 448 (incl. inf)
  if (a < 0x3c800000u) {                                   // < 2^-6: subnormal grid 2^-9
    float q = __builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scaling, RNE
    return sign | static_cast<uint32_t>(q);                // 8 -> 0x08 = 2^-6
  }
  uint32_t exp = (a >> 23) - 127u + 7u;                    // 1..15
  uint32_t m = (a >> 20) & 7u;
  uint32_t rem = a & 0xfffffu;
  m += (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ? 1u : 0u;
  uint32_t code = (exp << 3) + m;                          // carry m==8 into exponent
  return sign | (code > 0x7eu ? 0x7eu : code);
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

}  // namespace moe

// Host-side helpers
#define MOE_CHECK_LAUNCH()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return MOE_EDEVICE; \
  } while (0)
