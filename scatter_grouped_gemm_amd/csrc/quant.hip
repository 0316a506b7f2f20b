// Per-token UE8M0 FP8 quantisation, 128x128 weight block quantisation and
// SiLU-and-mul (with optional FP8 output).
//
// Row kernels use one wavefront per row: each lane owns 8 consecutive
// channels (16 bytes of bf16), so 16 lanes hold one 128-channel group and the
// group maximum is a 4-step butterfly inside those 16 lanes.
#include "common.h"

namespace moe {

// Quantise the 8 values a lane holds (part of a 128-wide group spread over 16
// lanes): returns the 8 e4m3 bytes packed little-endian; *e_out = exponent.
__device__ __forceinline__ uint2 quant8_group16(const float (&f)[8], int* e_out) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = group_max<16>(amax);
  const int e = ue8m0_exponent(amax);
  const uint32_t lo = e4m3x4(f[0], f[1], f[2], f[3], e);
  const uint32_t hi = e4m3x4(f[4], f[5], f[6], f[7], e);
  *e_out = e;
  return make_uint2(lo, hi);
}

__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xffffu));
    f[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
  }
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                         int K, int64_t ld_x,
                                                         const int32_t* __restrict__ m_indices,
                                                         uint8_t* __restrict__ q,
                                                         uint8_t* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= M) return;
  if (m_indices && m_indices[r] < 0) return;
  const uint16_t* xr = x + r * ld_x;
  for (int col = lane * 8; col < K; col += 512) {
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(xr + col), f);
    int e;
    const uint2 qq = quant8_group16(f, &e);
    *reinterpret_cast<uint2*>(q + r * K + col) = qq;
    if ((lane & 15) == 0) scale[static_cast<int64_t>(col / 128) * M + r] = static_cast<uint8_t>(e + 127);
  }
}

// Weight blocks: one workgroup per 128x128 block; thread t covers rows
// 8*(t/16) .. +8 and columns 8*(t%16) .. +8 of the block.  The block's bf16
// values f (held by the threads) get one UE8M0 exponent from the block
// maximum and are stored as e4m3.
struct BlockPos {
  int64_t g, blk;
  int r0, c0;
};
__device__ __forceinline__ BlockPos block_pos(int N, int K) {
  const int nb = N / 128, kb = K / 128;
  BlockPos b;
  b.blk = blockIdx.x;
  b.g = b.blk / (static_cast<int64_t>(nb) * kb);
  const int bn = static_cast<int>((b.blk / kb) % nb), bk = static_cast<int>(b.blk % kb);
  b.r0 = bn * 128 + (threadIdx.x >> 4) * 8;
  b.c0 = bk * 128 + (threadIdx.x & 15) * 8;
  return b;
}
__device__ __forceinline__ void quant_block_store(const float (&f)[8][8], const BlockPos& b, int N,
                                                  int K, uint8_t* __restrict__ q,
                                                  uint8_t* __restrict__ scale) {
  __shared__ float wmax[4];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[i][j]));
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e = ue8m0_exponent(amax);
  uint8_t* qg = q + b.g * N * static_cast<int64_t>(K);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo = e4m3x4(f[i][0], f[i][1], f[i][2], f[i][3], e);
    const uint32_t hi = e4m3x4(f[i][4], f[i][5], f[i][6], f[i][7], e);
    *reinterpret_cast<uint2*>(qg + static_cast<int64_t>(b.r0 + i) * K + b.c0) = make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) scale[b.blk] = static_cast<uint8_t>(e + 127);
}

__global__ __launch_bounds__(256) void quant_weight_kernel(const uint16_t* __restrict__ w, int N,
                                                           int K, uint8_t* __restrict__ q,
                                                           uint8_t* __restrict__ scale) {
  const BlockPos b = block_pos(N, K);
  const uint16_t* wg = w + b.g * N * static_cast<int64_t>(K);
  float f[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    unpack8(*reinterpret_cast<const uint4*>(wg + static_cast<int64_t>(b.r0 + i) * K + b.c0), f[i]);
  quant_block_store(f, b, N, K, q, scale);
}

// Block-FP8 weights (e4m3 codes, one fp32 scale per 128x128 block) to the
// UE8M0 block format: each element decode(q) * s in fp32, rounded to bf16,
// then the block quantisation above.  q_out may be q_in: every thread reads
// its 8x8 piece into registers before the block-wide barrier and writes the
// same piece after it.
__global__ __launch_bounds__(256) void requant_weight_kernel(const uint8_t* q_in,
                                                             const float* __restrict__ s_in, int N,
                                                             int K, uint8_t* q_out,
                                                             uint8_t* __restrict__ s_out) {
  const BlockPos b = block_pos(N, K);
  const uint8_t* qg = q_in + b.g * N * static_cast<int64_t>(K);
  const float sc = s_in[b.blk];
  float f[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint2 c = *reinterpret_cast<const uint2*>(qg + static_cast<int64_t>(b.r0 + i) * K + b.c0);
    // exact e4m3 -> fp32 by the hardware conversion, two codes per instruction
    const auto d0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c.x), false);
    const auto d1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c.x), true);
    const auto d2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c.y), false);
    const auto d3 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c.y), true);
    const float v[8] = {d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
#pragma unroll
    for (int j = 0; j < 8; ++j) f[i][j] = bf16_to_f32(f32_to_bf16(v[j] * sc));
  }
  quant_block_store(f, b, N, K, q_out, s_out);
}

// SiLU-and-mul over one row per wavefront.  gate = first I columns, up = last I.
template <bool FP8>
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t* __restrict__ gu, int64_t M,
                                                       int I, const int32_t* __restrict__ m_indices,
                                                       const int32_t* __restrict__ masked_m,
                                                       int max_m, uint8_t* __restrict__ out,
                                                       uint8_t* __restrict__ out_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= M) return;
  if (m_indices && m_indices[r] < 0) return;
  int64_t g = 0, rr = r;
  if (masked_m) {
    g = r / max_m;
    rr = r - g * max_m;
    if (rr >= masked_m[g]) return;
  }
  const uint16_t* row = gu + r * 2 * static_cast<int64_t>(I);
  // four 512-column passes per round: all loads of a round are issued before
  // any arithmetic so eight 16-byte loads per lane are in flight
  constexpr int U = 4;
  for (int c0 = lane * 8; c0 < I; c0 += U * 512) {
    uint4 gv[U], uv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int col = c0 + u * 512;
      if (col < I) {
        gv[u] = *reinterpret_cast<const uint4*>(row + col);
        uv[u] = *reinterpret_cast<const uint4*>(row + I + col);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int col = c0 + u * 512;
      if (col >= I) break;
      float gt[8], up[8], a[8];
      unpack8(gv[u], gt);
      unpack8(uv[u], up);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a[i] = bf16_to_f32(f32_to_bf16(silu_f32(gt[i]) * up[i]));  // the bf16 activation
      }
      if (!FP8) {
        *reinterpret_cast<uint4*>(out + (r * I + col) * 2) = pack8(a);
      } else {
        int e;
        const uint2 qq = quant8_group16(a, &e);
        *reinterpret_cast<uint2*>(out + r * I + col) = qq;
        if ((lane & 15) == 0) {
          const int b = col / 128;
          const int64_t si = masked_m ? (g * (I / 128) + b) * max_m + rr : static_cast<int64_t>(b) * M + r;
          out_scale[si] = static_cast<uint8_t>(e + 127);
        }
      }
    }
  }
}

// MX weights: byte offset of the scale of (row n of group g, 32-block b) in
// the tiled layout [G][N/64][K/128][4][16][4]: per 64 weight rows and 128 k, a
// 256-byte slot whose byte kq*64 + r16*4 + j16 holds row 16*j16 + r16 of the
// slot and k block 4*s + kq -- so a lane of the GEMM reads the four scales of
// its 16-row sub-tiles with one 4-byte LDS load.
__device__ __forceinline__ int64_t mx_scale_offset(int64_t g, int n, int b, int N, int K) {
  const int c = n & 63;
  return ((g * (N / 64) + n / 64) * (K / 128) + b / 4) * 256 + (b & 3) * 64 + (c & 15) * 4 +
         (c >> 4);
}

// UE8M0 rule for e2m1 elements (largest magnitude 6 = 1.5 * 2^2): the
// smallest e in [-126, 127] with amax <= 6 * 2^e.
__device__ __forceinline__ int mx_exponent_e2m1(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int ef = static_cast<int>(u >> 23);
  if (ef == 0) return -126;
  const int e = ef - 127 - 2 + ((u & 0x7fffffu) > 0x400000u ? 1 : 0);
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}

// e2m1 code of v (nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even
// code, saturating at 6, sign kept): the midpoints between neighbours decide.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
  const float a = fabsf(v);
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return sign | c;
}

// One thread per 32 consecutive k of a weight row: exponent from the block
// maximum, then e4m3 (fmt 0, 32 bytes) or e2m1 (fmt 1, 16 bytes, even k in
// the low nibble) codes.
__global__ __launch_bounds__(256) void quant_weight_mx_kernel(const uint16_t* __restrict__ w,
                                                              int64_t rows, int N, int K, int fmt,
                                                              uint8_t* __restrict__ q,
                                                              uint8_t* __restrict__ s_tiled) {
  const int kb = K / 32;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * kb) return;
  const int64_t row = i / kb;
  const int b = static_cast<int>(i - row * kb);
  const uint16_t* src = w + row * K + b * 32;
  float f[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float t[8];
    unpack8(*reinterpret_cast<const uint4*>(src + 8 * j), t);
#pragma unroll
    for (int u = 0; u < 8; ++u) f[8 * j + u] = t[u];
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(f[j]));
  const int64_t so = mx_scale_offset(row / N, static_cast<int>(row % N), b, N, K);
  if (fmt == MOE_MX_E4M3) {
    const int e = ue8m0_exponent(amax);
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = e4m3x4(f[4 * j], f[4 * j + 1], f[4 * j + 2], f[4 * j + 3], e);
    uint4* dst = reinterpret_cast<uint4*>(q + row * K + b * 32);
    dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
    dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
    s_tiled[so] = static_cast<uint8_t>(e + 127);
  } else {
    const int e = mx_exponent_e2m1(amax);
    uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j)
      c[j / 8] |= f32_to_e2m1(__builtin_amdgcn_ldexpf(f[j], -e)) << (4 * (j % 8));
    *reinterpret_cast<uint4*>(q + row * (K / 2) + b * 16) = make_uint4(c[0], c[1], c[2], c[3]);
    s_tiled[so] = static_cast<uint8_t>(e + 127);
  }
}

// Plain MX scales [G][N][K/32] -> the tiled layout, one thread per byte.
__global__ __launch_bounds__(256) void mx_scales_tile_kernel(const uint8_t* __restrict__ s_plain,
                                                             int64_t total, int N, int K,
                                                             uint8_t* __restrict__ s_tiled) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int kb = K / 32;
  const int64_t row = i / kb;
  const int b = static_cast<int>(i - row * kb);
  s_tiled[mx_scale_offset(row / N, static_cast<int>(row % N), b, N, K)] = s_plain[i];
}

}  // namespace moe

using namespace moe;

extern "C" int32_t moe_quant_fp8_ue8m0(const void* x, int64_t M, int32_t K, int64_t ld_x,
                                       const int32_t* m_indices, uint8_t* q, uint8_t* scale,
                                       void* stream) {
  if (M < 0 || K <= 0 || ld_x < K) return MOE_EINVAL;
  if (K % 128 != 0) return MOE_EUNSUPPORTED;
  if (M == 0) return MOE_OK;
  if (!x || !q || !scale) return MOE_EINVAL;
  const int64_t nb = (M + 3) / 4;
  if (nb >= (1ll << 31)) return MOE_EINVAL;
  quant_rows_kernel<<<static_cast<int>(nb), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(x), M, K, ld_x, m_indices, q, scale);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int32_t moe_quant_weight_mx(const void* w, int32_t G, int32_t N, int32_t K,
                                       int32_t fmt, uint8_t* q, uint8_t* scale_tiled,
                                       void* stream) {
  if (G < 0 || N <= 0 || K <= 0) return MOE_EINVAL;
  if (fmt != MOE_MX_E4M3 && fmt != MOE_MX_E2M1) return MOE_EUNSUPPORTED;
  if (N % 64 != 0 || K % 128 != 0) return MOE_EUNSUPPORTED;
  if (G == 0) return MOE_OK;
  if (!w || !q || !scale_tiled) return MOE_EINVAL;
  const int64_t threads = static_cast<int64_t>(G) * N * (K / 32);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks >= (1ll << 31)) return MOE_EINVAL;
  quant_weight_mx_kernel<<<static_cast<int>(blocks), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(w), static_cast<int64_t>(G) * N, N, K, fmt, q, scale_tiled);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int32_t moe_mx_scales_tile(const uint8_t* scale_plain, int32_t G, int32_t N, int32_t K,
                                      uint8_t* scale_tiled, void* stream) {
  if (G < 0 || N <= 0 || K <= 0) return MOE_EINVAL;
  if (N % 64 != 0 || K % 128 != 0) return MOE_EUNSUPPORTED;
  if (G == 0) return MOE_OK;
  if (!scale_plain || !scale_tiled) return MOE_EINVAL;
  const int64_t total = static_cast<int64_t>(G) * N * (K / 32);
  const int64_t blocks = (total + 255) / 256;
  if (blocks >= (1ll << 31)) return MOE_EINVAL;
  mx_scales_tile_kernel<<<static_cast<int>(blocks), 256, 0, static_cast<hipStream_t>(stream)>>>(
      scale_plain, total, N, K, scale_tiled);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int32_t moe_quant_weight_fp8_ue8m0(const void* w, int32_t G, int32_t N, int32_t K,
                                              uint8_t* q, uint8_t* scale, void* stream) {
  if (G < 0 || N <= 0 || K <= 0) return MOE_EINVAL;
  if (N % 128 != 0 || K % 128 != 0) return MOE_EUNSUPPORTED;
  if (G == 0) return MOE_OK;
  if (!w || !q || !scale) return MOE_EINVAL;
  const int64_t blocks = static_cast<int64_t>(G) * (N / 128) * (K / 128);
  if (blocks >= (1ll << 31)) return MOE_EINVAL;
  quant_weight_kernel<<<static_cast<int>(blocks), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(w), N, K, q, scale);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int32_t moe_requant_weight_fp8_ue8m0(const uint8_t* q_in, const float* s_in, int32_t G,
                                                int32_t N, int32_t K, uint8_t* q_out,
                                                uint8_t* s_out, void* stream) {
  if (G < 0 || N <= 0 || K <= 0) return MOE_EINVAL;
  if (N % 128 != 0 || K % 128 != 0) return MOE_EUNSUPPORTED;
  if (G == 0) return MOE_OK;
  if (!q_in || !s_in || !q_out || !s_out) return MOE_EINVAL;
  const int64_t blocks = static_cast<int64_t>(G) * (N / 128) * (K / 128);
  if (blocks >= (1ll << 31)) return MOE_EINVAL;
  requant_weight_kernel<<<static_cast<int>(blocks), 256, 0, static_cast<hipStream_t>(stream)>>>(
      q_in, s_in, N, K, q_out, s_out);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int32_t silu_and_mul(const void* gateup, int64_t M, int32_t I, const int32_t* m_indices,
                                const int32_t* masked_m, int32_t max_m, int32_t out_dtype, void* out,
                                uint8_t* out_scale, void* stream) {
  if (M < 0 || I <= 0) return MOE_EINVAL;
  if (I % 128 != 0) return MOE_EUNSUPPORTED;
  if (out_dtype != MOE_DTYPE_BF16 && out_dtype != MOE_DTYPE_FP8_E4M3_UE8M0) return MOE_EUNSUPPORTED;
  if (masked_m && m_indices) return MOE_EINVAL;
  if (masked_m && (max_m <= 0 || M % max_m != 0)) return MOE_EINVAL;
  if (M == 0) return MOE_OK;
  if (!gateup || !out) return MOE_EINVAL;
  if (out_dtype == MOE_DTYPE_FP8_E4M3_UE8M0 && !out_scale) return MOE_EINVAL;
  const int64_t nb = (M + 3) / 4;
  if (nb >= (1ll << 31)) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (out_dtype == MOE_DTYPE_FP8_E4M3_UE8M0)
    silu_mul_kernel<true><<<static_cast<int>(nb), 256, 0, s>>>(
        static_cast<const uint16_t*>(gateup), M, I, m_indices, masked_m, max_m,
        static_cast<uint8_t*>(out), out_scale);
  else
    silu_mul_kernel<false><<<static_cast<int>(nb), 256, 0, s>>>(
        static_cast<const uint16_t*>(gateup), M, I, m_indices, masked_m, max_m,
        static_cast<uint8_t*>(out), nullptr);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
