// Weighted combine back to token order: one workgroup per token, each thread
// 8 consecutive channels.  Slots are summed in order j = 0..k-1 with explicit
// round-to-nearest fp32 multiply and add (no contraction), so the result is
// the same for a token whatever batch it arrives in.
#include "common.cuh"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ Y,
                                                      int64_t num_rows,
                                                      const int32_t* __restrict__ src2dst,
                                                      const float* __restrict__ w, int k, int H,
                                                      uint16_t* __restrict__ out) {
#pragma clang fp contract(off)
  __shared__ int rows[32];
  __shared__ float wt[32];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    const int r = src2dst[static_cast<int64_t>(t) * k + threadIdx.x];
    rows[threadIdx.x] = r < num_rows ? r : -1;
    wt[threadIdx.x] = w[static_cast<int64_t>(t) * k + threadIdx.x];
  }
  __syncthreads();
  for (int col = threadIdx.x * 8; col < H; col += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = rows[j];
      if (r < 0) continue;
      const float wj = wt[j];
      const uint4 v = *reinterpret_cast<const uint4*>(Y + static_cast<int64_t>(r) * H + col);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __fadd_rn(acc[2 * i], __fmul_rn(wj, bf16_to_f32(static_cast<uint16_t>(u[i] & 0xffffu))));
        acc[2 * i + 1] = __fadd_rn(acc[2 * i + 1], __fmul_rn(wj, bf16_to_f32(static_cast<uint16_t>(u[i] >> 16))));
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(out + static_cast<int64_t>(t) * H + col) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace moe

extern "C" int32_t moe_combine(const void* Y, int64_t num_rows, const int32_t* src2dst,
                               const float* topk_weights, int32_t T, int32_t k, int32_t H, void* out,
                               void* stream) {
  if (T < 0 || k < 1 || k > 32 || H <= 0 || num_rows < 0) return MOE_EINVAL;
  if (H % 8 != 0) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!Y || !src2dst || !topk_weights || !out) return MOE_EINVAL;
  moe::combine_kernel<<<T, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(Y), num_rows, src2dst, topk_weights, k, H, static_cast<uint16_t*>(out));
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
