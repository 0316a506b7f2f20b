// Top-k routing: one wavefront per token.
//
// Selection is made on the fp32 logits (softmax is monotone, so the k most
// probable experts are the k largest logits); equal logits go to the lower
// expert index.  Weights are the chosen softmax terms renormalised over the k:
// w_j = exp(L_j - L_max) / sum_i exp(L_i - L_max), in fp32, summed in slot order.
#include "common.h"

namespace moe {

// order-preserving 32-bit key of a float (larger float -> larger key)
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int PER_LANE>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* L = logits + static_cast<int64_t>(t) * E;
  // candidate key: (ordered value << 32) | (~index), 0 = empty / taken
  uint64_t key[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    int e = lane + 64 * i;
    key[i] = e < E ? (static_cast<uint64_t>(ordered_key(L[e])) << 32) |
                         static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(e))
                   : 0ull;
  }
  int my_id = 0;
  float my_val = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      uint32_t lo = __shfl_xor(static_cast<uint32_t>(best), off, 64);
      uint32_t hi = __shfl_xor(static_cast<uint32_t>(best >> 32), off, 64);
      uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
      best = o > best ? o : best;
    }
    const int idx = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
      if (lane + 64 * i == idx) key[i] = 0;
    if (lane == j) {
      my_id = idx;
      my_val = L[idx];
    }
  }
  const float m = __shfl(my_val, 0, 64);
  const float s = lane < k ? expf(my_val - m) : 0.0f;
  float den = 0.0f;
  for (int j = 0; j < k; ++j) den = __fadd_rn(den, __shfl(s, j, 64));
  if (lane < k) {
    ids[static_cast<int64_t>(t) * k + lane] = my_id;
    weights[static_cast<int64_t>(t) * k + lane] = s / den;
  }
}

}  // namespace moe

extern "C" int32_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                                  int32_t* topk_ids, float* topk_weights, void* stream) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 32) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((T + 3) / 4), block(256);
  const int per = (E + 63) / 64;
  if (per <= 1)
    moe::route_topk_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, topk_ids, topk_weights);
  else if (per <= 2)
    moe::route_topk_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, topk_ids, topk_weights);
  else if (per <= 4)
    moe::route_topk_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, topk_ids, topk_weights);
  else if (per <= 8)
    moe::route_topk_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, topk_ids, topk_weights);
  else
    moe::route_topk_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, topk_ids, topk_weights);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
