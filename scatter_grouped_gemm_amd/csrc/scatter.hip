// Scatter of routed tokens into the compact or masked expert layout.
//
// Deterministic and atomic-free on the value path: row positions come from
// prefix sums, so the result is the same on every run.
//   1. count  : each wavefront counts the local expert ids of one chunk of
//               kChunk flat assignments (t*k + j) into per-chunk histograms.
//   2. scan   : one workgroup turns the histograms into per-chunk offsets, the
//               per-expert totals, padded sizes and expert start rows.
//   3. rank   : each wavefront walks its chunk in order, 64 assignments at a
//               time; lanes with the same expert are found with ballots and
//               ranked by lane order, so rows follow increasing (t, j).  Writes
//               src2dst and the assignment of each valid row (src, indexed by
//               the expert's first valid-row number plus the rank).
//               (compact) m_indices is filled by a grid-stride pass.
//   4. rows   : one workgroup per token reads its row once and writes it to
//               each destination row, optionally quantised to e4m3 with
//               per-128-channel UE8M0 scales; the scale bytes are staged
//               token-major.
//   5. scales : (FP8) one thread per destination row copies its token's
//               staged scale bytes into the K-block-major scale array, so
//               each block's line is written by consecutive threads.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace moe {

constexpr int kChunk = 256;    // assignments per wavefront chunk
constexpr int kWsHeader = 256;  // bytes: device error word, the scan's ticket, padding

struct ScatterWs {
  int32_t* err;
  int32_t* counts;  // [C][El]
  int32_t* start;   // [El] first row of expert e (compact; 0 for masked)
  int32_t* total;   // [El] assignments of expert e
  int32_t* vstart;  // [El] assignments of the experts before e
  int32_t* src;     // [A] assignment t*k + j of valid row vstart[e] + rank
  uint8_t* tscale;  // [T][tscale_ld(H)] FP8: each token's UE8M0 scale bytes
};

__host__ __device__ inline int64_t num_chunks(int64_t A) { return (A + kChunk - 1) / kChunk; }

inline size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// Row stride of the staged scale bytes: H/128 rounded up to whole 8-byte words.
__host__ __device__ inline int tscale_ld(int H) { return (H / 128 + 7) & ~7; }

// Scratch of a scatter of T tokens, top-k, El local experts, H channels.
inline size_t ws_bytes(int64_t T, int k, int El, int H) {
  const int64_t A = T * k;
  return kWsHeader + align256(static_cast<size_t>(num_chunks(A)) * El * 4) +
         3 * align256(static_cast<size_t>(El) * 4) + align256(static_cast<size_t>(A) * 4) +
         align256(static_cast<size_t>(T) * tscale_ld(H));
}

inline ScatterWs carve(void* ws, int64_t T, int k, int El) {
  const int64_t A = T * k;
  uint8_t* b = static_cast<uint8_t*>(ws);
  ScatterWs w;
  w.err = reinterpret_cast<int32_t*>(b);
  b += kWsHeader;
  w.counts = reinterpret_cast<int32_t*>(b);
  b += align256(static_cast<size_t>(num_chunks(A)) * El * 4);
  w.start = reinterpret_cast<int32_t*>(b);
  b += align256(static_cast<size_t>(El) * 4);
  w.total = reinterpret_cast<int32_t*>(b);
  b += align256(static_cast<size_t>(El) * 4);
  w.vstart = reinterpret_cast<int32_t*>(b);
  b += align256(static_cast<size_t>(El) * 4);
  w.src = reinterpret_cast<int32_t*>(b);
  b += align256(static_cast<size_t>(A) * 4);
  w.tscale = b;
  return w;
}

__global__ __launch_bounds__(256) void scatter_count_kernel(const int32_t* __restrict__ ids,
                                                            int64_t A, int expert_start, int El,
                                                            int C, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ err) {
  extern __shared__ int lds_i[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + w;
  int* cnt = lds_i + w * El;
  for (int e = lane; e < El; e += 64) cnt[e] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    err[0] = 0;
    err[1] = 0;  // the scan's ticket
  }
  __syncthreads();
  if (c < C) {
    const int64_t a0 = static_cast<int64_t>(c) * kChunk;
    const int64_t a1 = a0 + kChunk < A ? a0 + kChunk : A;
    for (int64_t a = a0 + lane; a < a1; a += 64) {
      const int e = ids[a] - expert_start;
      if (e >= 0 && e < El) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  if (c < C)
    for (int e = lane; e < El; e += 64) counts[static_cast<int64_t>(c) * El + e] = cnt[e];
}

// Step 2, over ceil(El / 4) workgroups: wavefront e takes expert e's chunk
// counts (lane l a contiguous run of ceil(C / 64) chunks, loads batched),
// writes the exclusive per-chunk offsets in place and the expert's total.
// The last workgroup to finish (a ticket in the workspace header, zeroed by
// the count kernel; release by a fence before the ticket, acquire by a fence
// after it) scans the padded and the plain sizes over the experts.
__global__ __launch_bounds__(256) void scatter_scan_kernel(int32_t* __restrict__ counts, int C,
                                                           int El, int block_e, int clamp,
                                                           int32_t* __restrict__ start,
                                                           int32_t* __restrict__ total,
                                                           int32_t* __restrict__ vstart,
                                                           int32_t* __restrict__ start_out,
                                                           int32_t* __restrict__ valid_out,
                                                           int32_t* __restrict__ ticket) {
  __shared__ int64_t wsum[4];
  __shared__ int64_t wsum_v[4];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int e = blockIdx.x * 4 + w;
  if (e < El) {
    const int per = (C + 63) / 64;
    const int c0 = min(lane * per, C), c1 = min(c0 + per, C);
    constexpr int B = 8;
    // runs of up to B chunks (C <= 512) stay in registers between the passes
    int keep[B] = {};
    int sum = 0;
    for (int cb = c0; cb < c1; cb += B) {
      int v[B];
#pragma unroll
      for (int j = 0; j < B; ++j) v[j] = cb + j < c1 ? counts[static_cast<int64_t>(cb + j) * El + e] : 0;
#pragma unroll
      for (int j = 0; j < B; ++j) {
        sum += v[j];
        keep[j] = v[j];
      }
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    int base = incl - sum;
    const int tot = __shfl(incl, 63, 64);
    if (per <= B) {
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (c0 + j < c1) counts[static_cast<int64_t>(c0 + j) * El + e] = base;
        base += keep[j];
      }
    } else {
      for (int cb = c0; cb < c1; cb += B) {
        int v[B];
#pragma unroll
        for (int j = 0; j < B; ++j) v[j] = cb + j < c1 ? counts[static_cast<int64_t>(cb + j) * El + e] : 0;
#pragma unroll
        for (int j = 0; j < B; ++j) {
          if (cb + j < c1) counts[static_cast<int64_t>(cb + j) * El + e] = base;
          base += v[j];
        }
      }
    }
    if (lane == 0) total[e] = tot;
  }
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    last = atomicAdd(ticket, 1) == static_cast<int>(gridDim.x) - 1;
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  // thread t takes experts 4t .. 4t + 3 (El <= 1024)
  int run[4];
  int64_t pad[4];
  int64_t sp = 0, sv = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ee = tid * 4 + j;
    run[j] = ee < El ? total[ee] : 0;
    pad[j] = static_cast<int64_t>(run[j] + block_e - 1) / block_e * block_e;
    sp += pad[j];
    sv += run[j];
  }
  int64_t incl = sp, incl_v = sv;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t v = __shfl_up(incl, off, 64);
    const int64_t vv = __shfl_up(incl_v, off, 64);
    if (lane >= off) {
      incl += v;
      incl_v += vv;
    }
  }
  if (lane == 63) {
    wsum[w] = incl;
    wsum_v[w] = incl_v;
  }
  __syncthreads();
  for (int q = 0; q < w; ++q) {
    incl += wsum[q];
    incl_v += wsum_v[q];
  }
  int64_t bp = incl - sp, bv = incl_v - sv;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ee = tid * 4 + j;
    if (ee < El) {
      start[ee] = static_cast<int32_t>(bp);
      vstart[ee] = static_cast<int32_t>(bv);
      if (start_out) start_out[ee] = static_cast<int32_t>(bp);
      if (valid_out) valid_out[ee] = static_cast<int32_t>(clamp > 0 && run[j] > clamp ? clamp : run[j]);
    }
    bp += pad[j];
    bv += run[j];
  }
}

template <bool MASKED>
__global__ __launch_bounds__(256) void scatter_rank_kernel(
    const int32_t* __restrict__ ids, int64_t A, int expert_start, int El, int C,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ start,
    const int32_t* __restrict__ vstart, int max_m, int32_t* __restrict__ src2dst,
    int32_t* __restrict__ src, int32_t* __restrict__ err) {
  extern __shared__ int lds_i[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + w;
  if (c >= C) return;  // whole wavefront
  int* base = lds_i + w * El;
  for (int e = lane; e < El; e += 64)
    base[e] = offsets[static_cast<int64_t>(c) * El + e] + (MASKED ? 0 : start[e]);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const int bits = 32 - __clz(El);  // enough bits for the sentinel value El
  const uint64_t below = (1ull << lane) - 1ull;
  const int64_t a0 = static_cast<int64_t>(c) * kChunk;
  for (int s = 0; s < kChunk; s += 64) {
    const int64_t a = a0 + s + lane;
    const bool valid = a < A;
    int e = valid ? ids[a] - expert_start : -1;
    const bool local = valid && e >= 0 && e < El;
    const int key = local ? e : El;
    uint64_t mask = ballot(true);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t bal = ballot(bit);
      mask &= bit ? bal : ~bal;
    }
    const int rank = __popcll(mask & below);
    const int cnt = __popcll(mask);
    int r = 0;
    if (local) r = base[key] + rank;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (local && rank == 0) base[key] = r + cnt;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      int out = -1;
      if (local) {
        // rank of the assignment inside its expert
        const int re = MASKED ? r : r - start[key];
        if (!MASKED) {
          out = r;
        } else if (r < max_m) {
          out = key * max_m + r;
        } else {
          atomicOr(err, MOE_DEVERR_MASKED_OVERFLOW);
        }
        if (out >= 0) src[vstart[key] + re] = static_cast<int32_t>(a);
      }
      src2dst[a] = out;
    }
  }
}

// Steps 1-3 in one workgroup for small batches (one launch instead of three):
// wavefront w counts, then ranks, the w-th sixteenth of the assignments;
// thread e scans expert e's per-wavefront counts and the padded expert sizes.
// Ranks are the same as the chunked kernels': a row's rank is the number of
// earlier assignments (in t*k + j order) of its expert.
constexpr int kSmallWaves = 16;
constexpr int64_t kSmallA = 16384;  // assignments handled by the one-workgroup path

// dynamic LDS of the one-workgroup kernel for El local experts
constexpr size_t small_lds_bytes(int El) {
  return (static_cast<size_t>(kSmallWaves) * El + 2 * 1024 + 2 * static_cast<size_t>(El)) * sizeof(int);
}

template <bool MASKED>
__global__ __launch_bounds__(1024) void scatter_front_small_kernel(
    const int32_t* __restrict__ ids, int A, int expert_start, int El, int block_e, int max_m,
    int32_t* __restrict__ start, int32_t* __restrict__ total, int32_t* __restrict__ vstart,
    int32_t* __restrict__ start_out, int32_t* __restrict__ valid_out,
    int32_t* __restrict__ src2dst, int32_t* __restrict__ src, int32_t* __restrict__ err) {
  extern __shared__ int lds_i[];
  int* const cnt = lds_i;                          // [kSmallWaves][El]
  int* const scan = lds_i + kSmallWaves * El;      // [1024]
  int* const scan_v = scan + 1024;                 // [1024]
  int* const st_l = scan_v + 1024;                 // [El]
  int* const vs_l = st_l + El;                     // [El]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int per = (A + kSmallWaves * 64 - 1) / (kSmallWaves * 64) * 64;
  const int a0 = w * per, a1 = a0 + per < A ? a0 + per : A;
  if (tid == 0) *err = 0;
  for (int i = tid; i < kSmallWaves * El; i += 1024) cnt[i] = 0;
  __syncthreads();
  for (int a = a0 + lane; a < a1; a += 64) {
    const int e = ids[a] - expert_start;
    if (e >= 0 && e < El) atomicAdd(&cnt[w * El + e], 1);
  }
  __syncthreads();
  int run = 0;
  if (tid < El) {
    for (int q = 0; q < kSmallWaves; ++q) {
      const int v = cnt[q * El + tid];
      cnt[q * El + tid] = run;
      run += v;
    }
  }
  const int padded = tid < El ? (run + block_e - 1) / block_e * block_e : 0;
  const int plain = tid < El ? run : 0;
  scan[tid] = padded;
  scan_v[tid] = plain;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    const int vv = tid >= off ? scan_v[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    scan_v[tid] += vv;
    __syncthreads();
  }
  if (tid < El) {
    const int st = scan[tid] - padded;
    st_l[tid] = st;
    vs_l[tid] = scan_v[tid] - plain;
    start[tid] = st;
    total[tid] = run;
    vstart[tid] = scan_v[tid] - plain;
    if (start_out) start_out[tid] = st;
    if (valid_out) valid_out[tid] = MASKED && run > max_m ? max_m : run;
  }
  __syncthreads();
  int* const base = cnt + w * El;
  if (!MASKED)
    for (int e = lane; e < El; e += 64) base[e] += st_l[e];
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const int bits = 32 - __clz(El);
  const uint64_t below = (1ull << lane) - 1ull;
  for (int s0 = a0; s0 < a1; s0 += 64) {
    const int a = s0 + lane;
    const bool valid = a < a1;
    const int e = valid ? ids[a] - expert_start : -1;
    const bool local = valid && e >= 0 && e < El;
    const int key = local ? e : El;
    uint64_t mask = ballot(true);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t bal = ballot(bit);
      mask &= bit ? bal : ~bal;
    }
    const int rank = __popcll(mask & below);
    const int cnt_e = __popcll(mask);
    int r = 0;
    if (local) r = base[key] + rank;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (local && rank == 0) base[key] = r + cnt_e;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      int out = -1;
      if (local) {
        const int re = MASKED ? r : r - st_l[key];
        if (!MASKED) {
          out = r;
        } else if (r < max_m) {
          out = key * max_m + r;
        } else {
          atomicOr(err, MOE_DEVERR_MASKED_OVERFLOW);
        }
        if (out >= 0) src[vs_l[key] + re] = a;
      }
      src2dst[a] = out;
    }
  }
}

__global__ __launch_bounds__(256) void fill_m_indices_kernel(const int32_t* __restrict__ start,
                                                             const int32_t* __restrict__ total,
                                                             int El, int64_t R,
                                                             int32_t* __restrict__ m_indices) {
  __shared__ int s_start[1024];
  __shared__ int s_total[1024];
  for (int e = threadIdx.x; e < El; e += blockDim.x) {
    s_start[e] = start[e];
    s_total[e] = total[e];
  }
  __syncthreads();
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; r < R;
       r += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    // last expert whose block starts at or before r (empty experts share the
    // start of the next one, so the last of equal starts owns the rows)
    int lo = 0, hi = El - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= r) lo = mid; else hi = mid - 1;
    }
    m_indices[r] = (r - s_start[lo] < s_total[lo]) ? lo : -1;
  }
}

// Destination scale index of row `row`, 128-channel block b.
__device__ __forceinline__ int64_t scale_index(int64_t row, int b, int64_t ld, int max_m, int HB) {
  if (max_m == 0) return static_cast<int64_t>(b) * ld + row;
  const int64_t g = row / max_m;
  return (g * HB + b) * max_m + (row - g * max_m);
}

// Step 4: the token's row, read once, copied (or quantised, FP8) to each of
// its destination rows.  FP8 scale bytes go to the token-major staging array
// tscale[t][H/128] (56 contiguous bytes per token instead of k * 56 scattered
// ones); scatter_scales_kernel moves them to the destination layout.
template <bool FP8>
__global__ __launch_bounds__(256) void scatter_rows_kernel(
    const uint16_t* __restrict__ x, int H, int k, const int32_t* __restrict__ src2dst,
    uint8_t* __restrict__ x_out, uint8_t* __restrict__ tscale) {
  __shared__ int rows[32];
  const int t = blockIdx.x;
  if (threadIdx.x < k) rows[threadIdx.x] = src2dst[static_cast<int64_t>(t) * k + threadIdx.x];
  __syncthreads();
  const uint16_t* xt = x + static_cast<int64_t>(t) * H;
  const int HB = H / 128;
  // up to four 2048-column passes per round, loads issued first
  constexpr int U = 4;
  for (int c0 = threadIdx.x * 8; c0 < H; c0 += U * 2048) {
    uint4 vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int col = c0 + u * 2048;
      if (col < H) vv[u] = *reinterpret_cast<const uint4*>(xt + col);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int col = c0 + u * 2048;
      if (col >= H) break;
      const uint4 v = vv[u];
      if (!FP8) {
        for (int j = 0; j < k; ++j) {
          const int r = rows[j];
          if (r >= 0) *reinterpret_cast<uint4*>(x_out + (static_cast<int64_t>(r) * H + col) * 2) = v;
        }
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float f[8];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xffffu));
          f[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
          amax = fmaxf(amax, fmaxf(fabsf(f[2 * i]), fabsf(f[2 * i + 1])));
        }
        amax = group_max<16>(amax);
        const int e = ue8m0_exponent(amax);
        const uint32_t lo = e4m3x4(f[0], f[1], f[2], f[3], e);
        const uint32_t hi = e4m3x4(f[4], f[5], f[6], f[7], e);
        const uint2 q = make_uint2(lo, hi);
        if ((threadIdx.x & 15) == 0)
          tscale[static_cast<int64_t>(t) * tscale_ld(H) + col / 128] = static_cast<uint8_t>(e + 127);
        for (int j = 0; j < k; ++j) {
          const int r = rows[j];
          if (r < 0) continue;
          *reinterpret_cast<uint2*>(x_out + static_cast<int64_t>(r) * H + col) = q;
        }
      }
    }
  }
}

// FP8 scale bytes in the destination layout, one thread per destination row
// (consecutive threads write consecutive bytes of each 128-channel block's
// scale line): valid row r of expert e has rank r_e inside e; its token is
// src[vstart[e] + r_e] / k, whose staged bytes are copied.  Compact rows take
// Compact: the expert of row r is found as fill_m_indices_kernel finds it,
// and m_indices[r] is written here too (the FP8 path has no separate fill
// launch); padding rows get -1 and no scales.  Masked row r belongs to group
// r / max_m and is valid below min(total, max_m).
template <bool MASKED>
__global__ __launch_bounds__(256) void scatter_scales_kernel(
    int32_t* __restrict__ m_indices, const int32_t* __restrict__ start,
    const int32_t* __restrict__ total, const int32_t* __restrict__ vstart,
    const int32_t* __restrict__ src, const uint8_t* __restrict__ tscale, int k, int HB,
    int64_t rows, int max_m, int El, uint8_t* __restrict__ scale_out) {
  __shared__ int s_start[MASKED ? 1 : 1024];
  __shared__ int s_total[MASKED ? 1 : 1024];
  if (!MASKED) {
    for (int e = threadIdx.x; e < El; e += blockDim.x) {
      s_start[e] = start[e];
      s_total[e] = total[e];
    }
    __syncthreads();
  }
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; r < rows;
       r += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    int e, re;
    if (MASKED) {
      e = static_cast<int>(r / max_m);
      re = static_cast<int>(r - static_cast<int64_t>(e) * max_m);
      if (re >= min(total[e], max_m)) continue;
    } else {
      int lo = 0, hi = El - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_start[mid] <= r) lo = mid; else hi = mid - 1;
      }
      const bool valid = r - s_start[lo] < s_total[lo];
      m_indices[r] = valid ? lo : -1;
      if (!valid) continue;
      e = lo;
      re = static_cast<int>(r - s_start[lo]);
    }
    const int64_t t = src[vstart[e] + re] / k;
    // the token's bytes as 8-byte words (rows of the staging array are whole
    // words), then one byte per 128-channel block
    const uint64_t* ts = reinterpret_cast<const uint64_t*>(tscale + t * ((HB + 7) & ~7));
    for (int b0 = 0; b0 < HB; b0 += 8) {
      const uint64_t v = ts[b0 >> 3];
      for (int b = b0; b < b0 + 8 && b < HB; ++b)
        scale_out[scale_index(r, b, rows, MASKED ? max_m : 0, HB)] = static_cast<uint8_t>(v >> (8 * (b - b0)));
    }
  }
}

int32_t validate_common(const void* x, int32_t T, int32_t H, const int32_t* ids, int32_t k,
                        int32_t El, int32_t out_dtype, void* x_out, const uint8_t* scale_out,
                        int32_t* src2dst) {
  if (T < 0 || H <= 0 || k < 1 || k > 32 || El < 1 || El > 1024) return MOE_EINVAL;
  if (static_cast<int64_t>(T) * k >= (1ll << 31)) return MOE_EINVAL;
  if (H % 128 != 0) return MOE_EUNSUPPORTED;
  if (out_dtype != MOE_DTYPE_BF16 && out_dtype != MOE_DTYPE_FP8_E4M3_UE8M0) return MOE_EUNSUPPORTED;
  if (out_dtype == MOE_DTYPE_FP8_E4M3_UE8M0 && !scale_out) return MOE_EINVAL;
  if (T > 0 && (!x || !ids || !x_out || !src2dst)) return MOE_EINVAL;
  return MOE_OK;
}

int32_t validate_ws(int32_t T, int32_t k, int32_t El, int32_t H, const void* ws,
                    size_t ws_bytes_given) {
  if (!ws || ws_bytes_given < ws_bytes(T, k, El, H)) return MOE_ECAPACITY;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_scatter_ws_bytes(int32_t T, int32_t k, int32_t num_local_experts, int32_t H) {
  if (T < 0 || k < 1 || num_local_experts < 1 || H < 0) return 0;
  return ws_bytes(T, k, num_local_experts, H);
}

extern "C" int64_t moe_compact_rows_bound(int64_t A, int32_t E, int32_t block_e) {
  if (A < 0 || E <= 0 || block_e <= 0) return -1;
  const int64_t n = A < E ? A : E;
  return static_cast<int64_t>(block_e) * (n + (A - n) / block_e);
}

extern "C" int32_t moe_use_masked_layout(int32_t num_experts, int32_t num_local_experts) {
  return (num_experts > num_local_experts && num_local_experts <= 32) ? 1 : 0;
}

// Measured on MI355X (whole expert path, both layouts, 16 .. 16384 tokens):
// masked wins while experts hold few rows (its 16/32/64-row tiles), compact
// from about 64 rows per expert on; masked buffers (E_local * max_tokens rows)
// are capped at kMaskedRowsFactor times the compact bound.
constexpr int64_t kMaskedMeanRows = 64;
constexpr int64_t kMaskedRowsFactor = 4;
extern "C" int32_t moe_choose_layout(int64_t max_tokens, int32_t top_k, int32_t num_experts,
                                     int32_t num_local_experts, int32_t block_e) {
  if (max_tokens <= 0 || top_k <= 0 || num_experts <= 0 || num_local_experts <= 0 ||
      num_local_experts > num_experts || top_k > num_experts || block_e <= 0 || max_tokens > (1ll << 40))
    return -1;
  const int64_t compact = moe_compact_rows_bound(max_tokens * top_k, num_local_experts, block_e);
  const bool few_rows = max_tokens * top_k <= kMaskedMeanRows * num_experts;
  const bool fits = max_tokens * num_local_experts <= kMaskedRowsFactor * compact;
  return (few_rows && fits) ? 1 : 0;
}

static int32_t launch_front(const int32_t* ids, int64_t A, int32_t expert_start, int32_t El,
                            int32_t block_e, const ScatterWs& w, int32_t* start_out,
                            int32_t* valid_out, bool masked, int32_t max_m, int32_t* src2dst,
                            hipStream_t s) {
  if (A <= kSmallA) {
    const size_t lds = small_lds_bytes(El);
    // The LDS limit is raised once per device and layout (thread-safe).
    static std::once_flag attr_once[64][2];
    static bool attr_ok[64][2] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_EDEVICE;
    auto kern = masked ? scatter_front_small_kernel<true> : scatter_front_small_kernel<false>;
    const int li = masked ? 1 : 0;
    std::call_once(attr_once[dev][li], [&]() {
      attr_ok[dev][li] =
          hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(small_lds_bytes(1024))) == hipSuccess;
    });
    if (!attr_ok[dev][li]) return MOE_EDEVICE;
    kern<<<1, 1024, lds, s>>>(ids, static_cast<int>(A), expert_start, El, masked ? 1 : block_e,
                              masked ? max_m : 0, w.start, w.total, w.vstart, start_out, valid_out,
                              src2dst, w.src, w.err);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  const int C = static_cast<int>(num_chunks(A));
  const int nb = (C + 3) / 4;
  const size_t lds = static_cast<size_t>(4) * El * sizeof(int);
  if (C > 0) {
    scatter_count_kernel<<<nb, 256, lds, s>>>(ids, A, expert_start, El, C, w.counts, w.err);
  } else {
    scatter_count_kernel<<<1, 256, lds, s>>>(ids, 0, expert_start, El, 0, w.counts, w.err);
  }
  MOE_CHECK_LAUNCH();
  scatter_scan_kernel<<<(El + 3) / 4, 256, 0, s>>>(w.counts, C, El, masked ? 1 : block_e,
                                                  masked ? max_m : 0, w.start, w.total, w.vstart,
                                                  start_out, valid_out, w.err + 1);
  MOE_CHECK_LAUNCH();
  if (C > 0) {
    if (masked)
      scatter_rank_kernel<true><<<nb, 256, lds, s>>>(ids, A, expert_start, El, C, w.counts,
                                                     w.start, w.vstart, max_m, src2dst, w.src,
                                                     w.err);
    else
      scatter_rank_kernel<false><<<nb, 256, lds, s>>>(ids, A, expert_start, El, C, w.counts,
                                                      w.start, w.vstart, 0, src2dst, w.src, w.err);
    MOE_CHECK_LAUNCH();
  }
  return MOE_OK;
}

// Everything after argument validation of the compact scatter: the workspace
// `ws` (at least ws_bytes(T, k, El, H) bytes) is supplied by the caller or is the
// library's static scratch array.
static int32_t scatter_compact_body(const void* x, int32_t T, int32_t H, const int32_t* topk_ids,
                                    int32_t k, int32_t expert_start, int32_t El, int32_t block_e,
                                    int64_t rows_capacity, int32_t out_dtype, void* x_out,
                                    uint8_t* scale_out, int32_t* m_indices,
                                    int32_t* expert_start_loc, int32_t* num_valid,
                                    int32_t* src2dst, void* ws, hipStream_t s) {
  const int64_t A = static_cast<int64_t>(T) * k;
  const ScatterWs w = carve(ws, T, k, El);
  int32_t st = launch_front(topk_ids, A, expert_start, El, block_e, w, expert_start_loc, num_valid, false, 0,
                    src2dst, s);
  if (st != MOE_OK) return st;
  const bool fp8 = out_dtype == MOE_DTYPE_FP8_E4M3_UE8M0;
  // the FP8 scale pass writes m_indices itself
  if (rows_capacity > 0 && !(fp8 && T > 0)) {
    int64_t nb = (rows_capacity + 255) / 256;
    if (nb > 2048) nb = 2048;
    fill_m_indices_kernel<<<static_cast<int>(nb), 256, 0, s>>>(w.start, w.total, El, rows_capacity,
                                                               m_indices);
    MOE_CHECK_LAUNCH();
  }
  if (T > 0) {
    if (fp8)
      scatter_rows_kernel<true><<<T, 256, 0, s>>>(static_cast<const uint16_t*>(x), H, k, src2dst,
                                                  static_cast<uint8_t*>(x_out), w.tscale);
    else
      scatter_rows_kernel<false><<<T, 256, 0, s>>>(static_cast<const uint16_t*>(x), H, k, src2dst,
                                                   static_cast<uint8_t*>(x_out), nullptr);
    MOE_CHECK_LAUNCH();
    if (fp8 && rows_capacity > 0) {
      const int64_t nb = std::min<int64_t>((rows_capacity + 255) / 256, 2048);
      scatter_scales_kernel<false><<<static_cast<int>(nb), 256, 0, s>>>(
          m_indices, w.start, w.total, w.vstart, w.src, w.tscale, k, H / 128, rows_capacity, 0, El,
          scale_out);
      MOE_CHECK_LAUNCH();
    }
  }
  return MOE_OK;
}

static int32_t validate_compact(int32_t T, int32_t k, int32_t El, int32_t block_e,
                                int64_t rows_capacity, const int32_t* m_indices,
                                const int32_t* expert_start_loc, const int32_t* num_valid) {
  if (block_e <= 0 || block_e % 128 != 0) return MOE_EUNSUPPORTED;
  if (!expert_start_loc || !num_valid || (rows_capacity > 0 && !m_indices)) return MOE_EINVAL;
  if (rows_capacity < moe_compact_rows_bound(static_cast<int64_t>(T) * k, El, block_e))
    return MOE_ECAPACITY;
  if (rows_capacity >= (1ll << 31)) return MOE_EINVAL;
  return MOE_OK;
}

extern "C" int32_t moe_scatter_compact(const void* x, int32_t T, int32_t H, const int32_t* topk_ids,
                                       int32_t k, int32_t expert_start, int32_t El,
                                       int32_t block_e, int64_t rows_capacity, int32_t out_dtype,
                                       void* x_out, uint8_t* scale_out, int32_t* m_indices,
                                       int32_t* expert_start_loc, int32_t* num_valid,
                                       int32_t* src2dst, void* ws, size_t ws_bytes_given,
                                       void* stream) {
  int32_t st = validate_common(x, T, H, topk_ids, k, El, out_dtype, x_out, scale_out, src2dst);
  if (st != MOE_OK) return st;
  st = validate_ws(T, k, El, H, ws, ws_bytes_given);
  if (st != MOE_OK) return st;
  st = validate_compact(T, k, El, block_e, rows_capacity, m_indices, expert_start_loc, num_valid);
  if (st != MOE_OK) return st;
  return scatter_compact_body(x, T, H, topk_ids, k, expert_start, El, block_e, rows_capacity,
                              out_dtype, x_out, scale_out, m_indices, expert_start_loc, num_valid,
                              src2dst, ws, static_cast<hipStream_t>(stream));
}

// Scratch of the allocation-free compact scatter: one copy per device, kept
// until the process ends.  Host code never passes this name to a kernel or a
// copy (on the host it is only a stand-in for the symbol); it uses the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_SCATTER_NOALLOC_MAX_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
static int32_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EDEVICE;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = p;
  });
  if (!g_scratch_ptr[dev]) return MOE_EDEVICE;
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

extern "C" int32_t moe_scatter_compact_noalloc(const void* x, int32_t T, int32_t H,
                                               const int32_t* topk_ids, int32_t k,
                                               int32_t expert_start, int32_t El, int32_t block_e,
                                               int64_t rows_capacity, int32_t out_dtype,
                                               void* x_out, uint8_t* scale_out,
                                               int32_t* m_indices, int32_t* expert_start_loc,
                                               int32_t* num_valid, int32_t* src2dst,
                                               void* stream) {
  int32_t st = validate_common(x, T, H, topk_ids, k, El, out_dtype, x_out, scale_out, src2dst);
  if (st != MOE_OK) return st;
  st = validate_compact(T, k, El, block_e, rows_capacity, m_indices, expert_start_loc, num_valid);
  if (st != MOE_OK) return st;
  if (ws_bytes(T, k, El, H) > MOE_SCATTER_NOALLOC_MAX_BYTES) return MOE_ECAPACITY;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  // Nothing in the scratch has to start at zero: the first kernel clears the
  // error word and every count is written before it is read.
  return scatter_compact_body(x, T, H, topk_ids, k, expert_start, El, block_e, rows_capacity,
                              out_dtype, x_out, scale_out, m_indices, expert_start_loc, num_valid,
                              src2dst, ws, static_cast<hipStream_t>(stream));
}

extern "C" int32_t moe_scatter_masked(const void* x, int32_t T, int32_t H, const int32_t* topk_ids,
                                      int32_t k, int32_t expert_start, int32_t El, int32_t max_m,
                                      int32_t out_dtype, void* x_out, uint8_t* scale_out,
                                      int32_t* masked_m, int32_t* src2dst, void* ws,
                                      size_t ws_bytes_given, void* stream) {
  int32_t st = validate_common(x, T, H, topk_ids, k, El, out_dtype, x_out, scale_out, src2dst);
  if (st != MOE_OK) return st;
  st = validate_ws(T, k, El, H, ws, ws_bytes_given);
  if (st != MOE_OK) return st;
  if (!masked_m || max_m <= 0) return MOE_EINVAL;
  if (max_m < T) return MOE_ECAPACITY;
  if (static_cast<int64_t>(El) * max_m >= (1ll << 31)) return MOE_EINVAL;
  const int64_t A = static_cast<int64_t>(T) * k;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ScatterWs w = carve(ws, T, k, El);
  st = launch_front(topk_ids, A, expert_start, El, 1, w, nullptr, masked_m, true, max_m, src2dst, s);
  if (st != MOE_OK) return st;
  if (T > 0) {
    const bool fp8 = out_dtype == MOE_DTYPE_FP8_E4M3_UE8M0;
    if (fp8)
      scatter_rows_kernel<true><<<T, 256, 0, s>>>(static_cast<const uint16_t*>(x), H, k, src2dst,
                                                  static_cast<uint8_t*>(x_out), w.tscale);
    else
      scatter_rows_kernel<false><<<T, 256, 0, s>>>(static_cast<const uint16_t*>(x), H, k, src2dst,
                                                   static_cast<uint8_t*>(x_out), nullptr);
    MOE_CHECK_LAUNCH();
    if (fp8) {
      const int64_t rows = static_cast<int64_t>(El) * max_m;
      const int64_t nb = std::min<int64_t>((rows + 255) / 256, 2048);
      scatter_scales_kernel<true><<<static_cast<int>(nb), 256, 0, s>>>(
          nullptr, w.start, w.total, w.vstart, w.src, w.tscale, k, H / 128, rows, max_m, El, scale_out);
      MOE_CHECK_LAUNCH();
    }
  }
  return MOE_OK;
}

extern "C" int32_t moe_get_device_error(const void* ws, int32_t* host_err, void* stream) {
  if (!ws || !host_err) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(host_err, ws, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
    return MOE_EDEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_EDEVICE;
  return MOE_OK;
}

extern "C" const char* moe_status_str(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported dtype or alignment";
    case MOE_ECAPACITY: return "buffer below the required capacity";
    case MOE_EDEVICE: return "HIP launch or copy failed";
    default: return "unknown status";
  }
}
