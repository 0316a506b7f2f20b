// Tile order of the compact-layout register-streamed grouped GEMM
// (gemm_wreg.hip): the run table each workgroup builds from m_indices, the
// position -> tile decoder, and the small LDS and wait helpers the kernel uses
// around it.
//
// Order: expert runs (maximal stretches of 128-row blocks with one expert id)
// in row order; a run of z valid rows is cut into ceil(z / 256) M-tiles of
// equal height (rounded up to the kernel's row quantum); inside a run, groups
// of up to kGM M-tiles, N-tiles in order, the group's M-tiles innermost, so
// the workgroups of an XCD running side by side share weight panels (few
// M-tiles per expert) or tile a block of M-tiles by N-tiles (hot experts).
// The positions are cut into eight contiguous shares, one per XCD (workgroup
// ids are dealt round-robin over the XCDs, each with its own L2); workgroup b
// takes positions lo + b / 8, lo + b / 8 + grid / 8, ... of its XCD's share.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

namespace moe {
namespace runs {

constexpr int kTileRows = 256;     // rows of an M-tile at most
constexpr int kGM = 8;             // M-tiles of a group in the order
constexpr int kTable = 1024;       // run-table entries (one XCD's share)
constexpr int kMaxBlocks = 8160;   // 128-row blocks of A (about a million rows)
// LDS bytes the set-up needs as scratch before the kernel's stages are used
constexpr int kSetupBytes = (2 * kMaxBlocks + 24) * 4;

// vmcnt <= N, lgkmcnt 0 (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}
// Run-table reads are hand-written: the compiler would otherwise order them
// after every outstanding direct-to-LDS load, which never touches the table.
__device__ __forceinline__ int4 lds_read_run(const int4* t) {
  int4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(t)) : "memory");
  return v;
}

// exclusive scans over the workgroup's 256 threads (scr: 8 ints of LDS)
__device__ __forceinline__ int scan_excl_max(int v, int* scr) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc = max(inc, o);
  }
  if (lane == 63) scr[w] = inc;
  __syncthreads();
  int ex = __shfl_up(inc, 1, 64);
  if (lane == 0) ex = INT_MIN;
  for (int q = 0; q < w; ++q) ex = max(ex, scr[q]);
  __syncthreads();
  return ex;
}
__device__ __forceinline__ int2 scan_excl_sum2(int a, int b, int* scr, int2& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int oa = __shfl_up(ia, off, 64), ob = __shfl_up(ib, off, 64);
    if (lane >= off) {
      ia += oa;
      ib += ob;
    }
  }
  if (lane == 63) {
    scr[2 * w] = ia;
    scr[2 * w + 1] = ib;
  }
  __syncthreads();
  int pa = 0, pb = 0, ta = 0, tb = 0;
  for (int q = 0; q < 4; ++q) {
    if (q < w) {
      pa += scr[2 * q];
      pb += scr[2 * q + 1];
    }
    ta += scr[2 * q];
    tb += scr[2 * q + 1];
  }
  __syncthreads();
  total = make_int2(ta, tb);
  return make_int2(pa + ia - a, pb + ib - b);
}

// M-tiles of a run with z valid rows: as few as the tile height allows, so an
// expert with at most 256 rows is one tile and its weights stream once
__device__ __forceinline__ int tiles_of(int z) { return (z + kTileRows - 1) / kTileRows; }

// A tile: rows [row, row + rows) of A/C, expert id, N-tile nt
struct Tile {
  int64_t row;
  int rows, id, nt;
};

// Position pos of the order -> tile (rows <= 0: an empty position).  Run-table
// entries (P = first position, first row, valid rows, expert) are sorted by P;
// the cursor only moves forward since a workgroup's positions increase.  Tile
// heights are rounded up to a multiple of Q rows.
template <int Q>
__device__ __forceinline__ Tile decode(const int4* table, int nr, int& cur, int pos, int ntn) {
  int4 r;
  int nt;
  for (;;) {
    r = lds_read_run(table + cur);
    r.x = __builtin_amdgcn_readfirstlane(r.x);
    r.y = __builtin_amdgcn_readfirstlane(r.y);
    r.z = __builtin_amdgcn_readfirstlane(r.z);
    r.w = __builtin_amdgcn_readfirstlane(r.w);
    nt = tiles_of(r.z);
    if (pos < r.x + nt * ntn || cur + 1 >= nr) break;
    ++cur;
  }
  Tile t;
  const int q = pos - r.x;
  const int mg = q / (kGM * ntn);
  const int m0 = mg * kGM;
  const int gsz = min(kGM, nt - m0);
  const int rest = q - mg * kGM * ntn;
  const int ntile = gsz > 0 ? rest / gsz : 0;
  const int m = m0 + rest - ntile * gsz;
  const int h = ((r.z + nt - 1) / nt + Q - 1) / Q * Q;
  const int r0 = m * h;
  t.rows = (q < 0 || q >= nt * ntn || gsz <= 0) ? 0 : min(h, r.z - r0);
  t.row = static_cast<int64_t>(r.y) + r0;
  t.id = r.w;
  t.nt = ntile;
  return t;
}

// This workgroup's share of the order: NR run-table entries in `table`,
// positions [lo, hi) of its XCD, grid / 8 workgroups per XCD.
struct Share {
  int NR, lo, hi, per_xcd;
};

// Builds the run table of this workgroup's XCD share into `table` (kTable
// entries of LDS), using `scratch` (kSetupBytes of LDS, free afterwards) for
// the per-block ids.  All 256 threads call it; it ends with a barrier.
// Returns false when the workgroup has no position to run.
__device__ __forceinline__ bool build_share(const int32_t* __restrict__ m_indices, int64_t M, int G,
                                            int ntn, uint8_t* scratch, int4* table, Share& sh) {
  constexpr int kThreads = 256;
  const int tid = threadIdx.x;
  const int nblk = static_cast<int>((M + 127) / 128);
  int* const ids = reinterpret_cast<int*>(scratch);  // [nblk] first-row ids
  int* const scr = ids + kMaxBlocks + 8;
  int* const zv = scr + 16;  // [nblk] valid rows of the run ending at block j
  for (int j = tid; j < nblk; j += kThreads) {
    const int v = m_indices[static_cast<int64_t>(j) * 128];
    ids[j] = (v >= 0 && v < G) ? v : -1;
  }
  __syncthreads();
  const int PB = (nblk + kThreads - 1) / kThreads;
  const int j0 = min(tid * PB, nblk), j1 = min(j0 + PB, nblk);
  // block j starts a run if its id differs from the block before; ends one if
  // the block after differs
  int ls = -1;
  for (int j = j0; j < j1; ++j)
    if (ids[j] >= 0 && (j == 0 || ids[j - 1] != ids[j])) ls = j;
  const int carry = max(scan_excl_max(ls, scr), -1);
  // runs ending in this thread's blocks: their valid rows (the last block's
  // valid rows come first, so a binary search for its first negative entry)
  // and M-tiles
  int cnt = 0, tsum = 0;
  {
    int S = carry;
    for (int j = j0; j < j1; ++j) {
      const int v = ids[j];
      if (v >= 0 && (j == 0 || ids[j - 1] != v)) S = j;
      if (v >= 0 && (j == nblk - 1 || ids[j + 1] != v)) {
        const int64_t r0 = static_cast<int64_t>(j) * 128;
        int lo = 1, hi = M - r0 < 128 ? static_cast<int>(M - r0) : 128;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (m_indices[r0 + mid] >= 0) lo = mid + 1;
          else hi = mid;
        }
        const int z = (j - S) * 128 + lo;
        zv[j] = z;
        ++cnt;
        tsum += tiles_of(z);
      }
    }
  }
  int2 tot;
  const int2 base = scan_excl_sum2(cnt, tsum, scr, tot);
  const int U = tot.y * ntn;  // positions of the whole order
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7;
  const int lo_x = static_cast<int>((static_cast<int64_t>(U) * xcd) >> 3);
  const int hi_x = static_cast<int>((static_cast<int64_t>(U) * (xcd + 1)) >> 3);
  // runs ending at or before lo_x, runs starting before hi_x
  int c_lo = 0, c_hi = 0;
  {
    int S = carry, mb = base.y;
    for (int j = j0; j < j1; ++j) {
      const int v = ids[j];
      if (v >= 0 && (j == 0 || ids[j - 1] != v)) S = j;
      if (v >= 0 && (j == nblk - 1 || ids[j + 1] != v)) {
        const int nt = tiles_of(zv[j]);
        if ((mb + nt) * ntn <= lo_x) ++c_lo;
        if (mb * ntn < hi_x) ++c_hi;
        mb += nt;
      }
    }
  }
  int2 cc;
  scan_excl_sum2(c_lo, c_hi, scr, cc);
  const int R0 = cc.x, NR = cc.y - cc.x;
  {
    int S = carry, mb = base.y, ri = base.x;
    for (int j = j0; j < j1; ++j) {
      const int v = ids[j];
      if (v >= 0 && (j == 0 || ids[j - 1] != v)) S = j;
      if (v >= 0 && (j == nblk - 1 || ids[j + 1] != v)) {
        const int z = zv[j];
        const int nt = tiles_of(z);
        const int P = mb * ntn, Pe = (mb + nt) * ntn;
        if (Pe > lo_x && P < hi_x && ri - R0 >= 0 && ri - R0 < kTable)
          table[ri - R0] = make_int4(P, S * 128, z, v);
        ++ri;
        mb += nt;
      }
    }
  }
  __syncthreads();  // table complete; the scratch is free
  sh.NR = NR;
  sh.lo = lo_x;
  sh.hi = hi_x;
  sh.per_xcd = per_xcd;
  return NR > 0 && NR <= kTable && lo_x + static_cast<int>(blockIdx.x >> 3) < hi_x;
}

}  // namespace runs
}  // namespace moe
