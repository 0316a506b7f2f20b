// Grouped NT GEMM for the expert layouts: C[r, :] = A[r, :] . B[g(r)]^T,
// BF16 or FP8 e4m3 with UE8M0 scales, fp32 accumulation, bf16 output.
//
// The compact-layout calls with BF16 or 128x128-block FP8 weights and N a
// multiple of 256 go to the register-streamed kernel (gemm_wreg.hip); the
// kernel here serves the masked layout, the MX weight formats and the other
// shapes, and holds the entry points and their argument checks for both.
//
// Design (gfx950, wave64, 160 KB LDS):
//   - Persistent workgroups of 512 threads (8 wavefronts, two per SIMD), one
//     per CU.  A tile of C is BM x BN (128 x 256; 128 x 128 when N % 256 != 0;
//     masked tiles are 64, 32 or 16 rows tall for small expected counts); each
//     wavefront owns a 64-row (or BM-row) by 64- or 32-column sub-tile.
//     When a stage is not a whole number of 1 KB loads per wavefront (16- and
//     32-row tiles), the first wavefronts issue one load more and wait accordingly.
//   - The k loop is one flat stream of k-steps over all of the workgroup's
//     tiles.  A k-step covers 128 bytes of every tile row (64 bf16 or 128
//     e4m3), moved from global memory straight into LDS (global_load_lds, 16
//     bytes per lane) through three stages.  The loads run three steps ahead
//     of the MFMAs and cross into the next tile while the current one
//     finishes, so a tile costs no pipeline fill or drain.  Each step waits for
//     its stage with one vmcnt count and one barrier, then reads the next
//     step's fragments from LDS while the current step's MFMAs run from
//     registers; the refill's loads are spread among those MFMAs.  16-byte
//     chunks of each 128-byte LDS row are XOR-permuted so the 16 lanes of a
//     fragment read hit distinct banks.
//   - MFMA: v_mfma_f32_16x16x32_bf16 for BF16 and the block-scaled
//     v_mfma_scale_f32_16x16x128_f8f6f4 for FP8.  The UE8M0 bytes are exactly
//     the E8M0 scales that instruction consumes; the per-128-channel activation
//     scale and the 128x128 weight-block scale are both constant over one
//     128-wide k step, so every lane supplies its row's (column's) byte and no
//     fp32 rescaling is done in the main loop.  The scale bytes of a step ride
//     with its data: one 1-byte direct load per lane (each lane's byte lands
//     zero-extended in its own LDS dword) into the stage's scale area.
//   - The weight tile is the MFMA "A" operand and the activation tile the "B"
//     operand, so the accumulator holds C^T: each lane owns 4 consecutive output
//     columns of one row and stores them (8 bytes) straight from registers at
//     the start of the step after the tile's last one, before that step's
//     loads, so the stores never sit behind a stage the next wait needs.  Rows
//     past the end of A (compact) or of the group (masked) are not written;
//     padding rows inside a tile are.
//   - Tile order, built on the device: only tiles holding valid rows are
//     listed, each expert's tiles form one run ordered N-tile-major with its
//     M-tiles innermost, so the workgroups that run at the same time share each
//     weight panel, and the list is cut into eight equal contiguous parts, one
//     per XCD (the hardware deals workgroup ids round-robin over the XCDs,
//     each with its own L2).  Compact layout: a run is a maximal range of
//     M-tiles whose first rows carry one id (BM divides the 128-row alignment,
//     so a tile never straddles experts); masked layout: group g has
//     ceil(masked_m[g] / BM) tiles.  Every workgroup first writes into LDS a
//     table of the runs covering its XCD's share (compact) or the prefix sums
//     of the group tile counts (masked), so finding a tile's expert and
//     offsets costs a few LDS reads, never a global load inside the loop.
//   - Batch invariance: the instruction shape and the k order are the same for
//     every tile size and layout; a row's result depends only on its own A row
//     and its expert's weights.
#include <climits>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "gemm_wreg.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

struct GemmArgs {
  const uint8_t* A;
  const uint8_t* A_scale;
  const uint8_t* B;
  const uint8_t* B_scale;
  void* C;                 // bf16 [rows][N]; fused SiLU-and-mul: the activation [rows][N/2]
  uint8_t* C_scale;        // fused SiLU-and-mul with FP8 output: its UE8M0 scales
  const int32_t* rowinfo;  // m_indices (contiguous) or masked_m (masked)
  int64_t M;               // contiguous: rows of A/C; masked: max_m
  int N, K, G;
  int m_tiles;             // contiguous: M tiles of A; masked: M tiles per group
  int n_tiles;
};

// Epilogues: the bf16 product, or SiLU-and-mul of its two halves (gate =
// columns [0, N/2), up = [N/2, N)) written as bf16 or as e4m3 + UE8M0.
constexpr int kEpiPlain = 0, kEpiSiluBf16 = 1, kEpiSiluFp8 = 2;

constexpr int kWaves = 8;             // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kStages = 3;
constexpr int kScaleSlot = 256;      // FP8: 64 dwords, one 1-byte load per lane
constexpr int kRunMax = 1024;         // run-table entries: M-tiles of one XCD's share
constexpr int kMaxMaskedGroups = 1024;
// masked layout: prefix sums of the group tile counts, padded so that the
// two-level search below reads in bounds
constexpr int kPrefixLen = kMaxMaskedGroups + 17;
static_assert(kPrefixLen * 4 <= kRunMax * 8, "the prefix array lives in the run-table space");

// Weight formats (template argument WF): 0 bf16; 1 e4m3 with one UE8M0
// exponent per 128x128 block; 2 e4m3 MX (one exponent per 32 k of a weight
// row, scales in the tiled layout of the MX quantiser); 3 e2m1 MX (two codes
// per byte, even k in the low nibble, same scales).
constexpr int kWfBf16 = 0, kWfFp8Block = 1, kWfMxFp8 = 2, kWfMxFp4 = 3;
// bytes of one weight row in one 128-byte activation k-step
constexpr int weight_row_bytes(int wf) { return wf == kWfMxFp4 ? 64 : 128; }
// Stage: the data rows, then for FP8 the scale slots of the BM/64 wavefronts
// fetching activation scales and the weight scales: one slot shared by the
// rest (128x128 blocks), or for MX one 256-byte slot per 64 tile columns.
template <int BM, int BN, int WF>
constexpr int gemm_stage_bytes() {
  return BM * 128 + BN * weight_row_bytes(WF) +
         (WF == kWfBf16 ? 0 : ((BM + 63) / 64 + (WF >= kWfMxFp8 ? BN / 64 : 1)) * kScaleSlot);
}
// LDS: stages, the run table and, for the FP8 SiLU epilogue, the per-row
// maxima of the column wavefronts.  Four stages (three in flight) where they
// fit in the 160 KB, else three.
template <int BM, int BN, int WF, int EPI>
constexpr int gemm_lds_fixed() {
  return kRunMax * 8 + (EPI == kEpiSiluFp8 ? BM * (kWaves / (BM >= 128 ? 2 : 1)) * 4 : 0);
}
template <int BM, int BN, int WF, int EPI>
constexpr int gemm_stages() {
  return 4 * gemm_stage_bytes<BM, BN, WF>() + gemm_lds_fixed<BM, BN, WF, EPI>() <= 160 * 1024
             ? 4 : kStages;
}
template <int BM, int BN, int WF, int EPI>
constexpr int gemm_lds_bytes() {
  return gemm_stages<BM, BN, WF, EPI>() * gemm_stage_bytes<BM, BN, WF>() +
         gemm_lds_fixed<BM, BN, WF, EPI>();
}

// chunk permutation of LDS stage row r (see the kernel's staging comment)
__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// vmcnt <= N and lgkmcnt == 0 (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 left at its maximum, lgkmcnt 11:8 = 0)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Expert id of the first row of M-tile j (every negative id reads as -1), or
// INT_MIN outside [0, used), which therefore never equals an id.
template <int BM>
__device__ __forceinline__ int tile_expert(const int32_t* m_indices, int j, int used) {
  if (j < 0 || j >= used) return INT_MIN;
  const int v = m_indices[static_cast<int64_t>(j) * BM];
  return v < 0 ? -1 : v;
}

// Position pos of the tile order -> expert g, M-tile mt (global index in the
// order's M-tile space), N-tile nt and the first M-tile of the run.  Table
// entry j describes M-tile i_lo + j: x = (first - i_lo) | (end - i_lo) << 16
// as two int16 fields, y = the run's expert id (bits 0-23; negative for
// padding) and, in bits 24-30, the token rows of the run's last tile minus 1
// (every other tile of a run is full).
struct TilePos {
  int g, mt, nt, first;
  int rows;  // compact: rows of the tile holding tokens (the rest is padding)
};
// The table is read with a hand-written ds_read: the compiler orders every LDS
// read it can see after all outstanding direct-to-LDS loads (a full vmcnt
// drain), but the table never overlaps the stages those loads fill.
__device__ __forceinline__ int2 read_table(const int2* table, int j) {
  int2 v;
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const int2*)(table + j)));
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}
__device__ __forceinline__ void lds_write_b64(const void* p, u32x2_t v) {
  asm volatile("ds_write_b64 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_write_b32(const void* p, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ u32x4_t lds_read_b128(const void* p) {
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
__device__ __forceinline__ int lds_read_b32(const void* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
// Masked layout: pre[g] = M-tiles of the groups before g (pre[G] = used, then
// INT_MAX up to kPrefixLen).  The group of M-tile i is the last g with
// pre[g] <= i (empty groups repeat a value and are passed over): lane j first
// tests pre[16 j], then pre[16 c + j] inside the 16-group window c found.
template <bool MASKED>
__device__ __forceinline__ TilePos map_pos(const int2* table, int i_lo, int n_tiles, int used,
                                           int pos) {
  TilePos t;
  const int i0 = pos / n_tiles;
  int run;
  if constexpr (MASKED) {
    const int* const pre = reinterpret_cast<const int*>(table);
    const int lane = __lane_id();
    const int c = __builtin_popcountll(ballot(lds_read_b32(pre + 16 * lane) <= i0)) - 1;
    const int v = lds_read_b32(pre + 16 * c + (lane <= 16 ? lane : 16));
    const int c2 = __builtin_popcountll(ballot(lane <= 16 && v <= i0)) - 1;
    if (c < 0 || c2 < 0 || c2 > 15) {
      t.g = -1;  // cannot happen: pre[0] = 0 <= i0 < pre[16 c + 16]
      t.nt = 0;
      t.mt = 0;
      t.first = 0;
      t.rows = 0;
      return t;
    }
    t.g = 16 * c + c2;
    t.first = __builtin_amdgcn_readlane(v, c2);
    run = __builtin_amdgcn_readlane(v, c2 + 1) - t.first;
  } else {
    const int2 e = read_table(table, i0 - i_lo);
    const int x = __builtin_amdgcn_readfirstlane(e.x);
    const int y = __builtin_amdgcn_readfirstlane(e.y);
    t.g = y < 0 ? y : (y & 0xffffff);
    t.rows = y < 0 ? 0 : ((y >> 24) & 0x7f) + 1;  // of the run's last tile
    t.first = i_lo + static_cast<int>(static_cast<int16_t>(x & 0xffff));
    run = i_lo + (x >> 16) - t.first;
  }
  const int local = pos - t.first * n_tiles;
  if (run <= 0 || t.first < 0 || t.first + run > used || local < 0 || local >= run * n_tiles) {
    t.g = -1;  // an inconsistent entry is never used (cannot happen for a well-built table)
    t.nt = 0;
    t.mt = 0;
    t.rows = 0;
    return t;
  }
  t.nt = local / run;
  t.mt = t.first + (local - t.nt * run);
  if (MASKED || t.mt != t.first + run - 1) t.rows = 1 << 30;  // full (masked: by group size)
  return t;
}

// First position at or after pos (stepping by `stride`) whose run is a valid
// expert, or a position >= end.
template <bool MASKED>
__device__ __forceinline__ int next_tile(const int2* table, int i_lo, int n_tiles, int used, int G,
                                         int pos, int end, int stride) {
  for (; pos < end; pos += stride) {
    const TilePos t = map_pos<MASKED>(table, i_lo, n_tiles, used, pos);
    if (t.g >= 0 && t.g < G) break;
  }
  return pos;
}

// Rows of the tile at t: first row in A / C, rows that exist (rows past the
// end of A or of the group are neither loaded nor stored), and the A-scale
// index of (k block 0, tile row 0); A-scale rows are p.M apart per k block.
template <int BM, bool MASKED>
__device__ __forceinline__ void tile_rows(const GemmArgs& p, const TilePos& t, int64_t& row0,
                                          int& rows, int64_t& as0) {
  if (!MASKED) {
    row0 = static_cast<int64_t>(t.mt) * BM;
    const int64_t left = p.M - row0;
    rows = left < BM ? static_cast<int>(left) : BM;
    rows = t.rows < rows ? t.rows : rows;  // padding rows are neither loaded nor stored
    as0 = row0;
  } else {
    const int r_in0 = (t.mt - t.first) * BM;
    row0 = static_cast<int64_t>(t.g) * p.M + r_in0;
    const int64_t left = p.M - r_in0;
    rows = left < BM ? static_cast<int>(left) : BM;
    as0 = static_cast<int64_t>(t.g) * (p.K / 128) * p.M + r_in0;
  }
}

template <int BM, int BN, int WF, bool MASKED, int EPI>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(const GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr bool FP8 = WF != kWfBf16;
  constexpr bool MX = WF >= kWfMxFp8;
  constexpr bool W4 = WF == kWfMxFp4;
  constexpr int BROW = weight_row_bytes(WF);             // stage bytes of a weight row
  constexpr int WAVES_M = BM >= 128 ? 2 : 1;
  constexpr int WAVES_N = kWaves / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int SDATA = BM * 128 + BN * BROW;            // stage data bytes
  constexpr int STAGE = gemm_stage_bytes<BM, BN, WF>();
  constexpr int NST = gemm_stages<BM, BN, WF, EPI>();     // LDS stages
  constexpr int NLDT = SDATA / 1024;        // 16-byte direct loads per stage
  constexpr int NLD = NLDT / kWaves;        // per wavefront; the first NLDX wavefronts one more
  constexpr int NLDX = NLDT % kWaves;
  constexpr int NLDM = NLD + (NLDX ? 1 : 0);
  constexpr int NVM = NLDM + (FP8 ? 1 : 0);  // vector memory instructions per wavefront per step (at most)
  constexpr int NB = BN / 128;              // weight-scale blocks per tile
  constexpr int ASW = (BM + 63) / 64;       // wavefronts fetching activation scales
  static_assert((BM % 64 == 0 || ((BM == 16 || BM == 32) && MASKED)) && BN % 128 == 0 && WN <= 128 &&
                WM % 16 == 0 && WN % 16 == 0, "tile shape");
  static_assert(SDATA % 1024 == 0, "stage bytes in whole direct loads");
  static_assert(ASW < kWaves, "a wavefront is left for the weight scales");
  // The SiLU epilogue takes gate block nt and up block nt into one tile, laid
  // out in the stage as chunks of CH = WN/2 rows gate, up, gate, up, ... so
  // that every wavefront holds CH gate columns and the matching CH up columns
  // (sub-tiles jn < TN/2: gate, jn + TN/2: the same channels of up).
  constexpr int CH = WN / 2;
  static_assert(EPI == kEpiPlain || (BN == 256 && (WN == 64 || WN == 32)), "SiLU tile shape");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int2* const table = reinterpret_cast<int2*>(smem + NST * STAGE);
  int* const scratch = reinterpret_cast<int*>(smem);  // set-up only (stage memory)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  // this wavefront's direct loads per stage and the first of them
  const int nldw = NLD + (wave < NLDX ? 1 : 0);
  const int qbase = wave * NLD + (wave < NLDX ? wave : NLDX);
  const int n_tiles = p.n_tiles;

  // ======== set-up: this workgroup's share of the tile order ========
  int used;  // M-tiles of the order (compact: up to the last valid first row)
  if (!MASKED) {
    int last = -1;
    for (int j = tid; j < p.m_tiles; j += kThreads)
      if (p.rowinfo[static_cast<int64_t>(j) * BM] >= 0) last = j;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) last = max(last, __shfl_xor(last, off, 64));
    if (lane == 0) scratch[wave] = last;
    __syncthreads();
    last = scratch[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) last = max(last, scratch[w]);
    used = __builtin_amdgcn_readfirstlane(last + 1);
    __syncthreads();  // scratch is rewritten below
  } else {
    // pre[g] = M-tiles of the groups before g, pre[G] = total, then INT_MAX
    int* const pre = reinterpret_cast<int*>(table);
    constexpr int PER = (kMaxMaskedGroups + kThreads - 1) / kThreads;
    int* const wsum = scratch + kMaxMaskedGroups + 8;
    int cnt[PER];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = tid * PER + i;
      int c = 0;
      if (g < p.G) {
        int mm = p.rowinfo[g];
        mm = mm < 0 ? 0 : (mm > p.M ? static_cast<int>(p.M) : mm);
        c = (mm + BM - 1) / BM;
      }
      cnt[i] = c;
      sum += c;
    }
    int incl = sum;  // inclusive scan over the wavefront
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = incl - sum;
    for (int w = 0; w < wave; ++w) base += wsum[w];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = tid * PER + i;
      if (g < p.G) pre[g] = base;
      base += cnt[i];
    }
    if (tid == kThreads - 1) pre[p.G] = base;  // groups >= G count 0
    for (int g = p.G + 1 + tid; g < kPrefixLen; g += kThreads) pre[g] = INT_MAX;
    __syncthreads();
    used = __builtin_amdgcn_readfirstlane(pre[p.G]);
  }
  // XCD x (= blockIdx % 8) takes the x-th eighth [lo_x, hi_x) of the order;
  // its workgroups step through it side by side.
  const int U = used * n_tiles;
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7;
  const int lo_x = static_cast<int>((static_cast<int64_t>(U) * xcd) >> 3);
  const int hi_x = static_cast<int>((static_cast<int64_t>(U) * (xcd + 1)) >> 3);
  if (lo_x + static_cast<int>(blockIdx.x >> 3) >= hi_x) return;
  const int i_lo = lo_x / n_tiles;
  const int R = (hi_x - 1) / n_tiles - i_lo + 1;  // compact: <= kRunMax (host bound)

  // ---- compact: run table for M-tiles [i_lo, i_lo + R) ----
  if (!MASKED) {
    int* const ids = scratch + 8;                  // [R]
    int* const wred = scratch + 8 + kRunMax;       // [2 * kWaves]
    for (int j = tid; j < R; j += kThreads) ids[j] = tile_expert<BM>(p.rowinfo, i_lo + j, used);
    if (wave == 0) {
      // start of the run holding i_lo: windows of 64 tiles below it
      const int e = tile_expert<BM>(p.rowinfo, i_lo, used);
      int lo = i_lo - 64;
      uint64_t d = ballot(tile_expert<BM>(p.rowinfo, lo + lane, used) != e);
      while (d == 0) {
        lo -= 64;
        d = ballot(tile_expert<BM>(p.rowinfo, lo + lane, used) != e);
      }
      if (lane == 0) scratch[0] = lo + (63 - __builtin_clzll(d)) + 1;
    } else if (wave == 1) {
      // end of the run holding the share's last M-tile
      const int ih = i_lo + R - 1;
      const int e = tile_expert<BM>(p.rowinfo, ih, used);
      int hi = ih + 1;
      uint64_t d = ballot(tile_expert<BM>(p.rowinfo, hi + lane, used) != e);
      while (d == 0) {
        hi += 64;
        d = ballot(tile_expert<BM>(p.rowinfo, hi + lane, used) != e);
      }
      if (lane == 0) scratch[1] = hi + __builtin_ctzll(d);
    }
    __syncthreads();
    const int first_lo = scratch[0], end_hi = scratch[1];
    // entries 2*tid, 2*tid+1: run starts are a prefix maximum of the start
    // marks, run ends a suffix minimum of the end marks
    int id[2], v[2], w[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = 2 * tid + q;
      if (j < R) {
        id[q] = ids[j];
        v[q] = j == 0 ? first_lo : (ids[j - 1] != id[q] ? i_lo + j : INT_MIN);
        w[q] = j == R - 1 ? end_hi : (ids[j + 1] != id[q] ? i_lo + j + 1 : INT_MAX);
      } else {
        id[q] = -1;
        v[q] = INT_MIN;
        w[q] = INT_MAX;
      }
    }
    int pre = max(v[0], v[1]);
    int suf = min(w[0], w[1]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int a = __shfl_up(pre, off, 64);
      const int b = __shfl_down(suf, off, 64);
      if (lane >= off) pre = max(pre, a);
      if (lane + off < 64) suf = min(suf, b);
    }
    if (lane == 63) wred[wave] = pre;
    if (lane == 0) wred[kWaves + wave] = suf;
    __syncthreads();
    int before = INT_MIN, after = INT_MAX;
    for (int q = 0; q < wave; ++q) before = max(before, wred[q]);
    for (int q = wave + 1; q < kWaves; ++q) after = min(after, wred[kWaves + q]);
    const int pre_x = __shfl_up(pre, 1, 64);
    const int suf_x = __shfl_down(suf, 1, 64);
    if (lane > 0) before = max(before, pre_x);
    if (lane < 63) after = min(after, suf_x);
    const int f0 = max(before, v[0]), f1 = max(f0, v[1]);
    const int e1 = min(after, w[1]), e0 = min(e1, w[0]);
    // token rows of a run's last tile: its valid rows come first, so a binary
    // search for the first padding row (-1)
    auto last_rows = [&](int end_tile) -> int {
      const int64_t r0 = static_cast<int64_t>(end_tile - 1) * BM;
      int lo = 1, hi = p.M - r0 < BM ? static_cast<int>(p.M - r0) : BM;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (p.rowinfo[r0 + mid] >= 0) lo = mid + 1;
        else hi = mid;
      }
      return lo;
    };
    if (2 * tid < R)
      table[2 * tid] = make_int2(((f0 - i_lo) & 0xffff) | ((e0 - i_lo) << 16),
                                 id[0] < 0 ? id[0] : id[0] | ((last_rows(e0) - 1) << 24));
    if (2 * tid + 1 < R)
      table[2 * tid + 1] = make_int2(((f1 - i_lo) & 0xffff) | ((e1 - i_lo) << 16),
                                     id[1] < 0 ? id[1] : id[1] | ((last_rows(e1) - 1) << 24));
  }
  __syncthreads();  // table complete; stage memory is free

  // ======== the flat k-step stream ========
  constexpr int ES = FP8 ? 1 : 2;
  const int64_t rowbytes = static_cast<int64_t>(p.K) * ES;  // activation row
  const int64_t browbytes = rowbytes / 128 * BROW;          // weight row
  const int nk = static_cast<int>(rowbytes / 128);
  const int KB = p.K / 128;
  const int G = p.G;

  // -- load side: the tile and k-step whose stage is filled next --
  int d_pos = next_tile<MASKED>(table, i_lo, n_tiles, used, G, lo_x + static_cast<int>(blockIdx.x >> 3),
                                hi_x, per_xcd);
  if (d_pos >= hi_x) return;
  int d_k = 0;
  int64_t d_aoff, d_boff, d_as0, d_bs0;  // byte offsets of the tile in A and B; scale indices
  // B columns (weight rows) a tile advances by per N-tile, and the distance in
  // the weight-scale array between the tile's two 128-column blocks
  constexpr int NBW = EPI == kEpiPlain ? BN : 128;
  const int64_t bs_stride = EPI == kEpiPlain ? KB : static_cast<int64_t>(p.N / 256) * KB;
  // MX weight scales: wavefront w >= ASW fetches the 256-byte slot of tile
  // column block c_w (64 columns; SiLU tiles: gate blocks 0-1, up blocks 2-3)
  constexpr int NMX = BN / 64;
  const int c_w = wave >= ASW ? (wave - ASW) % NMX : 0;
  int d_rows;
  uint32_t soff[NLDM];  // per-lane source offsets from the tile's A / B rows
  // A direct load moves 1 KB (64 lanes x 16 bytes) into LDS: 8 activation rows,
  // or 1024 / BROW weight rows; lane i carries the 16-byte chunk that belongs
  // at LDS position i, i.e. source chunk (i & 7) ^ swz(row) of a 128-byte row,
  // or (i & 3) ^ ((row >> 2) & 3) of a 64-byte e2m1 row.  The stage holds the
  // BM activation rows, then the BN weight rows.
#define MOE_DSET(pos_)                                                                        \
  do {                                                                                        \
    const TilePos t_ = map_pos<MASKED>(table, i_lo, n_tiles, used, (pos_));                         \
    int64_t r0_;                                                                              \
    tile_rows<BM, MASKED>(p, t_, r0_, d_rows, d_as0);                                         \
    d_pos = (pos_);                                                                           \
    d_aoff = r0_ * rowbytes;                                                                  \
    d_boff = (static_cast<int64_t>(t_.g) * p.N + static_cast<int64_t>(t_.nt) * NBW) * browbytes; \
    if constexpr (MX) {                                                                       \
      const int blk_ = EPI == kEpiPlain ? t_.nt * NMX + c_w                                   \
                                        : (c_w >= 2 ? p.N / 128 : 0) + t_.nt * 2 + (c_w & 1); \
      d_bs0 = (static_cast<int64_t>(t_.g) * (p.N / 64) + blk_) * KB * 256;                   \
    } else {                                                                                  \
      d_bs0 = (static_cast<int64_t>(t_.g) * (p.N / 128) + t_.nt * (NBW / 128)) * KB;          \
    }                                                                                         \
    _Pragma("unroll") for (int j = 0; j < NLDM; ++j) {                                        \
      const int q_ = qbase + j;                                                               \
      if (q_ * 1024 < BM * 128) {                                                             \
        const int R_ = q_ * 8 + (lane >> 3);                                                  \
        const int c_ = (lane & 7) ^ lds_swz(R_);                                              \
        const int r_ = R_ < d_rows ? R_ : d_rows - 1;                                         \
        soff[j] = static_cast<uint32_t>(r_ * rowbytes + c_ * 16);                             \
      } else {                                                                                \
        const int b_ = (q_ * 1024 - BM * 128) / BROW + lane / (BROW / 16);                    \
        const int c_ = W4 ? (lane & 3) ^ ((b_ >> 2) & 3) : (lane & 7) ^ lds_swz(b_);          \
        int r_ = b_;                                                                          \
        if (EPI != kEpiPlain)                                                                 \
          r_ = ((r_ / CH) & 1) * (p.N / 2) + (r_ / (2 * CH)) * CH + (r_ % CH);                \
        soff[j] = static_cast<uint32_t>(r_ * browbytes + c_ * 16);                            \
      }                                                                                       \
    }                                                                                         \
  } while (0)
  MOE_DSET(d_pos);

  // One k-step of loads into stage st_: for FP8 first the scale bytes (wave w
  // < ASW: activation scales of tile rows 64w..64w+63; wave ASW: the NB
  // weight-block scales; the rest repeat those into the same slot), then the
  // data rows.
#define MOE_ISSUE(st_)                                                                          \
  do {                                                                                          \
    uint8_t* const stg_ = smem + (st_) * STAGE;                                                 \
    if constexpr (FP8) {                                                                        \
      /* both candidates computed, one selected: no branch in the step */                      \
      int r_ = wave * 64 + lane;                                                                \
      r_ = r_ < d_rows ? r_ : d_rows - 1;                                                       \
      const int nb_ = lane < NB ? lane : NB - 1;                                                \
      const uint8_t* const sa_ = p.A_scale + d_as0 + static_cast<int64_t>(d_k) * p.M + r_;     \
      const uint8_t* const sb_ = p.B_scale + d_bs0 + nb_ * bs_stride + d_k;                     \
      const uint8_t* const src_ = wave < ASW ? sa_ : sb_;                                       \
      if (!MX || wave < ASW) {                                                                  \
        /* wavefronts past ASW all write the same bytes into one slot */                        \
        __builtin_amdgcn_global_load_lds(src_,                                                  \
            (__attribute__((address_space(3))) void*)(stg_ + SDATA + (wave < ASW ? wave : ASW) * kScaleSlot), \
            1, 0, 0);                                                                           \
      } else {                                                                                  \
        /* MX: the slot of block c_w for this k-step, 4 bytes per lane; waves */                \
        /* past ASW + NMX repeat a slot with the same bytes */                                  \
        __builtin_amdgcn_global_load_lds(p.B_scale + d_bs0 + static_cast<int64_t>(d_k) * 256 + lane * 4, \
            (__attribute__((address_space(3))) void*)(stg_ + SDATA + (ASW + c_w) * kScaleSlot), \
            4, 0, 0);                                                                           \
      }                                                                                         \
    }                                                                                           \
    const uint8_t* ab_ = p.A + d_aoff + static_cast<int64_t>(d_k) * 128;                        \
    const uint8_t* bb_ = p.B + d_boff + static_cast<int64_t>(d_k) * BROW;                       \
    uint8_t* const dst_ = stg_ + qbase * 1024;                                                  \
    _Pragma("unroll") for (int j = 0; j < NLDM; ++j) {                                          \
      if (j < NLD || j < nldw) {                                                                \
        const bool is_a_ = (qbase + j) * 1024 < BM * 128;                                       \
        __builtin_amdgcn_global_load_lds((is_a_ ? ab_ : bb_) + soff[j],                         \
            (__attribute__((address_space(3))) void*)(dst_ + j * 1024), 16, 0, 0);              \
      }                                                                                         \
    }                                                                                           \
  } while (0)
  // Move the load side to the next k-step; past the last tile keep re-reading
  // its last k-step (never used).
#define MOE_ADVANCE()                                                                           \
  do {                                                                                          \
    if (++d_k == nk) {                                                                          \
      d_k = 0;                                                                                  \
      const int np_ = next_tile<MASKED>(table, i_lo, n_tiles, used, G, d_pos + per_xcd, hi_x, per_xcd); \
      if (np_ < hi_x) MOE_DSET(np_);                                                            \
      else d_k = nk - 1;                                                                        \
    }                                                                                           \
  } while (0)

  // -- compute side: the tile being accumulated --
  int c_k = 0;
  int c_pos = d_pos;
  int c_next = next_tile<MASKED>(table, i_lo, n_tiles, used, G, c_pos + per_xcd, hi_x, per_xcd);
  int64_t c_row0;
  int c_rows, c_nt, c_g;
#define MOE_CSET(pos_)                                                                        \
  do {                                                                                        \
    const TilePos t_ = map_pos<MASKED>(table, i_lo, n_tiles, used, (pos_));                         \
    int64_t as0_;                                                                             \
    tile_rows<BM, MASKED>(p, t_, c_row0, c_rows, as0_);                                       \
    c_nt = t_.nt;                                                                             \
    c_g = t_.g;                                                                               \
    c_pos = (pos_);                                                                           \
  } while (0)
  MOE_CSET(c_pos);

  f32x4_t acc[TN][TM];
#pragma unroll
  for (int jn = 0; jn < TN; ++jn)
#pragma unroll
    for (int im = 0; im < TM; ++im) acc[jn][im] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int frag_row = lane & 15;
  const int frag_k = lane >> 4;
  const int wblk = (wn * WN) / 128;
  // MX: the wavefront's first weight-scale slot and byte: its columns start at
  // tile column wn*WN (SiLU tiles: gate column wn*CH, up slot two further on);
  // scale byte j16 of a slot dword serves the 16 columns 16*j16 .. of that block
  const int mx_c0 = (EPI == kEpiPlain ? wn * WN : wn * CH) / 64;
  const int mx_j0 = ((EPI == kEpiPlain ? wn * WN : wn * CH) % 64) / 16;
  // Fragment rows are (multiple of 16) + frag_row, so the chunk permutation
  // depends on the lane only: the byte offset of logical chunk c of the lane's
  // row in the sub-tile starting at stage row rb is rb*128 + frag_row*128 +
  // ((c ^ swz_l) << 4).
  const int swz_l = lds_swz(frag_row);
  const int swz4_l = (frag_row >> 2) & 3;  // e2m1 weight rows: 64 bytes, 4 chunks
  const int CK_LO = MX ? frag_k : 2 * frag_k, CK_HI = MX ? frag_k + 4 : 2 * frag_k + 1;
#define MOE_ROWOFF(rb_, c_) ((rb_) * 128 + frag_row * 128 + (((c_) ^ swz_l) << 4))

  // FP8 operands of the 16x16x128 MFMA: the hardware reads bytes 0-15 of lane
  // group g's 32 as k = 16g .. 16g+15 and bytes 16-31 as k = 64+16g .. (its
  // 32-wide scale blocks are k = 32b .. 32b+31, scale of row i, block b from
  // lane 16b + i).  With MX weights each lane takes 16-byte chunks g and g + 4
  // of the 128-byte k-step, so the instruction's k order is the memory order
  // and an MX scale byte per lane covers one contiguous 32-block.  With one
  // scale per 128-wide k-step the order is free, and chunks 2g, 2g + 1 read
  // about 3% faster (measured), so those kernels keep them.  BF16: the two
  // 16x16x32 MFMAs of a k-step take chunks 2g and 2g + 1 (even, then odd), the
  // order of the register-streamed kernel too, so a row's sums come out
  // bit-identical whichever kernel or layout computes them.
  using frag_t = typename std::conditional<FP8, i32x8_t, bf16x8_t>::type;
  constexpr int KS = FP8 ? 1 : 2;  // MFMA k-substeps per 128-byte stage
  struct Frags {
    frag_t a[KS][TM];
    frag_t b[KS][TN];
    int sa[TM];
    int sw, sw2;  // weight scales of the wavefront's columns (SiLU: gate, up)
  };
#define MOE_LOAD(F_, st_)                                                                        \
  do {                                                                                           \
    const uint8_t* S_ = smem + (st_) * STAGE;                                                    \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                          \
      _Pragma("unroll") for (int im = 0; im < TM; ++im) {                                        \
        const int rb_ = wm * WM + im * 16;                                                       \
        if constexpr (FP8) {                                                                     \
          const u32x4_t lo_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, CK_LO));          \
          const u32x4_t hi_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, CK_HI));          \
          F_.a[ks][im] = i32x8_t{(int)lo_[0], (int)lo_[1], (int)lo_[2], (int)lo_[3],             \
                                 (int)hi_[0], (int)hi_[1], (int)hi_[2], (int)hi_[3]};            \
        } else {                                                                                 \
          F_.a[ks][im] = *reinterpret_cast<const frag_t*>(S_ + MOE_ROWOFF(rb_, 2 * frag_k + ks)); \
        }                                                                                        \
      }                                                                                          \
      _Pragma("unroll") for (int jn = 0; jn < TN; ++jn) {                                        \
        const int rb_ = BM + wn * WN + jn * 16;                                                  \
        if constexpr (W4) {                                                                      \
          /* e2m1: lane group g holds k 32g .. 32g+31, 16 bytes of the 64-byte row */           \
          const u32x4_t v_ = *reinterpret_cast<const u32x4_t*>(                                  \
              S_ + BM * 128 + (wn * WN + jn * 16 + frag_row) * 64 + ((frag_k ^ swz4_l) << 4));   \
          F_.b[ks][jn] = i32x8_t{(int)v_[0], (int)v_[1], (int)v_[2], (int)v_[3], 0, 0, 0, 0};    \
        } else if constexpr (FP8) {                                                              \
          const u32x4_t lo_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, CK_LO));          \
          const u32x4_t hi_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, CK_HI));          \
          F_.b[ks][jn] = i32x8_t{(int)lo_[0], (int)lo_[1], (int)lo_[2], (int)lo_[3],             \
                                 (int)hi_[0], (int)hi_[1], (int)hi_[2], (int)hi_[3]};            \
        } else {                                                                                 \
          F_.b[ks][jn] = *reinterpret_cast<const frag_t*>(S_ + MOE_ROWOFF(rb_, 2 * frag_k + ks)); \
        }                                                                                        \
      }                                                                                          \
    }                                                                                            \
    if constexpr (FP8) {                                                                         \
      const uint8_t* X_ = S_ + SDATA;                                                            \
      _Pragma("unroll") for (int im = 0; im < TM; ++im)                                          \
        F_.sa[im] = X_[(wm * WM + im * 16 + frag_row) * 4];                                      \
      if constexpr (MX) {                                                                        \
        const uint8_t* M_ = X_ + ASW * kScaleSlot + frag_k * 64 + frag_row * 4;                 \
        F_.sw = *reinterpret_cast<const int*>(M_ + mx_c0 * kScaleSlot);                          \
        if (EPI != kEpiPlain) F_.sw2 = *reinterpret_cast<const int*>(M_ + (mx_c0 + 2) * kScaleSlot); \
      } else {                                                                                   \
        F_.sw = X_[ASW * kScaleSlot + (EPI == kEpiPlain ? wblk : 0) * 4];                        \
        F_.sw2 = X_[ASW * kScaleSlot + 4];                                                       \
      }                                                                                          \
    }                                                                                            \
  } while (0)
// One activation fragment (k-substep ks, row block im) of stage st_.
#define MOE_LOAD_A1(F_, st_, ks, im)                                                             \
  do {                                                                                           \
    const uint8_t* S_ = smem + (st_) * STAGE;                                                    \
    const int rb_ = wm * WM + (im) * 16;                                                         \
    if constexpr (FP8) {                                                                         \
      const u32x4_t lo_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, CK_LO));        \
      const u32x4_t hi_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, CK_HI));        \
      F_.a[ks][im] = i32x8_t{(int)lo_[0], (int)lo_[1], (int)lo_[2], (int)lo_[3],                 \
                             (int)hi_[0], (int)hi_[1], (int)hi_[2], (int)hi_[3]};                \
    } else {                                                                                     \
      F_.a[ks][im] = *reinterpret_cast<const frag_t*>(S_ + MOE_ROWOFF(rb_, 2 * frag_k + (ks)));  \
    }                                                                                            \
  } while (0)
// The weight fragments and the scales of stage st_.
#define MOE_LOAD_B(F_, st_)                                                                      \
  do {                                                                                           \
    const uint8_t* S_ = smem + (st_) * STAGE;                                                    \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                          \
      _Pragma("unroll") for (int jn = 0; jn < TN; ++jn) {                                        \
        const int rb_ = BM + wn * WN + jn * 16;                                                  \
        if constexpr (W4) {                                                                      \
          const u32x4_t v_ = *reinterpret_cast<const u32x4_t*>(                                  \
              S_ + BM * 128 + (wn * WN + jn * 16 + frag_row) * 64 + ((frag_k ^ swz4_l) << 4));   \
          F_.b[ks][jn] = i32x8_t{(int)v_[0], (int)v_[1], (int)v_[2], (int)v_[3], 0, 0, 0, 0};    \
        } else if constexpr (FP8) {                                                              \
          const u32x4_t lo_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, CK_LO));    \
          const u32x4_t hi_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, CK_HI));    \
          F_.b[ks][jn] = i32x8_t{(int)lo_[0], (int)lo_[1], (int)lo_[2], (int)lo_[3],             \
                                 (int)hi_[0], (int)hi_[1], (int)hi_[2], (int)hi_[3]};            \
        } else {                                                                                 \
          F_.b[ks][jn] = *reinterpret_cast<const frag_t*>(S_ + MOE_ROWOFF(rb_, 2 * frag_k + ks)); \
        }                                                                                        \
      }                                                                                          \
    }                                                                                            \
    if constexpr (FP8) {                                                                         \
      const uint8_t* X_ = S_ + SDATA;                                                            \
      _Pragma("unroll") for (int im = 0; im < TM; ++im)                                          \
        F_.sa[im] = X_[(wm * WM + im * 16 + frag_row) * 4];                                      \
      if constexpr (MX) {                                                                        \
        const uint8_t* M_ = X_ + ASW * kScaleSlot + frag_k * 64 + frag_row * 4;                 \
        F_.sw = *reinterpret_cast<const int*>(M_ + mx_c0 * kScaleSlot);                          \
        if (EPI != kEpiPlain) F_.sw2 = *reinterpret_cast<const int*>(M_ + (mx_c0 + 2) * kScaleSlot); \
      } else {                                                                                   \
        F_.sw = X_[ASW * kScaleSlot + (EPI == kEpiPlain ? wblk : 0) * 4];                        \
        F_.sw2 = X_[ASW * kScaleSlot + 4];                                                       \
      }                                                                                          \
    }                                                                                            \
  } while (0)
// The step's MFMAs row block by row block (FC_); once a block's MFMAs are
// issued, its activation fragment registers take the next step's (FN_, from
// stage st_), so the two steps' activation fragments share registers and only
// the weight fragments are held twice.
#define MOE_MMA_IM(FC_, FN_, st_)                                                                \
  do {                                                                                           \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks)                                            \
      _Pragma("unroll") for (int im = 0; im < TM; ++im) {                                        \
        _Pragma("unroll") for (int jn = 0; jn < TN; ++jn) {                                      \
          if constexpr (FP8)                                                                     \
            acc[jn][im] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                      \
                FC_.b[ks][jn], FC_.a[ks][im], acc[jn][im], W4 ? 4 : 0, 0, 0,                     \
                MX ? (((EPI != kEpiPlain && jn >= TN / 2) ? FC_.sw2 : FC_.sw) >>                 \
                      (8 * (mx_j0 + (EPI != kEpiPlain ? jn % (TN / 2) : jn))))                    \
                   : ((EPI != kEpiPlain && jn >= TN / 2) ? FC_.sw2 : FC_.sw),                    \
                0, FC_.sa[im]);                                                                  \
          else                                                                                   \
            acc[jn][im] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(FC_.b[ks][jn], FC_.a[ks][im],  \
                                                                  acc[jn][im], 0, 0, 0);         \
        }                                                                                        \
        MOE_LOAD_A1(FN_, st_, ks, im);                                                           \
      }                                                                                          \
  } while (0)
  // Stores of the finished compute tile (lane: 4 consecutive columns of a row
  // per 16x16 block), then a fresh accumulator.
  //   Plain: the bf16 product.
  //   SiLU: per row and channel c of the tile's 128-channel block nt, gate and
  //   up (sub-tiles jn and jn + TN/2 of the lane) are rounded to bf16 as the
  //   plain product would be stored, act = bf16(silu(gate) * up) in fp32 (the
  //   same silu_f32 as the stand-alone SiLU-and-mul); FP8 output
  //   then takes the row's maximum over the 128 channels (the four column
  //   wavefronts of the row meet in LDS) and quantises as moe_quant_fp8_ue8m0.
  float* const rowmax = reinterpret_cast<float*>(smem + NST * STAGE + kRunMax * 8);
#define MOE_EPILOGUE()                                                                           \
  do {                                                                                           \
    /* lane indices from an opaque copy: rebuilt here rather than held in */                     \
    /* registers across the main loop                                    */                     \
    int te_ = threadIdx.x;                                                                       \
    asm volatile("" : "+v"(te_));                                                                \
    const int frag_row = te_ & 15;                                                               \
    const int frag_k = (te_ >> 4) & 3;                                                           \
    if constexpr (EPI == kEpiPlain) {                                                            \
      uint16_t* const cg_ = static_cast<uint16_t*>(p.C) + c_row0 * p.N +                         \
                            static_cast<int64_t>(c_nt) * BN + wn * WN + frag_k * 4;              \
      _Pragma("unroll") for (int im = 0; im < TM; ++im) {                                        \
        const int r_ = wm * WM + im * 16 + frag_row;                                             \
        if (r_ < c_rows) {                                                                       \
          uint16_t* const crow_ = cg_ + static_cast<int64_t>(r_) * p.N;                          \
          _Pragma("unroll") for (int jn = 0; jn < TN; ++jn) {                                    \
            const f32x4_t v_ = acc[jn][im];                                                      \
            const uint32_t lo_ = pack_bf16x2(v_[0], v_[1]);                                      \
            const uint32_t hi_ = pack_bf16x2(v_[2], v_[3]);                                      \
            *reinterpret_cast<u32x2_t*>(crow_ + jn * 16) = u32x2_t{lo_, hi_};                    \
          }                                                                                      \
        }                                                                                        \
      }                                                                                          \
    } else {                                                                                     \
      const int I_ = p.N / 2;                                                                    \
      const int64_t ch0_ = static_cast<int64_t>(c_nt) * 128 + wn * CH + frag_k * 4;             \
      constexpr int TH = TN / 2;                                                                 \
      /* act of 4 channels of sub-tile pair (h, h + TH) of row block im, from the */           \
      /* accumulators (read only: the result lives in a few temporaries)         */           \
      auto act4_ = [&](int im, int h) -> f32x4_t {                                               \
        f32x4_t r_;                                                                              \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                          \
          const float gt_ = bf16_to_f32(f32_to_bf16(acc[h][im][e]));                             \
          const float up_ = bf16_to_f32(f32_to_bf16(acc[h + TH][im][e]));                        \
          r_[e] = bf16_to_f32(f32_to_bf16(silu_f32(gt_) * up_));                                 \
        }                                                                                        \
        return r_;                                                                               \
      };                                                                                         \
      if constexpr (EPI == kEpiSiluBf16) {                                                       \
        _Pragma("unroll") for (int im = 0; im < TM; ++im) {                                      \
          const int r_ = wm * WM + im * 16 + frag_row;                                           \
          if (r_ < c_rows) {                                                                     \
            uint16_t* const orow_ = static_cast<uint16_t*>(p.C) + (c_row0 + r_) * I_ + ch0_;     \
            _Pragma("unroll") for (int h = 0; h < TH; ++h) {                                     \
              const f32x4_t v_ = act4_(im, h);                                                   \
              const uint32_t lo_ = pack_bf16x2(v_[0], v_[1]);                                    \
              const uint32_t hi_ = pack_bf16x2(v_[2], v_[3]);                                    \
              *reinterpret_cast<u32x2_t*>(orow_ + h * 16) = u32x2_t{lo_, hi_};                   \
            }                                                                                    \
          }                                                                                      \
        }                                                                                        \
      } else {                                                                                   \
        /* Row maxima: over the lane's channels, the 4 lanes of the row       */                   \
        /* (shuffles), then the column wavefronts (a small LDS array, one     */                   \
        /* barrier); the activation is recomputed for the quantisation.       */                   \
        _Pragma("unroll") for (int im = 0; im < TM; ++im) {                                      \
          const int r_ = wm * WM + im * 16 + frag_row;                                           \
          float m_ = 0.0f;                                                                       \
          if (r_ < c_rows) {                                                                     \
            _Pragma("unroll") for (int h = 0; h < TH; ++h) {                                     \
              const f32x4_t v_ = act4_(im, h);                                                   \
              _Pragma("unroll") for (int e = 0; e < 4; ++e) m_ = fmaxf(m_, fabsf(v_[e]));        \
            }                                                                                    \
          }                                                                                      \
          m_ = fmaxf(m_, __shfl_xor(m_, 16, 64));                                                \
          m_ = fmaxf(m_, __shfl_xor(m_, 32, 64));                                                \
          if (frag_k == 0) lds_write_b32(rowmax + r_ * WAVES_N + wn, __float_as_uint(m_));       \
        }                                                                                        \
        __builtin_amdgcn_s_waitcnt(0xc07f); /* lgkmcnt(0): the maxima are in LDS */             \
        __builtin_amdgcn_s_barrier();                                                            \
        _Pragma("unroll") for (int jn = 0; jn < TN; ++jn)                                        \
          _Pragma("unroll") for (int im = 0; im < TM; ++im) asm volatile("" : "+v"(acc[jn][im])); \
        _Pragma("unroll") for (int im = 0; im < TM; ++im) {                                      \
          const int r_ = wm * WM + im * 16 + frag_row;                                           \
          if (r_ < c_rows) {                                                                     \
            float amax_ = 0.0f;                                                                  \
            _Pragma("unroll") for (int w_ = 0; w_ < WAVES_N; w_ += 4) {                          \
              const u32x4_t q4_ = lds_read_b128(rowmax + r_ * WAVES_N + w_);                     \
              amax_ = fmaxf(amax_, fmaxf(fmaxf(__uint_as_float(q4_[0]), __uint_as_float(q4_[1])), \
                                         fmaxf(__uint_as_float(q4_[2]), __uint_as_float(q4_[3])))); \
            }                                                                                    \
            const int ex_ = ue8m0_exponent(amax_);                                               \
            uint8_t* const orow_ = static_cast<uint8_t*>(p.C) + (c_row0 + r_) * I_ + ch0_;       \
            _Pragma("unroll") for (int h = 0; h < TH; ++h) {                                     \
              const f32x4_t v_ = act4_(im, h);                                                   \
              *reinterpret_cast<uint32_t*>(orow_ + h * 16) =                                     \
                  e4m3x4(v_[0], v_[1], v_[2], v_[3], ex_);                                       \
            }                                                                                    \
            if (wn == 0 && frag_k == 0) {                                                        \
              const int64_t si_ = MASKED                                                         \
                  ? (static_cast<int64_t>(c_g) * (I_ / 128) + c_nt) * p.M + (c_row0 - static_cast<int64_t>(c_g) * p.M) + r_ \
                  : static_cast<int64_t>(c_nt) * p.M + c_row0 + r_;                               \
              p.C_scale[si_] = static_cast<uint8_t>(ex_ + 127);                                  \
            }                                                                                    \
          }                                                                                      \
        }                                                                                        \
        /* the maxima are rewritten only by the next tile's epilogue, after at */                \
        /* least one step barrier                                               */               \
      }                                                                                          \
    }                                                                                            \
    _Pragma("unroll") for (int jn = 0; jn < TN; ++jn)                                            \
      _Pragma("unroll") for (int im = 0; im < TM; ++im) acc[jn][im] = f32x4_t{0.f, 0.f, 0.f, 0.f}; \
  } while (0)
  // One step s (FC_ holds its fragments, read during step s-1):
  //   wait until stage s+1 (and its scales) landed and this wavefront's LDS
  //   reads are done, barrier; if step s-1 finished a tile, store it and move
  //   the compute side on; read step s+1's weight fragments and scales into
  //   FN_; refill the stage step s used (its fragments are in FC_) with step
  //   s+NST; run step s's MFMAs row block by row block, each block followed by
  //   the read of step s+1's activation fragment into the registers it frees,
  //   with the refill's loads spread over the blocks; then move the load side
  //   on.  The reads and the refill touch different stages.
  //   The wait count is the number of vector memory instructions of NST-2
  //   refills: those of steps s+2 .. s+NST-1 may still be in flight, all older
  //   ones (the refill of step s+1, the stores) have completed because vector
  //   memory instructions complete in issue order.
  bool c_epi = false;
  bool done = false;
  // LDS reads per step: weight fragments and scales (NRB), one activation
  // fragment (NRA); refill loads per row-block group (VPG)
  constexpr int NRA = FP8 ? 2 : 1;
  constexpr int NRB = KS * TN * (W4 ? 1 : (FP8 ? 2 : 1)) + (FP8 ? TM + 2 : 0);
  constexpr int VPG = (NVM + KS * TM - 1) / (KS * TM);
#define MOE_STEP(FC_, FN_)                                                                       \
  do {                                                                                           \
    if (NLDX == 0 || wave < NLDX) wait_vm_lgkm0<(NST - 2) * NVM>();                              \
    else wait_vm_lgkm0<(NST - 2) * (NVM - 1)>();                                                 \
    __builtin_amdgcn_s_barrier();                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    if (c_epi) {                                                                                 \
      MOE_EPILOGUE();                                                                            \
      c_epi = false;                                                                             \
      MOE_CSET(c_next);                                                                          \
      c_next = next_tile<MASKED>(table, i_lo, n_tiles, used, G, c_pos + per_xcd, hi_x, per_xcd);       \
    }                                                                                            \
    const int st1_ = st + 1 == NST ? 0 : st + 1;                                                 \
    MOE_LOAD_B(FN_, st1_);                                                                       \
    MOE_ISSUE(st);                                                                               \
    MOE_MMA_IM(FC_, FN_, st1_);                                                                  \
    /* the weight-fragment reads first, then per row block its MFMAs with */                     \
    /* a share of the refill's loads, then the block's next-step reads    */                     \
    __builtin_amdgcn_sched_group_barrier(0x100, NRB, 0);                                         \
    _Pragma("unroll") for (int g_ = 0; g_ < KS * TM; ++g_) {                                     \
      __builtin_amdgcn_sched_group_barrier(0x020, VPG, 0);                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);                                        \
      __builtin_amdgcn_sched_group_barrier(0x100, NRA, 0);                                       \
    }                                                                                            \
    __builtin_amdgcn_sched_group_barrier(0x020, NVM, 0);                                         \
    /* keep the MFMAs in this block: the advance below branches */                               \
    _Pragma("unroll") for (int jn = 0; jn < TN; ++jn)                                            \
      _Pragma("unroll") for (int im = 0; im < TM; ++im) asm volatile("" : "+v"(acc[jn][im]));    \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    MOE_ADVANCE();                                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    st = st1_;                                                                                   \
    if (++c_k == nk) {                                                                           \
      c_k = 0;                                                                                   \
      c_epi = true;                                                                              \
      done = c_next >= hi_x;                                                                     \
    }                                                                                            \
  } while (0)

  // prologue: the first NST k-steps, fully landed
#pragma unroll
  for (int q = 0; q < NST; ++q) {
    MOE_ISSUE(q);
    MOE_ADVANCE();
  }
  wait_vm_lgkm0<0>();
  __syncthreads();
  Frags f0, f1;
  MOE_LOAD(f0, 0);
  int st = 0;  // stage holding the current step (its fragments are in registers)
  for (;;) {
    MOE_STEP(f0, f1);
    if (done) break;
    MOE_STEP(f1, f0);
    if (done) break;
  }
  MOE_EPILOGUE();
  wait_vm_lgkm0<0>();  // the trailing re-reads and the stores
#undef MOE_DSET
#undef MOE_ISSUE
#undef MOE_ADVANCE
#undef MOE_CSET
#undef MOE_ROWOFF
#undef MOE_LOAD
#undef MOE_LOAD_A1
#undef MOE_LOAD_B
#undef MOE_MMA_IM
#undef MOE_EPILOGUE
#undef MOE_STEP
#endif
}

// Persistent grid: one workgroup per CU (the LDS footprint allows no more),
// rounded down to a multiple of the 8 XCDs.
// Workgroups of the persistent grid: the CU count rounded down to a multiple
// of the 8 XCDs, looked up once per device (thread-safe).
static int persistent_grid() {
  static std::once_flag once[64];
  static int grid[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::call_once(once[dev], [dev]() {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      grid[dev] = cus >= 8 ? cus / 8 * 8 : 8;
  });
  return grid[dev];
}

template <int BM, int BN, int WF, bool MASKED, int EPI = kEpiPlain>
int32_t launch_gemm(GemmArgs a, hipStream_t s) {
  // The compact run table holds one XCD's share of the M-tiles (about a
  // million rows in all) and tile positions are 32-bit.
  const int64_t m_tiles = (a.M + BM - 1) / BM;
  const int64_t order_m = (MASKED ? a.G : 1) * m_tiles;
  if (!MASKED && order_m > 8 * (kRunMax - 2)) return MOE_EUNSUPPORTED;
  if (!MASKED && a.G >= (1 << 24)) return MOE_EUNSUPPORTED;  // expert ids share a table word
  if (MASKED && a.G > kMaxMaskedGroups) return MOE_EUNSUPPORTED;
  a.n_tiles = EPI == kEpiPlain ? a.N / BN : a.N / 256;
  a.m_tiles = static_cast<int>(m_tiles);
  const int64_t tiles = order_m * a.n_tiles;
  if (tiles == 0) return MOE_OK;
  if (tiles >= (1ll << 31)) return MOE_EUNSUPPORTED;
  constexpr int lds = gemm_lds_bytes<BM, BN, WF, EPI>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = grouped_gemm_kernel<BM, BN, WF, MASKED, EPI>;
  // the dynamic-LDS limit is raised once per device the kernel runs on (thread-safe)
  static std::once_flag once[64];
  static bool attr_ok[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_EDEVICE;
  std::call_once(once[dev], [dev, kern]() {
    attr_ok[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess;
  });
  if (!attr_ok[dev]) return MOE_EDEVICE;
  const int grid = persistent_grid();
  if (grid == 0) return MOE_EDEVICE;
  kern<<<grid, kThreads, lds, s>>>(a);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

// Weight format of a GEMM dtype -> the kernel instance.
template <int BM, int BN, bool MASKED, int EPI = kEpiPlain>
int32_t launch_dtype(int32_t dtype, const GemmArgs& a, hipStream_t s) {
  switch (dtype) {
    case MOE_DTYPE_BF16: return launch_gemm<BM, BN, kWfBf16, MASKED, EPI>(a, s);
    case MOE_DTYPE_FP8_E4M3_UE8M0: return launch_gemm<BM, BN, kWfFp8Block, MASKED, EPI>(a, s);
    case MOE_DTYPE_FP8_E4M3_MXFP8: return launch_gemm<BM, BN, kWfMxFp8, MASKED, EPI>(a, s);
    case MOE_DTYPE_FP8_MXFP4: return launch_gemm<BM, BN, kWfMxFp4, MASKED, EPI>(a, s);
    default: return MOE_EUNSUPPORTED;
  }
}

}  // namespace moe

using namespace moe;

static int32_t validate_gemm(int32_t dtype, const void* A, const uint8_t* A_scale, const void* B,
                             const uint8_t* B_scale, void* C, int32_t N, int32_t K, int32_t G) {
  if (N <= 0 || K <= 0 || G <= 0) return MOE_EINVAL;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3_UE8M0 &&
      dtype != MOE_DTYPE_FP8_E4M3_MXFP8 && dtype != MOE_DTYPE_FP8_MXFP4)
    return MOE_EUNSUPPORTED;
  if (N % 128 != 0 || K % 128 != 0) return MOE_EUNSUPPORTED;
  if (dtype != MOE_DTYPE_BF16 && (!A_scale || !B_scale)) return MOE_EUNSUPPORTED;
  if (K > (1 << 22)) return MOE_EUNSUPPORTED;  // per-lane 32-bit source offsets
  if (!A || !B || !C) return MOE_EINVAL;
  return MOE_OK;
}

extern "C" int32_t grouped_gemm_contig(int32_t dtype, const void* A, const uint8_t* A_scale,
                                       const void* B, const uint8_t* B_scale, void* C,
                                       const int32_t* m_indices, int64_t M, int32_t N, int32_t K,
                                       int32_t G, void* stream) {
  if (M < 0) return MOE_EINVAL;
  int32_t st = validate_gemm(dtype, A, A_scale, B, B_scale, C, N, K, G);
  if (st != MOE_OK) return st;
  if (M == 0) return MOE_OK;
  if (!m_indices) return MOE_EINVAL;
  GemmArgs a{};
  a.A = static_cast<const uint8_t*>(A);
  a.A_scale = A_scale;
  a.B = static_cast<const uint8_t*>(B);
  a.B_scale = B_scale;
  a.C = C;
  a.rowinfo = m_indices;
  a.M = M;
  a.N = N;
  a.K = K;
  a.G = G;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fp8 = dtype == MOE_DTYPE_FP8_E4M3_UE8M0;
  if ((fp8 || dtype == MOE_DTYPE_BF16) && wreg_supported(M, N, K, G, fp8)) {
    WregArgs w{a.A, a.A_scale, a.B, a.B_scale, C, nullptr, m_indices, M, N, K, G};
    return launch_wreg(w, fp8, kWrEpiPlain, s);
  }
  if (N % 256 == 0) return launch_dtype<128, 256, false>(dtype, a, s);
  return launch_dtype<128, 128, false>(dtype, a, s);
}

// Rows of tile height bm the masked kernels use for this hint (the rule the
// launches below apply; SiLU always has N = 2I % 256 == 0).
static int masked_tile_rows(int32_t expected_m, int32_t N) {
  if (expected_m > 0 && expected_m <= 16 && N % 256 == 0) return 16;
  if (expected_m > 0 && expected_m <= 32 && N % 256 == 0) return 32;
  if (expected_m > 0 && expected_m <= 64) return 64;
  return 128;
}

extern "C" int64_t grouped_gemm_rows_executed(int32_t dtype, int32_t masked, const int32_t* counts,
                                              int32_t G, int32_t expected_m, int64_t M, int32_t N,
                                              int32_t K) {
  if (!counts || G <= 0 || N <= 0 || K <= 0 || M < 0 || expected_m < 0) return -1;
  int64_t rows = 0;
  if (masked) {
    const int64_t bm = masked_tile_rows(expected_m, N);
    for (int g = 0; g < G; ++g) {
      if (counts[g] < 0) return -1;
      rows += (counts[g] + bm - 1) / bm * bm;
    }
    return rows;
  }
  const bool fp8 = dtype == MOE_DTYPE_FP8_E4M3_UE8M0;
  const bool wreg = (fp8 || dtype == MOE_DTYPE_BF16) && wreg_supported(M, N, K, G, fp8);
  for (int g = 0; g < G; ++g) {
    const int64_t z = counts[g];
    if (z < 0) return -1;
    if (z == 0) continue;
    if (!wreg) {
      rows += (z + 127) / 128 * 128;
      continue;
    }
    // the register-streamed kernel: ceil(z / 256) tiles of equal height
    // rounded up to 16, each running its MFMAs on whole 16-row blocks
    const int64_t nt = (z + 255) / 256;
    const int64_t h = ((z + nt - 1) / nt + 15) / 16 * 16;
    for (int64_t t = 0; t < nt; ++t) {
      const int64_t r = z - t * h < h ? z - t * h : h;
      if (r > 0) rows += (r + 15) / 16 * 16;
    }
  }
  return rows;
}

extern "C" int32_t grouped_gemm_masked(int32_t dtype, const void* A, const uint8_t* A_scale,
                                       const void* B, const uint8_t* B_scale, void* C,
                                       const int32_t* masked_m, int32_t expected_m, int32_t max_m,
                                       int32_t N, int32_t K, int32_t G, void* stream) {
  if (max_m <= 0 || expected_m < 0) return MOE_EINVAL;
  int32_t st = validate_gemm(dtype, A, A_scale, B, B_scale, C, N, K, G);
  if (st != MOE_OK) return st;
  if (!masked_m) return MOE_EINVAL;
  if (G > kMaxMaskedGroups) return MOE_EUNSUPPORTED;
  GemmArgs a{};
  a.A = static_cast<const uint8_t*>(A);
  a.A_scale = A_scale;
  a.B = static_cast<const uint8_t*>(B);
  a.B_scale = B_scale;
  a.C = C;
  a.rowinfo = masked_m;
  a.M = max_m;
  a.N = N;
  a.K = K;
  a.G = G;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool n256 = N % 256 == 0;
  // tile height from the hint: small expected counts waste less work on 64 rows
  switch (masked_tile_rows(expected_m, N)) {
    case 16: return launch_dtype<16, 256, true>(dtype, a, s);
    case 32: return launch_dtype<32, 256, true>(dtype, a, s);
    case 64: return n256 ? launch_dtype<64, 256, true>(dtype, a, s) : launch_dtype<64, 128, true>(dtype, a, s);
    default: return n256 ? launch_dtype<128, 256, true>(dtype, a, s) : launch_dtype<128, 128, true>(dtype, a, s);
  }
}

// The w13 GEMM with SiLU-and-mul in its epilogue: B holds [G][2I][K] (gate
// rows then up rows); out receives the activation [rows][I].
static int32_t validate_silu(int32_t out_dtype, void* out, uint8_t* out_scale, int32_t I) {
  if (I <= 0 || !out) return MOE_EINVAL;
  if (I % 128 != 0) return MOE_EUNSUPPORTED;
  if (out_dtype != MOE_DTYPE_BF16 && out_dtype != MOE_DTYPE_FP8_E4M3_UE8M0) return MOE_EUNSUPPORTED;
  if (out_dtype == MOE_DTYPE_FP8_E4M3_UE8M0 && !out_scale) return MOE_EINVAL;
  return MOE_OK;
}

extern "C" int32_t grouped_gemm_contig_silu(int32_t dtype, const void* A, const uint8_t* A_scale,
                                            const void* B, const uint8_t* B_scale, int32_t out_dtype,
                                            void* out, uint8_t* out_scale, const int32_t* m_indices,
                                            int64_t M, int32_t I, int32_t K, int32_t G, void* stream) {
  if (M < 0) return MOE_EINVAL;
  int32_t st = validate_silu(out_dtype, out, out_scale, I);
  if (st != MOE_OK) return st;
  if (I > (1 << 29)) return MOE_EUNSUPPORTED;
  // per-lane 32-bit offsets reach the up rows, I weight rows in
  if (static_cast<int64_t>(I + 256) * K * 2 >= (1ll << 32)) return MOE_EUNSUPPORTED;
  st = validate_gemm(dtype, A, A_scale, B, B_scale, out, 2 * I, K, G);
  if (st != MOE_OK) return st;
  if (M == 0) return MOE_OK;
  if (!m_indices) return MOE_EINVAL;
  GemmArgs a{};
  a.A = static_cast<const uint8_t*>(A);
  a.A_scale = A_scale;
  a.B = static_cast<const uint8_t*>(B);
  a.B_scale = B_scale;
  a.C = out;
  a.C_scale = out_scale;
  a.rowinfo = m_indices;
  a.M = M;
  a.N = 2 * I;
  a.K = K;
  a.G = G;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fp8 = dtype == MOE_DTYPE_FP8_E4M3_UE8M0;
  if ((fp8 || dtype == MOE_DTYPE_BF16) && wreg_supported(M, 2 * I, K, G, fp8)) {
    WregArgs w{a.A, a.A_scale, a.B, a.B_scale, out, out_scale, m_indices, M, 2 * I, K, G};
    return launch_wreg(w, fp8, out_dtype == MOE_DTYPE_FP8_E4M3_UE8M0 ? kWrEpiSiluFp8 : kWrEpiSiluBf16, s);
  }
  if (out_dtype == MOE_DTYPE_FP8_E4M3_UE8M0)
    return launch_dtype<128, 256, false, kEpiSiluFp8>(dtype, a, s);
  return launch_dtype<128, 256, false, kEpiSiluBf16>(dtype, a, s);
}

extern "C" int32_t grouped_gemm_masked_silu(int32_t dtype, const void* A, const uint8_t* A_scale,
                                            const void* B, const uint8_t* B_scale, int32_t out_dtype,
                                            void* out, uint8_t* out_scale, const int32_t* masked_m,
                                            int32_t expected_m, int32_t max_m, int32_t I, int32_t K,
                                            int32_t G, void* stream) {
  if (max_m <= 0 || expected_m < 0) return MOE_EINVAL;
  int32_t st = validate_silu(out_dtype, out, out_scale, I);
  if (st != MOE_OK) return st;
  if (I > (1 << 29)) return MOE_EUNSUPPORTED;
  if (static_cast<int64_t>(I + 256) * K * 2 >= (1ll << 32)) return MOE_EUNSUPPORTED;
  st = validate_gemm(dtype, A, A_scale, B, B_scale, out, 2 * I, K, G);
  if (st != MOE_OK) return st;
  if (!masked_m) return MOE_EINVAL;
  if (G > kMaxMaskedGroups) return MOE_EUNSUPPORTED;
  GemmArgs a{};
  a.A = static_cast<const uint8_t*>(A);
  a.A_scale = A_scale;
  a.B = static_cast<const uint8_t*>(B);
  a.B_scale = B_scale;
  a.C = out;
  a.C_scale = out_scale;
  a.rowinfo = masked_m;
  a.M = max_m;
  a.N = 2 * I;
  a.K = K;
  a.G = G;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool q8 = out_dtype == MOE_DTYPE_FP8_E4M3_UE8M0;
  switch (masked_tile_rows(expected_m, 2 * I)) {
    case 16: return q8 ? launch_dtype<16, 256, true, kEpiSiluFp8>(dtype, a, s)
                       : launch_dtype<16, 256, true, kEpiSiluBf16>(dtype, a, s);
    case 32: return q8 ? launch_dtype<32, 256, true, kEpiSiluFp8>(dtype, a, s)
                       : launch_dtype<32, 256, true, kEpiSiluBf16>(dtype, a, s);
    case 64: return q8 ? launch_dtype<64, 256, true, kEpiSiluFp8>(dtype, a, s)
                       : launch_dtype<64, 256, true, kEpiSiluBf16>(dtype, a, s);
    default: return q8 ? launch_dtype<128, 256, true, kEpiSiluFp8>(dtype, a, s)
                       : launch_dtype<128, 256, true, kEpiSiluBf16>(dtype, a, s);
  }
}
