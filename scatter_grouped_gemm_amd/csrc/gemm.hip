// Grouped NT GEMM for the expert layouts: C[r, :] = A[r, :] . B[g(r)]^T,
// BF16 or FP8 e4m3 with UE8M0 scales, fp32 accumulation, bf16 output.
//
// Design (gfx950, wave64, 160 KB LDS):
//   - One workgroup of 512 threads (8 wavefronts, two per SIMD) computes a
//     BM x BN tile of C; each wavefront owns a 64-row (or BM-row) by 64- or
//     32-column sub-tile.  The second wavefront on each SIMD issues MFMAs while
//     the first waits on LDS reads or the per-step barrier.
//   - A k-step covers 128 bytes of every tile row (64 bf16 or 128 e4m3).  The
//     rows go from global memory straight into LDS (global_load_lds, 16 bytes
//     per lane) through three stages: two k-steps are in flight while the
//     fragments of the next k-step are read from LDS and the current one is
//     multiplied from registers.
//   - MFMA: v_mfma_f32_16x16x32_bf16 for BF16 and the block-scaled
//     v_mfma_scale_f32_16x16x128_f8f6f4 for FP8.  The UE8M0 bytes are exactly
//     the E8M0 scales that instruction consumes; the per-128-channel activation
//     scale and the 128x128 weight-block scale are both constant over one
//     128-wide k step, so every lane supplies its row's (column's) byte and no
//     fp32 rescaling is done in the main loop.
//   - The weight tile is the MFMA "A" operand and the activation tile the "B"
//     operand, so the accumulator holds C^T: each lane owns 4 consecutive output
//     columns of one row, which pack into one 8-byte LDS write in the epilogue;
//     the tile then leaves LDS as 16-byte row-contiguous global stores.
//   - Persistent workgroups, one per CU, walk a tile order built on the device
//     from the layout: only tiles holding valid rows are listed, each expert's
//     tiles form one run ordered N-tile-major with its M-tiles innermost, so
//     the workgroups that run at the same time share each weight panel, and
//     the list is cut into eight equal contiguous parts, one per XCD (the
//     hardware deals workgroup ids round-robin over the XCDs, each with its
//     own L2).  Compact layout: an expert's run is the maximal range of M-tiles
//     whose first row carries its id (BM divides the 128-row alignment, so a
//     tile never straddles experts); masked layout: group g has
//     ceil(masked_m[g] / BM) tiles.
//   - Batch invariance: the instruction shape and the k order are the same for
//     every tile size and layout; a row's result depends only on its own A row
//     and its expert's weights.
#include <type_traits>

#include "common.cuh"

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
  uint16_t* C;
  const int32_t* rowinfo;  // m_indices (contiguous) or masked_m (masked)
  int64_t M;               // contiguous: rows of A/C; masked: max_m
  int N, K, G;
  int m_tiles;             // contiguous: M tiles of A; masked: M tiles per group
  int n_tiles;
};

constexpr int kMaxMaskedGroups = 1024;  // masked tile prefix lives in LDS

// Expert id of the first row of M-tile j, or INT_MIN outside [0, used).
template <int BM>
__device__ __forceinline__ int tile_expert(const int32_t* m_indices, int j, int used) {
  return (j >= 0 && j < used) ? m_indices[static_cast<int64_t>(j) * BM] : INT_MIN;
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

constexpr int kWaves = 8;             // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kMaxFp8K = 8192;  // FP8 scale staging in LDS covers K up to this

// LDS bytes: three k-stages (plus, for FP8, the tile's scales) or the bf16 C
// tile of the epilogue, whichever is larger.
template <int BM, int BN, bool FP8>
constexpr int gemm_lds_bytes() {
  constexpr int stages = 3 * (BM + BN) * 128 +
                         (FP8 ? (BM + BN / 128) * (kMaxFp8K / 128) : 0);
  constexpr int ctile = BM * (BN * 2 + 16);
  return stages > ctile ? stages : ctile;
}

template <int BM, int BN, bool FP8, bool MASKED>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(const GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int WAVES_M = BM >= 128 ? 2 : 1;
  constexpr int WAVES_N = kWaves / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  static_assert(BM % 64 == 0 && BN % 128 == 0 && WN <= 128 && WM % 16 == 0 && WN % 16 == 0,
                "tile shape");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_rowok[BM];

  const int tid0 = threadIdx.x, lane0 = tid0 & 63, wave0 = tid0 >> 6;

  // ---- tile order (see the file comment) --------------------------------------
  __shared__ int s_sched[MASKED ? kMaxMaskedGroups + 1 : 8];
  int used;  // compact: M-tiles up to the last one holding a valid first row
  if (!MASKED) {
    int last = -1;
    for (int j = tid0; j < p.m_tiles; j += kThreads)
      if (p.rowinfo[static_cast<int64_t>(j) * BM] >= 0) last = j;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) last = max(last, __shfl_xor(last, off, 64));
    if (lane0 == 0) s_sched[wave0] = last;
    __syncthreads();
    last = s_sched[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) last = max(last, s_sched[w]);
    used = __builtin_amdgcn_readfirstlane(last + 1);  // uniform: keep it scalar
  } else {
    // s_sched[g] = M-tiles of groups before g (exclusive prefix), s_sched[G] = total
    constexpr int PER = (kMaxMaskedGroups + kThreads - 1) / kThreads;
    int cnt[PER];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = tid0 * PER + i;
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
      if (lane0 >= off) incl += v;
    }
    __shared__ int s_wsum[kWaves];
    if (lane0 == 63) s_wsum[wave0] = incl;
    __syncthreads();
    int base = incl - sum;
    for (int w = 0; w < wave0; ++w) base += s_wsum[w];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = tid0 * PER + i;
      if (g < p.G) s_sched[g] = base;
      base += cnt[i];
    }
    if (tid0 == kThreads - 1) s_sched[p.G] = base;  // groups >= G count 0
    __syncthreads();
    used = __builtin_amdgcn_readfirstlane(s_sched[p.G]);
  }
  // this workgroup's share: XCD x (= blockIdx % 8) takes the x-th eighth of
  // the order, its workgroups stepping through it side by side
  const int64_t U = static_cast<int64_t>(used) * p.n_tiles;
  const int xcd = blockIdx.x & 7, per_xcd = gridDim.x >> 3;
  const int64_t pos_end = (U * (xcd + 1)) >> 3;
  for (int64_t pos = ((U * xcd) >> 3) + (blockIdx.x >> 3); pos < pos_end; pos += per_xcd) {
  // Per-thread indices come from an opaque copy in every iteration, so the
  // compiler rebuilds per-thread addressing inside the tile instead of keeping
  // it live (in registers) across the main loop.
  int tid = tid0;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int i0 = static_cast<int>(pos / p.n_tiles);
  int g, first, run;  // the run of M-tiles [first, first + run) that holds i0
  if (!MASKED) {
    // windows of 64 tiles below and above i0, widened until both ends of the
    // run are found (tiles outside [0, used) compare unequal to any id)
    const int vb = tile_expert<BM>(p.rowinfo, i0 - 63 + lane, used);
    const int vf = tile_expert<BM>(p.rowinfo, i0 + 1 + lane, used);
    g = __builtin_amdgcn_readlane(vb, 63);
    int lo = i0 - 63;
    uint64_t d = ballot(vb != g);
    while (d == 0) {
      lo -= 64;
      d = ballot(tile_expert<BM>(p.rowinfo, lo + lane, used) != g);
    }
    first = lo + (63 - __builtin_clzll(d)) + 1;
    int hi = i0 + 1;
    d = ballot(vf != g);
    while (d == 0) {
      hi += 64;
      d = ballot(tile_expert<BM>(p.rowinfo, hi + lane, used) != g);
    }
    run = hi + __builtin_ctzll(d) - first;
    if (g < 0 || g >= p.G) continue;  // a run of padding tiles
  } else {
    int lo = 0, hi = p.G;  // last group whose prefix is <= i0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_sched[mid] <= i0) lo = mid;
      else hi = mid;
    }
    g = __builtin_amdgcn_readfirstlane(lo);
    first = __builtin_amdgcn_readfirstlane(s_sched[g]);
    run = __builtin_amdgcn_readfirstlane(s_sched[g + 1]) - first;
  }
  const int64_t local = pos - static_cast<int64_t>(first) * p.n_tiles;
  const int nt = static_cast<int>(local / run);
  const int mt = first + static_cast<int>(local - static_cast<int64_t>(nt) * run);

  int64_t row0;      // first row of the tile in A / C
  int64_t row_last;  // last addressable row of this group (loads clamp to it)
  int rows_here;     // masked: valid rows from row0
  if (!MASKED) {
    row0 = static_cast<int64_t>(mt) * BM;
    row_last = p.M - 1;
    rows_here = BM;
  } else {
    const int r_in0 = (mt - first) * BM;
    int mm = p.rowinfo[g];
    mm = mm < 0 ? 0 : (mm > p.M ? static_cast<int>(p.M) : mm);
    row0 = static_cast<int64_t>(g) * p.M + r_in0;
    row_last = static_cast<int64_t>(g) * p.M + p.M - 1;
    rows_here = mm - r_in0;
  }
  if (tid < BM) {
    bool ok;
    if (!MASKED) {
      const int64_t r = row0 + tid;
      ok = r < p.M && p.rowinfo[r] == g;
    } else {
      ok = tid < rows_here;
    }
    s_rowok[tid] = ok ? 1 : 0;
  }

  constexpr int ES = FP8 ? 1 : 2;
  const int64_t rowbytes = static_cast<int64_t>(p.K) * ES;
  const int nk = static_cast<int>(rowbytes / 128);

  // ---- global -> LDS: direct loads, three stages -----------------------------------
  // A stage holds 128 bytes of every tile row: rows [0, BM) are A rows, rows
  // [BM, BM+BN) are B rows, 128 bytes apart, with the 16-byte chunks of row r
  // permuted by chunk ^ swz(r) so that 16 lanes reading one chunk of 16
  // consecutive rows hit distinct banks.  Each global_load_lds_dwordx4 moves
  // 8 rows (64 lanes x 16 bytes) straight into LDS; lane i carries the chunk
  // that belongs at LDS position i, so the permutation costs nothing.
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * 128;
  constexpr int NST = 3;
  constexpr int NLD = ROWS / (8 * kWaves);  // load instructions per wavefront per stage
  static_assert(ROWS % (8 * kWaves) == 0, "stage rows split evenly over the wavefronts");
  // per-lane source offsets (32-bit) from the A and B tile bases
  const int64_t brow0 = static_cast<int64_t>(g) * p.N + static_cast<int64_t>(nt) * BN;
  const uint8_t* const a_base = p.A + row0 * rowbytes;
  const uint8_t* const b_base = p.B + brow0 * rowbytes;
  uint32_t soff[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int R = (wave * NLD + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ lds_swz(R);
    if (R < BM) {
      int64_t r = row0 + R;
      r = r > row_last ? row_last : r;
      soff[j] = static_cast<uint32_t>((r - row0) * rowbytes + c * 16);
    } else {
      soff[j] = static_cast<uint32_t>((R - BM) * rowbytes + c * 16);
    }
  }
#define MOE_DMA(st_, kt_)                                                                  \
  do {                                                                                     \
    const int64_t off_ = static_cast<int64_t>(kt_) * 128;                                  \
    const uint8_t* ab_ = a_base + off_;                                                    \
    const uint8_t* bb_ = b_base + off_;                                                    \
    uint8_t* dst_ = smem + (st_) * STAGE + wave * NLD * 1024;                              \
    _Pragma("unroll") for (int j = 0; j < NLD; ++j) {                                      \
      const bool is_a_ = (wave * NLD + j) * 8 < BM;                                        \
      __builtin_amdgcn_global_load_lds((is_a_ ? ab_ : bb_) + soff[j],                      \
          (__attribute__((address_space(3))) void*)(dst_ + j * 1024), 16, 0, 0);           \
    }                                                                                      \
  } while (0)

  // ---- FP8 scales, staged in LDS once per tile ----------------------------------------
  // s_as[kb][r]: activation scale of tile row r for k block kb;
  // s_bs[nb][kb]: weight block scale of the tile's 128-column block nb.
  const int KB = p.K / 128;
  uint8_t* s_as = smem + NST * STAGE;
  uint8_t* s_bs = s_as + BM * KB;
  if (FP8) {
    for (int i = tid; i < KB * BM; i += kThreads) {
      const int kb = i / BM, r = i - kb * BM;
      int64_t row = row0 + r;
      row = row > row_last ? row_last : row;
      const int64_t idx = MASKED ? (static_cast<int64_t>(g) * KB + kb) * p.M + (row - static_cast<int64_t>(g) * p.M)
                                 : static_cast<int64_t>(kb) * p.M + row;
      s_as[i] = p.A_scale[idx];
    }
    for (int i = tid; i < (BN / 128) * KB; i += kThreads) {
      const int nb = i / KB, kb = i - nb * KB;
      s_bs[i] = p.B_scale[(static_cast<int64_t>(g) * (p.N / 128) + nt * (BN / 128) + nb) * KB + kb];
    }
  }
  const int wblk = (wn * WN) / 128;

  f32x4_t acc[TN][TM];
#pragma unroll
  for (int jn = 0; jn < TN; ++jn)
#pragma unroll
    for (int im = 0; im < TM; ++im) acc[jn][im] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int frag_row = lane & 15;
  const int frag_k = lane >> 4;
  // Fragment rows are (multiple of 16) + frag_row, so the chunk permutation
  // depends on the lane only: the byte offset of logical chunk c of the lane's
  // row in the sub-tile starting at stage row rb is rb*128 + frag_row*128 +
  // ((c ^ swz_l) << 4).
  const int swz_l = lds_swz(frag_row);
#define MOE_ROWOFF(rb_, c_) ((rb_) * 128 + frag_row * 128 + (((c_) ^ swz_l) << 4))

  // ---- fragments, software-pipelined one k-step ahead ------------------------------
  // Each step: wait for the next stage and for this wave's pending LDS reads,
  // barrier, refill the stage just consumed (k+3), issue the LDS reads of step
  // k+1 into the spare fragment set, then run step k's MFMAs from registers.
  // The reads of step k+1 thus overlap the MFMAs of step k.
  using frag_t = typename std::conditional<FP8, i32x8_t, bf16x8_t>::type;
  constexpr int KS = FP8 ? 1 : 2;  // MFMA k-substeps per 128-byte stage
  struct Frags {
    frag_t a[KS][TM];
    frag_t b[KS][TN];
    int sa[TM];
    int sw;
  };
#define MOE_LOAD(F_, st_, kt_)                                                                   \
  do {                                                                                           \
    const uint8_t* S_ = smem + (st_) * STAGE;                                                    \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                          \
      _Pragma("unroll") for (int im = 0; im < TM; ++im) {                                        \
        const int rb_ = wm * WM + im * 16;                                                       \
        if constexpr (FP8) {                                                                     \
          const u32x4_t lo_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, frag_k * 2));     \
          const u32x4_t hi_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, frag_k * 2 + 1)); \
          F_.a[ks][im] = i32x8_t{(int)lo_[0], (int)lo_[1], (int)lo_[2], (int)lo_[3],             \
                                 (int)hi_[0], (int)hi_[1], (int)hi_[2], (int)hi_[3]};            \
        } else {                                                                                 \
          F_.a[ks][im] = *reinterpret_cast<const frag_t*>(S_ + MOE_ROWOFF(rb_, ks * 4 + frag_k)); \
        }                                                                                        \
      }                                                                                          \
      _Pragma("unroll") for (int jn = 0; jn < TN; ++jn) {                                        \
        const int rb_ = BM + wn * WN + jn * 16;                                                  \
        if constexpr (FP8) {                                                                     \
          const u32x4_t lo_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, frag_k * 2));     \
          const u32x4_t hi_ = *reinterpret_cast<const u32x4_t*>(S_ + MOE_ROWOFF(rb_, frag_k * 2 + 1)); \
          F_.b[ks][jn] = i32x8_t{(int)lo_[0], (int)lo_[1], (int)lo_[2], (int)lo_[3],             \
                                 (int)hi_[0], (int)hi_[1], (int)hi_[2], (int)hi_[3]};            \
        } else {                                                                                 \
          F_.b[ks][jn] = *reinterpret_cast<const frag_t*>(S_ + MOE_ROWOFF(rb_, ks * 4 + frag_k)); \
        }                                                                                        \
      }                                                                                          \
    }                                                                                            \
    if constexpr (FP8) {                                                                         \
      _Pragma("unroll") for (int im = 0; im < TM; ++im)                                          \
        F_.sa[im] = s_as[(kt_) * BM + wm * WM + im * 16 + frag_row];                             \
      F_.sw = s_bs[wblk * KB + (kt_)];                                                           \
    }                                                                                            \
  } while (0)
#define MOE_MMA(F_)                                                                              \
  do {                                                                                           \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks)                                            \
      _Pragma("unroll") for (int jn = 0; jn < TN; ++jn)                                          \
        _Pragma("unroll") for (int im = 0; im < TM; ++im) {                                      \
          if constexpr (FP8)                                                                     \
            acc[jn][im] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                      \
                F_.b[ks][jn], F_.a[ks][im], acc[jn][im], 0, 0, 0, F_.sw, 0, F_.sa[im]);          \
          else                                                                                   \
            acc[jn][im] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(F_.b[ks][jn], F_.a[ks][im],    \
                                                                  acc[jn][im], 0, 0, 0);         \
        }                                                                                        \
  } while (0)
  // step k: FC_ holds step k's fragments, FN_ receives step k+1's.  The body
  // has no branches: near the end the refill re-reads the last k-step into a
  // stage that is never read again and the final fragment load reads a stale
  // stage, so every step issues the same number of direct loads and the wait
  // count is the same constant everywhere.
#define MOE_STEP(FC_, FN_, k_)                                                                   \
  do {                                                                                           \
    wait_vm_lgkm0<NLD>();   /* stage k+1 landed (k+2 may be in flight); reads done */            \
    __builtin_amdgcn_s_barrier();                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    MOE_DMA(st, ((k_) + 3 < nk ? (k_) + 3 : nk - 1));                                            \
    const int st1_ = st + 1 == NST ? 0 : st + 1;                                                 \
    MOE_LOAD(FN_, st1_, ((k_) + 1 < nk ? (k_) + 1 : (k_)));                                      \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    MOE_MMA(FC_);                                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    st = st1_;                                                                                   \
  } while (0)

  // Scales and row flags were written with ordinary stores: make them visible
  // before the first step (this also drains their global loads before the
  // direct loads start counting).
  __syncthreads();
  MOE_DMA(0, 0);
  MOE_DMA(1, (1 < nk ? 1 : nk - 1));
  MOE_DMA(2, (2 < nk ? 2 : nk - 1));
  wait_vm_lgkm0<2 * NLD>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  Frags f0, f1;
  MOE_LOAD(f0, 0, 0);
  int st = 0;  // stage holding step k (read into registers during step k-1)
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    MOE_STEP(f0, f1, kt);
    MOE_STEP(f1, f0, kt + 1);
  }
  if (kt < nk) MOE_STEP(f0, f1, kt);
  wait_vm_lgkm0<0>();
#undef MOE_DMA
#undef MOE_ROWOFF
#undef MOE_LOAD
#undef MOE_MMA
#undef MOE_STEP
  __syncthreads();

  // ---- epilogue: accumulators -> bf16 tile in LDS -> row-contiguous stores ----------
  constexpr int CROW = BN * 2 + 16;
  uint8_t* Cs = smem;
#pragma unroll
  for (int jn = 0; jn < TN; ++jn)
#pragma unroll
    for (int im = 0; im < TM; ++im) {
      const int m_local = wm * WM + im * 16 + frag_row;
      const int n_local = wn * WN + jn * 16 + frag_k * 4;
      const f32x4_t v = acc[jn][im];
      const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
      const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
      *reinterpret_cast<u32x2_t*>(Cs + m_local * CROW + n_local * 2) = u32x2_t{lo, hi};
    }
  __syncthreads();
  constexpr int CPR = BN / 8;  // 16-byte chunks per output row
  uint16_t* Cg = p.C + row0 * p.N + static_cast<int64_t>(nt) * BN;
  for (int idx = tid; idx < BM * CPR; idx += kThreads) {
    const int rr = idx / CPR, cc = idx - rr * CPR;
    if (s_rowok[rr])
      *reinterpret_cast<u32x4_t*>(Cg + static_cast<int64_t>(rr) * p.N + cc * 8) =
          *reinterpret_cast<const u32x4_t*>(Cs + rr * CROW + cc * 16);
  }
  __syncthreads();  // the C tile and the row flags are reused by the next tile
  }  // tile loop
#endif
}

// Persistent grid: one workgroup per CU (the LDS footprint allows no more),
// rounded down to a multiple of the 8 XCDs.
static int persistent_grid() {
  static int grid[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (grid[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    grid[dev] = cus >= 8 ? cus / 8 * 8 : 8;
  }
  return grid[dev];
}

template <int BM, int BN, bool FP8, bool MASKED>
int32_t launch_gemm(GemmArgs a, hipStream_t s) {
  constexpr int lds = gemm_lds_bytes<BM, BN, FP8>();
  auto kern = grouped_gemm_kernel<BM, BN, FP8, MASKED>;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
      return MOE_EDEVICE;
    attr_set = true;
  }
  a.n_tiles = a.N / BN;
  a.m_tiles = static_cast<int>((a.M + BM - 1) / BM);
  const int64_t tiles = static_cast<int64_t>(MASKED ? a.G : 1) * a.m_tiles * a.n_tiles;
  if (tiles == 0) return MOE_OK;
  if (tiles >= (1ll << 40)) return MOE_EINVAL;
  const int grid = persistent_grid();
  if (grid == 0) return MOE_EDEVICE;
  kern<<<grid, kThreads, lds, s>>>(a);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

static int32_t validate_gemm(int32_t dtype, const void* A, const uint8_t* A_scale, const void* B,
                             const uint8_t* B_scale, void* C, int32_t N, int32_t K, int32_t G) {
  if (N <= 0 || K <= 0 || G <= 0) return MOE_EINVAL;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3_UE8M0) return MOE_EUNSUPPORTED;
  if (N % 128 != 0 || K % 128 != 0) return MOE_EUNSUPPORTED;
  if (dtype == MOE_DTYPE_FP8_E4M3_UE8M0 && (!A_scale || !B_scale)) return MOE_EUNSUPPORTED;
  if (dtype == MOE_DTYPE_FP8_E4M3_UE8M0 && K > kMaxFp8K) return MOE_EUNSUPPORTED;
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
  a.C = static_cast<uint16_t*>(C);
  a.rowinfo = m_indices;
  a.M = M;
  a.N = N;
  a.K = K;
  a.G = G;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fp8 = dtype == MOE_DTYPE_FP8_E4M3_UE8M0;
  if (N % 256 == 0)
    return fp8 ? launch_gemm<128, 256, true, false>(a, s) : launch_gemm<128, 256, false, false>(a, s);
  return fp8 ? launch_gemm<128, 128, true, false>(a, s) : launch_gemm<128, 128, false, false>(a, s);
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
  a.C = static_cast<uint16_t*>(C);
  a.rowinfo = masked_m;
  a.M = max_m;
  a.N = N;
  a.K = K;
  a.G = G;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fp8 = dtype == MOE_DTYPE_FP8_E4M3_UE8M0;
  const bool n256 = N % 256 == 0;
  // tile height from the hint: small expected counts waste less work on 64 rows
  if (expected_m > 0 && expected_m <= 64) {
    if (n256) return fp8 ? launch_gemm<64, 256, true, true>(a, s) : launch_gemm<64, 256, false, true>(a, s);
    return fp8 ? launch_gemm<64, 128, true, true>(a, s) : launch_gemm<64, 128, false, true>(a, s);
  }
  if (n256) return fp8 ? launch_gemm<128, 256, true, true>(a, s) : launch_gemm<128, 256, false, true>(a, s);
  return fp8 ? launch_gemm<128, 128, true, true>(a, s) : launch_gemm<128, 128, false, true>(a, s);
}
