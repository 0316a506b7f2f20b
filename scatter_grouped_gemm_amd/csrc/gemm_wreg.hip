// Grouped NT GEMM for the compact expert layout with the weights streamed
// straight into registers: C[r, :] = A[r, :] . B[g(r)]^T, BF16 or FP8 e4m3
// with UE8M0 scales, fp32 accumulation, bf16 output (or SiLU-and-mul of the
// two halves of w13, as bf16 or e4m3 + UE8M0).
//
// Why this shape (gfx950, one MI355X):
//   - In the FP8 DeepSeek-V3-shaped prefill each expert holds about 256 token
//     rows against a 4096 x 7168 weight matrix, so every k-step a CU moves 64
//     KB (256 activation rows and 256 weight rows, 128 bytes each) for at most
//     256 x 256 x 128 multiply-adds.  Measured, a step is bound by issuing
//     those loads (about 72 vector memory instructions per CU) and by how
//     little that overlaps the MFMAs of the same wavefront, not by latency:
//     the per-step wait for data is short.  Every wavefront loads its own
//     weight columns straight into VGPRs in MFMA fragment order (16 bytes per
//     lane), three k-steps ahead in four register sets, so the weights never
//     pass through LDS; the activations go through four 32 KB LDS stages.
//   - Workgroup = 4 wavefronts (one per SIMD, 512 registers each).  A tile is
//     up to 256 rows of one expert run by 256 weight columns; wavefront w owns
//     64 columns and all rows, so the activations (shared by every wavefront)
//     go through LDS once (direct-to-LDS buffer loads, 16 bytes per lane) and
//     each weight byte sits in exactly one wavefront's registers.  LDS reads
//     per k-step are 64 bytes per MFMA cycle, half the LDS bandwidth.
//   - Tiles follow the expert runs of the compact layout rather than its
//     128-row blocks: a run of z valid rows is cut into ceil(z / 256) tiles of
//     equal height rounded up to 16 (gemm_runs.h), and only the 16-row blocks
//     holding rows run MFMAs.  An expert with up to 256 rows streams its
//     weights once, and no tile computes a whole padding block.
//   - A k-step is 128 bytes of a row (128 e4m3 or 64 bf16).  MFMA: the block-
//     scaled v_mfma_scale_f32_16x16x128_f8f6f4 (the UE8M0 bytes are its E8M0
//     scale operands: the 128-channel activation scale and the 128x128 weight
//     block scale are constant over one k-step) or two v_mfma_f32_16x16x32_bf16.
//     The weight fragment is the MFMA "A" operand, so each lane ends with four
//     consecutive output columns of one row; the weight rows a lane loads are
//     permuted so that two column blocks give eight consecutive columns (16
//     bytes of bf16).  The plain (w2) epilogue passes them through the stage
//     just consumed, 64 rows at a time, and stores whole 128-byte row segments
//     (8 rows per instruction): stores of 16 rows x 64 bytes cost the texture
//     unit several times more per byte, and staging took the FP8 w2 of the
//     DeepSeek-V3 prefill from 1.29 to 1.25 ms (the SiLU epilogues staged the
//     same way measured no faster, FP8 slower, and store directly).
//   - The k loop is one flat stream of k-steps over all of the workgroup's
//     tiles: loads cross into the next tile while the current one finishes.
//     Each step waits for its own loads with one vmcnt count (vector memory
//     instructions complete in issue order; every step issues the same
//     number), one barrier makes the activation stage visible, and the stage
//     and register set of the step before are refilled with the step three
//     ahead.
//   - Tile order (built once per workgroup from m_indices): expert runs in
//     row order; inside a run, groups of up to 8 M-tiles, N-tiles in order,
//     the group's M-tiles innermost, so the 32 workgroups of an XCD running
//     side by side share weight panels (few M-tiles per expert) or tile a
//     block of 8 M-tiles by 4 N-tiles (hot experts, where activations and
//     weights are both reused through L2).  The order is cut into eight
//     contiguous parts, one per XCD (workgroup ids are dealt round-robin over
//     the XCDs, each with its own L2).
//   - Batch invariance: one MFMA shape per dtype, one k order, no split-K; a
//     row's result depends only on its own A row and its expert's weights,
//     whatever the tile height.
#include <climits>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "gemm_runs.h"
#include "gemm_wreg.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

constexpr int kThreads = 256;               // four wavefronts, one per SIMD
constexpr int kRB = 16;                     // 16-row blocks of a tile at most
constexpr int kMT = kRB * 16;               // tile rows at most
constexpr int kNS = 4;                      // LDS stages = weight register sets
constexpr int kLA = kNS - 1;                // k-steps of lookahead
constexpr int kALD = kMT * 128 / 1024 / 4;  // activation loads per wavefront per step
using runs::decode;
using runs::kMaxBlocks;
using runs::kTable;
using runs::lds_off;
using runs::Tile;
using runs::wait_vm;
constexpr int kActBytes = kMT * 128;
static_assert(kALD * 4 * 1024 == kActBytes, "whole 1 KB loads per wavefront");

// FP8 stages also hold the scale bytes: one 256-byte slot per wavefront for
// the activation scales of its 64 tile rows, one per wavefront for its weight
// scales
template <bool FP8>
constexpr int stage_bytes() { return kActBytes + (FP8 ? 2048 : 0); }
template <bool FP8, int EPI>
constexpr int lds_bytes() {
  return kNS * stage_bytes<FP8>() + kTable * 16 + (EPI == kWrEpiSiluFp8 ? kMT * 16 : 0);
}
// vector memory instructions per wavefront per step: activation rows, the
// scale bytes (FP8), eight 16-byte weight loads
template <bool FP8>
constexpr int vm_per_step() { return kALD + (FP8 ? 2 : 0) + 8; }

// MFMA operand fragments of one 128-byte k-step: lane group g (lanes 16 g ..
// 16 g + 15) holds 16-byte chunks 2 g and 2 g + 1 of its row, 32 contiguous
// bytes.  FP8: one 32-byte operand of the 16x16x128 instruction (k order =
// memory order).  BF16: the two 16-byte operands of two 16x16x32
// instructions, the first over the even chunks of the row and the second over
// the odd ones; both operands use the same order, so together they form the
// whole dot product, and the contiguous 32-byte LDS reads avoid the bank
// conflicts that chunks g and g + 4 would cause.
struct Bf16Frag {
  u32x4 lo, hi;
};
template <bool FP8>
struct FragT {
  using type = Bf16Frag;
};
template <>
struct FragT<true> {
  using type = i32x8;
};
__device__ __forceinline__ i32x8 make_frag8(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
template <bool FP8>
__device__ __forceinline__ typename FragT<FP8>::type make_frag_t(u32x4 lo, u32x4 hi) {
  if constexpr (FP8) return make_frag8(lo, hi);
  else return Bf16Frag{lo, hi};
}

// The MFMAs of one 16-row block against the wavefront's four 16-column weight
// blocks, skipped as a whole when the block holds no rows of the tile
// (rb >= nrb).  Written as assembly so that the weight fragments are read
// straight from the AGPRs their loads filled and the accumulators stay in
// place across the skip (as builtins behind a branch the compiler merges them
// through register copies).  The inputs come from loads the compiler waits
// on before the statement; the accumulators are read by other code only
// after mfma_drain().
#define MOE_MFMA8(c, w, s0)                                                             \
  "v_mfma_scale_f32_16x16x128_f8f6f4 %[" #c "], %[" #w "], %[a], %[" #c "], %[" #s0 "], %[sb]\n\t"
#define MOE_MFMA16(c, w, a)                                                             \
  "v_mfma_f32_16x16x32_bf16 %[" #c "], %[" #w "], %[" #a "], %[" #c "]\n\t"
template <bool FP8, bool SILU>
__device__ __forceinline__ void mma_block(f32x4 (&c)[4], const typename FragT<FP8>::type (&w)[4],
                                          const typename FragT<FP8>::type& a, int swa, int swb, int sa,
                                          int nrb, int rb) {
  if constexpr (FP8) {
    asm volatile(
        "s_cmp_le_i32 %[nrb], %[rb]\n\t"
        "s_cbranch_scc1 1f\n\t"
        MOE_MFMA8(c0, w0, sa0) MOE_MFMA8(c1, w1, sa0) MOE_MFMA8(c2, w2, sa1) MOE_MFMA8(c3, w3, sa1)
        "1:"
        : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [c3] "+a"(c[3])
        : [w0] "v"(w[0]), [w1] "v"(w[1]), [w2] "v"(w[2]), [w3] "v"(w[3]), [a] "v"(a), [sa0] "v"(swa),
          [sa1] "v"(SILU ? swb : swa), [sb] "v"(sa), [nrb] "s"(nrb), [rb] "s"(rb)
        : "scc");
  } else {
    asm volatile(
        "s_cmp_le_i32 %[nrb], %[rb]\n\t"
        "s_cbranch_scc1 1f\n\t"
        MOE_MFMA16(c0, w0l, al) MOE_MFMA16(c1, w1l, al) MOE_MFMA16(c2, w2l, al) MOE_MFMA16(c3, w3l, al)
        MOE_MFMA16(c0, w0h, ah) MOE_MFMA16(c1, w1h, ah) MOE_MFMA16(c2, w2h, ah) MOE_MFMA16(c3, w3h, ah)
        "1:"
        : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [c3] "+a"(c[3])
        : [w0l] "v"(w[0].lo), [w1l] "v"(w[1].lo), [w2l] "v"(w[2].lo), [w3l] "v"(w[3].lo),
          [w0h] "v"(w[0].hi), [w1h] "v"(w[1].hi), [w2h] "v"(w[2].hi), [w3h] "v"(w[3].hi),
          [al] "v"(a.lo), [ah] "v"(a.hi), [nrb] "s"(nrb), [rb] "s"(rb)
        : "scc");
  }
}
#undef MOE_MFMA8
#undef MOE_MFMA16

// The accumulators live in AGPRs and only assembly writes them: these two
// helpers are the only other accesses.  acc_zero clears the four tiles of a
// row block with 4x4x4 MFMAs of zero operands and a zero C (two passes each).
// The zero operand is written inside the statement, followed by the wait
// states a VALU write needs before an MFMA reads it: the compiler's hazard
// recognizer does not see MFMAs inside assembly, so a zero register it
// materialised just before the statement could be read while still being
// written.  acc_read copies them into VGPRs at this point of the program (the
// tie makes the compiler emit the copies here rather than hoisting all 256 of
// them).
__device__ __forceinline__ void acc_zero(f32x4 (&c)[4]) {
  typedef __attribute__((ext_vector_type(2))) int i32x2;
  i32x2 z;
  asm volatile(
      "v_mov_b64 %4, 0\n\t"
      "s_nop 4\n\t"
      "v_mfma_f32_4x4x4_16b_f16 %0, %4, %4, 0\n\t"
      "v_mfma_f32_4x4x4_16b_f16 %1, %4, %4, 0\n\t"
      "v_mfma_f32_4x4x4_16b_f16 %2, %4, %4, 0\n\t"
      "v_mfma_f32_4x4x4_16b_f16 %3, %4, %4, 0"
      : "=a"(c[0]), "=a"(c[1]), "=a"(c[2]), "=a"(c[3]), "=&v"(z));
}
__device__ __forceinline__ void acc_read(const f32x4 (&c)[4], f32x4 (&o)[4]) {
  asm volatile("" : "=v"(o[0]), "=v"(o[1]), "=v"(o[2]), "=v"(o[3]) : "0"(c[0]), "1"(c[1]), "2"(c[2]), "3"(c[3]));
}
__device__ __forceinline__ void acc_write0(f32x4 (&c)[4], f32x4 v) {
  asm volatile("" : "=a"(c[0]) : "0"(v));
}

// Wait states between the last MFMA and VALU/accumulator reads of its result
// (the compiler does not see into the assembly above).
__device__ __forceinline__ void mfma_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
}

// The loads of one k-step are spread over the row blocks of the step before
// (one piece after each block, at most): the texture unit that every vector
// memory instruction of the CU passes through is the busiest part of the
// kernel, and a wavefront stalled on it also stops issuing its MFMAs, so
// bunching the loads into a few blocks left the matrix cores idle there.
// Entry rb: 1..3 the weights of column block rb (two 16-byte loads), 4 + j
// activation row group j (j < 8; FP8: 12 the activation scales, 13 the
// weight scales), -1 nothing.  Column block 0 is loaded in block 0.
constexpr int kLoadAt[kRB] = {-1, 4, 1, 5, 6, 2, 7, 12, 8, 3, 9, 10, 13, 11, -1, -1};

__device__ __forceinline__ void lds_write_f32(float* p, float v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(lds_off(p)), "v"(v) : "memory");
}
__device__ __forceinline__ f32x4 lds_read_f32x4(const float* p) {
  f32x4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(p)) : "memory");
  return v;
}

// chunk permutation of activation stage row r: the 16 lanes reading one
// 16-byte chunk of 16 consecutive rows hit distinct banks
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <bool FP8, int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_wreg_kernel(const WregArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int STAGE = stage_bytes<FP8>();
  constexpr int NVM = vm_per_step<FP8>();
  constexpr bool SILU = EPI != kWrEpiPlain;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int4* const table = reinterpret_cast<int4*>(smem + kNS * STAGE);
  float* const rowmax = reinterpret_cast<float*>(smem + kNS * STAGE + kTable * 16);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ES = FP8 ? 1 : 2;
  const int64_t rowbytes = static_cast<int64_t>(p.K) * ES;  // A row and B row
  const int nk = static_cast<int>(rowbytes / 128);
  const int KB = p.K / 128;
  const int ntn = p.N / 256;  // N-tiles (SiLU: 128 activation channels each)
  const int I = p.N / 2;

  // ======== set-up: the run table of this XCD's share of the order ========
  static_assert(runs::kSetupBytes <= kNS * kActBytes, "set-up arrays fit in the stages");
  runs::Share sh;
  if (!runs::build_share(p.m_indices, p.M, p.G, ntn, smem, table, sh)) return;
  const int NR = sh.NR, lo_x = sh.lo, hi_x = sh.hi, per_xcd = sh.per_xcd;

  // ======== per-lane constants ========
  const int fr = lane & 15, fg = lane >> 4;
  // activation loads: wavefront w moves stage rows 8q .. 8q+7 for q = 8w + j;
  // lane L carries source chunk (L & 7) ^ swz(row) into LDS position L
  uint32_t va[kALD];
#pragma unroll
  for (int j = 0; j < kALD; ++j) {
    const int row = (wave * kALD + j) * 8 + (lane >> 3);
    va[j] = static_cast<uint32_t>(row * rowbytes + (((lane & 7) ^ swz(row)) << 4));
  }
  // weight rows: column block cb, MFMA row i = fr holds tile column
  //   plain: 64 w + 32 (cb / 2) + 8 (i / 4) + 4 (cb % 2) + i % 4
  //   SiLU : channel 32 w + 8 (i / 4) + 4 cb' + i % 4 of gate (cb = cb') or up (cb = 2 + cb')
  // so that a lane's four columns of blocks 2p and 2p + 1 are eight in a row
  auto wrow = [&](int cb, int nt) __attribute__((always_inline)) -> int {
    if (!SILU) return nt * 256 + wave * 64 + 32 * (cb >> 1) + 8 * (fr >> 2) + 4 * (cb & 1) + (fr & 3);
    const int ch = nt * 128 + wave * 32 + 8 * (fr >> 2) + 4 * (cb & 1) + (fr & 3);
    return cb < 2 ? ch : I + ch;
  };

  // ======== load side: the tile and k-step whose loads are issued next ========
  int d_cur = 0, d_pos = lo_x + static_cast<int>(blockIdx.x >> 3);
  Tile dt = decode<16>(table, NR, d_cur, d_pos, ntn);
  while (dt.rows <= 0) {
    d_pos += per_xcd;
    if (d_pos >= hi_x) return;
    dt = decode<16>(table, NR, d_cur, d_pos, ntn);
  }
  int d_k = 0;
  __amdgpu_buffer_rsrc_t rs_a, rs_w;
  uint32_t vw[4];
  const uint8_t* wbase8 = p.B;
  // FP8 scale bytes at k-step 0: s_off this lane's activation scale (tile row
  // 64 w + lane), w_off its weight-block scale (advance per k-step: M and 1)
  uint32_t s_off = 0, w_off = 0;
  const __amdgpu_buffer_rsrc_t rs_as =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.A_scale), 0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_ws =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.B_scale), 0, -1, 0x00020000);
  auto dset = [&]() __attribute__((always_inline)) {
    rs_a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.A + dt.row * rowbytes), 0,
                                             static_cast<int>(dt.rows * rowbytes), 0x00020000);
    rs_w = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.B + static_cast<int64_t>(dt.id) * p.N * rowbytes), 0,
        static_cast<int>(static_cast<int64_t>(p.N) * rowbytes), 0x00020000);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) vw[cb] = static_cast<uint32_t>(wrow(cb, dt.nt) * rowbytes + fg * 32);
    wbase8 = p.B + static_cast<int64_t>(dt.id) * p.N * rowbytes;
    if constexpr (FP8) {
      const int r = min(wave * 64 + lane, dt.rows - 1);
      s_off = static_cast<uint32_t>(dt.row + r);
      // weight-block scales of this wavefront's columns: plain, its 128-column
      // block (lanes 0 and 1 alike); SiLU, the gate block (lane 0) and the up
      // block (lane 1)
      const int blk = SILU ? (lane == 0 ? dt.nt : I / 128 + dt.nt) : 2 * dt.nt + (wave >> 1);
      w_off = static_cast<uint32_t>((static_cast<int64_t>(dt.id) * (p.N / 128) + blk) * KB);
    }
  };
  dset();

  using Frag = typename FragT<FP8>::type;
  Frag wr[kNS][4];  // weight fragments of the steps in flight, one set per stage
  // The loads of one k-step into stage / register set st, issued in pieces
  // that the compute side spreads among its MFMAs: the two 16-byte weight
  // loads of column block cb (register set: private to the wavefront), and the
  // activation rows j (a 1 KB direct-to-LDS load; j == kALD, kALD + 1: the FP8
  // activation and weight scale bytes).
  auto issue_w = [&](Frag (&w)[4], int cb) __attribute__((always_inline)) {
    if constexpr (FP8) {
      w[cb] = *reinterpret_cast<const i32x8*>(wbase8 + d_k * 128 + vw[cb]);
    } else {
      const u32x4 lo_ = __builtin_amdgcn_raw_buffer_load_b128(rs_w, vw[cb], d_k * 128, 0);
      const u32x4 hi_ = __builtin_amdgcn_raw_buffer_load_b128(rs_w, vw[cb] + 16, d_k * 128, 0);
      w[cb] = make_frag_t<FP8>(lo_, hi_);
    }
  };
  auto issue_a = [&](int st, int j) __attribute__((always_inline)) {
    uint8_t* const stg = smem + st * STAGE;
    if (j < kALD) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_a, (__attribute__((address_space(3))) void*)(stg + (wave * kALD + j) * 1024), 16, va[j],
          d_k * 128, 0, 0);
    } else if constexpr (FP8) {
      if (j == kALD)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs_as, (__attribute__((address_space(3))) void*)(stg + kActBytes + wave * 256), 1,
            s_off + static_cast<uint32_t>(d_k * p.M), 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs_ws, (__attribute__((address_space(3))) void*)(stg + kActBytes + 1024 + wave * 256), 1,
            w_off + static_cast<uint32_t>(d_k), 0, 0, 0);
    }
  };
  // move the load side on; past the last tile keep re-reading its last k-step
  // (never used) so that every step issues the same instructions
  auto advance = [&]() __attribute__((always_inline)) {
    if (++d_k == nk) {
      d_k = 0;
      int np = d_pos + per_xcd;
      Tile t;
      t.rows = 0;
      while (np < hi_x) {
        t = decode<16>(table, NR, d_cur, np, ntn);
        if (t.rows > 0) break;
        np += per_xcd;
      }
      if (np < hi_x) {
        d_pos = np;
        dt = t;
        dset();
      } else {
        d_k = nk - 1;
      }
    }
  };

  // ======== compute side ========
  int c_cur = d_cur, c_pos = d_pos;
  Tile ct = dt;
  int c_k = 0;
  f32x4 acc[kRB][4];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) acc_zero(acc[rb]);

  // next compute tile after c_pos (rows 0: none)
  auto c_next = [&]() __attribute__((always_inline)) -> Tile {
    int np = c_pos + per_xcd;
    Tile t;
    t.rows = 0;
    while (np < hi_x) {
      t = decode<16>(table, NR, c_cur, np, ntn);
      if (t.rows > 0) break;
      np += per_xcd;
    }
    c_pos = np;
    return t;
  };

  // Stores of the finished tile ct, then zero accumulators.  The stores are
  // buffer stores bounded by the tile's rows (rows past the tile fall outside
  // the buffer and are dropped), so no lane-dependent branch guards them.
  // stg is the LDS stage of the tile's last k-step: every wavefront has read
  // its fragments once all have reached the epilogue, and its next refill is
  // issued only after the next step's barrier.
  auto epilogue = [&](uint8_t* const stg) __attribute__((always_inline)) {
    if constexpr (EPI == kWrEpiPlain) {
      const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<uint16_t*>(p.C) + ct.row * p.N, 0, static_cast<int>(ct.rows * p.N * 2), 0x00020000);
      // through LDS, 64 rows at a time: each wavefront writes its 64 x 64
      // block into its own 8 KB of the stage just consumed, then stores it as
      // 8 rows x 128 bytes per instruction
      __builtin_amdgcn_s_barrier();  // every wavefront is done reading the stage
      uint8_t* const reg = stg + wave * 8192;
      const int lr8 = lane >> 3;
#pragma unroll
      for (int ps = 0; ps < 4; ++ps) {
        if (ps * 64 >= ct.rows) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 av[4];
          acc_read(acc[ps * 4 + q], av);
          const int r = q * 16 + fr;
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const f32x4 a = av[2 * pr], b = av[2 * pr + 1];
            const u32x4 v{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                          pack_bf16x2(b[2], b[3])};
            *reinterpret_cast<u32x4*>(reg + r * 128 + (((pr * 4 + fg) ^ (r & 7)) << 4)) = v;
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = j * 8 + lr8;
          const u32x4 v = *reinterpret_cast<const u32x4*>(reg + r * 128 + (((lane & 7) ^ (r & 7)) << 4));
          __builtin_amdgcn_raw_buffer_store_b128(
              v, rc, static_cast<uint32_t>(((ps * 64 + r) * p.N + ct.nt * 256 + wave * 64) * 2 + (lane & 7) * 16),
              0, 0);
        }
      }
    } else {
      // act of channel 8 fg + 4 h + e (h = 0, 1) of the wavefront's 32: gate
      // and up rounded to bf16 as the plain product would be stored, then
      // bf16(silu(gate) * up)
      auto act = [&](const f32x4 (&av)[4], int h, int e) __attribute__((always_inline)) -> float {
        const float gt = bf16_to_f32(f32_to_bf16(av[h][e]));
        const float up = bf16_to_f32(f32_to_bf16(av[h + 2][e]));
        return bf16_to_f32(f32_to_bf16(silu_f32(gt) * up));
      };
      const int ch0 = ct.nt * 128 + wave * 32 + fg * 8;
      if constexpr (EPI == kWrEpiSiluBf16) {
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<uint16_t*>(p.C) + ct.row * I, 0, static_cast<int>(ct.rows * I * 2), 0x00020000);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          f32x4 av[4];
          acc_read(acc[rb], av);
          float v[8];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * h + e] = act(av, h, e);
          const u32x4 o{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                        pack_bf16x2(v[6], v[7])};
          __builtin_amdgcn_raw_buffer_store_b128(o, rc, static_cast<uint32_t>(((rb * 16 + fr) * I + ch0) * 2), 0, 0);
        }
      } else {
        // Row maxima over the 128 channels of the tile: the lane's 8, the four
        // lanes of the row, then the four wavefronts through LDS.  Each row
        // block's eight activations are kept as packed bf16 in its first
        // accumulator (they are bf16 values already) for the quantisation.
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          f32x4 av[4];
          acc_read(acc[rb], av);
          float v[8];
          float m = 0.0f;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[4 * h + e] = act(av, h, e);
              m = fmaxf(m, fabsf(v[4 * h + e]));
            }
          acc_write0(acc[rb], __builtin_bit_cast(f32x4, u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                             pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])}));
          m = fmaxf(m, __shfl_xor(m, 16, 64));
          m = fmaxf(m, __shfl_xor(m, 32, 64));
          if (fg == 0) lds_write_f32(rowmax + (rb * 16 + fr) * 4 + wave, m);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the maxima are in LDS
        __builtin_amdgcn_s_barrier();
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<uint8_t*>(p.C) + ct.row * I, 0, static_cast<int>(ct.rows * I), 0x00020000);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            p.C_scale + static_cast<int64_t>(ct.nt) * p.M + ct.row, 0, ct.rows, 0x00020000);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          const int r = rb * 16 + fr;
          const f32x4 q4 = lds_read_f32x4(rowmax + r * 4);
          const float amax = fmaxf(fmaxf(q4[0], q4[1]), fmaxf(q4[2], q4[3]));
          const int ex = ue8m0_exponent(amax);
          f32x4 av[4];
          acc_read(acc[rb], av);
          const u32x4 pk = __builtin_bit_cast(u32x4, av[0]);
          auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
          auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
          const u32x2 o{e4m3x4(lo(pk[0]), hi(pk[0]), lo(pk[1]), hi(pk[1]), ex),
                        e4m3x4(lo(pk[2]), hi(pk[2]), lo(pk[3]), hi(pk[3]), ex)};
          __builtin_amdgcn_raw_buffer_store_b64(o, rc, static_cast<uint32_t>(r * I + ch0), 0, 0);
          // the scale bytes of row block rb come from wavefront rb % 4 (the
          // lanes of lane group 0 hold the block's 16 rows)
          if (rb % 4 == wave)
            __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(ex + 127), rs,
                                                 static_cast<uint32_t>(fg == 0 ? r : 0x7fffffff), 0, 0);
        }
        // the maxima are rewritten only by the next tile's epilogue, after at
        // least one step barrier
      }
    }
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) acc_zero(acc[rb]);
  };

  // ---- the step: MFMAs row block by row block from the fragments read two
  // blocks earlier; after block 0 one vmcnt wait and one barrier make the next
  // step's stage visible (its loads were issued kLA - 1 steps ago) and free
  // the stage and register set of the step before, which take the loads of the
  // step kLA ahead, spread over blocks 1 .. 13; the step ends by reading the
  // next step's first two fragments.
  bool c_epi = false, done = false;
  int c_nrb = __builtin_amdgcn_readfirstlane((ct.rows + 15) >> 4);
  const int ck_lo = 2 * fg, ck_hi = 2 * fg + 1;
  const uint32_t a_lo = static_cast<uint32_t>(fr * 128 + ((ck_lo ^ swz(fr)) << 4));
  const uint32_t a_hi = static_cast<uint32_t>(fr * 128 + ((ck_hi ^ swz(fr)) << 4));
  // weight-scale dword of this wavefront's columns (plain: its 128-column block)
  const int sw_sel = 1024 + wave * 256;
  Frag af[2];
  int sa[2] = {0, 0};
  int swa = 0, swb = 0;
  auto read_a = [&](const uint8_t* S, int rb, int slot) __attribute__((always_inline)) {
    const uint8_t* const R = S + rb * 2048;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(R + a_lo);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(R + a_hi);
    af[slot] = make_frag_t<FP8>(lo, hi);
    if constexpr (FP8) sa[slot] = *reinterpret_cast<const int*>(S + kActBytes + rb * 64 + fr * 4);
  };
  auto read_first = [&](const uint8_t* S) __attribute__((always_inline)) {
    if constexpr (FP8) {
      swa = *reinterpret_cast<const int*>(S + kActBytes + sw_sel);
      if (SILU) swb = *reinterpret_cast<const int*>(S + kActBytes + sw_sel + 4);
    }
    read_a(S, 0, 0);
    read_a(S, 1, 1);
  };
  // The next step's loads were issued kLA - 1 steps ago (the last of them
  // after block 13); since then kLA - 2 whole steps and this step's first two
  // weight loads have issued, and vector memory instructions complete in order.
  constexpr int W0 = (kLA - 2) * vm_per_step<FP8>() + 2;
  auto step = [&](auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    static_assert(u >= 0 && u < kNS, "stage / register set index");
    constexpr int un = (u + kLA) % kNS;   // = the stage of the step before
    constexpr int u1 = (u + 1) % kNS;
    const uint8_t* const S = smem + u * STAGE;
    const int nrb = __builtin_amdgcn_readfirstlane(c_nrb);
    // block 0, the weights of column block 0 (the register set is the
    // wavefront's own: no barrier needed), the wait and the barrier
    mma_block<FP8, SILU>(acc[0], wr[u], af[0], swa, swb, sa[0], nrb, 0);
    issue_w(wr[un], 0);
    read_a(S, 2, 0);
    // the wait counts the vector memory instructions issued before it, so no
    // load may move across it (sched_barrier: a hard scheduling boundary)
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<W0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // blocks 1 .. 15, each followed by at most one piece of the step's loads
    // (kLoadAt) and the read of the fragment two blocks on
#pragma unroll
    for (int rb = 1; rb < kRB; ++rb) {
      __builtin_amdgcn_sched_barrier(0);
      mma_block<FP8, SILU>(acc[rb], wr[u], af[rb & 1], swa, swb, sa[rb & 1], nrb, rb);
      {
        const int it = kLoadAt[rb];
        if (it >= 1 && it <= 3) issue_w(wr[un], it);
        else if (it >= 4 && it - 4 < kALD + (FP8 ? 2 : 0)) issue_a(un, it - 4);
      }
      if (rb + 2 < kRB) read_a(S, rb + 2, rb & 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    read_first(smem + u1 * STAGE);
    advance();
    if (++c_k == nk) {
      c_k = 0;
      const Tile cn = c_next();
      mfma_drain();
      // the accumulator copies of the epilogue stay after the drain
      __builtin_amdgcn_sched_barrier(0);
      epilogue(const_cast<uint8_t*>(S));
      done = cn.rows <= 0;
      ct = cn;
      c_nrb = __builtin_amdgcn_readfirstlane((ct.rows + 15) >> 4);
    }
  };

  // prologue: the first kLA steps' loads, then the first step's stage
#pragma unroll
  for (int q = 0; q < kLA; ++q) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) issue_w(wr[q], cb);
#pragma unroll
    for (int j = 0; j < kALD + (FP8 ? 2 : 0); ++j) issue_a(q, j);
    advance();
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vm<(kLA - 1) * vm_per_step<FP8>()>();  // the first step's loads
  __syncthreads();
  read_first(smem);
  // the loop body runs one step per stage / register set
  static_assert(kNS == 4, "the unrolled loop below has one step per stage");
  for (;;) {
    step(std::integral_constant<int, 0>());
    if (done) break;
    step(std::integral_constant<int, 1>());
    if (done) break;
    step(std::integral_constant<int, 2>());
    if (done) break;
    step(std::integral_constant<int, 3>());
    if (done) break;
  }
  wait_vm<0>();  // the trailing re-reads and the stores
#endif
}

}  // namespace

bool wreg_supported(int64_t M, int N, int K, int G, bool fp8) {
  const int64_t rowbytes = static_cast<int64_t>(K) * (fp8 ? 1 : 2);
  if (N <= 0 || K <= 0 || N % 256 != 0 || K % 128 != 0) return false;
  if (static_cast<int64_t>(N) * rowbytes >= (1ll << 31)) return false;  // one expert's weights
  // the run table holds one XCD's share of the runs: at most an eighth of the
  // M-tiles plus three
  if ((M + 127) / 128 > kMaxBlocks) return false;
  // 32-bit scale offsets (activation scales [K/128][M], weight scales)
  if (static_cast<int64_t>(K / 128) * M >= (1ll << 31)) return false;
  if (static_cast<int64_t>(N / 256) * kMaxBlocks >= (1ll << 30)) return false;  // positions
  if (static_cast<int64_t>(G) * (N / 128) * (K / 128) >= (1ll << 31)) return false;
  return true;
}

namespace {
int persistent_grid_wreg() {
  static int grid[64] = {0};
  static std::once_flag once[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::call_once(once[dev], [dev]() {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      grid[dev] = cus >= 8 ? cus / 8 * 8 : 8;
  });
  return grid[dev];
}

template <bool FP8, int EPI>
int32_t launch_t(const WregArgs& a, hipStream_t s) {
  constexpr int lds = lds_bytes<FP8, EPI>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = gemm_wreg_kernel<FP8, EPI>;
  static std::once_flag once[64];
  static bool ok[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_EDEVICE;
  std::call_once(once[dev], [&]() __attribute__((always_inline)) {
    ok[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess;
  });
  if (!ok[dev]) return MOE_EDEVICE;
  const int grid = persistent_grid_wreg();
  if (grid == 0) return MOE_EDEVICE;
  kern<<<grid, kThreads, lds, s>>>(a);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
}  // namespace

int32_t launch_wreg(const WregArgs& a, bool fp8, int epi, hipStream_t s) {
  if (a.M == 0) return MOE_OK;
  if (fp8) {
    if (epi == kWrEpiSiluFp8) return launch_t<true, kWrEpiSiluFp8>(a, s);
    if (epi == kWrEpiSiluBf16) return launch_t<true, kWrEpiSiluBf16>(a, s);
    return launch_t<true, kWrEpiPlain>(a, s);
  }
  if (epi == kWrEpiSiluFp8) return launch_t<false, kWrEpiSiluFp8>(a, s);
  if (epi == kWrEpiSiluBf16) return launch_t<false, kWrEpiSiluBf16>(a, s);
  return launch_t<false, kWrEpiPlain>(a, s);
}

}  // namespace moe
