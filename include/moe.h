/*
 * libmoe -- routed-token scatter -> grouped GEMM MoE expert path for MI355X
 * (gfx950), as a C ABI.
 *
 * Sources ("the pages"): three sglang pull-request reports --
 *   [P1] "Support DeepGEMM for standard MoE dispatch" (PR #33128)
 *   [P2] "Add BF16 support to EP-MoE for DeepGEMM" (PR #17392)
 *   [P3] "[Feature] Support BF16 and batch-invariant inference with DeepEP v2"
 *        (PR #38160)
 *
 * General contract
 *   - Every pointer named "device" is a device pointer on the current HIP
 *     device; the caller owns all memory.  The library never allocates: scratch
 *     comes in through ws/ws_bytes (size from moe_scatter_ws_bytes); the one
 *     exception is moe_scatter_compact_noalloc, whose scratch is a static
 *     device array of fixed size.
 *   - Every compute call validates its arguments on the host first and returns
 *     a status without launching anything when they are wrong; otherwise it
 *     enqueues its kernels on `stream` (a hipStream_t; NULL = default stream)
 *     and returns without synchronising.  No call reads device data back to the
 *     host, so all sizes are fixed by the host arguments (static shapes, P1
 *     implementation breakdown item 2: buffers usable under graph capture).
 *   - Buffers may be uninitialised on entry (P1 implementation breakdown item 4):
 *     every valid row is written before it is read.  Rows marked -1 in
 *     m_indices, and masked rows at or past masked_m, hold unspecified values in
 *     every output.
 *   - Sizes and byte offsets are 64-bit inside the library.
 *   - bf16 tensors are raw 16-bit patterns; e4m3 is OCP float8 e4m3fn (bias 7,
 *     max 448); a UE8M0 scale byte s stands for 2^(s-127).
 *   - Activation scale layout ("K-block major"): compact rows use
 *     scale[b * M + r] for row r of M and 128-channel block b; masked rows use
 *     scale[(g * (K/128) + b) * max_m + r] for row r of group g.  Weight scales
 *     are [G][N/128][K/128].
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK 0
#define MOE_EINVAL 1          /* null pointer, negative or inconsistent size */
#define MOE_EUNSUPPORTED 2    /* dtype / alignment the kernels do not cover */
#define MOE_ECAPACITY 3       /* a static buffer is below the required bound */
#define MOE_EDEVICE 4         /* a HIP launch or copy failed */

/* element types */
#define MOE_DTYPE_BF16 0
#define MOE_DTYPE_FP8_E4M3_UE8M0 1
/* GEMM operand dtype: activations as MOE_DTYPE_FP8_E4M3_UE8M0, weights e4m3
 * with MX scales (one UE8M0 exponent per 32 k of a weight row) in the tiled
 * layout of moe_quant_weight_mx. */
#define MOE_DTYPE_FP8_E4M3_MXFP8 2
/* GEMM operand dtype: activations as MOE_DTYPE_FP8_E4M3_UE8M0, weights e2m1
 * [G][N][K/2] (moe_quant_weight_mx with MOE_MX_E2M1) with the same tiled MX
 * scales. */
#define MOE_DTYPE_FP8_MXFP4 3

/* device error word bits (see moe_get_device_error) */
#define MOE_DEVERR_MASKED_OVERFLOW 1  /* an expert received more than max_m rows */

/* ---------------------------------------------------------------------------
 * Host helpers (no device work)
 * ------------------------------------------------------------------------- */

/* Static row bound of the compact layout, P1 key source excerpt of
 * _get_compact_all_tokens: block_e * (min(A, E) + (A - min(A, E)) / block_e)
 * with A = num_assignments and E = num_local_experts.  No routing of A
 * assignments over E experts can need more rows when every non-empty expert is
 * padded to a multiple of block_e.  Returns -1 for negative or zero sizes. */
int64_t moe_compact_rows_bound(int64_t num_assignments, int32_t num_local_experts,
                               int32_t block_e);

/* Layout rule, P1 key source excerpt of _should_use_masked_standard_layout:
 * 1 (masked) when num_experts > num_local_experts and num_local_experts <= 32,
 * else 0 (compact). */
int32_t moe_use_masked_layout(int32_t num_experts, int32_t num_local_experts);

/* Layout policy measured on MI355X in place of the rule above, which the pages
 * leave open ("Support DeepGEMM for standard MoE dispatch", comments section:
 * compact slower than masked up to a crossover in token count).  Timing the
 * whole path in both layouts over 16 .. 16384 tokens (DeepSeek-V3 with 256 and
 * 32 local experts, BF16 with 128 and 8) put the masked layout ahead while the
 * experts hold few rows (up to about 64 per expert on average) and the
 * compact layout level or ahead beyond, while the masked buffers grow as
 * num_local_experts * max_tokens rows.  Returns 1 (masked) when
 *   max_tokens * top_k <= 64 * num_experts            (mean rows per expert)
 *   and num_local_experts * max_tokens <= 4 * moe_compact_rows_bound(
 *       max_tokens * top_k, num_local_experts, block_e)   (memory cap),
 * else 0 (compact); -1 for a zero or negative argument, more local experts
 * than experts, or top_k above num_experts. */
int32_t moe_choose_layout(int64_t max_tokens, int32_t top_k, int32_t num_experts,
                          int32_t num_local_experts, int32_t block_e);

/* Scratch bytes moe_scatter_compact / moe_scatter_masked need for T tokens,
 * top-k, num_local_experts local experts and H hidden channels (per-chunk
 * expert counts, per-expert starts and totals, the assignment of each valid
 * row, and FP8 scale bytes staged per token).  0 on a negative size. */
size_t moe_scatter_ws_bytes(int32_t T, int32_t k, int32_t num_local_experts, int32_t H);

/* Static text for a status code. */
const char* moe_status_str(int32_t status);

/* Copies the device error word kept at the start of a scatter workspace to
 * *host_err after waiting for `stream`; 0 means no data-dependent error was
 * seen by the last scatter call that used this workspace.  Synchronises: this
 * is the one call that blocks the host (it waits for `stream` itself), unlike
 * the enqueue-only contract of every other call, where synchronising is left
 * to the caller. */
int32_t moe_get_device_error(const void* ws, int32_t* host_err, void* stream);

/* ---------------------------------------------------------------------------
 * Routing
 * ------------------------------------------------------------------------- */

/* Top-k routing: softmax over E experts, the k most probable kept and their
 * probabilities renormalised to sum to 1 (the router output the pages feed
 * into dispatch as topk_output; P3 related-PR note keeps the router in fp32).
 *   logits        device fp32 [T][E]
 *   topk_ids      device int32 [T][k], out: slot j holds the j-th most
 *                 probable expert; equal logits go to the lower index.
 *   topk_weights  device fp32 [T][k], out.
 * Limits: 1 <= E <= 1024, 1 <= k <= min(E, 32), T >= 0. */
int32_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                       int32_t* topk_ids, float* topk_weights, void* stream);

/* ---------------------------------------------------------------------------
 * Scatter into the expert layouts
 * ------------------------------------------------------------------------- */

/* Compact ("contiguous") layout, P1 implementation breakdown items 2-4 and the
 * key source excerpt of _fwd_kernel_ep_scatter_1.  Assignment (t, j) is local
 * when e = topk_ids[t][j] - expert_start lies in [0, num_local_experts)
 * (P3 implementation breakdown item 1).  Local rows are grouped by expert e in
 * increasing e; inside an expert they follow increasing (t, j).  Each
 * non-empty expert is padded to a multiple of block_e rows.
 *   x                 device bf16 [T][H]
 *   rows_capacity     rows of every per-row output; must be at least
 *                     moe_compact_rows_bound(T*k, num_local_experts, block_e)
 *                     (else MOE_ECAPACITY)
 *   out_dtype         MOE_DTYPE_BF16: x_out bf16 [rows_capacity][H] copies;
 *                     MOE_DTYPE_FP8_E4M3_UE8M0: x_out e4m3 [rows_capacity][H]
 *                     with scale_out [H/128][rows_capacity] (the token's own
 *                     per-128-channel UE8M0 quantisation, see
 *                     moe_quant_fp8_ue8m0)
 *   m_indices         device int32 [rows_capacity], out: e on valid rows, -1 on
 *                     padding rows and on every row past the last expert block
 *   expert_start_loc  device int32 [num_local_experts], out: first row of e
 *   num_valid         device int32 [num_local_experts], out: rows of e
 *   src2dst           device int32 [T][k], out: row of (t, j), -1 if not local
 *   ws, ws_bytes      scratch, at least moe_scatter_ws_bytes(T, k, El, H)
 * Limits: H % 128 == 0, block_e a positive multiple of 128 (the grouped GEMM
 * tiles never straddle experts), 1 <= num_local_experts <= 1024,
 * rows_capacity < 2^31. */
int32_t moe_scatter_compact(const void* x, int32_t T, int32_t H, const int32_t* topk_ids,
                            int32_t k, int32_t expert_start, int32_t num_local_experts,
                            int32_t block_e, int64_t rows_capacity, int32_t out_dtype,
                            void* x_out, uint8_t* scale_out, int32_t* m_indices,
                            int32_t* expert_start_loc, int32_t* num_valid, int32_t* src2dst,
                            void* ws, size_t ws_bytes, void* stream);

/* Largest scratch (bytes, as moe_scatter_ws_bytes counts it) that
 * moe_scatter_compact_noalloc serves: 4 MiB, e.g. T = 32768 tokens, top-8,
 * H = 7168 with 256 local experts (about 3.75 MiB). */
#define MOE_SCATTER_NOALLOC_MAX_BYTES (4u << 20)

/* moe_scatter_compact without the ws/ws_bytes arguments, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, outputs, limits
 * and status codes as moe_scatter_compact; the scratch is a static device
 * array of MOE_SCATTER_NOALLOC_MAX_BYTES per device, held until the process
 * ends.  The call allocates nothing.
 *   Returns MOE_ECAPACITY when moe_scatter_ws_bytes(T, k, num_local_experts, H)
 *   exceeds MOE_SCATTER_NOALLOC_MAX_BYTES, and MOE_EDEVICE when the scratch's
 *   device address cannot be obtained.
 * Every call on one device shares that device's scratch: calls that may run
 * at the same time on one device (different streams without ordering, other
 * threads) race and give undefined results; calls in one stream are fine.
 * The compact scatter sets no device error bits, so there is no error word to
 * read back. */
int32_t moe_scatter_compact_noalloc(const void* x, int32_t T, int32_t H, const int32_t* topk_ids,
                                    int32_t k, int32_t expert_start, int32_t num_local_experts,
                                    int32_t block_e, int64_t rows_capacity, int32_t out_dtype,
                                    void* x_out, uint8_t* scale_out, int32_t* m_indices,
                                    int32_t* expert_start_loc, int32_t* num_valid,
                                    int32_t* src2dst, void* stream);

/* Masked layout, P1 implementation breakdown item 2 (masked branch) and P2 key
 * source excerpt of _BF16GroupedMaskedWarmupExecutor: expert e's rows are
 * x_out[e][0 .. masked_m[e]) in increasing (t, j); src2dst holds the flat row
 * e*max_m + rank so moe_combine serves both layouts.
 *   x_out      [num_local_experts][max_m][H] bf16 or e4m3
 *   scale_out  FP8 only: [num_local_experts][H/128][max_m]
 *   masked_m   device int32 [num_local_experts], out
 * max_m must be >= T (a token contributes at most one row per expert when its
 * k ids are distinct), else MOE_ECAPACITY.  Repeated ids inside one token that
 * push an expert past max_m set MOE_DEVERR_MASKED_OVERFLOW in the device error
 * word; the overflowing rows are dropped (src2dst = -1) and masked_m is
 * clamped to max_m. */
int32_t moe_scatter_masked(const void* x, int32_t T, int32_t H, const int32_t* topk_ids,
                           int32_t k, int32_t expert_start, int32_t num_local_experts,
                           int32_t max_m, int32_t out_dtype, void* x_out, uint8_t* scale_out,
                           int32_t* masked_m, int32_t* src2dst, void* ws, size_t ws_bytes,
                           void* stream);

/* ---------------------------------------------------------------------------
 * Quantisation
 * ------------------------------------------------------------------------- */

/* Per-token, per-128-channel FP8 e4m3 with UE8M0 scales computed directly
 * (P1 implementation breakdown item 3; P3 key source excerpt of the dispatch
 * path calling per-token-group quantisation with ue8m0): for each group the
 * exponent e is the smallest integer in [-126, 127] with amax <= 448 * 2^e, then
 * each value is x * 2^-e rounded to nearest-even e4m3.
 *   x          device bf16, row r at x + r*ld_x (elements)
 *   m_indices  optional device int32 [M]; rows with a negative entry are skipped
 *   q          device e4m3 [M][K]
 *   scale      device u8 [K/128][M]
 * Limits: K % 128 == 0, ld_x >= K. */
int32_t moe_quant_fp8_ue8m0(const void* x, int64_t M, int32_t K, int64_t ld_x,
                            const int32_t* m_indices, uint8_t* q, uint8_t* scale,
                            void* stream);

/* Expert weights to 128x128 block-scaled e4m3 with UE8M0 block scales (the same
 * rule over each block; P1 implementation breakdown item 1 expresses both w13
 * and w2 with power-of-two block scales).
 *   w      device bf16 [G][N][K];  q  device e4m3 [G][N][K]
 *   scale  device u8 [G][N/128][K/128]
 * Limits: N % 128 == 0, K % 128 == 0. */
int32_t moe_quant_weight_fp8_ue8m0(const void* w, int32_t G, int32_t N, int32_t K,
                                   uint8_t* q, uint8_t* scale, void* stream);

/* MX expert weights (OCP microscaling: every 32 consecutive k of a weight row
 * share one power-of-two scale), the weight format the pages flag as not yet
 * covered ("Support DeepGEMM for standard MoE dispatch", comments section on
 * FP4 and MX weights).  The exponent follows the pages' direct UE8M0 rule
 * (implementation breakdown item 3) over each 32-value block: the smallest e in
 * [-126, 127] with max|w| <= fmax * 2^e, fmax = 448 (e4m3) or 6 (e2m1); each
 * value w * 2^-e is then rounded to nearest, ties to even.
 *   w            device bf16 [G][N][K]
 *   fmt          MOE_MX_E4M3: q e4m3 [G][N][K];
 *                MOE_MX_E2M1: q e2m1 [G][N][K/2], two codes per byte, even k in
 *                the low nibble (OCP FP4: sign, 2 exponent bits with bias 1,
 *                1 mantissa bit)
 *   scale_tiled  device u8 exponents + 127, tiled for the GEMM:
 *                [G][N/64][K/128][4][16][4], the byte of (row n, 32-block b) at
 *                ((g*(N/64) + n/64)*(K/128) + b/4)*256 + (b%4)*64 + (n%16)*4 + (n%64)/16
 * Limits: N % 64 == 0, K % 128 == 0.  Non-finite weights: unspecified codes. */
#define MOE_MX_E4M3 0
#define MOE_MX_E2M1 1
int32_t moe_quant_weight_mx(const void* w, int32_t G, int32_t N, int32_t K, int32_t fmt,
                            uint8_t* q, uint8_t* scale_tiled, void* stream);
/* Plain MX scales [G][N][K/32] (one byte per row and 32-block, as a checkpoint
 * stores them) -> the tiled layout above. */
int32_t moe_mx_scales_tile(const uint8_t* scale_plain, int32_t G, int32_t N, int32_t K,
                           uint8_t* scale_tiled, void* stream);

/* Requantise block-FP8 expert weights (a checkpoint's e4m3 codes with one
 * fp32 scale per 128x128 block) to the UE8M0 block format, through a bf16
 * intermediate ("Support DeepGEMM for standard MoE dispatch", implementation
 * breakdown item 1: both w13 and w2 of the standard layer are requantised with
 * bf16 as the output dtype): w = bf16(decode(q) * s) in fp32, then exactly
 * moe_quant_weight_fp8_ue8m0 of w.
 *   q_in   device e4m3 [G][N][K];  s_in  device fp32 [G][N/128][K/128]
 *   q_out  device e4m3 [G][N][K] (may be q_in);  s_out  device u8 [G][N/128][K/128]
 *   Non-finite codes or products give unspecified results.
 * Limits: N % 128 == 0, K % 128 == 0. */
int32_t moe_requant_weight_fp8_ue8m0(const uint8_t* q_in, const float* s_in, int32_t G, int32_t N,
                                     int32_t K, uint8_t* q_out, uint8_t* s_out, void* stream);

/* Rows on which a grouped GEMM call runs its MFMAs (whole 16-row blocks of
 * its tiles, padding included), for throughput accounting: the tile choice of
 * grouped_gemm_masked(_silu) with this expected_m (masked != 0), or of
 * grouped_gemm_contig(_silu) on a layout with M rows in which each of the G
 * experts is one run of counts[g] valid rows (what moe_scatter_compact
 * writes).  counts: host int32 [G].  N is the GEMM's output width (2I for
 * the SiLU variants).  Returns -1 on a null pointer or negative size. */
int64_t grouped_gemm_rows_executed(int32_t dtype, int32_t masked, const int32_t* counts, int32_t G,
                                   int32_t expected_m, int64_t M, int32_t N, int32_t K);

/* ---------------------------------------------------------------------------
 * Grouped GEMMs ("NT": C = A . B[g]^T), fp32 accumulation, bf16 output
 * ------------------------------------------------------------------------- */

/* Contiguous layout, P2 key source excerpts of _BF16GroupedContWarmupExecutor
 * and _run_bf16_contiguous_gemm: C[r, :] = A[r, :] . B[m_indices[r]]^T.
 *   dtype     MOE_DTYPE_BF16 (A bf16 [M][K], B bf16 [G][N][K]; scales NULL),
 *             MOE_DTYPE_FP8_E4M3_UE8M0 (A e4m3 [M][K] with A_scale [K/128][M],
 *             B e4m3 [G][N][K] with B_scale [G][N/128][K/128]) or
 *             MOE_DTYPE_FP8_E4M3_MXFP8 (A as before, B e4m3 [G][N][K] with MX
 *             B_scale tiled as moe_quant_weight_mx writes it) or
 *             MOE_DTYPE_FP8_MXFP4 (A as before, B e2m1 [G][N][K/2], MX scales)
 *   C         device bf16 [M][N].  Rows of an aligned 128-row block whose
 *             first row is -1 are not written; other rows with m_indices < 0
 *             (the padding at the end of an expert) receive unspecified values.
 *   m_indices device int32 [M]; layout contract: every aligned 128-row block
 *             holds one expert id on its valid rows, valid rows come first
 *             (what moe_scatter_compact produces with block_e % 128 == 0)
 * Limits: N % 128 == 0, K % 128 == 0, K <= 4194304, 0 <= m_indices < G,
 * ceil(M / 128) <= 8176 (about one million rows) -> else MOE_EUNSUPPORTED.
 * FP8 without scales -> MOE_EUNSUPPORTED (the dtype follows the weights and a
 * contradiction is an error, P3 implementation breakdown item 2). */
int32_t grouped_gemm_contig(int32_t dtype, const void* A, const uint8_t* A_scale,
                            const void* B, const uint8_t* B_scale, void* C,
                            const int32_t* m_indices, int64_t M, int32_t N, int32_t K,
                            int32_t G, void* stream);

/* Masked layout, P2 key source excerpt of _BF16GroupedMaskedWarmupExecutor:
 * C[g, r, :] = A[g, r, :] . B[g]^T for r < masked_m[g].
 *   A [G][max_m][K], C [G][max_m][N]; FP8 A_scale [G][K/128][max_m].
 *   expected_m  a hint of typical masked_m (sizes tiles: 16 or 32 rows when
 *               1 <= expected_m <= 16 or <= 32 and N % 256 == 0, 64 rows when
 *               1 <= expected_m <= 64, else 128); it never changes a result.
 *               0 = no hint.
 *   Rows at or past masked_m[g] receive unspecified values, except that rows
 *   at or past masked_m[g] rounded up to 128 are never written.
 * Limits: N, K as grouped_gemm_contig; G <= 1024; the tile count, at most
 * G * ceil(max_m / 64) * N / 128, below 2^31 -> else MOE_EUNSUPPORTED. */
int32_t grouped_gemm_masked(int32_t dtype, const void* A, const uint8_t* A_scale,
                            const void* B, const uint8_t* B_scale, void* C,
                            const int32_t* masked_m, int32_t expected_m, int32_t max_m,
                            int32_t N, int32_t K, int32_t G, void* stream);

/* The w13 GEMM with SiLU-and-mul in its epilogue (the two steps of P2 key
 * source excerpt _run_bf16_contiguous_gemm, w13 then silu_and_mul, in one
 * pass): B is w13 [G][2I][K] (gate rows [0, I), up rows [I, 2I)) and the
 * result is the activation act[r][i] = silu(C[r][i]) * C[r][I + i] with
 * C = A . B[g]^T rounded to bf16 first, exactly as grouped_gemm_* followed by
 * silu_and_mul computes it (bit for bit).
 *   out_dtype  MOE_DTYPE_BF16: out bf16 [rows][I];
 *              MOE_DTYPE_FP8_E4M3_UE8M0: out e4m3 [rows][I] with out_scale
 *              laid out as silu_and_mul's (compact [I/128][M], masked
 *              [G][I/128][max_m]).
 *   Rows follow the underlying GEMM: rows of blocks whose first row is -1
 *   (compact) or at or past masked_m rounded up to 128 (masked) are not
 *   written; other rows past an expert's valid rows receive unspecified values.
 * Limits: I % 128 == 0, (I + 256) * K * 2 < 2^32; the rest as the underlying
 * GEMM. */
int32_t grouped_gemm_contig_silu(int32_t dtype, const void* A, const uint8_t* A_scale,
                                 const void* B, const uint8_t* B_scale, int32_t out_dtype,
                                 void* out, uint8_t* out_scale, const int32_t* m_indices,
                                 int64_t M, int32_t I, int32_t K, int32_t G, void* stream);
int32_t grouped_gemm_masked_silu(int32_t dtype, const void* A, const uint8_t* A_scale,
                                 const void* B, const uint8_t* B_scale, int32_t out_dtype,
                                 void* out, uint8_t* out_scale, const int32_t* masked_m,
                                 int32_t expected_m, int32_t max_m, int32_t I, int32_t K,
                                 int32_t G, void* stream);

/* ---------------------------------------------------------------------------
 * Activation and combine
 * ------------------------------------------------------------------------- */

/* SiLU-and-mul, P2 key source excerpt of _run_bf16_contiguous_gemm (the w13
 * output [M][2I] is halved): out[r][i] = silu(gateup[r][i]) * gateup[r][I+i],
 * computed in fp32 (silu(g) = g * 1/(1 + 2^(-g log2 e)) with the hardware
 * exp2 and reciprocal, each within about one fp32 ulp) and rounded to bf16;
 * for FP8 output that bf16 row is then quantised as moe_quant_fp8_ue8m0 does.
 *   Row selection: m_indices (compact; rows with -1 skipped) or masked_m with
 *   max_m (masked; M = G*max_m, rows r % max_m >= masked_m[r / max_m] skipped);
 *   both NULL = every row.
 *   out_scale  FP8 only: compact [I/128][M], masked [G][I/128][max_m].
 * Limits: I % 128 == 0. */
int32_t silu_and_mul(const void* gateup, int64_t M, int32_t I, const int32_t* m_indices,
                     const int32_t* masked_m, int32_t max_m, int32_t out_dtype, void* out,
                     uint8_t* out_scale, void* stream);

/* Weighted combine back to token order (P1 risks item 2: the post-permute
 * reads src2dst; P3 review notes: combine follows per-slot pointers):
 * out[t][h] = sum over j = 0..k-1 with src2dst[t][j] >= 0 of
 * topk_weights[t][j] * Y[src2dst[t][j]][h], each product and partial sum
 * rounded to fp32 in slot order, then one rounding to bf16; tokens with no
 * local slot get 0.
 *   Y bf16 [num_rows][H]; out bf16 [T][H].  A src2dst entry >= num_rows is
 *   treated as -1 (never read).  Limits: H % 8 == 0, 1 <= k <= 32. */
int32_t moe_combine(const void* Y, int64_t num_rows, const int32_t* src2dst,
                    const float* topk_weights, int32_t T, int32_t k, int32_t H, void* out,
                    void* stream);


#ifdef __cplusplus
}
#endif
#endif
