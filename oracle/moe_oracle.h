/*
 * CPU oracle for the routed-token scatter -> grouped GEMM MoE expert path.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously-correct
 * reference that the HIP path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * Conventions
 *   bf16 values are passed as their raw 16-bit patterns (uint16_t).
 *   e4m3 values are OCP float8 e4m3fn bytes (bias 7, max 448, no inf,
 *   0x7F/0xFF = NaN).
 *   UE8M0 scale bytes hold e + 127 and stand for the factor 2^e.
 *   Activation scales are row-major here: scale[r * (K/128) + b] for row r and
 *   128-channel group b.  Weight scales are [G][N/128][K/128].
 *
 * Sources (the "pages"): three sglang pull-request reports --
 *   P1 "Support DeepGEMM for standard MoE dispatch" (PR #33128),
 *   P2 "Add BF16 support to EP-MoE for DeepGEMM" (PR #17392),
 *   P3 "[Feature] Support BF16 and batch-invariant inference with DeepEP v2"
 *      (PR #38160).
 * Each function below names the section of the page it follows.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Scalar helpers, exported so the tests can pin them. */
float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_f64_to_bf16(double v);
double   orc_e4m3_to_f64(uint8_t q);
uint8_t  orc_e4m3_from_f64(double v);
int32_t  orc_ue8m0_exponent(double amax);

/* P1, key source excerpt of _get_compact_all_tokens. */
int64_t orc_compact_rows_bound(int64_t num_assignments, int32_t num_experts, int32_t block_e);
/* P1, key source excerpt of _should_use_masked_standard_layout. */
int32_t orc_use_masked_layout(int32_t num_experts, int32_t num_local_experts);

/* softmax over E, top-k, renormalised over the k chosen experts. */
void orc_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                    int32_t* topk_ids, float* topk_weights);

/* Per row, per 128 channels: UE8M0 exponent chosen first, then e4m3 codes. */
void orc_quant_rows(const uint16_t* x, int64_t M, int32_t K, int64_t ld_x,
                    uint8_t* q, uint8_t* scale_rowmajor);

/* Same rule over 128x128 blocks of w[G][N][K]. */
void orc_quant_weight_blocks(const uint16_t* w, int32_t G, int32_t N, int32_t K,
                             uint8_t* q, uint8_t* scale);
/* Requantise block-FP8 weights (e4m3 codes, fp32 scale per 128x128 block) to
 * UE8M0 block scales through a bf16 intermediate. */
void orc_requant_weight_blocks(const uint8_t* q_in, const float* s_in, int32_t G, int32_t N,
                               int32_t K, uint8_t* q_out, uint8_t* s_out);

/* MX weights (OCP microscaling: 32 consecutive k of a weight row share one
 * E8M0 exponent, chosen with the UE8M0 rule; element format fmt 0 = e4m3,
 * fmt 1 = e2m1 packed two per byte, even k in the low nibble).  Scales
 * s[G][N][K/32]. */
double   orc_e2m1_to_f64(uint8_t q);
uint8_t  orc_e2m1_from_f64(double v);
int32_t  orc_mx_exponent(double amax, double fmax);
void orc_quant_weight_mx(const uint16_t* w, int32_t G, int32_t N, int32_t K, int32_t fmt,
                         uint8_t* q, uint8_t* s);
/* FP8 rows (UE8M0 per 128) times MX weights, blocks of 32 summed in fp32. */
void orc_gemm_mx_rows(const uint8_t* A, const uint8_t* A_scale_rowmajor, int64_t M,
                      const uint8_t* B, const uint8_t* B_scale, int32_t fmt,
                      int32_t N, int32_t K, const int32_t* row_group, uint16_t* C);

/* Compact layout (P1 implementation breakdown items 2-4). Returns 0, or 3 when
 * rows_capacity is below the rows the routing needs.  fp8 != 0 quantises each
 * scattered row (scale_out row-major [R][H/128]). */
int32_t orc_scatter_compact(const uint16_t* x, int32_t T, int32_t H,
                            const int32_t* topk_ids, int32_t k,
                            int32_t expert_start, int32_t num_local_experts,
                            int32_t block_e, int64_t rows_capacity, int32_t fp8,
                            void* x_out, uint8_t* scale_out, int32_t* m_indices,
                            int32_t* expert_start_loc, int32_t* num_valid,
                            int32_t* src2dst);

/* Masked layout [E_local][max_m][H].  Returns 0, or 3 when an expert would
 * receive more than max_m rows. */
int32_t orc_scatter_masked(const uint16_t* x, int32_t T, int32_t H,
                           const int32_t* topk_ids, int32_t k,
                           int32_t expert_start, int32_t num_local_experts,
                           int32_t max_m, int32_t fp8,
                           void* x_out, uint8_t* scale_out, int32_t* masked_m,
                           int32_t* src2dst);

/* Grouped NT GEMM over rows: C[r,:] = A[r,:] . B[g]^T with g = row_group[r];
 * rows with g < 0 are not computed (C left untouched). */
void orc_gemm_bf16_rows(const uint16_t* A, int64_t M, const uint16_t* B,
                        int32_t N, int32_t K, const int32_t* row_group,
                        uint16_t* C);
void orc_gemm_fp8_rows(const uint8_t* A, const uint8_t* A_scale_rowmajor, int64_t M,
                       const uint8_t* B, const uint8_t* B_scale,
                       int32_t N, int32_t K, const int32_t* row_group,
                       uint16_t* C);

/* act = silu(gate) * up over [M][2I] -> [M][I] bf16; rows with g < 0 skipped. */
void orc_silu_and_mul(const uint16_t* gateup, int64_t M, int32_t I,
                      const int32_t* row_group, uint16_t* out);

/* out[t] = sum_j w[t,j] * Y[src2dst[t,j]]  (slots with src2dst < 0 skipped). */
void orc_combine(const uint16_t* Y, const int32_t* src2dst, const float* w,
                 int32_t T, int32_t k, int32_t H, uint16_t* out);

/* Layout-free MoE expert computation, token by token.  Weights are indexed by
 * local expert id.  fp8 != 0: w13q/w2q are e4m3 with block scales, else
 * w13/w2 bf16.  Tokens whose slots are all non-local get a zero row. */
void orc_moe_dense(const uint16_t* x, int32_t T, int32_t H, int32_t I,
                   const int32_t* topk_ids, const float* topk_weights, int32_t k,
                   int32_t expert_start, int32_t num_local_experts, int32_t fp8,
                   const uint16_t* w13, const uint16_t* w2,
                   const uint8_t* w13q, const uint8_t* w13s,
                   const uint8_t* w2q, const uint8_t* w2s,
                   uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
