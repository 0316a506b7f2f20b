/*
 * CPU oracle for the routed-token scatter -> grouped GEMM MoE expert path.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h).  Plain scalar C: every loop is
 * written in the order the definition states, floating point is evaluated
 * without contraction (built with -ffp-contract=off, no fast-math), and the
 * only parallelism is OpenMP over independent output rows or tokens, so the
 * results do not depend on the thread count.
 *
 * Numerics, per step:
 *   routing      softmax in fp64, top-k by probability (ties -> lower expert
 *                index), renormalised over the k chosen in fp64, rounded to fp32.
 *   quant        UE8M0 exponent = smallest e in [-126,127] with amax <= 448*2^e,
 *                then e4m3fn round-to-nearest-even of x*2^-e (exact in fp64).
 *   GEMM         fp32 products (exact for bf16*bf16 and e4m3*e4m3), summed in
 *                fp32 in increasing k; FP8 sums each 128-wide k block in fp32,
 *                scales it by 2^(eA+eB) and adds the blocks in increasing order;
 *                bf16 round-to-nearest-even at the end.
 *   SiLU-mul     fp64 from bf16 inputs, one bf16 rounding.
 *   combine      fp32 product w*y, fp32 sum over slots j = 0..k-1, one bf16
 *                rounding.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* number formats                                                            */
/* ------------------------------------------------------------------------ */

float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round a double to the nearest bf16 (8 significant bits, ties to even), in one
 * step, so no double rounding through fp32 can occur. */
uint16_t orc_f64_to_bf16(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  if (isnan(v)) return (uint16_t)(sign | 0x7FC0);
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80);
  int E;
  double m = frexp(a, &E); /* a = m * 2^E, m in [0.5, 1) */
  double q;
  int p;
  if (E - 1 >= -126) { /* normal: 8 significant bits */
    q = nearbyint(ldexp(m, 8));
    p = E - 8;
  } else { /* subnormal: spacing 2^-133 */
    q = nearbyint(ldexp(a, 133));
    p = -133;
  }
  double r = ldexp(q, p);
  if (r >= 0x1p128) return (uint16_t)(sign | 0x7F80);
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

/* OCP e4m3fn: bias 7, 3 mantissa bits, subnormals m*2^-9, max 448,
 * S.1111.111 = NaN. */
double orc_e4m3_to_f64(uint8_t q) {
  int s = q >> 7, ef = (q >> 3) & 15, mf = q & 7;
  double v;
  if (ef == 15 && mf == 7) return NAN;
  if (ef == 0)
    v = ldexp((double)mf, -9);
  else
    v = ldexp((double)(8 + mf), ef - 7 - 3);
  return s ? -v : v;
}

/* Round an exactly-held value to e4m3fn, ties to even; beyond the largest
 * finite value it saturates to +-448.  The sign of zero is kept. */
uint8_t orc_e4m3_from_f64(double v) {
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (isinf(a)) return (uint8_t)(sign | 0x7E);
  if (a < 0x1p-6) { /* subnormal range, spacing 2^-9; 8*2^-9 is the min normal */
    double q = nearbyint(ldexp(a, 9));
    return (uint8_t)(sign | (uint8_t)q);
  }
  int E;
  double m = frexp(a, &E); /* a = (2m) * 2^(E-1), 2m in [1,2) */
  int p = E - 1;
  double q = nearbyint(ldexp(m, 4)); /* (2m)*8 rounded: 8..16 */
  if (q == 16.0) {
    q = 8.0;
    p += 1;
  }
  if (p > 8 || (p == 8 && q > 14.0)) return (uint8_t)(sign | 0x7E);
  return (uint8_t)(sign | (uint8_t)(((p + 7) << 3) | ((int)q - 8)));
}

/* UE8M0: the smallest power of two 2^e that lets the group's largest magnitude
 * fit the e4m3 range (amax <= 448 * 2^e), with e kept inside [-126, 127] so the
 * factor is a normal fp32 number.  The scale is chosen before any value is
 * quantised (P1, implementation breakdown item 3: quantise with UE8M0 scales
 * directly instead of rounding a scale afterwards). */
int32_t orc_ue8m0_exponent(double amax) {
  int32_t e = -126;
  while (e < 127 && amax > ldexp(448.0, e)) ++e;
  return e;
}

/* ------------------------------------------------------------------------ */
/* host rules                                                                */
/* ------------------------------------------------------------------------ */

/* P1 key source excerpt of _get_compact_all_tokens: each non-empty expert takes
 * at least one block_e block and the remaining assignments fill further whole
 * blocks. */
int64_t orc_compact_rows_bound(int64_t num_assignments, int32_t num_experts, int32_t block_e) {
  int64_t n = num_assignments < (int64_t)num_experts ? num_assignments : (int64_t)num_experts;
  return (int64_t)block_e * (n + (num_assignments - n) / block_e);
}

/* P1 key source excerpt of _should_use_masked_standard_layout. */
int32_t orc_use_masked_layout(int32_t num_experts, int32_t num_local_experts) {
  return (num_experts > num_local_experts && num_local_experts <= 32) ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* routing                                                                   */
/* ------------------------------------------------------------------------ */

void orc_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                    int32_t* topk_ids, float* topk_weights) {
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
      const float* L = logits + (int64_t)t * E;
      /* softmax over all E experts */
      double mx = -INFINITY;
      for (int32_t e = 0; e < E; ++e)
        if ((double)L[e] > mx) mx = (double)L[e];
      double den = 0.0;
      for (int32_t e = 0; e < E; ++e) {
        p[e] = exp((double)L[e] - mx);
        den += p[e];
      }
      for (int32_t e = 0; e < E; ++e) p[e] /= den;
      /* top-k by probability, ties -> lower expert index */
      memset(taken, 0, (size_t)E);
      double sel = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e)
          if (!taken[e] && (best < 0 || p[e] > p[best])) best = e;
        taken[best] = 1;
        topk_ids[(int64_t)t * k + j] = best;
        sel += p[best];
      }
      /* renormalise over the chosen k */
      for (int32_t j = 0; j < k; ++j)
        topk_weights[(int64_t)t * k + j] = (float)(p[topk_ids[(int64_t)t * k + j]] / sel);
    }
    free(p);
    free(taken);
  }
}

/* ------------------------------------------------------------------------ */
/* quantisation                                                              */
/* ------------------------------------------------------------------------ */

static void quant_row(const uint16_t* x, int32_t K, uint8_t* q, uint8_t* s) {
  for (int32_t b = 0; b < K / 128; ++b) {
    double amax = 0.0;
    for (int32_t i = 0; i < 128; ++i) {
      double a = fabs((double)orc_bf16_to_f32(x[b * 128 + i]));
      if (a > amax) amax = a;
    }
    int32_t e = orc_ue8m0_exponent(amax);
    s[b] = (uint8_t)(e + 127);
    for (int32_t i = 0; i < 128; ++i)
      q[b * 128 + i] = orc_e4m3_from_f64(ldexp((double)orc_bf16_to_f32(x[b * 128 + i]), -e));
  }
}

void orc_quant_rows(const uint16_t* x, int64_t M, int32_t K, int64_t ld_x,
                    uint8_t* q, uint8_t* scale_rowmajor) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < M; ++r)
    quant_row(x + r * ld_x, K, q + r * K, scale_rowmajor + r * (K / 128));
}

void orc_quant_weight_blocks(const uint16_t* w, int32_t G, int32_t N, int32_t K,
                             uint8_t* q, uint8_t* scale) {
  int32_t nb = N / 128, kb = K / 128;
#pragma omp parallel for collapse(3) schedule(static)
  for (int32_t g = 0; g < G; ++g)
    for (int32_t bn = 0; bn < nb; ++bn)
      for (int32_t bk = 0; bk < kb; ++bk) {
        const uint16_t* wg = w + (int64_t)g * N * K;
        uint8_t* qg = q + (int64_t)g * N * K;
        double amax = 0.0;
        for (int32_t n = bn * 128; n < bn * 128 + 128; ++n)
          for (int32_t kk = bk * 128; kk < bk * 128 + 128; ++kk) {
            double a = fabs((double)orc_bf16_to_f32(wg[(int64_t)n * K + kk]));
            if (a > amax) amax = a;
          }
        int32_t e = orc_ue8m0_exponent(amax);
        scale[((int64_t)g * nb + bn) * kb + bk] = (uint8_t)(e + 127);
        for (int32_t n = bn * 128; n < bn * 128 + 128; ++n)
          for (int32_t kk = bk * 128; kk < bk * 128 + 128; ++kk)
            qg[(int64_t)n * K + kk] =
                orc_e4m3_from_f64(ldexp((double)orc_bf16_to_f32(wg[(int64_t)n * K + kk]), -e));
      }
}

/* P1 implementation breakdown item 1 (the standard MoE layer requantises both
 * expert weight sets, w13 and w2, to UE8M0 block scales, with a bf16 output
 * dtype): each element of a block-FP8 checkpoint is dequantised as
 * decode(q) * s in fp32 (one fp32 rounding, as a tensor multiply in that
 * dtype does) and rounded to bf16; the bf16 weights then take the same direct
 * UE8M0 128x128 block quantisation as orc_quant_weight_blocks. */
void orc_requant_weight_blocks(const uint8_t* q_in, const float* s_in, int32_t G, int32_t N,
                               int32_t K, uint8_t* q_out, uint8_t* s_out) {
  int32_t nb = N / 128, kb = K / 128;
  int64_t n_el = (int64_t)G * N * K;
  uint16_t* w = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n_el > 0 ? n_el : 1));
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_el; ++i) {
    int64_t g = i / ((int64_t)N * K);
    int64_t n = (i / K) % N, k = i % K;
    float s = s_in[(g * nb + n / 128) * kb + k / 128];
    float v = (float)orc_e4m3_to_f64(q_in[i]) * s;  /* fp32 product */
    w[i] = orc_f64_to_bf16((double)v);
  }
  orc_quant_weight_blocks(w, G, N, K, q_out, s_out);
  free(w);
}

/* ------------------------------------------------------------------------ */
/* MX expert weights (microscaling: one power-of-two scale per 32 values)     */
/* ------------------------------------------------------------------------ */

/* OCP microscaling FP4 element, e2m1: sign bit 3, two exponent bits (bias 1),
 * one mantissa bit; exponent field 0 holds 0 and 0.5, otherwise the value is
 * 2^(E-1) * (1 + M/2).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no inf or NaN. */
double orc_e2m1_to_f64(uint8_t q) {
  int s = (q >> 3) & 1, ef = (q >> 1) & 3, mf = q & 1;
  double v = ef == 0 ? 0.5 * mf : ldexp(1.0 + 0.5 * mf, ef - 1);
  return s ? -v : v;
}

/* Nearest e2m1 value of an exactly-held v, ties to the even code (mantissa bit
 * 0), saturating at +-6; the sign of zero is kept.  A plain search over the
 * eight magnitudes. */
uint8_t orc_e2m1_from_f64(double v) {
  uint8_t sign = signbit(v) ? 8 : 0;
  double a = fabs(v);
  if (!(a < 6.0)) return (uint8_t)(sign | 7);
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c < 8; ++c) {
    double d = fabs(orc_e2m1_to_f64((uint8_t)c) - a);
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return (uint8_t)(sign | best);
}

/* The UE8M0 rule of orc_ue8m0_exponent for an element format whose largest
 * magnitude is fmax: the smallest e in [-126, 127] with amax <= fmax * 2^e. */
int32_t orc_mx_exponent(double amax, double fmax) {
  int32_t e = -126;
  while (e < 127 && amax > ldexp(fmax, e)) ++e;
  return e;
}

/* MX weights: every 32 consecutive k of one row of w[G][N][K] share the
 * exponent chosen directly from their largest magnitude, then each value is
 * rounded to the element format.  fmt 0: e4m3 codes q[G][N][K]; fmt 1: e2m1
 * codes two per byte, q[G][N][K/2], even k in the low nibble.  Scale bytes
 * s[G][N][K/32] hold e + 127. */
void orc_quant_weight_mx(const uint16_t* w, int32_t G, int32_t N, int32_t K, int32_t fmt,
                         uint8_t* q, uint8_t* s) {
  int32_t kb = K / 32;
  double fmax = fmt == 0 ? 448.0 : 6.0;
#pragma omp parallel for collapse(2) schedule(static)
  for (int32_t g = 0; g < G; ++g)
    for (int32_t n = 0; n < N; ++n) {
      const uint16_t* row = w + ((int64_t)g * N + n) * K;
      for (int32_t b = 0; b < kb; ++b) {
        double amax = 0.0;
        for (int32_t i = 0; i < 32; ++i) {
          double a = fabs((double)orc_bf16_to_f32(row[b * 32 + i]));
          if (a > amax) amax = a;
        }
        int32_t e = orc_mx_exponent(amax, fmax);
        s[((int64_t)g * N + n) * kb + b] = (uint8_t)(e + 127);
        for (int32_t i = 0; i < 32; ++i) {
          int32_t kk = b * 32 + i;
          double v = ldexp((double)orc_bf16_to_f32(row[kk]), -e);
          if (fmt == 0) {
            q[((int64_t)g * N + n) * K + kk] = orc_e4m3_from_f64(v);
          } else {
            uint8_t c = orc_e2m1_from_f64(v);
            uint8_t* byte = q + ((int64_t)g * N + n) * (K / 2) + kk / 2;
            *byte = (kk & 1) ? (uint8_t)((*byte & 0x0F) | (c << 4)) : (uint8_t)((*byte & 0xF0) | c);
          }
        }
      }
    }
}

/* ------------------------------------------------------------------------ */
/* scatter                                                                   */
/* ------------------------------------------------------------------------ */

/* local expert of an id, or -1 when the id is outside this share (P3,
 * implementation breakdown item 1: expert ids are rebased by expert_start and
 * only num_experts local experts are kept). */
static int32_t local_of(int32_t id, int32_t expert_start, int32_t num_local) {
  int32_t e = id - expert_start;
  return (e >= 0 && e < num_local) ? e : -1;
}

static void put_row(const uint16_t* xt, int32_t H, int32_t fp8, void* x_out,
                    uint8_t* scale_out, int64_t row) {
  if (!x_out) return; /* index-only call */
  if (fp8) {
    quant_row(xt, H, (uint8_t*)x_out + row * H, scale_out + row * (H / 128));
  } else {
    memcpy((uint16_t*)x_out + row * H, xt, sizeof(uint16_t) * (size_t)H);
  }
}

/* P1 implementation breakdown items 2-4 and the key source excerpt of
 * _fwd_kernel_ep_scatter_1: rows grouped by expert, each non-empty expert padded
 * to a multiple of block_e, m_indices = expert id on valid rows and -1 on padding.
 * Row order inside an expert: ascending (token, slot).  Rows past the last
 * expert block are also marked -1 so a fixed-size buffer is fully described. */
int32_t orc_scatter_compact(const uint16_t* x, int32_t T, int32_t H,
                            const int32_t* topk_ids, int32_t k,
                            int32_t expert_start, int32_t num_local_experts,
                            int32_t block_e, int64_t rows_capacity, int32_t fp8,
                            void* x_out, uint8_t* scale_out, int32_t* m_indices,
                            int32_t* expert_start_loc, int32_t* num_valid,
                            int32_t* src2dst) {
  int32_t El = num_local_experts;
  int64_t* cnt = (int64_t*)calloc((size_t)El, sizeof(int64_t));
  int64_t* start = (int64_t*)calloc((size_t)El, sizeof(int64_t));
  int64_t* cur = (int64_t*)calloc((size_t)El, sizeof(int64_t));
  for (int64_t a = 0; a < (int64_t)T * k; ++a) {
    int32_t e = local_of(topk_ids[a], expert_start, El);
    if (e >= 0) cnt[e]++;
  }
  int64_t total = 0;
  for (int32_t e = 0; e < El; ++e) {
    start[e] = total;
    total += (cnt[e] + block_e - 1) / block_e * block_e;
  }
  if (total > rows_capacity) {
    free(cnt);
    free(start);
    free(cur);
    return 3;
  }
  for (int64_t r = 0; r < rows_capacity; ++r) m_indices[r] = -1;
  for (int32_t e = 0; e < El; ++e) {
    expert_start_loc[e] = (int32_t)start[e];
    num_valid[e] = (int32_t)cnt[e];
    for (int64_t r = start[e]; r < start[e] + cnt[e]; ++r) m_indices[r] = e;
  }
  for (int32_t t = 0; t < T; ++t)
    for (int32_t j = 0; j < k; ++j) {
      int64_t a = (int64_t)t * k + j;
      int32_t e = local_of(topk_ids[a], expert_start, El);
      if (e < 0) {
        src2dst[a] = -1;
        continue;
      }
      int64_t row = start[e] + cur[e]++;
      src2dst[a] = (int32_t)row;
      put_row(x + (int64_t)t * H, H, fp8, x_out, scale_out, row);
    }
  free(cnt);
  free(start);
  free(cur);
  return 0;
}

/* Masked layout: expert e's rows are e*max_m + rank, masked_m[e] = count
 * (P2 key source excerpt of _BF16GroupedMaskedWarmupExecutor: A is
 * [groups, max_m, k] with a masked_m count per group). */
int32_t orc_scatter_masked(const uint16_t* x, int32_t T, int32_t H,
                           const int32_t* topk_ids, int32_t k,
                           int32_t expert_start, int32_t num_local_experts,
                           int32_t max_m, int32_t fp8,
                           void* x_out, uint8_t* scale_out, int32_t* masked_m,
                           int32_t* src2dst) {
  int32_t El = num_local_experts;
  int64_t* cnt = (int64_t*)calloc((size_t)El, sizeof(int64_t));
  for (int64_t a = 0; a < (int64_t)T * k; ++a) {
    int32_t e = local_of(topk_ids[a], expert_start, El);
    if (e >= 0) cnt[e]++;
  }
  for (int32_t e = 0; e < El; ++e)
    if (cnt[e] > max_m) {
      free(cnt);
      return 3;
    }
  for (int32_t e = 0; e < El; ++e) {
    masked_m[e] = (int32_t)cnt[e];
    cnt[e] = 0;
  }
  for (int32_t t = 0; t < T; ++t)
    for (int32_t j = 0; j < k; ++j) {
      int64_t a = (int64_t)t * k + j;
      int32_t e = local_of(topk_ids[a], expert_start, El);
      if (e < 0) {
        src2dst[a] = -1;
        continue;
      }
      int64_t row = (int64_t)e * max_m + cnt[e]++;
      src2dst[a] = (int32_t)row;
      put_row(x + (int64_t)t * H, H, fp8, x_out, scale_out, row);
    }
  free(cnt);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* grouped GEMM, SiLU-and-mul, combine                                       */
/* ------------------------------------------------------------------------ */

/* e4m3 code -> float, filled once from orc_e4m3_to_f64 (every code is exact in
 * fp32); only a faster way to read the same values. */
static float g_e4m3[256];
static int g_e4m3_ready = 0;
static void e4m3_table_init(void) {
  if (g_e4m3_ready) return;
  for (int c = 0; c < 256; ++c) g_e4m3[c] = (float)orc_e4m3_to_f64((uint8_t)c);
  g_e4m3_ready = 1;
}

/* One output row of the NT product: c[n] = sum_k a[k] * b[n][k]. */
static void gemm_row_bf16(const uint16_t* a, const uint16_t* b, int32_t N, int32_t K, uint16_t* c) {
  for (int32_t n = 0; n < N; ++n) {
    const uint16_t* bn = b + (int64_t)n * K;
    float acc = 0.0f;
    for (int32_t kk = 0; kk < K; ++kk) acc += orc_bf16_to_f32(a[kk]) * orc_bf16_to_f32(bn[kk]);
    c[n] = orc_f64_to_bf16((double)acc);
  }
}

/* FP8 row with UE8M0 scales: per 128-wide k block the e4m3 products are summed in
 * fp32, the block sum is scaled by 2^(eA + eB) (exact power of two), and the
 * blocks are accumulated in fp32. */
static void gemm_row_fp8(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                         const uint8_t* bs, int32_t N, int32_t K, uint16_t* c) {
  int32_t kb = K / 128;
  for (int32_t n = 0; n < N; ++n) {
    const uint8_t* bn = b + (int64_t)n * K;
    float acc = 0.0f;
    for (int32_t blk = 0; blk < kb; ++blk) {
      float part = 0.0f;
      for (int32_t kk = blk * 128; kk < blk * 128 + 128; ++kk)
        part += g_e4m3[a[kk]] * g_e4m3[bn[kk]];
      int32_t ea = (int32_t)as[blk] - 127;
      int32_t eb = (int32_t)bs[(int64_t)(n / 128) * kb + blk] - 127;
      acc += (float)ldexp((double)part, ea + eb);
    }
    c[n] = orc_f64_to_bf16((double)acc);
  }
}

void orc_gemm_bf16_rows(const uint16_t* A, int64_t M, const uint16_t* B,
                        int32_t N, int32_t K, const int32_t* row_group, uint16_t* C) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < M; ++r) {
    int32_t g = row_group[r];
    if (g < 0) continue;
    gemm_row_bf16(A + r * K, B + (int64_t)g * N * K, N, K, C + r * N);
  }
}

void orc_gemm_fp8_rows(const uint8_t* A, const uint8_t* A_scale_rowmajor, int64_t M,
                       const uint8_t* B, const uint8_t* B_scale,
                       int32_t N, int32_t K, const int32_t* row_group, uint16_t* C) {
  int32_t kb = K / 128;
  e4m3_table_init();
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < M; ++r) {
    int32_t g = row_group[r];
    if (g < 0) continue;
    gemm_row_fp8(A + r * K, A_scale_rowmajor + r * kb, B + (int64_t)g * N * K,
                 B_scale + (int64_t)g * (N / 128) * kb, N, K, C + r * N);
  }
}

/* FP8 activations (UE8M0 per 128 channels) times MX weights (one exponent per
 * 32 k of a weight row): per 32-wide k block the products are summed in fp32
 * (exact products), scaled by 2^(eA + eB) and the blocks accumulated in fp32
 * in increasing order, as for the 128-block FP8 product. */
void orc_gemm_mx_rows(const uint8_t* A, const uint8_t* A_scale_rowmajor, int64_t M,
                      const uint8_t* B, const uint8_t* B_scale, int32_t fmt,
                      int32_t N, int32_t K, const int32_t* row_group, uint16_t* C) {
  int32_t ka = K / 128, kb = K / 32;
  int64_t brow = fmt == 0 ? K : K / 2;
  e4m3_table_init();
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < M; ++r) {
    int32_t g = row_group[r];
    if (g < 0) continue;
    const uint8_t* a = A + r * K;
    const uint8_t* as = A_scale_rowmajor + r * ka;
    for (int32_t n = 0; n < N; ++n) {
      const uint8_t* bn = B + ((int64_t)g * N + n) * brow;
      const uint8_t* bs = B_scale + ((int64_t)g * N + n) * kb;
      float acc = 0.0f;
      for (int32_t blk = 0; blk < kb; ++blk) {
        float part = 0.0f;
        for (int32_t kk = blk * 32; kk < blk * 32 + 32; ++kk) {
          float bv = fmt == 0 ? g_e4m3[bn[kk]]
                              : (float)orc_e2m1_to_f64((uint8_t)((bn[kk / 2] >> (4 * (kk & 1))) & 15));
          part += g_e4m3[a[kk]] * bv;
        }
        int32_t ea = (int32_t)as[blk / 4] - 127;
        int32_t eb = (int32_t)bs[blk] - 127;
        acc += (float)ldexp((double)part, ea + eb);
      }
      C[r * N + n] = orc_f64_to_bf16((double)acc);
    }
  }
}

/* P2 key source excerpt of _run_bf16_contiguous_gemm: the w13 output of width N
 * is halved by SiLU-and-mul; the first half is the gate, the second the up
 * projection. */
static void silu_row(const uint16_t* gu, int32_t I, uint16_t* out) {
  for (int32_t i = 0; i < I; ++i) {
    double g = (double)orc_bf16_to_f32(gu[i]);
    double u = (double)orc_bf16_to_f32(gu[I + i]);
    out[i] = orc_f64_to_bf16(g / (1.0 + exp(-g)) * u);
  }
}

void orc_silu_and_mul(const uint16_t* gateup, int64_t M, int32_t I,
                      const int32_t* row_group, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < M; ++r) {
    if (row_group[r] < 0) continue;
    silu_row(gateup + r * 2 * I, I, out + r * I);
  }
}

/* P1 risks item 2 (post-permute reads src2dst) and P3 review notes (combine
 * follows per-slot pointers): gather the k expert rows of a token and sum them
 * with the routing weights, slot by slot. */
void orc_combine(const uint16_t* Y, const int32_t* src2dst, const float* w,
                 int32_t T, int32_t k, int32_t H, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t)
    for (int32_t h = 0; h < H; ++h) {
      float acc = 0.0f;
      for (int32_t j = 0; j < k; ++j) {
        int32_t r = src2dst[(int64_t)t * k + j];
        if (r < 0) continue;
        float prod = w[(int64_t)t * k + j] * orc_bf16_to_f32(Y[(int64_t)r * H + h]);
        acc = acc + prod;
      }
      out[(int64_t)t * H + h] = orc_f64_to_bf16((double)acc);
    }
}

/* Layer without any layout: for each token and each local slot, w13 row ->
 * SiLU-and-mul -> (requantise) -> w2 row, then the weighted sum over slots.
 * Intermediates are rounded to bf16 exactly where the layout path stores them,
 * so this equals the scatter/GEMM/combine chain bit for bit. */
void orc_moe_dense(const uint16_t* x, int32_t T, int32_t H, int32_t I,
                   const int32_t* topk_ids, const float* topk_weights, int32_t k,
                   int32_t expert_start, int32_t num_local_experts, int32_t fp8,
                   const uint16_t* w13, const uint16_t* w2,
                   const uint8_t* w13q, const uint8_t* w13s,
                   const uint8_t* w2q, const uint8_t* w2s,
                   uint16_t* out) {
  int32_t N13 = 2 * I;
  e4m3_table_init();
#pragma omp parallel
  {
    uint16_t* h1 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)N13);
    uint16_t* act = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
    uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
    float* acc = (float*)malloc(sizeof(float) * (size_t)H);
    uint8_t* xq = (uint8_t*)malloc((size_t)H);
    uint8_t* xs = (uint8_t*)malloc((size_t)(H / 128));
    uint8_t* aq = (uint8_t*)malloc((size_t)I);
    uint8_t* as = (uint8_t*)malloc((size_t)(I / 128 + 1));
#pragma omp for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
      const uint16_t* xt = x + (int64_t)t * H;
      for (int32_t h = 0; h < H; ++h) acc[h] = 0.0f;
      if (fp8) quant_row(xt, H, xq, xs);
      for (int32_t j = 0; j < k; ++j) {
        int32_t e = local_of(topk_ids[(int64_t)t * k + j], expert_start, num_local_experts);
        if (e < 0) continue;
        if (fp8) {
          gemm_row_fp8(xq, xs, w13q + (int64_t)e * N13 * H,
                       w13s + (int64_t)e * (N13 / 128) * (H / 128), N13, H, h1);
          silu_row(h1, I, act);
          quant_row(act, I, aq, as);
          gemm_row_fp8(aq, as, w2q + (int64_t)e * H * I,
                       w2s + (int64_t)e * (H / 128) * (I / 128), H, I, y);
        } else {
          gemm_row_bf16(xt, w13 + (int64_t)e * N13 * H, N13, H, h1);
          silu_row(h1, I, act);
          gemm_row_bf16(act, w2 + (int64_t)e * H * I, H, I, y);
        }
        float wj = topk_weights[(int64_t)t * k + j];
        for (int32_t h = 0; h < H; ++h) {
          float prod = wj * orc_bf16_to_f32(y[h]);
          acc[h] = acc[h] + prod;
        }
      }
      for (int32_t h = 0; h < H; ++h) out[(int64_t)t * H + h] = orc_f64_to_bf16((double)acc[h]);
    }
    free(h1);
    free(act);
    free(y);
    free(acc);
    free(xq);
    free(xs);
    free(aq);
    free(as);
  }
}
