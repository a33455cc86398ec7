/*
 * dg_oracle.c -- plain, slow, obviously-correct CPU reference for the FP8
 * fine-grained-scaled NT GEMM family (dense, MoE contiguous, MoE masked,
 * weight gradient, K-grouped weight gradient).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load this file
 * or its shared library: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * What it computes (DeepSeek DeepGEMM 中文讲解, "主要特点" -- FP8 GEMM with
 * fine-grained scaling and two-level accumulation; "使用示例" -- operand
 * tuples (fp8 [M,K], fp32 [M,K/128]) and (fp8 [N,K], fp32 [N/128 rounded up,
 * K/128]), bf16 output; "适用条件" -- K is a multiple of 128):
 *
 *   C[m,n] = bf16( sum_kb sa[m,kb] * sb[n/128,kb] * sum_{k in kb} A[m,k]*B[n,k] )
 *
 * Steps, in the order the definition states them:
 *   1. decode e4m3 (OCP E4M3FN) from its closed form;
 *   2. per 128-wide K block, sum the 128 products in fp64.  Every e4m3 value
 *      is an integer multiple of 2^-9 and |value| <= 448, so every product is
 *      a multiple of 2^-18 and every partial sum is an integer times 2^-18
 *      below 2^43: the fp64 block sum is exact, whatever the order;
 *   3. multiply by sa*sb (exact in fp64: 24+24 significant bits) and add the
 *      blocks in ascending kb order in fp64;
 *   4. round once, fp64 -> bf16 with round-to-nearest-even (fp64 -> fp32 for
 *      the weight-gradient kinds, which add into an existing fp32 D first).
 *
 * The grouped kinds reduce to the dense one row by row (DeepGEMM pages:
 * contiguous layout = every row names its expert, padding rows are -1;
 * masked layout = per-group valid row count masked_m[g]).  Rows that are not
 * computed are left untouched.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC dg_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define BK 128

/* ---- step 1: e4m3 decode ------------------------------------------------ */

/* OCP E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
 * Exponent 0 is subnormal: f/8 * 2^-6.  Exponent 15 with mantissa 7 is NaN;
 * there are no infinities, so the largest finite magnitude is 1.75*2^8 = 448. */
static double e4m3_closed_form(unsigned code) {
  unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, f = code & 7u;
  double mag;
  if (e == 15u && f == 7u) return NAN;
  if (e == 0u)
    mag = ldexp((double)f / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)f / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

static double g_table[256];
static int g_table_ready = 0;

static void table_init(void) {
  if (g_table_ready) return;
  for (unsigned c = 0; c < 256; ++c) g_table[c] = e4m3_closed_form(c);
  g_table_ready = 1;
}

void dgo_e4m3_table(double* out) {
  table_init();
  for (int c = 0; c < 256; ++c) out[c] = g_table[c];
}

/* ---- step 4: rounding ---------------------------------------------------- */

/* fp64 -> bf16 bits, round to nearest, ties to even, in one rounding.
 * bf16 = 8 significant bits, fp32's exponent range (normal >= 2^-126,
 * subnormal quantum 2^-133, largest finite (2-2^-7)*2^127). */
static uint16_t round_bf16(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
  double ax = fabs(x), y;
  if (isinf(x) || ax >= ldexp(2.0 - ldexp(1.0, -8), 127)) {
    y = INFINITY; /* at or beyond the halfway point above the largest finite */
  } else if (ax < ldexp(1.0, -126)) {
    y = nearbyint(ldexp(ax, 133));      /* subnormal: quantum 2^-133 */
    y = ldexp(y, -133);
  } else {
    int e = ilogb(ax);                  /* ax in [2^e, 2^(e+1)) */
    y = nearbyint(ldexp(ax, 7 - e));    /* 8 significant bits */
    y = ldexp(y, e - 7);
  }
  float f = (float)(signbit(x) ? -y : y); /* exact: y has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

void dgo_round_bf16(const double* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = round_bf16(x[i]);
}

/* fp64 -> fp32, round to nearest even (the C conversion under the default mode). */
void dgo_round_f32(const double* x, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = (float)x[i];
}

/* ---- step 2: block sums (exposed for the exactness cross-check) ---------- */

static double block_sum(const uint8_t* arow, const uint8_t* brow, int64_t kb) {
  double p = 0.0;
  for (int64_t k = kb * BK; k < (kb + 1) * BK; ++k) p += g_table[arow[k]] * g_table[brow[k]];
  return p;
}

/* out[(i*n + j)*KB + kb] = fp64 sum of the 128 products of block kb. */
int dgo_block_sums_f64(const uint8_t* a, const uint8_t* b, int64_t m, int64_t n, int64_t k,
                       double* out) {
  if (m < 0 || n < 0 || k <= 0 || k % BK) return -1;
  table_init();
  int64_t KB = k / BK;
  for (int64_t i = 0; i < m; ++i)
    for (int64_t j = 0; j < n; ++j)
      for (int64_t kb = 0; kb < KB; ++kb)
        out[(i * n + j) * KB + kb] = block_sum(a + i * k, b + j * k, kb);
  return 0;
}

/* The same block sums in integers: each e4m3 value times 2^9 is an integer,
 * so products and sums are exact in int64 (result in units of 2^-18).
 * Returns 1 if any operand byte is a NaN code (sum then undefined). */
int dgo_block_sums_i64(const uint8_t* a, const uint8_t* b, int64_t m, int64_t n, int64_t k,
                       int64_t* out) {
  if (m < 0 || n < 0 || k <= 0 || k % BK) return -1;
  int64_t iv[256];
  int nan_seen = 0;
  for (unsigned c = 0; c < 256; ++c) {
    unsigned s = (c >> 7) & 1u, e = (c >> 3) & 15u, f = c & 7u;
    int64_t mag;
    if (e == 15u && f == 7u) { iv[c] = 0; continue; }
    if (e == 0u)
      mag = (int64_t)f;                          /* f/8 * 2^-6 * 2^9 = f */
    else
      mag = (int64_t)(8 + f) << (e - 1);         /* (8+f)/8 * 2^(e-7) * 2^9 */
    iv[c] = s ? -mag : mag;
  }
  int64_t KB = k / BK;
  for (int64_t i = 0; i < m; ++i)
    for (int64_t j = 0; j < n; ++j)
      for (int64_t kb = 0; kb < KB; ++kb) {
        int64_t acc = 0;
        for (int64_t kk = kb * BK; kk < (kb + 1) * BK; ++kk) {
          uint8_t x = a[i * k + kk], y = b[j * k + kk];
          if ((x & 0x7F) == 0x7F || (y & 0x7F) == 0x7F) nan_seen = 1;
          acc += iv[x] * iv[y];
        }
        out[(i * n + j) * KB + kb] = acc;
      }
  return nan_seen;
}

/* ---- steps 2+3: one output element before rounding ----------------------- */

/* sum over blocks kb in [kb0, kb1) of sa_row[kb] * sb_row[kb] * block_sum(kb).
 * sa_row and sb_row are indexed by absolute kb. */
static double element(const uint8_t* arow, const float* sa_row, const uint8_t* brow,
                      const float* sb_row, int64_t kb0, int64_t kb1) {
  double acc = 0.0;
  for (int64_t kb = kb0; kb < kb1; ++kb) {
    double p = block_sum(arow, brow, kb);
    double s = (double)sa_row[kb] * (double)sb_row[kb];
    acc += s * p;
  }
  return acc;
}

/* ---- dense ---------------------------------------------------------------- */

/* C bf16 [m,n] (all written); c_exact (nullable) gets the fp64 value. */
int dgo_gemm_fp8_nt(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                    int64_t m, int64_t n, int64_t k, uint16_t* c, double* c_exact) {
  if (m < 0 || n < 0 || k <= 0 || k % BK) return -1;
  table_init();
  int64_t KB = k / BK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < m; ++i)
    for (int64_t j = 0; j < n; ++j) {
      double v = element(a + i * k, sa + i * KB, b + j * k, sb + (j / BK) * KB, 0, KB);
      if (c_exact) c_exact[i * n + j] = v;
      if (c) c[i * n + j] = round_bf16(v);
    }
  return 0;
}

/* fp64 values of the dense output at `count` (row, col) positions. */
int dgo_gemm_fp8_nt_at(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                       int64_t m, int64_t n, int64_t k, const int64_t* rows,
                       const int64_t* cols, int64_t count, double* out) {
  if (m < 0 || n < 0 || k <= 0 || k % BK) return -1;
  table_init();
  int64_t KB = k / BK;
  for (int64_t t = 0; t < count; ++t)
    if (rows[t] < 0 || rows[t] >= m || cols[t] < 0 || cols[t] >= n) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < count; ++t) {
    int64_t i = rows[t], j = cols[t];
    out[t] = element(a + i * k, sa + i * KB, b + j * k, sb + (j / BK) * KB, 0, KB);
  }
  return 0;
}

/* ---- MoE contiguous --------------------------------------------------------- */

/* A [m_total,k] + sa [m_total,KB]; B [g,n,k] + sb [g,NB,KB]; C bf16 [m_total,n].
 * Row r uses expert e = m_indices[r]; rows with e outside [0,g) are untouched. */
int dgo_grouped_contiguous(const uint8_t* a, const float* sa, const uint8_t* b,
                           const float* sb, const int32_t* m_indices, int64_t m_total,
                           int64_t n, int64_t k, int64_t g, uint16_t* c, double* c_exact) {
  if (m_total < 0 || n < 0 || k <= 0 || k % BK || g <= 0) return -1;
  table_init();
  int64_t KB = k / BK, NB = (n + BK - 1) / BK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < m_total; ++r) {
    int64_t e = m_indices[r];
    if (e < 0 || e >= g) continue;
    for (int64_t j = 0; j < n; ++j) {
      double v = element(a + r * k, sa + r * KB, b + (e * n + j) * k,
                         sb + (e * NB + j / BK) * KB, 0, KB);
      if (c_exact) c_exact[r * n + j] = v;
      if (c) c[r * n + j] = round_bf16(v);
    }
  }
  return 0;
}

/* fp64 values at (row, col); written[t] = 0 where the row is padding. */
int dgo_grouped_contiguous_at(const uint8_t* a, const float* sa, const uint8_t* b,
                              const float* sb, const int32_t* m_indices, int64_t m_total,
                              int64_t n, int64_t k, int64_t g, const int64_t* rows,
                              const int64_t* cols, int64_t count, double* out,
                              int8_t* written) {
  if (m_total < 0 || n < 0 || k <= 0 || k % BK || g <= 0) return -1;
  table_init();
  int64_t KB = k / BK, NB = (n + BK - 1) / BK;
  for (int64_t t = 0; t < count; ++t)
    if (rows[t] < 0 || rows[t] >= m_total || cols[t] < 0 || cols[t] >= n) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < count; ++t) {
    int64_t r = rows[t], j = cols[t], e = m_indices[r];
    if (e < 0 || e >= g) {
      written[t] = 0;
      out[t] = 0.0;
      continue;
    }
    written[t] = 1;
    out[t] = element(a + r * k, sa + r * KB, b + (e * n + j) * k,
                     sb + (e * NB + j / BK) * KB, 0, KB);
  }
  return 0;
}

/* ---- MoE masked ------------------------------------------------------------- */

static int64_t valid_rows(const int32_t* masked_m, int64_t gi, int64_t m_max) {
  int64_t v = masked_m[gi];
  if (v < 0) v = 0;
  if (v > m_max) v = m_max;
  return v;
}

/* A [g,m_max,k] + sa [g,m_max,KB]; B [g,n,k] + sb [g,NB,KB]; C bf16 [g,m_max,n].
 * Only rows r < min(max(masked_m[gi],0), m_max) of group gi are written. */
int dgo_grouped_masked(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                       const int32_t* masked_m, int64_t g, int64_t m_max, int64_t n, int64_t k,
                       uint16_t* c, double* c_exact) {
  if (g <= 0 || m_max < 0 || n < 0 || k <= 0 || k % BK) return -1;
  table_init();
  int64_t KB = k / BK, NB = (n + BK - 1) / BK;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t gi = 0; gi < g; ++gi)
    for (int64_t r = 0; r < m_max; ++r) {
      if (r >= valid_rows(masked_m, gi, m_max)) continue;
      int64_t row = gi * m_max + r;
      for (int64_t j = 0; j < n; ++j) {
        double v = element(a + row * k, sa + row * KB, b + (gi * n + j) * k,
                           sb + (gi * NB + j / BK) * KB, 0, KB);
        if (c_exact) c_exact[row * n + j] = v;
        if (c) c[row * n + j] = round_bf16(v);
      }
    }
  return 0;
}

int dgo_grouped_masked_at(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                          const int32_t* masked_m, int64_t g, int64_t m_max, int64_t n,
                          int64_t k, const int64_t* groups, const int64_t* rows,
                          const int64_t* cols, int64_t count, double* out, int8_t* written) {
  if (g <= 0 || m_max < 0 || n < 0 || k <= 0 || k % BK) return -1;
  table_init();
  int64_t KB = k / BK, NB = (n + BK - 1) / BK;
  for (int64_t t = 0; t < count; ++t)
    if (groups[t] < 0 || groups[t] >= g || rows[t] < 0 || rows[t] >= m_max || cols[t] < 0 ||
        cols[t] >= n)
      return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < count; ++t) {
    int64_t gi = groups[t], r = rows[t], j = cols[t];
    if (r >= valid_rows(masked_m, gi, m_max)) {
      written[t] = 0;
      out[t] = 0.0;
      continue;
    }
    int64_t row = gi * m_max + r;
    written[t] = 1;
    out[t] = element(a + row * k, sa + row * KB, b + (gi * n + j) * k,
                     sb + (gi * NB + j / BK) * KB, 0, KB);
  }
  return 0;
}

/* ---- weight gradient ---------------------------------------------------------- */

/* DeepGEMM pages, "反向传播中的梯度计算": dW from FP8 inputs with an fp32
 * result.  Both operands are scaled per row and per 128 tokens (K = tokens):
 * A [m,k] + sa [m,KB], B [n,k] + sb [n,KB].  D fp32 [m,n] becomes
 * fp32( D + sum_kb sa[i,kb]*sb[j,kb]*block_sum ), with the addition in fp64. */
int dgo_wgrad(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
              int64_t m, int64_t n, int64_t k, float* d, double* d_exact) {
  if (m < 0 || n < 0 || k <= 0 || k % BK) return -1;
  table_init();
  int64_t KB = k / BK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < m; ++i)
    for (int64_t j = 0; j < n; ++j) {
      double v = (double)d[i * n + j] +
                 element(a + i * k, sa + i * KB, b + j * k, sb + j * KB, 0, KB);
      if (d_exact) d_exact[i * n + j] = v;
      d[i * n + j] = (float)v;
    }
  return 0;
}

int dgo_wgrad_at(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                 int64_t m, int64_t n, int64_t k, const float* d0, const int64_t* rows,
                 const int64_t* cols, int64_t count, double* out) {
  if (m < 0 || n < 0 || k <= 0 || k % BK) return -1;
  table_init();
  int64_t KB = k / BK;
  for (int64_t t = 0; t < count; ++t)
    if (rows[t] < 0 || rows[t] >= m || cols[t] < 0 || cols[t] >= n) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < count; ++t) {
    int64_t i = rows[t], j = cols[t];
    double base = d0 ? (double)d0[i * n + j] : 0.0;
    out[t] = base + element(a + i * k, sa + i * KB, b + j * k, sb + j * KB, 0, KB);
  }
  return 0;
}

/* K-grouped weight gradient (DeepGEMM pages, "反向传播中的梯度计算": per-expert
 * gradients in one call).  Tokens of all groups are concatenated along K:
 * group gi owns tokens [o, o+ks[gi]) with o = ks[0]+...+ks[gi-1], each ks a
 * multiple of 128.  A [m,T] + sa [m,T/128], B [n,T] + sb [n,T/128],
 * D fp32 [g,m,n]; D[gi] is updated as dgo_wgrad over that token range. */
int dgo_k_grouped_wgrad(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                        const int64_t* ks, int64_t g, int64_t m, int64_t n, float* d,
                        double* d_exact) {
  if (g <= 0 || m < 0 || n < 0) return -1;
  int64_t T = 0;
  for (int64_t gi = 0; gi < g; ++gi) {
    if (ks[gi] < 0 || ks[gi] % BK) return -1;
    T += ks[gi];
  }
  table_init();
  int64_t TB = T / BK;
  int64_t kb0 = 0;
  for (int64_t gi = 0; gi < g; ++gi) {
    int64_t kb1 = kb0 + ks[gi] / BK;
    float* dg = d + gi * m * n;
    double* dx = d_exact ? d_exact + gi * m * n : NULL;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i)
      for (int64_t j = 0; j < n; ++j) {
        double v = (double)dg[i * n + j] +
                   element(a + i * T, sa + i * TB, b + j * T, sb + j * TB, kb0, kb1);
        if (dx) dx[i * n + j] = v;
        dg[i * n + j] = (float)v;
      }
    kb0 = kb1;
  }
  return 0;
}

int dgo_k_grouped_wgrad_at(const uint8_t* a, const float* sa, const uint8_t* b,
                           const float* sb, const int64_t* ks, int64_t g, int64_t m, int64_t n,
                           const float* d0, const int64_t* groups, const int64_t* rows,
                           const int64_t* cols, int64_t count, double* out) {
  if (g <= 0 || m < 0 || n < 0) return -1;
  int64_t T = 0;
  for (int64_t gi = 0; gi < g; ++gi) {
    if (ks[gi] < 0 || ks[gi] % BK) return -1;
    T += ks[gi];
  }
  for (int64_t t = 0; t < count; ++t)
    if (groups[t] < 0 || groups[t] >= g || rows[t] < 0 || rows[t] >= m || cols[t] < 0 ||
        cols[t] >= n)
      return -1;
  table_init();
  int64_t TB = T / BK;
  int64_t* kb_start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(g + 1));
  if (!kb_start) return -2;
  kb_start[0] = 0;
  for (int64_t gi = 0; gi < g; ++gi) kb_start[gi + 1] = kb_start[gi] + ks[gi] / BK;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < count; ++t) {
    int64_t gi = groups[t], i = rows[t], j = cols[t];
    double base = d0 ? (double)d0[(gi * m + i) * n + j] : 0.0;
    out[t] = base + element(a + i * T, sa + i * TB, b + j * T, sb + j * TB, kb_start[gi],
                            kb_start[gi + 1]);
  }
  free(kb_start);
  return 0;
}

/* ---- BF16 NT GEMM ---------------------------------------------------------
 * The pages list BF16 GEMM beside FP8 (aikraft.ru, support table: formats FP8,
 * FP4, BF16; DeepSeek DeepGEMM 中文讲解, "未来计划": BF16 support).  Same NT
 * layouts, no scales:
 *
 *   C[m,n] = bf16( sum_k A[m,k] * B[n,k] ),  A [M,K], B [N,K] bf16, C [M,N] bf16
 *
 * A bf16 value is the fp32 value whose upper 16 bits it holds, exact in fp64;
 * each product (8 x 8 significant bits) is exact in fp64; the K products are
 * added in ascending k in fp64 (rounding error below k * 2^-53 * sum|terms|,
 * far below half a bf16 step except within that distance of a tie); one
 * rounding to bf16 (round to nearest even). */
static double bf16_value(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double bf16_element(const uint16_t* arow, const uint16_t* brow, int64_t k) {
  double acc = 0.0;
  for (int64_t t = 0; t < k; ++t) acc += bf16_value(arow[t]) * bf16_value(brow[t]);
  return acc;
}

int dgo_gemm_bf16_nt(const uint16_t* a, const uint16_t* b, int64_t m, int64_t n, int64_t k, uint16_t* c,
                     double* c_exact) {
  if (m < 0 || n < 0 || k < 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i)
    for (int64_t j = 0; j < n; ++j) {
      const double v = bf16_element(a + i * k, b + j * k, k);
      if (c_exact) c_exact[i * n + j] = v;
      c[i * n + j] = round_bf16(v);
    }
  return 0;
}

/* the elements (rows[i], cols[i]) only, unrounded */
int dgo_gemm_bf16_nt_at(const uint16_t* a, const uint16_t* b, int64_t m, int64_t n, int64_t k,
                        const int64_t* rows, const int64_t* cols, int64_t count, double* out) {
  for (int64_t i = 0; i < count; ++i)
    if (rows[i] < 0 || rows[i] >= m || cols[i] < 0 || cols[i] >= n) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = bf16_element(a + rows[i] * k, b + cols[i] * k, k);
  return 0;
}
