/*
 * dg_quant_oracle.c -- plain CPU reference for the FP8 (e4m3) quantiser that
 * produces the GEMM's operands and their fine-grained fp32 scales.
 *
 * TEST INFRASTRUCTURE ONLY, like dg_oracle.c (built into the same library):
 * nothing on the product path loads it, and it shares no code, header or
 * table with the HIP library.
 *
 * What it computes.  The DeepGEMM pages (DeepSeek DeepGEMM 中文讲解,
 * "注意事项") say FP8 needs dynamic scale factors taken from amax; their
 * usage example ("使用示例") fixes the scale granularity: one fp32 scale per
 * row and 128-wide K group for activations ([M, K/128]) and one per 128x128
 * block for weights ([ceil(N/128), K/128]).  Per group G of inputs:
 *
 *   amax = max_{x in G} |x|
 *   s    = fp32(amax / 448)            (448 = largest finite e4m3fn value;
 *                                        s = 1 for an all-zero group)
 *   q(x) = e4m3_RNE( clamp(fp32(x / s), -448, 448) )
 *
 * fp32(.) is one IEEE-754 binary32 operation, rounded to nearest even.  The
 * clamp catches the few quotients that exceed 448 because s was rounded.
 * e4m3_RNE is the nearest OCP E4M3FN value, ties to the code whose mantissa
 * is even.  Inputs must be finite.
 *
 * Layouts (row-major, last dimension contiguous):
 *   1x128:            x [M, K] -> q [M, K], s [M, K/128]
 *   128x128:          x [N, K] -> q [N, K], s [ceil(N/128), K/128]
 *                     (the last row block holds the rows that exist)
 *   1x128 transposed: x [T, F] -> q [F, T], s [F, T/128]: the 1x128 rule
 *                     applied to the transpose of x, i.e. groups of 128
 *                     consecutive rows (tokens) of one column (feature), the
 *                     token-contiguous operands of the weight-gradient GEMM.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QG 128
#define E4M3_LARGEST 448.0f

/* The nearest e4m3fn value to y (|y| <= 448), ties to an even mantissa.
 * Magnitudes below 2^-6 are subnormal: integer multiples n of 2^-9, n in
 * [0, 8] (n = 8 is the smallest normal, code 0x08).  Above, a magnitude in
 * [2^E, 2^(E+1)) is n * 2^(E-3) with n in [8, 16]; n = 16 moves to the next
 * binade with mantissa 0.  Both scalings by powers of two are exact, and
 * nearbyint rounds half-way cases to even in the default rounding mode. */
static uint8_t e4m3_encode(float y) {
  const unsigned sign = signbit(y) ? 0x80u : 0u;
  if (isnan(y)) return (uint8_t)(sign | 0x7Fu);
  const double a = fabs((double)y);
  if (a < ldexp(1.0, -6)) {
    const double n = nearbyint(ldexp(a, 9));
    return (uint8_t)(sign | (unsigned)n);
  }
  int e;
  (void)frexp(a, &e);   /* a = f * 2^e with f in [0.5, 1) */
  int E = e - 1;        /* a in [2^E, 2^(E+1)) */
  double n = nearbyint(ldexp(a, 3 - E));
  if (n == 16.0) {
    E += 1;
    n = 8.0;
  }
  return (uint8_t)(sign | ((unsigned)(E + 7) << 3) | ((unsigned)n - 8u));
}

void dgo_e4m3_encode(const float* y, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(y[i]);
}

static float scale_of(float amax) { return amax == 0.0f ? 1.0f : amax / E4M3_LARGEST; }

static uint8_t quantize_one(float x, float s) {
  float y = x / s;
  if (y > E4M3_LARGEST) y = E4M3_LARGEST;
  if (y < -E4M3_LARGEST) y = -E4M3_LARGEST;
  return e4m3_encode(y);
}

/* x [m, k] -> q [m, k], s [m, k/128] */
int dgo_quantize_1x128(const float* x, int64_t m, int64_t k, uint8_t* q, float* s) {
  if (m < 0 || k < 0 || k % QG) return -1;
  const int64_t kg = k / QG;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t g = 0; g < kg; ++g) {
      const float* xg = x + r * k + g * QG;
      float amax = 0.0f;
      for (int i = 0; i < QG; ++i) amax = fmaxf(amax, fabsf(xg[i]));
      const float sc = scale_of(amax);
      s[r * kg + g] = sc;
      for (int i = 0; i < QG; ++i) q[r * k + g * QG + i] = quantize_one(xg[i], sc);
    }
  }
  return 0;
}

/* x [n, k] -> q [n, k], s [ceil(n/128), k/128] */
int dgo_quantize_128x128(const float* x, int64_t n, int64_t k, uint8_t* q, float* s) {
  if (n < 0 || k < 0 || k % QG) return -1;
  const int64_t kg = k / QG, nb = (n + QG - 1) / QG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    for (int64_t g = 0; g < kg; ++g) {
      const int64_t r0 = b * QG, r1 = (r0 + QG < n) ? r0 + QG : n;
      float amax = 0.0f;
      for (int64_t r = r0; r < r1; ++r)
        for (int i = 0; i < QG; ++i) amax = fmaxf(amax, fabsf(x[r * k + g * QG + i]));
      const float sc = scale_of(amax);
      s[b * kg + g] = sc;
      for (int64_t r = r0; r < r1; ++r)
        for (int i = 0; i < QG; ++i) q[r * k + g * QG + i] = quantize_one(x[r * k + g * QG + i], sc);
    }
  }
  return 0;
}

/* x [t, f] -> q [f, t], s [f, t/128]: the 1x128 rule on the transpose of x */
int dgo_quantize_1x128_transposed(const float* x, int64_t t, int64_t f, uint8_t* q, float* s) {
  if (t < 0 || f < 0 || t % QG) return -1;
  float* xt = (float*)malloc(sizeof(float) * (size_t)(t * f > 0 ? t * f : 1));
  if (!xt) return -2;
  for (int64_t i = 0; i < t; ++i)
    for (int64_t j = 0; j < f; ++j) xt[j * t + i] = x[i * f + j];
  const int rc = dgo_quantize_1x128(xt, f, t, q, s);
  free(xt);
  return rc;
}

/* ---- power-of-two (UE8M0) scales, packed four to an int32 --------------
 *
 * DeepGEMM pages (aikraft.ru, support table: the scale format of the newer
 * architecture is packed UE8M0, four values in one torch.int).  The pages
 * give no rule for choosing such a scale.  Reading taken: the scale of a
 * group is the smallest E8M0 value 2^(E - 127), E in [0, 254], that is not
 * below the fp32 scale above (so no element is clipped harder than with it):
 *
 *   s0   = fp32(amax / 448)                  (1 for an all-zero group)
 *   E    = least E in [0, 254] with 2^(E - 127) >= s0
 *   q(x) = e4m3_RNE( clamp(x / 2^(E - 127), -448, 448) )
 *
 * The quotient by a power of two is exact in fp64; handed to the encoder as
 * fp32 it stays exact down to 2^-126, and anything smaller encodes to zero
 * either way (the smallest e4m3 magnitude is 2^-9).  The codes E go to packed
 * words [rows, ceil(groups/4)] int32: group g of a row is byte g mod 4 (bits
 * 8(g mod 4) .. +7) of word g/4; the bytes past the last group are 0. */
static unsigned ue8m0_of(float amax) {
  const double s0 = (double)scale_of(amax);
  for (unsigned e = 0; e < 254; ++e)
    if (ldexp(1.0, (int)e - 127) >= s0) return e;
  return 254;
}

static uint8_t quantize_pow2(float x, unsigned e) {
  double y = (double)x / ldexp(1.0, (int)e - 127);
  if (y > E4M3_LARGEST) y = E4M3_LARGEST;
  if (y < -E4M3_LARGEST) y = -E4M3_LARGEST;
  return e4m3_encode((float)y);
}

static void put_code(int32_t* words, int64_t kw, int64_t row, int64_t g, unsigned e) {
  uint32_t w = (uint32_t)words[row * kw + g / 4];
  w |= (uint32_t)e << (8 * (g % 4));
  words[row * kw + g / 4] = (int32_t)w;
}

/* x [m, k] -> q [m, k], s [m, ceil(k/512)] packed codes of the 1x128 groups */
int dgo_quantize_1x128_ue8m0(const float* x, int64_t m, int64_t k, uint8_t* q, int32_t* s) {
  if (m < 0 || k < 0 || k % QG) return -1;
  const int64_t kg = k / QG, kw = (kg + 3) / 4;
  memset(s, 0, sizeof(int32_t) * (size_t)(m * kw));
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t g = 0; g < kg; ++g) {
      const float* xg = x + r * k + g * QG;
      float amax = 0.0f;
      for (int i = 0; i < QG; ++i) {
        const float v = fabsf(xg[i]);
        if (v > amax) amax = v;
      }
      const unsigned e = ue8m0_of(amax);
      put_code(s, kw, r, g, e);
      for (int i = 0; i < QG; ++i) q[r * k + g * QG + i] = quantize_pow2(xg[i], e);
    }
  }
  return 0;
}

/* x [n, k] -> q [n, k], s [ceil(n/128), ceil(k/512)] packed codes of the 128x128 blocks */
int dgo_quantize_128x128_ue8m0(const float* x, int64_t n, int64_t k, uint8_t* q, int32_t* s) {
  if (n < 0 || k < 0 || k % QG) return -1;
  const int64_t kg = k / QG, nb = (n + QG - 1) / QG, kw = (kg + 3) / 4;
  memset(s, 0, sizeof(int32_t) * (size_t)(nb * kw));
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    for (int64_t g = 0; g < kg; ++g) {
      const int64_t r0 = b * QG, r1 = (r0 + QG < n) ? r0 + QG : n;
      float amax = 0.0f;
      for (int64_t rr = r0; rr < r1; ++rr)
        for (int i = 0; i < QG; ++i) {
          const float v = fabsf(x[rr * k + g * QG + i]);
          if (v > amax) amax = v;
        }
      const unsigned e = ue8m0_of(amax);
      put_code(s, kw, b, g, e);
      for (int64_t rr = r0; rr < r1; ++rr)
        for (int i = 0; i < QG; ++i) q[rr * k + g * QG + i] = quantize_pow2(x[rr * k + g * QG + i], e);
    }
  }
  return 0;
}

/* ---- SwiGLU on the first linear's output, then the 1x128 rule ----------
 *
 * DeepGEMM pages (the Russian overview "DeepSeek выложила в открытый доступ
 * библиотеку…", section "Ключевые функции: Mega MoE и индексация": Mega MoE
 * runs an expert's first linear layer, the SwiGLU activation and the second
 * linear layer in one kernel).  Between the two FP8 GEMMs the
 * activation's output must be re-quantised, since the second GEMM takes FP8
 * operands with 1x128 scales.  Reading taken (the pages give no layout):
 *
 *   c [M, 2I] bf16, the first GEMM's output; gate g = c[:, 0:I],
 *   up u = c[:, I:2I] (the two halves of the stacked projection);
 *   h = silu(g) * u,  silu(x) = x / (1 + e^-x)   evaluated in fp64,
 *   rounded once to fp32, then the 1x128 rule above on h [M, I]:
 *   q [M, I] e4m3, s [M, I/128] fp32.
 *
 * h_exact (optional, [M, I] fp64) receives h before the fp32 rounding. */
static double bf16_to_double(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double silu(double x) { return x / (1.0 + exp(-x)); }

int dgo_swiglu_quantize_1x128(const uint16_t* c, int64_t m, int64_t i, uint8_t* q, float* s,
                              double* h_exact) {
  if (m < 0 || i < 0 || i % QG) return -1;
  float* h = (float*)malloc(sizeof(float) * (size_t)(m * i > 0 ? m * i : 1));
  if (!h) return -2;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < m; ++r) {
    const uint16_t* gate = c + r * 2 * i;
    const uint16_t* up = gate + i;
    for (int64_t j = 0; j < i; ++j) {
      const double v = silu(bf16_to_double(gate[j])) * bf16_to_double(up[j]);
      if (h_exact) h_exact[r * i + j] = v;
      h[r * i + j] = (float)v;
    }
  }
  const int rc = dgo_quantize_1x128(h, m, i, q, s);
  free(h);
  return rc;
}
