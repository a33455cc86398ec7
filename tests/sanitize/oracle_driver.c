/* oracle_driver.c -- host-sanitizer driver (tests/test_host_sanitizers.py) for
 * the CPU oracle (oracle/dg_oracle.c, oracle/dg_quant_oracle.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer: every entry point on small
 * seeded inputs with ragged shapes, empty groups, padding ids and masked
 * counts outside [0, M_max], plus cross-checks between entry points (sampled
 * against full results, fp64 against int64 block sums). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void dgo_e4m3_table(double* out);
void dgo_round_bf16(const double* x, uint16_t* out, int64_t n);
void dgo_round_f32(const double* x, float* out, int64_t n);
int dgo_block_sums_f64(const uint8_t* a, const uint8_t* b, int64_t m, int64_t n, int64_t k, double* out);
int dgo_block_sums_i64(const uint8_t* a, const uint8_t* b, int64_t m, int64_t n, int64_t k, int64_t* out);
int dgo_gemm_fp8_nt(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int64_t m, int64_t n,
                    int64_t k, uint16_t* c, double* c_exact);
int dgo_gemm_fp8_nt_at(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int64_t m, int64_t n,
                       int64_t k, const int64_t* rows, const int64_t* cols, int64_t count, double* out);
int dgo_grouped_contiguous(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                           const int32_t* m_indices, int64_t m_total, int64_t n, int64_t k, int64_t g, uint16_t* c,
                           double* c_exact);
int dgo_grouped_contiguous_at(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                              const int32_t* m_indices, int64_t m_total, int64_t n, int64_t k, int64_t g,
                              const int64_t* rows, const int64_t* cols, int64_t count, double* out, int8_t* written);
int dgo_grouped_masked(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, const int32_t* masked_m,
                       int64_t g, int64_t m_max, int64_t n, int64_t k, uint16_t* c, double* c_exact);
int dgo_grouped_masked_at(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                          const int32_t* masked_m, int64_t g, int64_t m_max, int64_t n, int64_t k,
                          const int64_t* groups, const int64_t* rows, const int64_t* cols, int64_t count, double* out,
                          int8_t* written);
int dgo_wgrad(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int64_t m, int64_t n, int64_t k,
              float* d, double* d_exact);
int dgo_wgrad_at(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int64_t m, int64_t n,
                 int64_t k, const float* d0, const int64_t* rows, const int64_t* cols, int64_t count, double* out);
int dgo_k_grouped_wgrad(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, const int64_t* ks,
                        int64_t g, int64_t m, int64_t n, float* d, double* d_exact);
int dgo_k_grouped_wgrad_at(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, const int64_t* ks,
                           int64_t g, int64_t m, int64_t n, const float* d0, const int64_t* groups,
                           const int64_t* rows, const int64_t* cols, int64_t count, double* out);
int dgo_gemm_bf16_nt(const uint16_t* a, const uint16_t* b, int64_t m, int64_t n, int64_t k, uint16_t* c,
                     double* c_exact);
int dgo_gemm_bf16_nt_at(const uint16_t* a, const uint16_t* b, int64_t m, int64_t n, int64_t k, const int64_t* rows,
                        const int64_t* cols, int64_t count, double* out);
void dgo_e4m3_encode(const float* y, uint8_t* out, int64_t n);
int dgo_quantize_1x128(const float* x, int64_t m, int64_t k, uint8_t* q, float* s);
int dgo_quantize_128x128(const float* x, int64_t n, int64_t k, uint8_t* q, float* s);
int dgo_quantize_1x128_transposed(const float* x, int64_t t, int64_t f, uint8_t* q, float* s);
int dgo_swiglu_quantize_1x128(const uint16_t* c, int64_t m, int64_t i, uint8_t* q, float* s, double* h_exact);

static int bad = 0;
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);  \
      bad++;                                                         \
    }                                                                \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {  /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static uint8_t code(void) {  /* a finite e4m3 code (no 0x7F / 0xFF) */
  uint8_t c = (uint8_t)(rnd() & 0xff);
  return (c & 0x7f) == 0x7f ? (uint8_t)(c - 1) : c;
}
static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) exit(3);
  return p;
}
static uint8_t* codes(size_t n) {
  uint8_t* p = (uint8_t*)xmalloc(n);
  for (size_t i = 0; i < n; ++i) p[i] = code();
  return p;
}
static float* scales(size_t n) {
  float* p = (float*)xmalloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = ldexpf(1.0f + (float)(rnd() % 1000) / 1000.0f, (int)(rnd() % 16) - 8);
  return p;
}

int main(void) {
  double table[256];
  dgo_e4m3_table(table);
  CHECK(table[0x7e] == 448.0 && table[0x01] == ldexp(1.0, -9) && isnan(table[0x7f]));

  /* dense, ragged N, three K blocks */
  const int64_t m = 17, n = 130, k = 384, kb = k / 128, nb = (n + 127) / 128;
  uint8_t *a = codes(m * k), *b = codes(n * k);
  float *sa = scales(m * kb), *sb = scales(nb * kb);
  uint16_t* c = (uint16_t*)xmalloc(m * n * 2);
  double* cx = (double*)xmalloc(m * n * 8);
  CHECK(dgo_gemm_fp8_nt(a, sa, b, sb, m, n, k, c, cx) == 0);
  int64_t rows[64], cols[64], groups[64];
  double out[64];
  int8_t wr[64];
  for (int i = 0; i < 64; ++i) rows[i] = rnd() % m, cols[i] = rnd() % n;
  CHECK(dgo_gemm_fp8_nt_at(a, sa, b, sb, m, n, k, rows, cols, 64, out) == 0);
  for (int i = 0; i < 64; ++i) CHECK(out[i] == cx[rows[i] * n + cols[i]]);
  double* bs = (double*)xmalloc(m * n * kb * 8);
  int64_t* bi = (int64_t*)xmalloc(m * n * kb * 8);
  CHECK(dgo_block_sums_f64(a, b, m, n, k, bs) == 0);
  CHECK(dgo_block_sums_i64(a, b, m, n, k, bi) == 0);
  for (int64_t i = 0; i < m * n * kb; ++i) CHECK(bs[i] == ldexp((double)bi[i], -18));
  uint16_t r16[4];
  float r32[4];
  const double vals[4] = {1.0, -0.0, 1e38, 3.0e-39};
  dgo_round_bf16(vals, r16, 4);
  dgo_round_f32(vals, r32, 4);
  CHECK(r16[0] == 0x3f80 && r32[0] == 1.0f);

  /* contiguous: two experts, padding rows, an out-of-range id, an empty expert */
  const int64_t g = 3, mt = 256;
  uint8_t *ga = codes(mt * k), *gb = codes(g * n * k);
  float *gsa = scales(mt * kb), *gsb = scales(g * nb * kb);
  int32_t ids[256];
  for (int i = 0; i < 256; ++i) ids[i] = i < 100 ? 0 : i < 128 ? -1 : i < 200 ? 2 : i < 210 ? 7 : -1;
  uint16_t* gc = (uint16_t*)xmalloc(mt * n * 2);
  double* gx = (double*)xmalloc(mt * n * 8);
  memset(gc, 0xff, mt * n * 2);
  CHECK(dgo_grouped_contiguous(ga, gsa, gb, gsb, ids, mt, n, k, g, gc, gx) == 0);
  for (int i = 0; i < 64; ++i) rows[i] = rnd() % mt, cols[i] = rnd() % n;
  CHECK(dgo_grouped_contiguous_at(ga, gsa, gb, gsb, ids, mt, n, k, g, rows, cols, 64, out, wr) == 0);
  for (int i = 0; i < 64; ++i) {
    const int valid = ids[rows[i]] >= 0 && ids[rows[i]] < g;
    CHECK(wr[i] == valid);
    if (valid) CHECK(out[i] == gx[rows[i] * n + cols[i]]);
    else CHECK(gc[rows[i] * n + cols[i]] == 0xffff);
  }

  /* masked: counts 0, 5, M_max and beyond, negative */
  const int64_t mg = 4, mmax = 40;
  const int32_t mm[4] = {0, 5, 40, 99};
  const int32_t mm_neg[4] = {-3, 1, 2, 3};
  uint8_t *ma = codes(mg * mmax * k), *mb = codes(mg * n * k);
  float *msa = scales(mg * mmax * kb), *msb = scales(mg * nb * kb);
  uint16_t* mc = (uint16_t*)xmalloc(mg * mmax * n * 2);
  double* mx = (double*)xmalloc(mg * mmax * n * 8);
  CHECK(dgo_grouped_masked(ma, msa, mb, msb, mm, mg, mmax, n, k, mc, mx) == 0);
  CHECK(dgo_grouped_masked(ma, msa, mb, msb, mm_neg, mg, mmax, n, k, mc, mx) == 0);
  for (int i = 0; i < 64; ++i) groups[i] = rnd() % mg, rows[i] = rnd() % mmax, cols[i] = rnd() % n;
  CHECK(dgo_grouped_masked_at(ma, msa, mb, msb, mm, mg, mmax, n, k, groups, rows, cols, 64, out, wr) == 0);

  /* weight gradients: fp32 D, row scales on both operands, K-grouped with an empty group */
  const int64_t wm = 24, wn = 20, wt = 512, wkb = wt / 128;
  uint8_t *wa = codes(wm * wt), *wb = codes(wn * wt);
  float *wsa = scales(wm * wkb), *wsb = scales(wn * wkb), *d = scales(4 * wm * wn);
  float* d0 = (float*)xmalloc(4 * wm * wn * 4);
  memcpy(d0, d, 4 * wm * wn * 4);
  double* dx = (double*)xmalloc(4 * wm * wn * 8);
  CHECK(dgo_wgrad(wa, wsa, wb, wsb, wm, wn, wt, d, dx) == 0);
  for (int i = 0; i < 64; ++i) rows[i] = rnd() % wm, cols[i] = rnd() % wn, groups[i] = rnd() % 4;
  CHECK(dgo_wgrad_at(wa, wsa, wb, wsb, wm, wn, wt, d0, rows, cols, 64, out) == 0);
  const int64_t kgs[4] = {128, 0, 256, 128};
  memcpy(d, d0, 4 * wm * wn * 4);
  CHECK(dgo_k_grouped_wgrad(wa, wsa, wb, wsb, kgs, 4, wm, wn, d, dx) == 0);
  CHECK(dgo_k_grouped_wgrad_at(wa, wsa, wb, wsb, kgs, 4, wm, wn, d0, groups, rows, cols, 64, out) == 0);
  for (int i = 0; i < 64; ++i) CHECK(fabs(out[i] - dx[(groups[i] * wm + rows[i]) * wn + cols[i]]) <= 0.0);

  /* BF16 GEMM */
  const int64_t bk = 192;
  uint16_t *ba = (uint16_t*)xmalloc(m * bk * 2), *bb = (uint16_t*)xmalloc(n * bk * 2), *bc = (uint16_t*)xmalloc(m * n * 2);
  for (int64_t i = 0; i < m * bk; ++i) ba[i] = (uint16_t)(0x3c00 + rnd() % 0x800);
  for (int64_t i = 0; i < n * bk; ++i) bb[i] = (uint16_t)(0xbc00 + rnd() % 0x800);
  double* bx = (double*)xmalloc(m * n * 8);
  CHECK(dgo_gemm_bf16_nt(ba, bb, m, n, bk, bc, bx) == 0);
  for (int i = 0; i < 64; ++i) rows[i] = rnd() % m, cols[i] = rnd() % n;
  CHECK(dgo_gemm_bf16_nt_at(ba, bb, m, n, bk, rows, cols, 64, out) == 0);
  for (int i = 0; i < 64; ++i) CHECK(out[i] == bx[rows[i] * n + cols[i]]);

  /* quantisers: ragged rows, a zero group, transposed, SwiGLU */
  const int64_t qm = 130, qk = 256;
  float* x = (float*)xmalloc(qm * qk * 4);
  for (int64_t i = 0; i < qm * qk; ++i) x[i] = ldexpf((float)((int)(rnd() % 2001) - 1000) / 1000.0f, (int)(rnd() % 8));
  for (int64_t i = 0; i < 128; ++i) x[i] = 0.0f;
  uint8_t* q = (uint8_t*)xmalloc(qm * qk);
  float* s = (float*)xmalloc(qm * qk * 4);
  CHECK(dgo_quantize_1x128(x, qm, qk, q, s) == 0);
  CHECK(s[0] == 1.0f);
  CHECK(dgo_quantize_128x128(x, qm, qk, q, s) == 0);
  CHECK(dgo_quantize_1x128_transposed(x, 128, 130, q, s) == 0);
  float y[8] = {0.f, 448.f, -448.f, 1e-9f, 0.0078125f, 3.5f, 447.9f, -0.f};
  uint8_t yc[8];
  dgo_e4m3_encode(y, yc, 8);
  CHECK(yc[1] == 0x7e && yc[2] == 0xfe);
  uint16_t* sw = (uint16_t*)xmalloc(3 * 512 * 2);
  for (int i = 0; i < 3 * 512; ++i) sw[i] = (uint16_t)(rnd() & 0x7fff) | (uint16_t)((rnd() & 1) << 15);
  for (int i = 0; i < 3 * 512; ++i) if ((sw[i] & 0x7f80) == 0x7f80) sw[i] = 0x3f80;  /* finite */
  double* hx = (double*)xmalloc(3 * 256 * 8);
  CHECK(dgo_swiglu_quantize_1x128(sw, 3, 256, q, s, hx) == 0);

  free(a); free(b); free(sa); free(sb); free(c); free(cx); free(bs); free(bi);
  free(ga); free(gb); free(gsa); free(gsb); free(gc); free(gx);
  free(ma); free(mb); free(msa); free(msb); free(mc); free(mx);
  free(wa); free(wb); free(wsa); free(wsb); free(d); free(d0); free(dx);
  free(ba); free(bb); free(bc); free(bx); free(x); free(q); free(s); free(sw); free(hx);
  printf("bad=%d\n", bad);
  return bad != 0;
}
