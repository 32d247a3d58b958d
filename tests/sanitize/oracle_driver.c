/*
 * Runs every function of oracle/q4_oracle.c on small seeded inputs, the
 * edge cases included (one row, one group, ragged sample lists, rejected
 * lengths, the first and last cache positions, an out-of-range token), so
 * that a build with AddressSanitizer and UndefinedBehaviorSanitizer checks
 * the oracle's memory accesses and arithmetic on the host.  Exits 0 when
 * every call returned what its contract says.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float orc_tree(const float *v, int64_t n);
void orc_group_sums(const float *x, int64_t n, float *xs);
uint32_t orc_code(const uint32_t *q, int64_t cols, int64_t r, int64_t c);
void orc_q4mv(const uint32_t *q, const float *s, const float *b, const float *x, const float *xs,
              float *y, int64_t rows, int64_t cols, int nthreads);
void orc_q4mv_sample(const uint32_t *q, const float *s, const float *b, const float *x,
                     const float *xs, float *y, int64_t cols, const int64_t *idx, int64_t count);
int orc_rmsq(const float *h, const float *w, int64_t n, float eps, float *u, float *us);
double orc_exp(double t);
int orc_swq(const float *a, int64_t n, float *o, float *os);
int32_t orc_argmax(const float *v, int64_t n);
void orc_embed(const uint32_t *q, const float *s, const float *b, int64_t rows, int64_t cols,
               int64_t tok, float *e);
void orc_add(const float *a, const float *b, float *out, int64_t n);
uint32_t orc_fnv1a32(const void *data, int64_t nbytes);
int orc_atq(const float *q, const float *g, const float *k, const float *v, const float *wq,
            const float *wk, float eps, const float *cs, const float *sn, float *kc, float *vc,
            int64_t pos, int64_t max_pos, int64_t hq, int64_t hkv, float *o, float *os);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(state >> 32);
}
static float uniform(float lo, float hi) { return lo + (hi - lo) * (float)(next32() >> 8) / 16777216.0f; }
static float *floats(int64_t n, float lo, float hi) {
  float *p = (float *)malloc(sizeof(float) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) p[i] = uniform(lo, hi);
  return p;
}

static int failures = 0;
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

static void product(int64_t rows, int64_t cols) {
  const int64_t G = cols / 64;
  uint32_t *q = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(rows * cols / 8));
  for (int64_t i = 0; i < rows * cols / 8; ++i) q[i] = next32();
  float *s = floats(rows * G, 0.001f, 0.02f), *b = floats(rows * G, -0.2f, 0.0f);
  float *x = floats(cols, -2.0f, 2.0f), *xs = (float *)malloc(sizeof(float) * (size_t)G);
  orc_group_sums(x, cols, xs);
  float *y1 = (float *)malloc(sizeof(float) * (size_t)rows);
  float *y3 = (float *)malloc(sizeof(float) * (size_t)rows);
  orc_q4mv(q, s, b, x, xs, y1, rows, cols, 1);
  orc_q4mv(q, s, b, x, xs, y3, rows, cols, 3);
  CHECK(memcmp(y1, y3, sizeof(float) * (size_t)rows) == 0);
  int64_t idx[3] = {rows - 1, 0, rows / 2};
  float ys[3];
  orc_q4mv_sample(q, s, b, x, xs, ys, cols, idx, 3);
  for (int k = 0; k < 3; ++k) CHECK(memcmp(&ys[k], &y1[idx[k]], sizeof(float)) == 0);
  CHECK(orc_code(q, cols, rows - 1, cols - 1) == (q[rows * cols / 8 - 1] >> 28));
  float *e = (float *)malloc(sizeof(float) * (size_t)cols);
  orc_embed(q, s, b, rows, cols, rows - 1, e);
  orc_embed(q, s, b, rows, cols, rows, e); /* outside: NaNs */
  CHECK(isnan(e[0]) && isnan(e[cols - 1]));
  CHECK(orc_argmax(y1, rows) >= 0);
  free(q), free(s), free(b), free(x), free(xs), free(y1), free(y3), free(e);
}

int main(void) {
  /* trees over every small length and a few large ones */
  for (int64_t n = 1; n <= 200; ++n) {
    float *v = floats(n, -1.0f, 1.0f);
    (void)orc_tree(v, n);
    free(v);
  }
  /* products: one row, one group, ragged rows, the split widths */
  product(1, 64);
  product(13, 128);
  product(7, 2048);
  product(5, 6144);
  product(3, 2112);
  /* rmsq: accepted and rejected lengths */
  {
    float *h = floats(2048, -3.0f, 3.0f), *w = floats(2048, 0.5f, 1.5f);
    float *u = (float *)malloc(sizeof(float) * 2048), us[32];
    CHECK(orc_rmsq(h, w, 2048, 1e-6f, u, us) == 0);
    CHECK(orc_rmsq(h, w, 64, 1e-6f, u, us) == 0);
    CHECK(orc_rmsq(h, w, 96, 1e-6f, u, us) == -1);
    CHECK(orc_rmsq(h, w, 0, 1e-6f, u, us) == -1);
    free(h), free(w), free(u);
  }
  /* exp over its range and past both ends */
  for (double t = -800.0; t <= 800.0; t += 0.37) (void)orc_exp(t);
  CHECK(orc_exp(-1000.0) == 0.0 && isinf(orc_exp(1000.0)));
  /* swq: n = 64 and 6144; n = 32 rejected */
  {
    float *a = floats(2 * 6144, -50.0f, 50.0f), *o = (float *)malloc(sizeof(float) * 6144);
    float os[96];
    CHECK(orc_swq(a, 6144, o, os) == 0);
    CHECK(orc_swq(a, 64, o, os) == 0);
    CHECK(orc_swq(a, 32, o, os) == -1);
    float c[4] = {1.0f, 2.0f, 2.0f, 0.5f};
    CHECK(orc_argmax(c, 4) == 1);
    c[3] = NAN;
    CHECK(orc_argmax(c, 4) == -1);
    orc_add(a, a + 6144, o, 6144);
    CHECK(orc_fnv1a32(a, 0) == 0x811C9DC5u);
    free(a), free(o);
  }
  /* atq: first and last cache positions, several head groupings, rejected
     shapes */
  {
    const int64_t max_pos = 300, D = 128;
    const int64_t shapes[3][2] = {{16, 4}, {4, 2}, {2, 2}};
    for (int sh = 0; sh < 3; ++sh) {
      const int64_t hq = shapes[sh][0], hkv = shapes[sh][1];
      float *q = floats(hq * D, -1, 1), *g = floats(hq * D, -4, 4), *k = floats(hkv * D, -1, 1);
      float *v = floats(hkv * D, -1, 1), *wq = floats(D, 0.8f, 1.2f), *wk = floats(D, 0.8f, 1.2f);
      float *cs = floats(D / 2, -1, 1), *sn = floats(D / 2, -1, 1);
      float *kc = floats(hkv * max_pos * D, -1, 1), *vc = floats(hkv * max_pos * D, -1, 1);
      float *o = (float *)malloc(sizeof(float) * (size_t)(hq * D));
      float *os = (float *)malloc(sizeof(float) * (size_t)(hq * 2));
      CHECK(orc_atq(q, g, k, v, wq, wk, 1e-6f, cs, sn, kc, vc, 0, max_pos, hq, hkv, o, os) == 0);
      CHECK(orc_atq(q, g, k, v, wq, wk, 1e-6f, cs, sn, kc, vc, max_pos - 1, max_pos, hq, hkv, o,
                    os) == 0);
      CHECK(orc_atq(q, g, k, v, wq, wk, 1e-6f, cs, sn, kc, vc, max_pos, max_pos, hq, hkv, o,
                    os) == -1);
      CHECK(orc_atq(q, g, k, v, wq, wk, 1e-6f, cs, sn, kc, vc, 5, max_pos, hq, hkv + 1, o,
                    os) == -1);
      free(q), free(g), free(k), free(v), free(wq), free(wk), free(cs), free(sn), free(kc);
      free(vc), free(o), free(os);
    }
  }
  if (failures) fprintf(stderr, "%d checks failed\n", failures);
  else printf("oracle driver: ok\n");
  return failures ? 1 : 0;
}
