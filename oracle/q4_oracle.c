/*
 * q4_oracle.c -- plain CPU oracle for the affine 4-bit matvec (q4mv) and its
 * producers (rmsq, swq), plus the greedy-decode glue (argmax, embed).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * reference that the GPU library is checked against.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code with the HIP library: no header, helper, table or
 * constant is common to both.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 *        (x86-64, SSE2 scalar float: every float operation below is one
 *        IEEE-754 binary32 operation with round-to-nearest-even; no FMA
 *        contraction, no flush-to-zero).
 *
 * Sources (bendlang/bend pull requests, as quoted in the source pages):
 *  - "Array.q4mv on Metal: one kernel thread per row ..." (#1435), Why and
 *    Change: the product is an affine 4-bit matvec over rows of packed codes.
 *  - "Metal: queued rmsq, swq, gdn and atq kernels and a 4-row q4mv, so a
 *    decode token is one command buffer with one wait" (#1440), Change:
 *    rmsq is an RMS norm with binary32 weights that also produces the
 *    per-64-column group sums q4mv consumes; swq is SwiGLU (silu of each
 *    gate value times its up value, rounded) with group sums; q4mv sums
 *    each row in a fixed order that the pages name but never print.
 *  - The pages never print the summation tree, the nibble order or the
 *    precision of swq.  The readings taken here (canonical tree T, low
 *    nibble first, swq in binary64 with one rounding to binary32, exp by a
 *    fixed binary64 method) are listed with the design notes.
 *
 * Parity pins for every function are in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 64

/* ------------------------------------------------------------------------
 * Canonical summation tree T: the reading taken of the fixed summation
 * order that #1436's title (cited on the #1440 page, Change) names.
 *   T(v[0..1)) = v[0]
 *   T(v[0..n)) = T(v[0..m)) + T(v[m..n)),  m = largest power of two < n
 * Every '+' is one binary32 addition.
 * ---------------------------------------------------------------------- */
static int64_t largest_pow2_below(int64_t n) {
    int64_t m = 1;
    while (m * 2 < n) m *= 2;
    return m;
}

float orc_tree(const float *v, int64_t n) {
    if (n == 1) return v[0];
    int64_t m = largest_pow2_below(n);
    float left = orc_tree(v, m);
    float right = orc_tree(v + m, n - m);
    return left + right;
}

/* ------------------------------------------------------------------------
 * Group sums of an activation vector: xs[g] = T(x[64g .. 64g+63]).
 * These are the group sums the producers hand to q4mv (#1440, Change, rmsq
 * bullet).  n must be a multiple of 64.
 * ---------------------------------------------------------------------- */
void orc_group_sums(const float *x, int64_t n, float *xs) {
    for (int64_t g = 0; g < n / GROUP; ++g) xs[g] = orc_tree(x + g * GROUP, GROUP);
}

/* ------------------------------------------------------------------------
 * Code of row r, column c.  Layout: row-major, cols/8 words per row, column
 * 8j+k held in bits 4k..4k+3 of word j (low nibble first).
 * ---------------------------------------------------------------------- */
uint32_t orc_code(const uint32_t *q, int64_t cols, int64_t r, int64_t c) {
    uint32_t word = q[r * (cols / 8) + c / 8];
    return (word >> (4 * (c % 8))) & 15u;
}

/* ------------------------------------------------------------------------
 * q4mv, fixed order.  For each row r:
 *   p_i  = float(q(r, 64g+i)) * x[64g+i]              (64 binary32 products)
 *   d_g  = T(p_0 .. p_63)
 *   t_g  = (s[r,g] * d_g) + (b[r,g] * xs[g])          (two products, one add)
 *   y[r] = T(t_0 .. t_{G-1})
 * i.e. y[r] = sum_g s*(q.x_g) + b*sum(x_g), the affine dequantised dot.
 * xs is an input (the producers emit it); it is never recomputed here.
 * ---------------------------------------------------------------------- */
/* One output row; p holds 64 scratch floats, t holds G scratch floats. */
static float q4mv_row(const uint32_t *q, const float *s, const float *b,
                      const float *x, const float *xs, int64_t cols, int64_t r,
                      float *p, float *t) {
    const int64_t G = cols / GROUP;
    for (int64_t g = 0; g < G; ++g) {
        for (int64_t i = 0; i < GROUP; ++i) {
            int64_t c = g * GROUP + i;
            float code = (float)orc_code(q, cols, r, c);
            p[i] = code * x[c];
        }
        float d = orc_tree(p, GROUP);
        float sd = s[r * G + g] * d;
        float bx = b[r * G + g] * xs[g];
        t[g] = sd + bx;
    }
    return orc_tree(t, G);
}

static void q4mv_rows(const uint32_t *q, const float *s, const float *b,
                      const float *x, const float *xs, float *y,
                      int64_t cols, int64_t r0, int64_t r1) {
    float p[GROUP];
    float *t = (float *)malloc(sizeof(float) * (size_t)(cols / GROUP));
    for (int64_t r = r0; r < r1; ++r) y[r] = q4mv_row(q, s, b, x, xs, cols, r, p, t);
    free(t);
}

typedef struct {
    const uint32_t *q;
    const float *s, *b, *x, *xs;
    float *y;
    int64_t cols, r0, r1;
} q4mv_job;

static void *q4mv_worker(void *arg) {
    q4mv_job *j = (q4mv_job *)arg;
    q4mv_rows(j->q, j->s, j->b, j->x, j->xs, j->y, j->cols, j->r0, j->r1);
    return NULL;
}

/* Rows are independent and each row's operation order is fixed, so the
 * thread count (rows split into contiguous ranges) never changes the bits. */
void orc_q4mv(const uint32_t *q, const float *s, const float *b,
              const float *x, const float *xs, float *y,
              int64_t rows, int64_t cols, int nthreads) {
    if (nthreads <= 1 || rows < 2 * nthreads) {
        q4mv_rows(q, s, b, x, xs, y, cols, 0, rows);
        return;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    q4mv_job *jobs = (q4mv_job *)malloc(sizeof(q4mv_job) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (q4mv_job){q, s, b, x, xs, y, cols,
                             rows * i / nthreads, rows * (i + 1) / nthreads};
        pthread_create(&th[i], NULL, q4mv_worker, &jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(jobs);
    free(th);
}

/* Same product on a subset of rows (sampled parity checks): y[k] is row
 * idx[k]. */
void orc_q4mv_sample(const uint32_t *q, const float *s, const float *b,
                     const float *x, const float *xs, float *y,
                     int64_t cols, const int64_t *idx, int64_t count) {
    float p[GROUP];
    float *t = (float *)malloc(sizeof(float) * (size_t)(cols / GROUP));
    for (int64_t k = 0; k < count; ++k) y[k] = q4mv_row(q, s, b, x, xs, cols, idx[k], p, t);
    free(t);
}

/* ------------------------------------------------------------------------
 * rmsq: RMS norm with F32 weights plus group sums (#1440, Change, rmsq
 * bullet; exact on the GPU per the same page).  Reading: binary32 only,
 * correctly rounded divide and square root:
 *   ss   = T(h_i * h_i)
 *   ms   = ss / float(n)
 *   rho  = 1 / sqrt(ms + eps)
 *   u_i  = (h_i * rho) * w_i
 *   us_g = T(u[64g .. 64g+63])
 * Returns 0, or -1 when n is not a positive multiple of 64.
 * ---------------------------------------------------------------------- */
int orc_rmsq(const float *h, const float *w, int64_t n, float eps,
             float *u, float *us) {
    if (n <= 0 || n % GROUP != 0) return -1;
    float *sq = (float *)malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) sq[i] = h[i] * h[i];
    float ss = orc_tree(sq, n);
    free(sq);
    float ms = ss / (float)n;
    float rho = 1.0f / sqrtf(ms + eps);
    for (int64_t i = 0; i < n; ++i) {
        float hr = h[i] * rho;
        u[i] = hr * w[i];
    }
    orc_group_sums(u, n, us);
    return 0;
}

/* ------------------------------------------------------------------------
 * exp in binary64 by a fixed method, so that every implementation that
 * follows the same steps gets the same bits (the pages put swq's Metal
 * mismatch down to Metal's exp, #1440 Change):
 *   t >= 710  -> +inf ;  t <= -746 -> +0 ;  NaN -> NaN
 *   k = rint(t * INV_LN2)                      (nearest, ties to even)
 *   r = (t - k*LN2_HI) - k*LN2_LO              (Cody-Waite reduction)
 *   p = sum_{j=0..13} r^j / j!                 (Horner, fused multiply-add)
 *   E = ldexp(p, k)
 * INV_LN2 = RN64(1/ln 2).  LN2_HI = ln 2 truncated to 32 significant bits,
 * so k*LN2_HI is exact for |k| < 2^21.  LN2_LO = RN64(ln 2 - LN2_HI).
 * 1/j! is the correctly rounded quotient (j! is exact in binary64 for
 * j <= 18).
 * ---------------------------------------------------------------------- */
static const double INV_LN2 = 0x1.71547652b82fep+0;
static const double LN2_HI = 0x1.62e42fee00000p-1;
static const double LN2_LO = 0x1.a39ef35793c76p-33;

double orc_exp(double t) {
    if (t != t) return t;
    if (t >= 710.0) return INFINITY;
    if (t <= -746.0) return 0.0;
    double k = rint(t * INV_LN2);
    double hi = t - k * LN2_HI;
    double lo = k * LN2_LO;
    double r = hi - lo;
    double coef[14];
    double fact = 1.0;
    for (int j = 0; j < 14; ++j) {
        if (j > 0) fact = fact * (double)j;
        coef[j] = 1.0 / fact;
    }
    double p = coef[13];
    for (int j = 12; j >= 0; --j) p = fma(p, r, coef[j]);
    return ldexp(p, (int)k);
}

/* ------------------------------------------------------------------------
 * swq: SwiGLU over a = [gate (n) | up (n)]: silu of each gate value times
 * its up value, rounded, plus group sums (#1440, Change, swq bullet).  Reading: the product is
 * formed in binary64 and rounded once to binary32:
 *   sig_i = a_i / (1 + E(-a_i))                 (binary64)
 *   o_i   = RN32(sig_i * a_{n+i})               (binary64 product, one
 *                                                rounding to binary32)
 *   os_g  = T(o[64g .. 64g+63])                 (binary32)
 * Returns 0, or -1 when n is not a positive multiple of 64 (the pages' n=32
 * case silently left o untouched; here it is an error).
 * ---------------------------------------------------------------------- */
int orc_swq(const float *a, int64_t n, float *o, float *os) {
    if (n <= 0 || n % GROUP != 0) return -1;
    for (int64_t i = 0; i < n; ++i) {
        double g = (double)a[i];
        double up = (double)a[n + i];
        double sig = g / (1.0 + orc_exp(-g));
        o[i] = (float)(sig * up);
    }
    orc_group_sums(o, n, os);
    return 0;
}

/* ------------------------------------------------------------------------
 * Greedy pick (the pages' engine decodes greedily, #1440 Verification):
 * lowest index of the largest value; -1 when any value is NaN or n < 1.
 * ---------------------------------------------------------------------- */
int32_t orc_argmax(const float *v, int64_t n) {
    if (n < 1) return -1;
    int64_t best = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (v[i] != v[i]) return -1;
        if (v[i] > v[best]) best = i;
    }
    return (int32_t)best;
}

/* ------------------------------------------------------------------------
 * Embedding lookup from a tied Q4 matrix: dequantise row t,
 *   e[c] = (s[t, c/64] * float(q(t, c))) + b[t, c/64].
 * A token outside [0, rows) yields quiet NaNs.
 * ---------------------------------------------------------------------- */
void orc_embed(const uint32_t *q, const float *s, const float *b,
               int64_t rows, int64_t cols, int64_t tok, float *e) {
    const int64_t G = cols / GROUP;
    for (int64_t c = 0; c < cols; ++c) {
        if (tok < 0 || tok >= rows) {
            e[c] = NAN;
            continue;
        }
        float code = (float)orc_code(q, cols, tok, c);
        float sq = s[tok * G + c / GROUP] * code;
        e[c] = sq + b[tok * G + c / GROUP];
    }
}

/* Elementwise binary32 add (the chain's residual): out = a + b. */
void orc_add(const float *a, const float *b, float *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = a[i] + b[i];
}

/* FNV-1a 32-bit over a byte buffer (hash of an output's bits). */
uint32_t orc_fnv1a32(const void *data, int64_t nbytes) {
    const uint8_t *p = (const uint8_t *)data;
    uint32_t h = 2166136261u;
    for (int64_t i = 0; i < nbytes; ++i) {
        h ^= p[i];
        h *= 16777619u;
    }
    return h;
}

/* ------------------------------------------------------------------------
 * atq: one decode token of gated attention over key and value caches
 * ("Metal: queued rmsq, swq, gdn and atq kernels ..." (#1440), Change, atq
 * bullet).  That bullet names the parts only: the query and the new key are
 * normalised and rotated, the new key and value are appended to the caches,
 * each cached position is weighted by a softmax of its score, the weighted
 * sum of values is gated by a sigmoid, and the 64-value sums are emitted;
 * the Metal kernel runs a threadgroup per query head, and several query
 * heads share one key/value head.  The pages give no formulas; the
 * readings (listed with the design notes):
 *   D = 128 values per head; hq query heads, hkv key/value heads with
 *   hq % hkv == 0; query head h uses key/value head h / (hq / hkv).
 *   qn = rmsq(q_h, wq), kn = rmsq(k_j, wk)     (rmsq's definition over D)
 *   rotation by the position's table c_i, s_i (i < D/2), pairing dims i
 *   and i + D/2 (a = x_i, b = x_{i+D/2}):
 *     r_i       = (a * c_i) - (b * s_i)
 *     r_{i+D/2} = (a * s_i) + (b * c_i)
 *   caches (rows of D floats, [hkv][max_pos][D]): K[j][pos] = rotated kn,
 *   V[j][pos] = v_j
 *   score   s_t = T(qr_i * K[j][t]_i, i < D) * SCALE, t = 0..pos,
 *           SCALE = RN32(1/sqrt(D))
 *   m = the largest s_t; e_t = RN32(E(s_t - m)), the difference in binary32,
 *   E the fixed binary64 exp above
 *   Z = T(e_0 .. e_pos)
 *   w_i = T(e_t * V[j][t]_i, t = 0..pos) / Z
 *   o_i = w_i * RN32(1 / (1 + E(-g_i)))      (the sigmoid in binary64)
 *   os  = T over each 64 values of o
 * Returns 0, or -1 for shapes outside these readings.
 * ---------------------------------------------------------------------- */
#define ATQ_D 128

static void atq_rotate(const float *x, const float *c, const float *s, float *r) {
    for (int i = 0; i < ATQ_D / 2; ++i) {
        const float a = x[i], b = x[i + ATQ_D / 2];
        const float ac = a * c[i], bs = b * s[i];
        const float as = a * s[i], bc = b * c[i];
        r[i] = ac - bs;
        r[i + ATQ_D / 2] = as + bc;
    }
}

int orc_atq(const float *q, const float *g, const float *k, const float *v,
            const float *wq, const float *wk, float eps, const float *cs,
            const float *sn, float *kc, float *vc, int64_t pos, int64_t max_pos,
            int64_t hq, int64_t hkv, float *o, float *os) {
    if (hq < 1 || hkv < 1 || hq % hkv != 0 || pos < 0 || pos >= max_pos) return -1;
    const int64_t group = hq / hkv;
    const int64_t n = pos + 1;
    const float scale = (float)(1.0 / sqrt((double)ATQ_D));
    float kn[ATQ_D], knu[2], qn[ATQ_D], qnu[2], qr[ATQ_D];
    float *prod = (float *)malloc(sizeof(float) * ATQ_D);
    float *sc = (float *)malloc(sizeof(float) * (size_t)n);
    float *ev = (float *)malloc(sizeof(float) * (size_t)n);
    /* the new key and value rows of every key/value head */
    for (int64_t j = 0; j < hkv; ++j) {
        orc_rmsq(k + j * ATQ_D, wk, ATQ_D, eps, kn, knu);
        atq_rotate(kn, cs, sn, kc + (j * max_pos + pos) * ATQ_D);
        memcpy(vc + (j * max_pos + pos) * ATQ_D, v + j * ATQ_D, sizeof(float) * ATQ_D);
    }
    for (int64_t h = 0; h < hq; ++h) {
        const int64_t j = h / group;
        orc_rmsq(q + h * ATQ_D, wq, ATQ_D, eps, qn, qnu);
        atq_rotate(qn, cs, sn, qr);
        const float *K = kc + j * max_pos * ATQ_D;
        const float *V = vc + j * max_pos * ATQ_D;
        float m = 0.0f;
        for (int64_t t = 0; t < n; ++t) {
            for (int i = 0; i < ATQ_D; ++i) prod[i] = qr[i] * K[t * ATQ_D + i];
            sc[t] = orc_tree(prod, ATQ_D) * scale;
            if (t == 0 || sc[t] > m) m = sc[t];
        }
        for (int64_t t = 0; t < n; ++t) ev[t] = (float)orc_exp((double)(sc[t] - m));
        const float z = orc_tree(ev, n);
        float *wv = (float *)malloc(sizeof(float) * (size_t)n);
        for (int i = 0; i < ATQ_D; ++i) {
            for (int64_t t = 0; t < n; ++t) wv[t] = ev[t] * V[t * ATQ_D + i];
            const float w = orc_tree(wv, n) / z;
            const double gi = (double)g[h * ATQ_D + i];
            const float sig = (float)(1.0 / (1.0 + orc_exp(-gi)));
            o[h * ATQ_D + i] = w * sig;
        }
        free(wv);
    }
    orc_group_sums(o, hq * ATQ_D, os);
    free(prod);
    free(sc);
    free(ev);
    return 0;
}
