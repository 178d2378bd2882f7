/*
 * fp64 CPU oracle for causal differential attention, forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load or call this file.  It shares no
 * code, header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * What it computes (per batch b, head h and query row), following the Motif
 * 2.6B explainer, section "Differential attention" and the caption of figure 1
 * ("The block"): two softmax attention maps are formed from the two query/key
 * pairs (Q1, K1) and (Q2, K2), the second is scaled by lambda and subtracted
 * from the first, the difference multiplies the single value tensor V, and a
 * GroupNorm follows.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - scores carry the usual 1/sqrt(d_qk) factor (passed in as `scale`);
 *   - the model is decoder-only (edgentiq article on Motif-2.6B), so query i
 *     attends to keys j <= i; decode attends to all n cached keys;
 *   - sliding window (Motif 3's sliding-window layers, picx.dev summary of the
 *     Motif 3 report, section 2.1): with window W > 0, query i attends keys
 *     i-W+1 .. i, and decode the last W cached keys;
 *   - lambda is an input (scalar or one value per head) that scales the
 *     normalised second map; no clamping;
 *   - "GroupNorm" acts on the head output (after the product with V), with one
 *     group per head over its d_v channels: mean, biased variance (two-pass),
 *     eps inside the square root, a per-channel gain and no bias.
 *
 * Each row materialises its row of both maps in full (every j, softmax
 * normalised over the causal range), then the difference map's row, then the
 * product with V, then the norm: the plain definition, no streaming, no
 * blocking, no reordering.  Inputs are bf16 bit patterns, widened exactly to
 * fp64.  Rows are independent; OpenMP spreads them over host threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static inline double bf16_to_f64(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Softmax of x[0..n) in place: exp(x - max) / sum (the textbook definition). */
static void softmax_inplace(double* x, int64_t n) {
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) if (x[j] > m) m = x[j];
    double s = 0.0;
    for (int64_t j = 0; j < n; ++j) { x[j] = exp(x[j] - m); s += x[j]; }
    for (int64_t j = 0; j < n; ++j) x[j] /= s;
}

/*
 * One query row.  q1, q2 point at the row's d_qk-vectors; k1, k2, v at key
 * position 0 of this (b, h), with `kstride`/`vstride` elements between
 * consecutive positions.  p1 and p2 are scratch of length >= n_keys.
 * Writes o[d_v] (pre-norm) and y[d_v] (after GroupNorm).
 */
static void diff_attention_row(const uint16_t* q1, const uint16_t* q2,
                               const uint16_t* k1, const uint16_t* k2, const uint16_t* v,
                               int64_t kstride, int64_t vstride, int64_t n_keys,
                               int d_qk, int d_v, double scale, double lam,
                               const float* gain, double eps,
                               double* p1, double* p2, double* o, double* y) {
    /* Scores of both maps over the causal range. */
    for (int64_t j = 0; j < n_keys; ++j) {
        double a = 0.0, b = 0.0;
        for (int c = 0; c < d_qk; ++c) {
            a += bf16_to_f64(q1[c]) * bf16_to_f64(k1[j * kstride + c]);
            b += bf16_to_f64(q2[c]) * bf16_to_f64(k2[j * kstride + c]);
        }
        p1[j] = scale * a;
        p2[j] = scale * b;
    }
    /* The two attention maps' rows. */
    softmax_inplace(p1, n_keys);
    softmax_inplace(p2, n_keys);
    /* Difference map: first map minus lambda times the second. */
    for (int64_t j = 0; j < n_keys; ++j) p1[j] = p1[j] - lam * p2[j];
    /* Times V. */
    for (int c = 0; c < d_v; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        const uint16_t* vj = v + j * vstride;
        for (int c = 0; c < d_v; ++c) o[c] += p1[j] * bf16_to_f64(vj[c]);
    }
    /* GroupNorm, one group = this head's d_v channels. */
    double mu = 0.0;
    for (int c = 0; c < d_v; ++c) mu += o[c];
    mu /= d_v;
    double var = 0.0;
    for (int c = 0; c < d_v; ++c) var += (o[c] - mu) * (o[c] - mu);
    var /= d_v;
    double inv = 1.0 / sqrt(var + eps);
    for (int c = 0; c < d_v; ++c) y[c] = (o[c] - mu) * inv * (double)gain[c];
}

/*
 * Causal prefill.  q1, q2, k1, k2: bf16 [B, T, H, d_qk]; v: bf16 [B, T, H, d_v],
 * all C-contiguous.  lam: fp64 [H].  gain: fp32 [H, d_v].  window: > 0 for a
 * sliding window of that many keys, 0 for every key <= i.
 * rows: n_rows flat indices ((b * T + i) * H + h), or NULL for every row in
 * that order (then n_rows must be B*T*H).  o_pre, y: fp64 [n_rows, d_v].
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or -1 on bad arguments
 * or failed scratch allocation.
 */
int oracle_prefill(const uint16_t* q1, const uint16_t* q2, const uint16_t* k1,
                   const uint16_t* k2, const uint16_t* v, int B, int T, int H,
                   int d_qk, int d_v, const double* lam, const float* gain,
                   double eps, double scale, int window, const int64_t* rows, int64_t n_rows,
                   double* o_pre, double* y, int nthreads) {
    if (B <= 0 || T <= 0 || H <= 0 || d_qk <= 0 || d_v <= 0 || window < 0) return -1;
    if (!rows && n_rows != (int64_t)B * T * H) return -1;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double* p1 = (double*)malloc(sizeof(double) * (size_t)T);
        double* p2 = (double*)malloc(sizeof(double) * (size_t)T);
        if (!p1 || !p2) {
            bad = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t flat = rows ? rows[r] : r;
                if (flat < 0 || flat >= (int64_t)B * T * H) { bad = 1; continue; }
                int h = (int)(flat % H);
                int64_t i = (flat / H) % T;
                int64_t b = flat / ((int64_t)H * T);
                int64_t first = (window > 0 && i + 1 > window) ? i + 1 - window : 0;
                int64_t qoff = ((b * T + i) * H + h) * d_qk;
                int64_t koff = ((b * T + first) * H + h) * (int64_t)d_qk;
                int64_t voff = ((b * T + first) * H + h) * (int64_t)d_v;
                diff_attention_row(q1 + qoff, q2 + qoff, k1 + koff, k2 + koff, v + voff,
                                   (int64_t)H * d_qk, (int64_t)H * d_v, i + 1 - first, d_qk, d_v,
                                   scale, lam[h], gain + (int64_t)h * d_v, eps, p1, p2,
                                   o_pre + r * d_v, y + r * d_v);
            }
        }
        free(p1);
        free(p2);
    }
    return bad ? -1 : 0;
}

/*
 * Decode: one query per (b, h) against a cache of length L.
 * q1, q2: bf16 [B, H, d_qk]; k1, k2: bf16 [B, L, H, d_qk]; v: bf16 [B, L, H, d_v].
 * seqlens: [B] cached lengths (NULL = L for all).  A length <= 0 leaves no
 * key to attend to and gives all-zero outputs.
 * window: > 0 attends only the last `window` positions.
 * ring = 0: slot p holds position p; a length above L counts as L.
 * ring != 0: the L slots are a ring buffer, position p in slot p % L, so the
 * length may exceed L; window 0 then means window L, and window > L is an
 * error (those positions are overwritten).  The visible positions are
 * gathered, oldest first, into a contiguous copy before the row is computed.
 * o_pre, y: fp64 [B, H, d_v].
 */
int oracle_decode(const uint16_t* q1, const uint16_t* q2, const uint16_t* k1,
                  const uint16_t* k2, const uint16_t* v, const int32_t* seqlens,
                  int B, int L, int H, int d_qk, int d_v, const double* lam,
                  const float* gain, double eps, double scale, int window, int ring,
                  double* o_pre, double* y, int nthreads) {
    if (B <= 0 || L <= 0 || H <= 0 || d_qk <= 0 || d_v <= 0 || window < 0) return -1;
    if (ring && window > L) return -1;
    if (ring && window == 0) window = L;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double* p1 = (double*)malloc(sizeof(double) * (size_t)L);
        double* p2 = (double*)malloc(sizeof(double) * (size_t)L);
        uint16_t* g1 = ring ? (uint16_t*)malloc(sizeof(uint16_t) * (size_t)L * d_qk) : NULL;
        uint16_t* g2 = ring ? (uint16_t*)malloc(sizeof(uint16_t) * (size_t)L * d_qk) : NULL;
        uint16_t* gv = ring ? (uint16_t*)malloc(sizeof(uint16_t) * (size_t)L * d_v) : NULL;
        if (!p1 || !p2 || (ring && (!g1 || !g2 || !gv))) {
            bad = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t r = 0; r < (int64_t)B * H; ++r) {
                int h = (int)(r % H);
                int64_t b = r / H;
                int64_t n = seqlens ? seqlens[b] : L;
                if (!ring && n > L) n = L;
                if (n <= 0) {
                    for (int c = 0; c < d_v; ++c) { o_pre[r * d_v + c] = 0.0; y[r * d_v + c] = 0.0; }
                    continue;
                }
                int64_t first = (window > 0 && n > window) ? n - window : 0;
                int64_t qoff = (b * H + h) * (int64_t)d_qk;
                if (ring) {
                    for (int64_t p = first; p < n; ++p) {
                        int64_t slot = p % L;
                        memcpy(g1 + (p - first) * d_qk, k1 + ((b * L + slot) * H + h) * d_qk, 2 * (size_t)d_qk);
                        memcpy(g2 + (p - first) * d_qk, k2 + ((b * L + slot) * H + h) * d_qk, 2 * (size_t)d_qk);
                        memcpy(gv + (p - first) * d_v, v + ((b * L + slot) * H + h) * d_v, 2 * (size_t)d_v);
                    }
                    diff_attention_row(q1 + qoff, q2 + qoff, g1, g2, gv, d_qk, d_v, n - first, d_qk, d_v,
                                       scale, lam[h], gain + (int64_t)h * d_v, eps, p1, p2,
                                       o_pre + r * d_v, y + r * d_v);
                    continue;
                }
                int64_t koff = ((b * L + first) * H + h) * (int64_t)d_qk;
                int64_t voff = ((b * L + first) * H + h) * (int64_t)d_v;
                diff_attention_row(q1 + qoff, q2 + qoff, k1 + koff, k2 + koff, v + voff,
                                   (int64_t)H * d_qk, (int64_t)H * d_v, n - first, d_qk, d_v, scale,
                                   lam[h], gain + (int64_t)h * d_v, eps, p1, p2,
                                   o_pre + r * d_v, y + r * d_v);
            }
        }
        free(p1);
        free(p2);
        free(g1);
        free(g2);
        free(gv);
    }
    return bad ? -1 : 0;
}
