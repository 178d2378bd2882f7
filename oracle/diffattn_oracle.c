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
 *   - rotary position embedding (Motif 2.6B explainer, section "The block":
 *     RoPE with base 500,000; the pages fix neither the pairing nor where it
 *     is applied): each d_qk-wide vector of Q1, Q2, K1, K2 is rotated on its
 *     own, pair c turning by the angle pos * theta^(-2c/d_qk), with either
 *     the split-half pairing (c, c + d_qk/2) or the interleaved pairing
 *     (2c, 2c + 1); token t of a prefill sits at position pos0 + t, and a
 *     decode query at pos0 + n - 1 (the cache holds keys already rotated);
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

/*
 * Rotary position embedding of one d-vector x (fp64, in place) at position
 * pos: pair c = (i0, i1) turns by the angle pos * theta^(-2c/d), i.e.
 * (x[i0], x[i1]) -> (x[i0] cos a - x[i1] sin a, x[i0] sin a + x[i1] cos a).
 * mode 1 pairs (c, c + d/2), mode 2 pairs (2c, 2c + 1); mode 0 leaves x.
 */
static void rope_rotate(double* x, int d, int mode, double theta, double pos) {
    if (mode == 0) return;
    for (int c = 0; c < d / 2; ++c) {
        double a = pos * pow(theta, -2.0 * c / d);
        double cs = cos(a), sn = sin(a);
        int i0 = mode == 1 ? c : 2 * c;
        int i1 = mode == 1 ? c + d / 2 : 2 * c + 1;
        double x0 = x[i0], x1 = x[i1];
        x[i0] = x0 * cs - x1 * sn;
        x[i1] = x0 * sn + x1 * cs;
    }
}

/* One d-vector of bf16 bits widened to fp64 and rotated at position pos. */
static void load_rotated(const uint16_t* src, double* dst, int d, int mode, double theta, double pos) {
    for (int c = 0; c < d; ++c) dst[c] = bf16_to_f64(src[c]);
    rope_rotate(dst, d, mode, theta, pos);
}

/*
 * Standalone rotation of x: bf16 [B, T, H, d] -> fp64 out [B, T, H, d], token
 * t of batch row b at position pos0 + (pos_start ? pos_start[b] : 0) + t.
 */
int oracle_rope(const uint16_t* x, double* out, int B, int T, int H, int d, int mode,
                double theta, int64_t pos0, const int32_t* pos_start) {
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || d % 2 || mode < 0 || mode > 2) return -1;
    if (mode && !(theta > 0)) return -1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t h = 0; h < H; ++h) {
                int64_t off = ((b * T + t) * H + h) * d;
                double pos = (double)(pos0 + (pos_start ? pos_start[b] : 0) + t);
                load_rotated(x + off, out + off, d, mode, theta, pos);
            }
    return 0;
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
 * Keys of one (b, h): either bf16 bits (b16) or, when rotated, fp64 values
 * (f64); element (j, c) at [j * stride + c].
 */
typedef struct {
    const uint16_t* b16;
    const double* f64;
} keys_t;

static inline double key_at(keys_t k, int64_t idx) { return k.f64 ? k.f64[idx] : bf16_to_f64(k.b16[idx]); }

/*
 * One query row.  q1, q2: the row's d_qk-vectors in fp64 (already rotated
 * when RoPE is on); k1, k2, v at key position 0 of this (b, h), with
 * `kstride`/`vstride` elements between consecutive positions.  p1 and p2 are
 * scratch of length >= n_keys.  Writes o[d_v] (pre-norm) and y[d_v] (after
 * GroupNorm).
 */
static void diff_attention_row(const double* q1, const double* q2, keys_t k1, keys_t k2, const uint16_t* v,
                               int64_t kstride, int64_t vstride, int64_t n_keys,
                               int d_qk, int d_v, double scale, double lam,
                               const float* gain, double eps,
                               double* p1, double* p2, double* o, double* y) {
    /* Scores of both maps over the causal range. */
    for (int64_t j = 0; j < n_keys; ++j) {
        double a = 0.0, b = 0.0;
        for (int c = 0; c < d_qk; ++c) {
            a += q1[c] * key_at(k1, j * kstride + c);
            b += q2[c] * key_at(k2, j * kstride + c);
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
 * sliding window of that many keys, 0 for every key <= i.  rope: 0 none,
 * 1 split-half, 2 interleaved pairs, base theta, token t at position pos0 + t.
 * rows: n_rows flat indices ((b * T + i) * H + h), or NULL for every row in
 * that order (then n_rows must be B*T*H).  o_pre, y: fp64 [n_rows, d_v].
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or -1 on bad arguments
 * or failed scratch allocation.
 */
int oracle_prefill(const uint16_t* q1, const uint16_t* q2, const uint16_t* k1,
                   const uint16_t* k2, const uint16_t* v, int B, int T, int H,
                   int d_qk, int d_v, const double* lam, const float* gain,
                   double eps, double scale, int window, int rope, double theta, int64_t pos0,
                   const int64_t* rows, int64_t n_rows, double* o_pre, double* y, int nthreads) {
    if (B <= 0 || T <= 0 || H <= 0 || d_qk <= 0 || d_v <= 0 || window < 0) return -1;
    if (rope < 0 || rope > 2 || (rope && (!(theta > 0) || d_qk % 2))) return -1;
    if (!rows && n_rows != (int64_t)B * T * H) return -1;
    /* With RoPE, every key is rotated once, up front, into fp64 copies. */
    double* k1r = NULL;
    double* k2r = NULL;
    if (rope) {
        size_t n = (size_t)B * T * H * d_qk;
        k1r = (double*)malloc(sizeof(double) * n);
        k2r = (double*)malloc(sizeof(double) * n);
        if (!k1r || !k2r) { free(k1r); free(k2r); return -1; }
        oracle_rope(k1, k1r, B, T, H, d_qk, rope, theta, pos0, NULL);
        oracle_rope(k2, k2r, B, T, H, d_qk, rope, theta, pos0, NULL);
    }
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double* p1 = (double*)malloc(sizeof(double) * (size_t)T);
        double* p2 = (double*)malloc(sizeof(double) * (size_t)T);
        double* qa = (double*)malloc(sizeof(double) * 2 * (size_t)d_qk);
        if (!p1 || !p2 || !qa) {
            bad = 1;
        } else {
            double* qb = qa + d_qk;
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
                load_rotated(q1 + qoff, qa, d_qk, rope, theta, (double)(pos0 + i));
                load_rotated(q2 + qoff, qb, d_qk, rope, theta, (double)(pos0 + i));
                keys_t kk1 = {k1 + koff, rope ? k1r + koff : NULL};
                keys_t kk2 = {k2 + koff, rope ? k2r + koff : NULL};
                diff_attention_row(qa, qb, kk1, kk2, v + voff,
                                   (int64_t)H * d_qk, (int64_t)H * d_v, i + 1 - first, d_qk, d_v,
                                   scale, lam[h], gain + (int64_t)h * d_v, eps, p1, p2,
                                   o_pre + r * d_v, y + r * d_v);
            }
        }
        free(p1);
        free(p2);
        free(qa);
    }
    free(k1r);
    free(k2r);
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
 * rope, theta, pos0: the query of sequence b is rotated at position
 * pos0 + n - 1; cached keys are used as given (already rotated).
 * o_pre, y: fp64 [B, H, d_v].
 */
int oracle_decode(const uint16_t* q1, const uint16_t* q2, const uint16_t* k1,
                  const uint16_t* k2, const uint16_t* v, const int32_t* seqlens,
                  int B, int L, int H, int d_qk, int d_v, const double* lam,
                  const float* gain, double eps, double scale, int window, int ring,
                  int rope, double theta, int64_t pos0, double* o_pre, double* y, int nthreads) {
    if (B <= 0 || L <= 0 || H <= 0 || d_qk <= 0 || d_v <= 0 || window < 0) return -1;
    if (rope < 0 || rope > 2 || (rope && (!(theta > 0) || d_qk % 2))) return -1;
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
        double* qa = (double*)malloc(sizeof(double) * 2 * (size_t)d_qk);
        if (!p1 || !p2 || !qa || (ring && (!g1 || !g2 || !gv))) {
            bad = 1;
        } else {
            double* qb = qa + d_qk;
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
                load_rotated(q1 + qoff, qa, d_qk, rope, theta, (double)(pos0 + n - 1));
                load_rotated(q2 + qoff, qb, d_qk, rope, theta, (double)(pos0 + n - 1));
                if (ring) {
                    for (int64_t p = first; p < n; ++p) {
                        int64_t slot = p % L;
                        memcpy(g1 + (p - first) * d_qk, k1 + ((b * L + slot) * H + h) * d_qk, 2 * (size_t)d_qk);
                        memcpy(g2 + (p - first) * d_qk, k2 + ((b * L + slot) * H + h) * d_qk, 2 * (size_t)d_qk);
                        memcpy(gv + (p - first) * d_v, v + ((b * L + slot) * H + h) * d_v, 2 * (size_t)d_v);
                    }
                    keys_t kk1 = {g1, NULL}, kk2 = {g2, NULL};
                    diff_attention_row(qa, qb, kk1, kk2, gv, d_qk, d_v, n - first, d_qk, d_v,
                                       scale, lam[h], gain + (int64_t)h * d_v, eps, p1, p2,
                                       o_pre + r * d_v, y + r * d_v);
                    continue;
                }
                int64_t koff = ((b * L + first) * H + h) * (int64_t)d_qk;
                int64_t voff = ((b * L + first) * H + h) * (int64_t)d_v;
                keys_t kk1 = {k1 + koff, NULL}, kk2 = {k2 + koff, NULL};
                diff_attention_row(qa, qb, kk1, kk2, v + voff,
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
        free(qa);
    }
    return bad ? -1 : 0;
}

/*
 * Grouped differential attention with token-wise lambda and an output gate
 * (picx.dev summary of the Motif 3 report, section 2.2, "Grouped Differential
 * Attention" and "Output Gating"): n_H heads split into n_S = g n_N signal
 * heads and n_N = n_H / (g + 1) noise heads.  Each head is ordinary causal
 * softmax attention with its own query, key and value, H = softmax(Q K^T
 * scale) V.  Signal head s is paired with noise head Repeat_g(s):
 *     D_s = H_S,s - lambda_t[s] * H_N,(s / g)
 *     out_s = sigmoid(G_s) * D_s          (elementwise over d_v; no gate: D_s)
 * Readings (the pages fix none of these): heads 0 .. n_S-1 are the signal
 * heads and n_S .. n_H-1 the noise heads; Repeat_g repeats each noise head g
 * times in place (signal head s uses noise head s / g); no GroupNorm follows
 * (the GDLA formula applies only the gate).
 * q, k: bf16 [B, T, n_H, d_qk]; v: bf16 [B, T, n_H, d_v]; lam: fp32 [B, T, n_S];
 * gate: fp32 [B, T, n_S, d_v] or NULL; rows: flat ((b * T + i) * n_S + s) or NULL
 * for all; out: fp64 [n_rows, d_v].
 */
static void head_row(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t kstride, int64_t vstride,
                     int64_t n_keys, int d_qk, int d_v, double scale, double* p, double* o) {
    for (int64_t j = 0; j < n_keys; ++j) {
        double a = 0.0;
        for (int c = 0; c < d_qk; ++c) a += bf16_to_f64(q[c]) * bf16_to_f64(k[j * kstride + c]);
        p[j] = scale * a;
    }
    softmax_inplace(p, n_keys);
    for (int c = 0; c < d_v; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j)
        for (int c = 0; c < d_v; ++c) o[c] += p[j] * bf16_to_f64(v[j * vstride + c]);
}

int oracle_grouped(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int T, int n_H, int g,
                   int d_qk, int d_v, const float* lam, const float* gate, double scale, const int64_t* rows,
                   int64_t n_rows, double* out, int nthreads) {
    if (B <= 0 || T <= 0 || n_H <= 0 || g <= 0 || n_H % (g + 1) || d_qk <= 0 || d_v <= 0) return -1;
    const int n_N = n_H / (g + 1), n_S = g * n_N;
    if (!rows && n_rows != (int64_t)B * T * n_S) return -1;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)T);
        double* hs = (double*)malloc(sizeof(double) * (size_t)d_v);
        double* hn = (double*)malloc(sizeof(double) * (size_t)d_v);
        if (!p || !hs || !hn) {
            bad = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t flat = rows ? rows[r] : r;
                if (flat < 0 || flat >= (int64_t)B * T * n_S) { bad = 1; continue; }
                int s = (int)(flat % n_S);
                int64_t i = (flat / n_S) % T;
                int64_t b = flat / ((int64_t)n_S * T);
                int hn_head = n_S + s / g;
                int64_t ks = (int64_t)n_H * d_qk, vs = (int64_t)n_H * d_v;
                head_row(q + ((b * T + i) * n_H + s) * d_qk, k + (b * T * n_H + s) * (int64_t)d_qk,
                         v + (b * T * n_H + s) * (int64_t)d_v, ks, vs, i + 1, d_qk, d_v, scale, p, hs);
                head_row(q + ((b * T + i) * n_H + hn_head) * d_qk, k + (b * T * n_H + hn_head) * (int64_t)d_qk,
                         v + (b * T * n_H + hn_head) * (int64_t)d_v, ks, vs, i + 1, d_qk, d_v, scale, p, hn);
                double l = (double)lam[(b * T + i) * n_S + s];
                for (int c = 0; c < d_v; ++c) {
                    double d = hs[c] - l * hn[c];
                    if (gate) {
                        double gv = (double)gate[((b * T + i) * n_S + s) * (int64_t)d_v + c];
                        d *= 1.0 / (1.0 + exp(-gv));
                    }
                    out[r * d_v + c] = d;
                }
            }
        }
        free(p);
        free(hs);
        free(hn);
    }
    return bad ? -1 : 0;
}
