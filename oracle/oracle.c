/*
 * CPU oracle for the batched causal long convolution -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the smoke check in __graft_entry__ and the cpu_baseline leg of bench.py
 * may load this library.  The product path (libspecconv) never links, loads or calls it,
 * and it shares no source, header, table or helper with the HIP kernels.
 *
 * What it computes (all plain definitions, no blocking, no fusion, no reordering):
 *
 *   oracle_conv_f64   r[t] = sum_{j=0..t} v[j] * g[t-j]          (float64)
 *                     s[t] = sum_{j=0..t} |v[j]| * |g[t-j]|       (float64, the error scale)
 *     The causal convolution that the Caracal notes ("Caracal: Causal Architecture via
 *     Spectral Mixing", key design 1, the multi-head Fourier module) state the frequency-
 *     domain product is equivalent to, and that key design 2 (the frequency-domain causal
 *     mask) says the pad-to-2L / truncate-to-L geometry reduces to.
 *
 *   oracle_conv_i64   the same sum in exact int64 arithmetic (reference for the exact
 *                     number-theoretic path of "Catastrophic Token Leakage in Convolutional
 *                     Sequence Modeling and How to Mitigate It", abstract).
 *
 *   oracle_conv_f64_at  the same sum for individually sampled (channel, t) outputs.
 *
 *   oracle_circular_dft_f64  the pages' recipe written out plainly: zero-pad both
 *                     sequences on the right to length n, take the O(n^2) DFT of each,
 *                     multiply bin by bin, take the O(n^2) inverse DFT (with 1/n), return
 *                     the real part of all n outputs (the caller truncates).  Used only to
 *                     pin the claim of key design 2 against the direct sum.
 *
 *   oracle_circular_ntt  the same recipe over Z_p: O(n^2) number-theoretic transforms with
 *                     omega = root^((p-1)/n), pointwise product, inverse with n^{-1} mod p.
 *                     Residues in [0, p).
 *
 *   oracle_conv_bwd_f64  the gradients of the scalar sum_t dr[t] r[t] with respect to v
 *                     and g (the pages' models are trained end to end with a next-token
 *                     loss, "Caracal", loss function / training strategy, so the
 *                     primitive's backward pass is needed):
 *                       dv[j] = sum_{t=j..L-1} dr[t] g[t-j],  dg[k] = sum_{t=k..L-1} dr[t] v[t-k]
 *                     with the error scales sv, sg (the same sums of absolute values).
 *
 *   oracle_conv_bwd_i64  the same two sums in exact int64.
 *
 *   oracle_conv_i128  r[t] = sum_{j<=t} v[j] * g[t-j] for int64 inputs in exact signed
 *                     128-bit arithmetic (returned as high and low 64-bit halves): the
 *                     exact sum of fixed-point encodings of real inputs, for the exactly
 *                     causal real-valued path (number-theoretic transforms on integers,
 *                     "Catastrophic Token Leakage ...", abstract, applied to real
 *                     activations through a fixed-point encoding).
 *
 * Loop order of the direct sums is "for j: for t >= j: r[t] += v[j]*g[t-j]" (an axpy per
 * input tap), which fixes the rounding order and touches r[t] only with v[0..t].  The
 * gradient sums run "for t: for j <= t: dv[j] += dr[t]*g[t-j]" (an axpy per output tap).
 * Build flags: -O2 -ffp-contract=off (no fused multiply-add contraction).
 *
 * Threads: channels are independent, so a channel range is given to each POSIX thread.
 * The result does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- thread helper */

typedef void (*chan_fn)(void *ctx, int64_t c);

typedef struct {
    chan_fn fn;
    void *ctx;
    int64_t c0, c1;
} span_t;

static void *run_span(void *p)
{
    span_t *s = (span_t *)p;
    for (int64_t c = s->c0; c < s->c1; ++c) s->fn(s->ctx, c);
    return NULL;
}

static int for_channels(chan_fn fn, void *ctx, int64_t nch, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nch) nthreads = (int)(nch > 0 ? nch : 1);
    if (nthreads == 1) {
        for (int64_t c = 0; c < nch; ++c) fn(ctx, c);
        return 0;
    }
    pthread_t tid[256];
    span_t span[256];
    int joined[256];
    for (int i = 0; i < nthreads; ++i) {
        span[i].fn = fn;
        span[i].ctx = ctx;
        span[i].c0 = nch * i / nthreads;
        span[i].c1 = nch * (i + 1) / nthreads;
        joined[i] = pthread_create(&tid[i], NULL, run_span, &span[i]) == 0;
        if (!joined[i]) run_span(&span[i]); /* no thread: run the span here */
    }
    for (int i = 0; i < nthreads; ++i)
        if (joined[i]) pthread_join(tid[i], NULL);
    return 0;
}

/* ---------------------------------------------------------------- float64 direct sum */

typedef struct {
    const double *v, *g;
    double *r, *s;
    int64_t L;
} f64_ctx;

static void conv_f64_channel(void *p, int64_t c)
{
    f64_ctx *k = (f64_ctx *)p;
    const int64_t L = k->L;
    const double *v = k->v + c * L;
    const double *g = k->g + c * L;
    double *r = k->r + c * L;
    double *s = k->s ? k->s + c * L : NULL;
    for (int64_t t = 0; t < L; ++t) r[t] = 0.0;
    if (s)
        for (int64_t t = 0; t < L; ++t) s[t] = 0.0;
    for (int64_t j = 0; j < L; ++j) {
        const double vj = v[j];
        for (int64_t t = j; t < L; ++t) r[t] += vj * g[t - j];
        if (s) {
            const double aj = fabs(vj);
            for (int64_t t = j; t < L; ++t) s[t] += aj * fabs(g[t - j]);
        }
    }
}

/* r, s: [nch][L]; s may be NULL.  Returns 0, or -1 on a bad argument. */
int oracle_conv_f64(const double *v, const double *g, double *r, double *s, int64_t nch,
                    int64_t L, int nthreads)
{
    if (nch < 0 || L < 0) return -1;
    if (nch == 0 || L == 0) return 0;
    if (!v || !g || !r) return -1;
    f64_ctx k = {v, g, r, s, L};
    return for_channels(conv_f64_channel, &k, nch, nthreads);
}

/* ---------------------------------------------------------------- int64 direct sum */

typedef struct {
    const int64_t *v, *g;
    int64_t *r;
    int64_t L;
} i64_ctx;

static void conv_i64_channel(void *p, int64_t c)
{
    i64_ctx *k = (i64_ctx *)p;
    const int64_t L = k->L;
    const int64_t *v = k->v + c * L;
    const int64_t *g = k->g + c * L;
    int64_t *r = k->r + c * L;
    for (int64_t t = 0; t < L; ++t) r[t] = 0;
    for (int64_t j = 0; j < L; ++j) {
        const int64_t vj = v[j];
        for (int64_t t = j; t < L; ++t) r[t] += vj * g[t - j];
    }
}

/* Exact while every partial sum fits in int64 (callers keep |v|,|g| small). */
int oracle_conv_i64(const int64_t *v, const int64_t *g, int64_t *r, int64_t nch, int64_t L,
                    int nthreads)
{
    if (nch < 0 || L < 0) return -1;
    if (nch == 0 || L == 0) return 0;
    if (!v || !g || !r) return -1;
    i64_ctx k = {v, g, r, L};
    return for_channels(conv_i64_channel, &k, nch, nthreads);
}

/* ---------------------------------------------------------------- gradients */

typedef struct {
    const double *dr, *v, *g;
    double *dv, *dg, *sv, *sg;
    int64_t L;
} bwd_f64_ctx;

static void bwd_f64_channel(void *p, int64_t c)
{
    bwd_f64_ctx *k = (bwd_f64_ctx *)p;
    const int64_t L = k->L;
    const double *dr = k->dr + c * L, *v = k->v + c * L, *g = k->g + c * L;
    double *dv = k->dv + c * L, *dg = k->dg + c * L;
    double *sv = k->sv ? k->sv + c * L : NULL, *sg = k->sg ? k->sg + c * L : NULL;
    for (int64_t j = 0; j < L; ++j) dv[j] = dg[j] = 0.0;
    if (sv)
        for (int64_t j = 0; j < L; ++j) sv[j] = sg[j] = 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const double d = dr[t];
        for (int64_t j = 0; j <= t; ++j) {
            dv[j] += d * g[t - j];
            dg[j] += d * v[t - j];
        }
        if (sv) {
            const double a = fabs(d);
            for (int64_t j = 0; j <= t; ++j) {
                sv[j] += a * fabs(g[t - j]);
                sg[j] += a * fabs(v[t - j]);
            }
        }
    }
}

/* dv, dg (and sv, sg when not NULL): [nch][L].  Returns 0, or -1 on a bad argument. */
int oracle_conv_bwd_f64(const double *dr, const double *v, const double *g, double *dv,
                        double *dg, double *sv, double *sg, int64_t nch, int64_t L,
                        int nthreads)
{
    if (nch < 0 || L < 0) return -1;
    if (nch == 0 || L == 0) return 0;
    if (!dr || !v || !g || !dv || !dg || (!sv) != (!sg)) return -1;
    bwd_f64_ctx k = {dr, v, g, dv, dg, sv, sg, L};
    return for_channels(bwd_f64_channel, &k, nch, nthreads);
}

typedef struct {
    const int64_t *dr, *v, *g;
    int64_t *dv, *dg;
    int64_t L;
} bwd_i64_ctx;

static void bwd_i64_channel(void *p, int64_t c)
{
    bwd_i64_ctx *k = (bwd_i64_ctx *)p;
    const int64_t L = k->L;
    const int64_t *dr = k->dr + c * L, *v = k->v + c * L, *g = k->g + c * L;
    int64_t *dv = k->dv + c * L, *dg = k->dg + c * L;
    for (int64_t j = 0; j < L; ++j) dv[j] = dg[j] = 0;
    for (int64_t t = 0; t < L; ++t) {
        const int64_t d = dr[t];
        for (int64_t j = 0; j <= t; ++j) {
            dv[j] += d * g[t - j];
            dg[j] += d * v[t - j];
        }
    }
}

/* Exact while every partial sum fits in int64. */
int oracle_conv_bwd_i64(const int64_t *dr, const int64_t *v, const int64_t *g, int64_t *dv,
                        int64_t *dg, int64_t nch, int64_t L, int nthreads)
{
    if (nch < 0 || L < 0) return -1;
    if (nch == 0 || L == 0) return 0;
    if (!dr || !v || !g || !dv || !dg) return -1;
    bwd_i64_ctx k = {dr, v, g, dv, dg, L};
    return for_channels(bwd_i64_channel, &k, nch, nthreads);
}

/* ---------------------------------------------------------------- int128 direct sum */

typedef struct {
    const int64_t *v, *g;
    int64_t *hi;
    uint64_t *lo;
    int64_t L;
} i128_ctx;

static void conv_i128_channel(void *p, int64_t c)
{
    i128_ctx *k = (i128_ctx *)p;
    const int64_t L = k->L;
    const int64_t *v = k->v + c * L, *g = k->g + c * L;
    __int128 *acc = (__int128 *)calloc((size_t)(L > 0 ? L : 1), sizeof(__int128));
    if (!acc) return;
    for (int64_t j = 0; j < L; ++j) {
        const __int128 vj = v[j];
        for (int64_t t = j; t < L; ++t) acc[t] += vj * (__int128)g[t - j];
    }
    for (int64_t t = 0; t < L; ++t) {
        const unsigned __int128 u = (unsigned __int128)acc[t];
        k->lo[c * L + t] = (uint64_t)u;
        k->hi[c * L + t] = (int64_t)(uint64_t)(u >> 64);
    }
    free(acc);
}

/* Exact while |v|, |g| < 2^63 and every partial sum fits in 127 bits.  r = hi * 2^64 + lo. */
int oracle_conv_i128(const int64_t *v, const int64_t *g, int64_t *hi, uint64_t *lo, int64_t nch,
                     int64_t L, int nthreads)
{
    if (nch < 0 || L < 0) return -1;
    if (nch == 0 || L == 0) return 0;
    if (!v || !g || !hi || !lo) return -1;
    i128_ctx k = {v, g, hi, lo, L};
    return for_channels(conv_i128_channel, &k, nch, nthreads);
}

/* ---------------------------------------------------------------- sampled outputs */

/* For each sample i: r[i] = sum_{j=0..t} v[c*L + j] * g[c*L + t - j], s[i] likewise with
 * absolute values, where c = ch[i], t = tt[i].  s may be NULL. */
int oracle_conv_f64_at(const double *v, const double *g, int64_t L, const int64_t *ch,
                       const int64_t *tt, int64_t npts, double *r, double *s)
{
    if (L <= 0 || npts < 0) return -1;
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t c = ch[i], t = tt[i];
        if (c < 0 || t < 0 || t >= L) return -1;
        const double *vc = v + c * L;
        const double *gc = g + c * L;
        double acc = 0.0, sacc = 0.0;
        for (int64_t j = 0; j <= t; ++j) {
            acc += vc[j] * gc[t - j];
            sacc += fabs(vc[j]) * fabs(gc[t - j]);
        }
        r[i] = acc;
        if (s) s[i] = sacc;
    }
    return 0;
}

/* ---------------------------------------------------------------- naive DFT recipe */

/* v, g: length L (L <= n).  out: n real values of the inverse DFT of DFT(v0) * DFT(g0),
 * where v0, g0 are v, g zero-padded on the right to length n.  O(n^2), float64. */
int oracle_circular_dft_f64(const double *v, const double *g, int64_t L, int64_t n,
                            double *out)
{
    if (L < 0 || n <= 0 || L > n) return -1;
    double *vr = calloc((size_t)n, sizeof(double)), *vi = calloc((size_t)n, sizeof(double));
    double *gr = calloc((size_t)n, sizeof(double)), *gi = calloc((size_t)n, sizeof(double));
    if (!vr || !vi || !gr || !gi) {
        free(vr); free(vi); free(gr); free(gi);
        return -1;
    }
    const double two_pi = 6.283185307179586476925286766559;
    for (int64_t k = 0; k < n; ++k) {
        double ar = 0, ai = 0, br = 0, bi = 0;
        for (int64_t m = 0; m < L; ++m) {
            /* exponent e^{-2 pi i m k / n}; reduce m*k mod n first for accuracy */
            const double ang = -two_pi * (double)((m * k) % n) / (double)n;
            const double c = cos(ang), sn = sin(ang);
            ar += v[m] * c;
            ai += v[m] * sn;
            br += g[m] * c;
            bi += g[m] * sn;
        }
        /* X_k = V_k * G_k */
        vr[k] = ar * br - ai * bi;
        vi[k] = ar * bi + ai * br;
    }
    for (int64_t m = 0; m < n; ++m) {
        double acc = 0;
        for (int64_t k = 0; k < n; ++k) {
            const double ang = two_pi * (double)((m * k) % n) / (double)n;
            /* real part of X_k e^{+2 pi i m k / n} */
            acc += vr[k] * cos(ang) - vi[k] * sin(ang);
        }
        out[m] = acc / (double)n;
    }
    free(vr); free(vi); free(gr); free(gi);
    return 0;
}

/* ---------------------------------------------------------------- naive NTT recipe */

static uint64_t mulmod(uint64_t a, uint64_t b, uint64_t p) { return (a * b) % p; }

static uint64_t powmod(uint64_t b, uint64_t e, uint64_t p)
{
    uint64_t r = 1 % p;
    b %= p;
    while (e) {
        if (e & 1) r = mulmod(r, b, p);
        b = mulmod(b, b, p);
        e >>= 1;
    }
    return r;
}

/* v, g: length L signed integers, reduced into [0,p).  out: n residues in [0,p) of the
 * inverse NTT of NTT(v0) * NTT(g0) over Z_p with omega = root^((p-1)/n).  Requires
 * p < 2^32 (so products fit in uint64) and n | p-1.  O(n^2). */
int oracle_circular_ntt(const int64_t *v, const int64_t *g, int64_t L, int64_t n,
                        uint32_t p, uint32_t root, int64_t *out)
{
    if (L < 0 || n <= 0 || L > n || p < 3) return -1;
    if ((uint64_t)(p - 1) % (uint64_t)n != 0) return -1;
    uint64_t *a = calloc((size_t)n, sizeof(uint64_t)), *b = calloc((size_t)n, sizeof(uint64_t));
    uint64_t *x = calloc((size_t)n, sizeof(uint64_t));
    if (!a || !b || !x) {
        free(a); free(b); free(x);
        return -1;
    }
    const uint64_t P = p;
    for (int64_t m = 0; m < L; ++m) {
        int64_t vm = v[m] % (int64_t)P, gm = g[m] % (int64_t)P;
        a[m] = (uint64_t)(vm < 0 ? vm + (int64_t)P : vm);
        b[m] = (uint64_t)(gm < 0 ? gm + (int64_t)P : gm);
    }
    const uint64_t w = powmod(root, (P - 1) / (uint64_t)n, P);
    const uint64_t winv = powmod(w, P - 2, P);
    const uint64_t ninv = powmod((uint64_t)n % P, P - 2, P);
    for (int64_t k = 0; k < n; ++k) {
        uint64_t A = 0, B = 0;
        for (int64_t m = 0; m < n; ++m) {
            const uint64_t wk = powmod(w, (uint64_t)((m * k) % n), P);
            A = (A + mulmod(a[m], wk, P)) % P;
            B = (B + mulmod(b[m], wk, P)) % P;
        }
        x[k] = mulmod(A, B, P);
    }
    for (int64_t m = 0; m < n; ++m) {
        uint64_t acc = 0;
        for (int64_t k = 0; k < n; ++k)
            acc = (acc + mulmod(x[k], powmod(winv, (uint64_t)((m * k) % n), P), P)) % P;
        out[m] = (int64_t)mulmod(acc, ninv, P);
    }
    free(a); free(b); free(x);
    return 0;
}

int oracle_abi_version(void) { return 1; }
