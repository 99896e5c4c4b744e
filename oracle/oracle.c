/*
 * oracle.c -- fp64 CPU oracle for Parallax attention.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no source,
 * header, helper or table with the GPU library and includes none of it.
 * Parity pinned: every function here is checked in the CPU test suite
 * against closed forms, a library attention routine, a weighted
 * least-squares intercept and hand-derived fixtures.
 *
 * What is computed. The zubnet.ai news item on Parallax (second paragraph)
 * states that the layer output is softmax attention minus a projected
 * covariance term: the key-value covariance is contracted with a learned probe
 * rho_i = W_R x_i, and W_R = 0 gives back plain softmax attention. The
 * q2bstudio page ("Parallax: Atencion Local Lineal que Mantiene Softmax y
 * Corrige", second paragraph) describes the same sum of softmax attention
 * and a learned projection of the key-value covariance.
 *
 * For one query i with key set J_i:
 *   s_j   = scale * (q_i . k_j)
 *   p_j   = softmax_j(s)                      (max-subtracted)
 *   vbar  = sum_j p_j v_j ,  kbar = sum_j p_j k_j
 *   C     = sum_j p_j (v_j - vbar)(k_j - kbar)^T          (D x D, explicit)
 *   o_i   = vbar - C rho_i
 *
 * Readings where the pages are silent (each is also pinned by a test):
 *   - covariance is centred and weighted by the same softmax weights,
 *     with no n/(n-1) factor;
 *   - rho contracts the key side of C, so C rho is a value-space vector;
 *   - the softmax scale multiplies q.k only, rho is used unscaled;
 *   - causal prefill lets query i see keys 0..i;
 *   - an empty key set gives a zero output row.
 *
 * The one-pass functions (oracle_decode_partial_f64, oracle_merge_f64,
 * oracle_decode_onepass_f64) restate the same output through the identity
 * C rho = sum_j p_j r_j v_j - rbar vbar with r_j = rho . k_j, accumulated by
 * online softmax; the pages say both branches share one pass over K and V
 * (zubnet.ai item, second paragraph; encorp.ai blog "Integraciones de IA
 * personalizadas tras la atencion Parallax", section on Hopper GPUs).
 *
 * oracle_bwd_f64 is the gradient of the prefill output with respect to q, k,
 * v and rho, obtained by the chain rule on the one-pass form of the same
 * output, o = vbar (1 + rbar) - u with rbar = sum_j p_j r_j and
 * u = sum_j p_j r_j v_j (the pages give no backward pass; the derivative of
 * the forward definition is unique). Its pins do not reuse these formulas:
 * central finite differences of oracle_fwd_f64, the closed form
 * d rho_i = -C_i^T g_i (o is linear in rho), shift invariances, and a
 * library autograd of plain softmax attention at rho = 0.
 *
 * oracle_lla_probe_f64 is the probe that exact Local Linear Attention would
 * use, for comparison (the pages say Parallax replaces LLA's per-query
 * conjugate-gradient solve with the learned projection W_R: encorp.ai blog,
 * the paragraph on removing the solver; zubnet.ai item, first paragraph, on
 * LLA as a local linear estimate). Reading taken: the local linear fit at
 * the query, v ~ a + B (k - q) weighted by the softmax weights with a ridge
 * penalty lam |B|^2 on the slope, whose intercept is
 *   a = vbar - C (S + lam I)^-1 (kbar - q),  S = sum_j p_j (k_j - kbar)(k_j - kbar)^T,
 * i.e. the Parallax output with rho = (S + lam I)^-1 (kbar - q). The system is
 * solved by conjugate gradient without forming S: every product streams the
 * query's keys once more. Pinned against the intercept of a textbook
 * weighted least-squares fit with the ridge rows appended, and closed forms.
 *
 * Everything is double precision. Nothing is blocked, fused or reordered
 * beyond the formulas above.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 * ORACLE_MUTANT=<n> builds a deliberately wrong variant used only by the
 * mutation test that checks the pins catch plausible mistakes (n = 20: an
 * out-of-bounds read with unchanged results, which only the sanitizer build
 * catches).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* Explicit two-pass Parallax output for one query.
 * K, V: n rows with row strides ks, vs (in elements); D columns contiguous.
 * work: n + 2*D + D*D doubles. */
static void one_query(const double *qi, const double *rhoi, const double *K,
                      long ks, const double *V, long vs, long n, int D,
                      double scale, double *out, double *work) {
    if (n <= 0) {
        for (int a = 0; a < D; ++a) out[a] = 0.0;
        return;
    }
    double *p = work;
    double *vbar = p + n;
    double *kbar = vbar + D;
    double *C = kbar + D;
#if ORACLE_MUTANT == 20
    {   /* mutant for the sanitizer test: reads one double before the work
           buffer; the result is unchanged, only a memory checker sees it */
        volatile double before = work[-1];
        (void)before;
    }
#endif

    /* logits and their maximum */
    double m = -INFINITY;
    for (long j = 0; j < n; ++j) {
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += qi[d] * K[j * ks + d];
#if ORACLE_MUTANT == 6
        (void)scale;           /* mutant: scale dropped from the logits */
#else
        s *= scale;
#endif
        p[j] = s;
        if (s > m) m = s;
    }
    /* softmax weights */
    double z = 0.0;
    for (long j = 0; j < n; ++j) {
        p[j] = exp(p[j] - m);
        z += p[j];
    }
    for (long j = 0; j < n; ++j) p[j] /= z;

    /* weighted means of values and keys */
    for (int a = 0; a < D; ++a) { vbar[a] = 0.0; kbar[a] = 0.0; }
    for (long j = 0; j < n; ++j) {
        for (int a = 0; a < D; ++a) {
            vbar[a] += p[j] * V[j * vs + a];
            kbar[a] += p[j] * K[j * ks + a];
        }
    }

    /* explicit weighted value-key covariance, C[a][b] (value a, key b) */
    memset(C, 0, sizeof(double) * (size_t)D * (size_t)D);
    for (long j = 0; j < n; ++j) {
#if ORACLE_MUTANT == 7
        double w = 1.0 / (double)n;   /* mutant: uniform weights */
#else
        double w = p[j];
#endif
        for (int a = 0; a < D; ++a) {
#if ORACLE_MUTANT == 3
            double dv = w * V[j * vs + a];          /* mutant: uncentred */
#else
            double dv = w * (V[j * vs + a] - vbar[a]);
#endif
            for (int b = 0; b < D; ++b) {
#if ORACLE_MUTANT == 3
                C[(size_t)a * D + b] += dv * K[j * ks + b];
#else
                C[(size_t)a * D + b] += dv * (K[j * ks + b] - kbar[b]);
#endif
            }
        }
    }
#if ORACLE_MUTANT == 4
    if (n > 1)  /* mutant: Bessel factor */
        for (long e = 0; e < (long)D * D; ++e) C[e] *= (double)n / (double)(n - 1);
#endif

    /* o = vbar - C rho */
    for (int a = 0; a < D; ++a) {
        double acc = 0.0;
        for (int b = 0; b < D; ++b) {
#if ORACLE_MUTANT == 2
            acc += C[(size_t)b * D + a] * rhoi[b];   /* mutant: C transposed */
#elif ORACLE_MUTANT == 10
            acc += C[(size_t)a * D + b] * qi[b];     /* mutant: q instead of rho */
#else
            acc += C[(size_t)a * D + b] * rhoi[b];
#endif
        }
#if ORACLE_MUTANT == 1
        out[a] = vbar[a] + acc;                      /* mutant: sign */
#elif ORACLE_MUTANT == 5
        out[a] = vbar[a] - scale * acc;              /* mutant: scaled probe */
#else
        out[a] = vbar[a] - acc;
#endif
    }
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Decode: one query per (b, h) against a cache.
 * q, rho: [B, H, D]; k, v: [B, H, Lmax, D]; out: [B, H, D]; all contiguous.
 * seqlens: int32[B] or NULL (then every sequence has Lmax keys). Positions
 * at or beyond seqlens[b] are not read. */
int oracle_decode_f64(const double *q, const double *rho, const double *k,
                      const double *v, const int32_t *seqlens, double *out,
                      int B, int H, int D, long Lmax, double scale,
                      int nthreads) {
    if (B < 0 || H < 0 || D <= 0 || Lmax < 0) return 1;
    set_threads(nthreads);
    long nbh = (long)B * H;
    int err = 0;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) *
                                        ((size_t)Lmax + 2 * (size_t)D + (size_t)D * D + 1));
        if (!work) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long bh = 0; bh < nbh; ++bh) {
                long b = bh / H;
                long n = seqlens ? (long)seqlens[b] : Lmax;
                if (n > Lmax) n = Lmax;
                const double *kb = k + bh * Lmax * D;
                const double *vb = v + bh * Lmax * D;
                one_query(q + bh * D, rho + bh * D, kb, D, vb, D, n, D, scale,
                          out + bh * D, work);
            }
            free(work);
        }
    }
    return err;
}

/* Prefill over [B, N, H, D] contiguous tensors. Query i sees keys 0..i when
 * causal != 0, all N keys otherwise. */
int oracle_fwd_f64(const double *q, const double *k, const double *v,
                   const double *rho, double *out, int B, int N, int H, int D,
                   double scale, int causal, int nthreads) {
    if (B < 0 || N < 0 || H < 0 || D <= 0) return 1;
    set_threads(nthreads);
    long rs = (long)H * D;                 /* stride between positions */
    long total = (long)B * N * H;
    int err = 0;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) *
                                        ((size_t)N + 2 * (size_t)D + (size_t)D * D + 1));
        if (!work) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (long t = 0; t < total; ++t) {
                long h = t % H;
                long i = (t / H) % N;
                long b = t / ((long)H * N);
                long n;
#if ORACLE_MUTANT == 8
                n = causal ? i : N;                /* mutant: diagonal excluded */
#else
                n = causal ? i + 1 : N;
#endif
                const double *base_k = k + b * (long)N * rs + h * D;
                const double *base_v = v + b * (long)N * rs + h * D;
                long off = ((b * N + i) * (long)H + h) * D;
                one_query(q + off, rho + off, base_k, rs, base_v, rs, n, D,
                          scale, out + off, work);
            }
            free(work);
        }
    }
    return err;
}

/* Selected prefill rows. rows: nrows triples (b, i, h) as int64; out: [nrows, D]. */
int oracle_fwd_rows_f64(const double *q, const double *k, const double *v,
                        const double *rho, const int64_t *rows, long nrows,
                        double *out, int B, int N, int H, int D, double scale,
                        int causal, int nthreads) {
    if (B < 0 || N < 0 || H < 0 || D <= 0 || nrows < 0) return 1;
    for (long r = 0; r < nrows; ++r) {
        int64_t b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
        if (b < 0 || b >= B || i < 0 || i >= N || h < 0 || h >= H) return 1;
    }
    set_threads(nthreads);
    long rs = (long)H * D;
    int err = 0;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) *
                                        ((size_t)N + 2 * (size_t)D + (size_t)D * D + 1));
        if (!work) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long r = 0; r < nrows; ++r) {
                long b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
                long n = causal ? i + 1 : N;
                const double *base_k = k + b * (long)N * rs + h * D;
                const double *base_v = v + b * (long)N * rs + h * D;
                long off = ((b * N + i) * (long)H + h) * D;
                one_query(q + off, rho + off, base_k, rs, base_v, rs, n, D,
                          scale, out + r * D, work);
            }
            free(work);
        }
    }
    return err;
}

/* ---------------------------------------------------------------------
 * One-pass form. State for a key range: [m, l, A_r, A_v[D], A_rv[D]] with
 *   l = sum e^{s-m},  A_r = sum e^{s-m} r,  A_v = sum e^{s-m} v,
 *   A_rv = sum e^{s-m} r v,   r = rho . k,   s = scale * q . k.
 * Keys are consumed in chunks of `chunk`; before a chunk the running max is
 * raised to cover it and the sums are rescaled by e^{m_old - m_new}.
 * An empty range gives m = -inf and zero sums.
 * --------------------------------------------------------------------- */
int oracle_decode_partial_f64(const double *qi, const double *rhoi,
                              const double *K, const double *V, long j0,
                              long j1, int D, double scale, long chunk,
                              double *state) {
    if (D <= 0 || chunk <= 0) return 1;
    double m = -INFINITY, l = 0.0, ar = 0.0;
    double *av = state + 3;
    double *arv = state + 3 + D;
    for (int a = 0; a < D; ++a) { av[a] = 0.0; arv[a] = 0.0; }
    for (long c0 = j0; c0 < j1; c0 += chunk) {
        long c1 = c0 + chunk < j1 ? c0 + chunk : j1;
        double mc = m;
        for (long j = c0; j < c1; ++j) {
            double s = 0.0;
            for (int d = 0; d < D; ++d) s += qi[d] * K[j * D + d];
            s *= scale;
            if (s > mc) mc = s;
        }
        double alpha = (m == -INFINITY) ? 0.0 : exp(m - mc);
        l *= alpha;
        ar *= alpha;
        for (int a = 0; a < D; ++a) { av[a] *= alpha; arv[a] *= alpha; }
        m = mc;
        for (long j = c0; j < c1; ++j) {
            double s = 0.0, r = 0.0;
            for (int d = 0; d < D; ++d) {
                s += qi[d] * K[j * D + d];
                r += rhoi[d] * K[j * D + d];
            }
            double p = exp(s * scale - m);
            l += p;
            ar += p * r;
            for (int a = 0; a < D; ++a) {
                av[a] += p * V[j * D + a];
                arv[a] += p * r * V[j * D + a];
            }
        }
    }
    state[0] = m;
    state[1] = l;
    state[2] = ar;
    return 0;
}

/* Merge nstates partial states (each 3 + 2D doubles) and finish:
 *   vbar = A_v / l, rbar = A_r / l, o = vbar (1 + rbar) - A_rv / l.
 * All-empty input gives zeros. */
int oracle_merge_f64(const double *states, int nstates, int D, double *out) {
    if (D <= 0 || nstates < 0) return 1;
    long w = 3 + 2L * D;
    double m = -INFINITY;
    for (int s = 0; s < nstates; ++s)
        if (states[s * w] > m) m = states[s * w];
    if (m == -INFINITY) {
        for (int a = 0; a < D; ++a) out[a] = 0.0;
        return 0;
    }
    double l = 0.0, ar = 0.0;
    for (int s = 0; s < nstates; ++s) {
        const double *st = states + s * w;
        if (st[0] == -INFINITY) continue;
        double f = exp(st[0] - m);
        l += f * st[1];
        ar += f * st[2];
    }
    for (int a = 0; a < D; ++a) {
        double av = 0.0, arv = 0.0;
        for (int s = 0; s < nstates; ++s) {
            const double *st = states + s * w;
            if (st[0] == -INFINITY) continue;
            double f = exp(st[0] - m);
            av += f * st[3 + a];
            arv += f * st[3 + D + a];
        }
        double vbar = av / l;
        out[a] = vbar * (1.0 + ar / l) - arv / l;
    }
    return 0;
}

/* One-pass decode over whole arrays (same layout as oracle_decode_f64). */
int oracle_decode_onepass_f64(const double *q, const double *rho,
                              const double *k, const double *v,
                              const int32_t *seqlens, double *out, int B,
                              int H, int D, long Lmax, double scale,
                              long chunk, int nthreads) {
    if (B < 0 || H < 0 || D <= 0 || Lmax < 0 || chunk <= 0) return 1;
    set_threads(nthreads);
    long nbh = (long)B * H;
    int err = 0;
#pragma omp parallel
    {
        double *st = (double *)malloc(sizeof(double) * (3 + 2 * (size_t)D));
        if (!st) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long bh = 0; bh < nbh; ++bh) {
                long b = bh / H;
                long n = seqlens ? (long)seqlens[b] : Lmax;
                if (n > Lmax) n = Lmax;
                if (n < 0) n = 0;
                oracle_decode_partial_f64(q + bh * D, rho + bh * D,
                                          k + bh * Lmax * D, v + bh * Lmax * D,
                                          0, n, D, scale, chunk, st);
                oracle_merge_f64(st, 1, D, out + bh * D);
            }
            free(st);
        }
    }
    return err;
}

/* Backward of the prefill forward for the loss L = sum_i dout_i . o_i.
 * All tensors [B, N, H, D] contiguous; dq, dk, dv, drho are overwritten.
 * For query i with visible keys j (g = dout_i, sigma = scale):
 *   s_j = sigma q_i.k_j,  p = softmax(s),  r_j = rho_i.k_j
 *   vbar = sum p_j v_j,  rbar = sum p_j r_j,  u = sum p_j r_j v_j,
 *   o = vbar (1 + rbar) - u                        (= vbar - C rho_i)
 *   a_j = g.v_j,  b = g.vbar
 *   dL/dp_j  = a_j (1 + rbar - r_j) + b r_j
 *   dL/ds_j  = p_j (dL/dp_j - sum_l p_l dL/dp_l),  sum_l p_l dL/dp_l = g.o + rbar b
 *   dL/dr_j  = p_j (b - a_j)
 *   dq_i   += sigma dL/ds_j k_j          drho_i += dL/dr_j k_j
 *   dk_j   += sigma dL/ds_j q_i + dL/dr_j rho_i
 *   dv_j   += p_j (1 + rbar - r_j) g
 * An empty key set contributes nothing. */
int oracle_bwd_f64(const double *q, const double *k, const double *v,
                   const double *rho, const double *dout, double *dq,
                   double *dk, double *dv, double *drho, int B, int N, int H,
                   int D, double scale, int causal, int nthreads) {
    if (B < 0 || N < 0 || H < 0 || D <= 0) return 1;
    set_threads(nthreads);
    long rs = (long)H * D;
    size_t all = (size_t)B * (size_t)N * (size_t)rs;
    memset(dq, 0, sizeof(double) * all);
    memset(dk, 0, sizeof(double) * all);
    memset(dv, 0, sizeof(double) * all);
    memset(drho, 0, sizeof(double) * all);
    long nbh = (long)B * H;
    int err = 0;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * (3 * (size_t)N + 3 * (size_t)D + 1));
        if (!work) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long bh = 0; bh < nbh; ++bh) {
                long b = bh / H, h = bh % H;
                double *p = work, *r = p + N, *a = r + N;
                double *vbar = a + N, *u = vbar + D, *o = u + D;
                const long base = b * (long)N * rs + h * D;  /* row 0 of (b, h) */
                for (long i = 0; i < N; ++i) {
                    const long n = causal ? i + 1 : N;
                    const double *qi = q + base + i * rs;
                    const double *ri = rho + base + i * rs;
                    const double *g = dout + base + i * rs;
                    /* forward quantities */
                    double m = -INFINITY;
                    for (long j = 0; j < n; ++j) {
                        const double *kj = k + base + j * rs;
                        double sq = 0.0, sr = 0.0;
                        for (int d = 0; d < D; ++d) { sq += qi[d] * kj[d]; sr += ri[d] * kj[d]; }
                        p[j] = scale * sq;
                        r[j] = sr;
                        if (p[j] > m) m = p[j];
                    }
                    double z = 0.0;
                    for (long j = 0; j < n; ++j) { p[j] = exp(p[j] - m); z += p[j]; }
                    for (long j = 0; j < n; ++j) p[j] /= z;
                    double rbar = 0.0;
                    for (int d = 0; d < D; ++d) { vbar[d] = 0.0; u[d] = 0.0; }
                    for (long j = 0; j < n; ++j) {
                        const double *vj = v + base + j * rs;
                        rbar += p[j] * r[j];
                        for (int d = 0; d < D; ++d) {
                            vbar[d] += p[j] * vj[d];
                            u[d] += p[j] * r[j] * vj[d];
                        }
                    }
                    for (int d = 0; d < D; ++d) o[d] = vbar[d] * (1.0 + rbar) - u[d];
                    /* incoming gradient projections */
                    double bg = 0.0, go = 0.0;
                    for (int d = 0; d < D; ++d) { bg += g[d] * vbar[d]; go += g[d] * o[d]; }
#if ORACLE_MUTANT == 15
                    const double Dsum = go;                  /* mutant: rbar b dropped */
#else
                    const double Dsum = go + rbar * bg;
#endif
                    for (long j = 0; j < n; ++j) {
                        const double *vj = v + base + j * rs;
                        double aj = 0.0;
                        for (int d = 0; d < D; ++d) aj += g[d] * vj[d];
                        a[j] = aj;
                    }
                    double *dqi = dq + base + i * rs;
                    double *dri = drho + base + i * rs;
                    for (long j = 0; j < n; ++j) {
#if ORACLE_MUTANT == 11
                        const double dp = a[j] * (1.0 + rbar - r[j]);   /* mutant: b r dropped */
#else
                        const double dp = a[j] * (1.0 + rbar - r[j]) + bg * r[j];
#endif
                        const double ds = p[j] * (dp - Dsum);
#if ORACLE_MUTANT == 12
                        const double dr = p[j] * (a[j] - bg);           /* mutant: sign */
#else
                        const double dr = p[j] * (bg - a[j]);
#endif
#if ORACLE_MUTANT == 14
                        const double wv = p[j] * (1.0 + r[j] - rbar);   /* mutant: swapped */
#else
                        const double wv = p[j] * (1.0 + rbar - r[j]);
#endif
                        const double *kj = k + base + j * rs;
#if ORACLE_MUTANT == 16
                        const double *vj = v + base + j * rs;
#endif
                        double *dkj = dk + base + j * rs;
                        double *dvj = dv + base + j * rs;
                        for (int d = 0; d < D; ++d) {
#if ORACLE_MUTANT == 16
                            dqi[d] += scale * ds * vj[d];               /* mutant: v for k */
#else
                            dqi[d] += scale * ds * kj[d];
#endif
                            dri[d] += dr * kj[d];
#if ORACLE_MUTANT == 13
                            dkj[d] += ds * qi[d] + dr * ri[d];          /* mutant: scale dropped */
#else
                            dkj[d] += scale * ds * qi[d] + dr * ri[d];
#endif
                            dvj[d] += wv * g[d];
                        }
                    }
                }
            }
            free(work);
        }
    }
    return err;
}

/* Exact local-linear probe per query by conjugate gradient (matrix-free).
 * q, k: [B, N, H, D]; rho_out: [B, N, H, D]; iters (nullable): [B, N, H].
 * For query i (causal: keys 0..i, else all N): p = softmax(scale q.k),
 * kbar = sum p k, and (S + lam I) rho = kbar - q with
 * S x = sum_j p_j (k_j - kbar) ((k_j - kbar) . x). CG from rho = 0 stops when
 * |residual| <= tol |kbar - q| or after maxit iterations (the last iterate is
 * kept). Returns 0; 1 for bad arguments; 2 if memory runs out; 3 if some
 * query did not reach tol. lam > 0 makes the system positive definite. */
int oracle_lla_probe_f64(const double *q, const double *k, double *rho_out,
                         int32_t *iters, int B, int N, int H, int D, double scale,
                         int causal, double lam, int maxit, double tol,
                         int nthreads) {
    if (B < 0 || N < 0 || H < 0 || D <= 0 || maxit < 0 || !(lam >= 0.0) || !(tol >= 0.0))
        return 1;
    set_threads(nthreads);
    long rs = (long)H * D;
    long total = (long)B * N * H;
    int err = 0, unconverged = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * ((size_t)N + 6 * (size_t)D));
        if (!w) {
#pragma omp atomic write
            err = 2;
        } else {
            double *p = w, *kbar = w + N, *rhs = kbar + D, *x = rhs + D;
            double *r = x + D, *dir = r + D, *ad = dir + D;
#pragma omp for schedule(dynamic, 4)
            for (long t = 0; t < total; ++t) {
                long h = t % H;
                long i = (t / H) % N;
                long b = t / ((long)H * N);
                long n = causal ? i + 1 : N;
                const double *K = k + b * (long)N * rs + h * D;
                long off = ((b * N + i) * (long)H + h) * D;
                const double *qi = q + off;
                /* softmax weights */
                double mx = -INFINITY;
                for (long j = 0; j < n; ++j) {
                    double s = 0.0;
                    for (int d = 0; d < D; ++d) s += qi[d] * K[j * rs + d];
                    p[j] = scale * s;
                    if (p[j] > mx) mx = p[j];
                }
                double l = 0.0;
                for (long j = 0; j < n; ++j) { p[j] = exp(p[j] - mx); l += p[j]; }
                for (long j = 0; j < n; ++j) p[j] /= l;
                for (int d = 0; d < D; ++d) kbar[d] = 0.0;
                for (long j = 0; j < n; ++j)
                    for (int d = 0; d < D; ++d) kbar[d] += p[j] * K[j * rs + d];
                double bn = 0.0;
                for (int d = 0; d < D; ++d) {
#if ORACLE_MUTANT == 18
                    rhs[d] = qi[d] - kbar[d];           /* mutant: sign */
#else
                    rhs[d] = kbar[d] - qi[d];
#endif
                    x[d] = 0.0;
                    r[d] = rhs[d];
                    dir[d] = rhs[d];
                    bn += rhs[d] * rhs[d];
                }
                bn = sqrt(bn);
                double rr = bn * bn;
                int it = 0;
                while (it < maxit && sqrt(rr) > tol * bn) {
                    /* ad = (S + lam I) dir, streaming the keys */
                    for (int d = 0; d < D; ++d) ad[d] = lam * dir[d];
#if ORACLE_MUTANT == 17
                    for (int d = 0; d < D; ++d) ad[d] = 0.0;  /* mutant: no ridge */
#endif
                    for (long j = 0; j < n; ++j) {
                        double c = 0.0;
                        for (int d = 0; d < D; ++d) {
#if ORACLE_MUTANT == 19
                            c += K[j * rs + d] * dir[d];      /* mutant: uncentred */
#else
                            c += (K[j * rs + d] - kbar[d]) * dir[d];
#endif
                        }
                        c *= p[j];
                        for (int d = 0; d < D; ++d) {
#if ORACLE_MUTANT == 19
                            ad[d] += c * K[j * rs + d];
#else
                            ad[d] += c * (K[j * rs + d] - kbar[d]);
#endif
                        }
                    }
                    double dad = 0.0;
                    for (int d = 0; d < D; ++d) dad += dir[d] * ad[d];
                    if (!(dad > 0.0)) break;                /* breakdown */
                    double alpha = rr / dad;
                    double rr2 = 0.0;
                    for (int d = 0; d < D; ++d) {
                        x[d] += alpha * dir[d];
                        r[d] -= alpha * ad[d];
                        rr2 += r[d] * r[d];
                    }
                    double beta = rr2 / rr;
                    for (int d = 0; d < D; ++d) dir[d] = r[d] + beta * dir[d];
                    rr = rr2;
                    ++it;
                }
                if (sqrt(rr) > tol * bn) {
#pragma omp atomic write
                    unconverged = 1;
                }
                for (int d = 0; d < D; ++d) rho_out[off + d] = x[d];
                if (iters) iters[(b * N + i) * (long)H + h] = it;
            }
            free(w);
        }
    }
    if (err) return err;
    return unconverged ? 3 : 0;
}
