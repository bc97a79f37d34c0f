/* CPU oracle for the bounded-decay gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links, loads or calls
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header or constant with the GPU path.
 *
 * Three independent formulations of the same result, all plain loops:
 *
 *   gdn_oracle_recurrent_f64 / _f32   the token-by-token recurrence (the
 *       definition; see gdn_oracle_impl.h).  f64 is the parity reference,
 *       f32 is what the benchmark times on the host cores.
 *
 *   gdn_oracle_chunked_f64   the same result reached chunk by chunk.  Inside
 *       a chunk the decay is carried as a cumulative log-decay that restarts at
 *       every chunk (the cumulative decay factor of "Architecture Evolution and
 *       Training Engineering for Trillion-Scale Sparse Multimodal Models",
 *       section 3.2, taken per fixed-size tile as that section frames it); the
 *       causal part inside a chunk is a matrix product and chunks are linked
 *       through the carried state (section 3, item 1 of "How to Think About
 *       Trillion-Parameter Sparse Multimodal LLMs"); and the delta-rule
 *       coupling between the tokens of one chunk is removed by a unit
 *       lower-triangular solve (a reading: the pages do not spell out the
 *       solve that a delta rule needs).  Exponents are always formed as
 *       differences exp(G_t - G_s), never as a product of a factor and a
 *       reciprocal, so fp64 cannot overflow for any chunk length.
 *
 *   gdn_oracle_bruteforce_f64   for very short sequences: every state is the
 *       explicit unrolled sum  S_t = A_t...A_1 S0 + sum_s A_t...A_{s+1} B_s
 *       with dense transition matrices A_t = (I - beta_t k_t k_t^T) diag(alpha_t)
 *       and writes B_s = beta_s k_s v_s^T, built from scratch for each t.
 *
 * Layouts (row-major, host memory): q, k, g [T, H, dk]; v, o [T, H, dv];
 * beta [T, H]; states [num_seqs, H, dk, dv]; cu_seqlens [num_seqs + 1] with
 * cu_seqlens[0] = 0, non-decreasing.
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REAL double
#define FN(name) gdn_oracle_##name##_f64
#include "gdn_oracle_impl.h"
#undef REAL
#undef FN

#define REAL float
#define FN(name) gdn_oracle_##name##_f32
#include "gdn_oracle_impl.h"
#undef REAL
#undef FN

/* ---------------------------------------------------------------------------
 * Chunked form, fp64.
 *
 * For one chunk of L tokens starting from state S (dk x dv), with
 * G_t = sum_{r <= t, r in chunk} g_r (inclusive, per key channel):
 *
 *   A[t][s]  = beta_t * sum_i k_t,i k_s,i exp(G_t,i - G_s,i)        (s < t)
 *   solve (I + A) X = diag(beta) [Kt | V]   with Kt_t,i = k_t,i exp(G_t,i)
 *            giving W = X[:, :dk] and Ut = X[:, dk:]
 *   U        = Ut - W S                       (the chunk's corrected writes)
 *   o_t      = sum_i q_t,i exp(G_t,i) S[i][:] + sum_{s <= t} P[t][s] U_s
 *              with P[t][s] = sum_i q_t,i k_s,i exp(G_t,i - G_s,i)
 *   S       <- diag(exp(G_L)) S + sum_s (k_s * exp(G_L - G_s)) U_s^T
 *
 * Derivation: unrolling the recurrence inside the chunk gives
 *   S_t = D_t S + sum_{s<=t} diag(exp(G_t - G_s)) k_s u_s^T,
 * and u_t = beta_t (v_t - (diag(alpha_t) S_{t-1})^T k_t) becomes
 *   u_t + beta_t sum_{s<t} (k_t exp(G_t)) . (k_s exp(-G_s)) u_s = beta_t (v_t - S^T (k_t exp(G_t))),
 * i.e. (I + A) U = diag(beta) (V - Kt S), so U = Ut - W S.
 * ------------------------------------------------------------------------- */
static void chunk_step_f64(const double* q, const double* k, const double* v, const double* g,
                           const double* beta, int64_t t0, int32_t L, int32_t H, int32_t h, int32_t dk,
                           int32_t dv, double* S, double* o, double* work)
{
    double* G = work;                      /* L x dk */
    double* A = G + (int64_t)L * dk;       /* L x L  */
    double* X = A + (int64_t)L * L;        /* L x (dk + dv) */
    double* U = X + (int64_t)L * (dk + dv); /* L x dv */
    const int32_t nx = dk + dv;
#define Q_(t, i) q[((t0 + (t)) * H + h) * (int64_t)dk + (i)]
#define K_(t, i) k[((t0 + (t)) * H + h) * (int64_t)dk + (i)]
#define V_(t, j) v[((t0 + (t)) * H + h) * (int64_t)dv + (j)]
#define g_(t, i) g[((t0 + (t)) * H + h) * (int64_t)dk + (i)]
#define B_(t) beta[(t0 + (t)) * H + h]

    /* local cumulative log-decay */
    for (int32_t i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int32_t t = 0; t < L; ++t) {
            acc += g_(t, i);
            G[(int64_t)t * dk + i] = acc;
        }
    }
    /* A (strictly lower) */
    for (int32_t t = 0; t < L; ++t)
        for (int32_t s = 0; s < L; ++s) {
            double a = 0.0;
            if (s < t)
                for (int32_t i = 0; i < dk; ++i)
                    a += K_(t, i) * K_(s, i) * exp(G[(int64_t)t * dk + i] - G[(int64_t)s * dk + i]);
            A[(int64_t)t * L + s] = B_(t) * a;
        }
    /* right-hand side diag(beta) [Kt | V], then forward substitution */
    for (int32_t t = 0; t < L; ++t) {
        double* xt = X + (int64_t)t * nx;
        for (int32_t i = 0; i < dk; ++i) xt[i] = B_(t) * K_(t, i) * exp(G[(int64_t)t * dk + i]);
        for (int32_t j = 0; j < dv; ++j) xt[dk + j] = B_(t) * V_(t, j);
        for (int32_t s = 0; s < t; ++s) {
            const double a = A[(int64_t)t * L + s];
            const double* xs = X + (int64_t)s * nx;
            for (int32_t c = 0; c < nx; ++c) xt[c] -= a * xs[c];
        }
    }
    /* U = Ut - W S */
    for (int32_t t = 0; t < L; ++t) {
        const double* xt = X + (int64_t)t * nx;
        for (int32_t j = 0; j < dv; ++j) {
            double ws = 0.0;
            for (int32_t i = 0; i < dk; ++i) ws += xt[i] * S[(int64_t)i * dv + j];
            U[(int64_t)t * dv + j] = xt[dk + j] - ws;
        }
    }
    /* outputs */
    for (int32_t t = 0; t < L; ++t) {
        double* ot = o + ((t0 + t) * H + h) * (int64_t)dv;
        for (int32_t j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int32_t i = 0; i < dk; ++i) acc += Q_(t, i) * exp(G[(int64_t)t * dk + i]) * S[(int64_t)i * dv + j];
            ot[j] = acc;
        }
        for (int32_t s = 0; s <= t; ++s) {
            double p = 0.0;
            for (int32_t i = 0; i < dk; ++i)
                p += Q_(t, i) * K_(s, i) * exp(G[(int64_t)t * dk + i] - G[(int64_t)s * dk + i]);
            for (int32_t j = 0; j < dv; ++j) ot[j] += p * U[(int64_t)s * dv + j];
        }
    }
    /* state carried to the next chunk */
    const double* GL = G + (int64_t)(L - 1) * dk;
    for (int32_t i = 0; i < dk; ++i) {
        double* Si = S + (int64_t)i * dv;
        const double d = exp(GL[i]);
        for (int32_t j = 0; j < dv; ++j) Si[j] *= d;
        for (int32_t s = 0; s < L; ++s) {
            const double kd = K_(s, i) * exp(GL[i] - G[(int64_t)s * dk + i]);
            for (int32_t j = 0; j < dv; ++j) Si[j] += kd * U[(int64_t)s * dv + j];
        }
    }
#undef Q_
#undef K_
#undef V_
#undef g_
#undef B_
}

int gdn_oracle_chunked_f64(const double* q, const double* k, const double* v, const double* g,
                           const double* beta, const int32_t* cu_seqlens, int32_t num_seqs, int32_t H,
                           int32_t dk, int32_t dv, int32_t chunk, const double* S0, double* o,
                           double* S_final, int32_t nthreads)
{
    if (chunk < 1) return -2;
    const int64_t units = (int64_t)num_seqs * H;
    const int64_t state = (int64_t)dk * dv;
    const int64_t per = (int64_t)chunk * dk + (int64_t)chunk * chunk + (int64_t)chunk * (dk + dv) +
                        (int64_t)chunk * dv;
    int failed = 0;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)(state + per));
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!S) { failed = 1; continue; }
            const int32_t n = (int32_t)(u / H), h = (int32_t)(u % H);
            if (S0) memcpy(S, S0 + u * state, sizeof(double) * (size_t)state);
            else memset(S, 0, sizeof(double) * (size_t)state);
            for (int64_t t0 = cu_seqlens[n]; t0 < cu_seqlens[n + 1]; t0 += chunk) {
                int64_t L = cu_seqlens[n + 1] - t0;
                if (L > chunk) L = chunk;
                chunk_step_f64(q, k, v, g, beta, t0, (int32_t)L, H, h, dk, dv, S, o, S + state);
            }
            if (S_final) memcpy(S_final + u * state, S, sizeof(double) * (size_t)state);
        }
        free(S);
    }
    return failed ? -1 : 0;
}

/* ---------------------------------------------------------------------------
 * Brute force for short sequences (L <= 16 per sequence): no state is carried
 * from one token to the next; each S_t is rebuilt from the unrolled sum.
 * ------------------------------------------------------------------------- */
static void matmul_sq(const double* X, const double* Y, double* Z, int32_t n)
{
    for (int32_t a = 0; a < n; ++a)
        for (int32_t b = 0; b < n; ++b) {
            double acc = 0.0;
            for (int32_t c = 0; c < n; ++c) acc += X[(int64_t)a * n + c] * Y[(int64_t)c * n + b];
            Z[(int64_t)a * n + b] = acc;
        }
}

int gdn_oracle_bruteforce_f64(const double* q, const double* k, const double* v, const double* g,
                              const double* beta, const int32_t* cu_seqlens, int32_t num_seqs, int32_t H,
                              int32_t dk, int32_t dv, const double* S0, double* o, double* S_final)
{
    const int64_t nn = (int64_t)dk * dk;
    for (int32_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] - cu_seqlens[n] > 16) return -2;
    double* Tr = (double*)malloc(sizeof(double) * (size_t)(16 * nn)); /* A_1..A_L */
    double* P = (double*)malloc(sizeof(double) * (size_t)nn);         /* running product */
    double* Pn = (double*)malloc(sizeof(double) * (size_t)nn);
    double* St = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    if (!Tr || !P || !Pn || !St) {
        free(Tr); free(P); free(Pn); free(St);
        return -1;
    }
    for (int32_t n = 0; n < num_seqs; ++n)
        for (int32_t h = 0; h < H; ++h) {
            const int64_t t0 = cu_seqlens[n];
            const int32_t L = (int32_t)(cu_seqlens[n + 1] - t0);
            const double* s0 = S0 ? S0 + ((int64_t)n * H + h) * dk * dv : NULL;
            /* A_t = (I - beta_t k_t k_t^T) diag(exp(g_t)) */
            for (int32_t t = 0; t < L; ++t) {
                const double* kt = k + ((t0 + t) * H + h) * (int64_t)dk;
                const double* gt = g + ((t0 + t) * H + h) * (int64_t)dk;
                const double bt = beta[(t0 + t) * H + h];
                double* At = Tr + (int64_t)t * nn;
                for (int32_t a = 0; a < dk; ++a)
                    for (int32_t b = 0; b < dk; ++b)
                        At[(int64_t)a * dk + b] = ((a == b ? 1.0 : 0.0) - bt * kt[a] * kt[b]) * exp(gt[b]);
            }
            for (int32_t t = 0; t < L; ++t) {
                /* S_t = (A_t ... A_1) S0 + sum_{s<=t} (A_t ... A_{s+1}) beta_s k_s v_s^T.
                   Term index s = -1 stands for the S0 term, whose product starts at A_1
                   (index 0); the write of token s has the product A_{s+1} ... A_t. */
                memset(St, 0, sizeof(double) * (size_t)dk * dv);
                for (int32_t s = -1; s <= t; ++s) {
                    if (s < 0 && !s0) continue;
                    for (int64_t e = 0; e < nn; ++e) P[e] = 0.0;
                    for (int32_t a = 0; a < dk; ++a) P[(int64_t)a * dk + a] = 1.0;
                    for (int32_t r = s + 1; r <= t; ++r) { /* P <- A_r P */
                        matmul_sq(Tr + (int64_t)r * nn, P, Pn, dk);
                        memcpy(P, Pn, sizeof(double) * (size_t)nn);
                    }
                    if (s < 0) {
                        for (int32_t a = 0; a < dk; ++a)
                            for (int32_t j = 0; j < dv; ++j) {
                                double acc = 0.0;
                                for (int32_t c = 0; c < dk; ++c) acc += P[(int64_t)a * dk + c] * s0[(int64_t)c * dv + j];
                                St[(int64_t)a * dv + j] += acc;
                            }
                    } else {
                        const double* ks = k + ((t0 + s) * H + h) * (int64_t)dk;
                        const double* vs = v + ((t0 + s) * H + h) * (int64_t)dv;
                        const double bs = beta[(t0 + s) * H + h];
                        for (int32_t a = 0; a < dk; ++a) {
                            double pk = 0.0;
                            for (int32_t c = 0; c < dk; ++c) pk += P[(int64_t)a * dk + c] * ks[c];
                            for (int32_t j = 0; j < dv; ++j) St[(int64_t)a * dv + j] += bs * pk * vs[j];
                        }
                    }
                }
                const double* qt = q + ((t0 + t) * H + h) * (int64_t)dk;
                double* ot = o + ((t0 + t) * H + h) * (int64_t)dv;
                for (int32_t j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int32_t a = 0; a < dk; ++a) acc += St[(int64_t)a * dv + j] * qt[a];
                    ot[j] = acc;
                }
            }
            if (S_final) {
                double* sf = S_final + ((int64_t)n * H + h) * dk * dv;
                if (L == 0) {
                    if (s0) memmove(sf, s0, sizeof(double) * (size_t)dk * dv);
                    else memset(sf, 0, sizeof(double) * (size_t)dk * dv);
                } else {
                    memcpy(sf, St, sizeof(double) * (size_t)dk * dv);
                }
            }
        }
    free(Tr); free(P); free(Pn); free(St);
    return 0;
}
