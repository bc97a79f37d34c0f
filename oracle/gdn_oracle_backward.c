/* CPU oracle for the gradients of the gated delta rule (reverse mode).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links, loads or calls
 * this file: only the tests use it.  It shares no code, header or constant
 * with the GPU path.
 *
 * The forward map is the token-by-token recurrence of gdn_oracle_impl.h:
 *
 *   X_t = diag(alpha_t) S_{t-1},  alpha_t = exp(g_t)      (decay first)
 *   r_t = X_t^T k_t,  u_t = beta_t (v_t - r_t)            (correct on write)
 *   S_t = X_t + k_t u_t^T,  o_t = S_t^T q_t
 *
 * Given the gradient of a scalar loss with respect to every o_t (dO) and to the
 * final state (dS_T, or zero), this file returns its gradient with respect to
 * q, k, v, g, beta and the initial state, by the chain rule applied to those
 * four lines in reverse order, one token at a time (the method is trained by
 * back-propagation, "What a Trillion-Parameter MoE Model Reveals About the
 * Next Stage of LLM Scaling", section 3.2, and "Architecture Evolution and
 * Training Engineering for Trillion-Scale Sparse Multimodal Models", section
 * 3.3; the pages do not write the backward pass out, so this is the plain
 * adjoint of the forward recurrence).  With dS = dL/dS_t:
 *
 *   dS   += q_t dO_t^T                   dq_t  = S_t dO_t
 *   du    = dS^T k_t                     dk_t  = dS u_t
 *   dbeta = du . (v_t - r_t)             dv_t  = beta_t du
 *   dr    = -beta_t du                   dk_t += X_t dr
 *   dX    = dS + k_t dr^T                dg_t,i = sum_j dX_ij X_ij
 *   dS_{t-1} = diag(alpha_t) dX
 *
 * States S_{t-1} are recomputed forward from checkpoints taken every
 * `interval` tokens, so memory stays bounded for long sequences; the
 * recomputation repeats the same operations, so the result does not depend
 * on the interval.
 *
 * Layouts (row-major, host memory) as in gdn_oracle.c; gradients have the
 * layouts of their inputs.
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* S_t from S_{t-1} for token t of head h (the forward recurrence). */
static void forward_token(const double* q, const double* k, const double* v, const double* g, const double* beta,
                          int64_t t, int32_t H, int32_t h, int32_t dk, int32_t dv, const double* Sp, double* S,
                          double* r)
{
    (void)q;
    const double* kt = k + (t * H + h) * (int64_t)dk;
    const double* vt = v + (t * H + h) * (int64_t)dv;
    const double* gt = g + (t * H + h) * (int64_t)dk;
    const double bt = beta[t * H + h];
    for (int32_t i = 0; i < dk; ++i) {
        const double a = exp(gt[i]);
        for (int32_t j = 0; j < dv; ++j) S[(int64_t)i * dv + j] = a * Sp[(int64_t)i * dv + j];
    }
    for (int32_t j = 0; j < dv; ++j) r[j] = 0.0;
    for (int32_t i = 0; i < dk; ++i)
        for (int32_t j = 0; j < dv; ++j) r[j] += S[(int64_t)i * dv + j] * kt[i];
    for (int32_t j = 0; j < dv; ++j) {
        const double u = bt * (vt[j] - r[j]);
        for (int32_t i = 0; i < dk; ++i) S[(int64_t)i * dv + j] += kt[i] * u;
    }
}

/* The adjoint of token t: dS holds dL/dS_t on entry and dL/dS_{t-1} on exit. */
static void backward_token(const double* q, const double* k, const double* v, const double* g,
                           const double* beta, const double* dO, int64_t t, int32_t H, int32_t h, int32_t dk,
                           int32_t dv, const double* Sp, double* dS, double* X, double* vec, double* dq,
                           double* dkk, double* dvv, double* dg, double* dbeta)
{
    const double* qt = q + (t * H + h) * (int64_t)dk;
    const double* kt = k + (t * H + h) * (int64_t)dk;
    const double* vt = v + (t * H + h) * (int64_t)dv;
    const double* gt = g + (t * H + h) * (int64_t)dk;
    const double* dot = dO + (t * H + h) * (int64_t)dv;
    const double bt = beta[t * H + h];
    double* r = vec;         /* dv */
    double* u = vec + dv;    /* dv */
    double* du = u + dv;     /* dv */
    double* dr = du + dv;    /* dv */
    double* a = dr + dv;     /* dk */
    /* recompute X, r, u (S_t = X + k u^T is used through X and u) */
    for (int32_t i = 0; i < dk; ++i) {
        a[i] = exp(gt[i]);
        for (int32_t j = 0; j < dv; ++j) X[(int64_t)i * dv + j] = a[i] * Sp[(int64_t)i * dv + j];
    }
    for (int32_t j = 0; j < dv; ++j) r[j] = 0.0;
    for (int32_t i = 0; i < dk; ++i)
        for (int32_t j = 0; j < dv; ++j) r[j] += X[(int64_t)i * dv + j] * kt[i];
    for (int32_t j = 0; j < dv; ++j) u[j] = bt * (vt[j] - r[j]);

    /* o_t = S_t^T q_t */
    double* dqt = dq + (t * H + h) * (int64_t)dk;
    for (int32_t i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int32_t j = 0; j < dv; ++j) {
            const double St = X[(int64_t)i * dv + j] + kt[i] * u[j];
            acc += St * dot[j];
            dS[(int64_t)i * dv + j] += qt[i] * dot[j];
        }
        dqt[i] = acc;
    }
    /* S_t = X + k u^T */
    double* dkt = dkk + (t * H + h) * (int64_t)dk;
    for (int32_t j = 0; j < dv; ++j) du[j] = 0.0;
    for (int32_t i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int32_t j = 0; j < dv; ++j) {
            du[j] += dS[(int64_t)i * dv + j] * kt[i];
            acc += dS[(int64_t)i * dv + j] * u[j];
        }
        dkt[i] = acc;
    }
    /* u = beta (v - r) */
    double db = 0.0;
    double* dvt = dvv + (t * H + h) * (int64_t)dv;
    for (int32_t j = 0; j < dv; ++j) {
        db += du[j] * (vt[j] - r[j]);
        dvt[j] = bt * du[j];
        dr[j] = -bt * du[j];
    }
    dbeta[t * H + h] = db;
    /* r = X^T k;  X = diag(a) S_{t-1} */
    double* dgt = dg + (t * H + h) * (int64_t)dk;
    for (int32_t i = 0; i < dk; ++i) {
        double acck = 0.0, accg = 0.0;
        for (int32_t j = 0; j < dv; ++j) {
            const double x = X[(int64_t)i * dv + j];
            acck += x * dr[j];
            const double dx = dS[(int64_t)i * dv + j] + kt[i] * dr[j];
            accg += dx * x;
            dS[(int64_t)i * dv + j] = a[i] * dx;
        }
        dkt[i] += acck;
        dgt[i] = accg;
    }
}

/* One (sequence, head): tokens t0 .. t1-1. */
static void backward_head(const double* q, const double* k, const double* v, const double* g, const double* beta,
                          const double* dO, int64_t t0, int64_t t1, int32_t H, int32_t h, int32_t dk, int32_t dv,
                          int32_t interval, const double* S0, const double* dSf, double* dS0, double* dq,
                          double* dkk, double* dvv, double* dg, double* dbeta, double* mem)
{
    const int64_t st = (int64_t)dk * dv, len = t1 - t0;
    const int64_t nblk = (len + interval - 1) / interval;
    double* ckpt = mem;                      /* nblk x st: state at each block start */
    double* blk = ckpt + nblk * st;          /* (interval + 1) x st: states inside a block */
    double* dS = blk + (interval + 1) * st;  /* st */
    double* X = dS + st;                     /* st */
    double* vec = X + st;                    /* 4 dv + dk */
    /* forward: the state at the start of every block */
    if (nblk > 0) {
        if (S0) memcpy(ckpt, S0, sizeof(double) * (size_t)st);
        else memset(ckpt, 0, sizeof(double) * (size_t)st);
    }
    for (int64_t b = 0; b + 1 < nblk; ++b) {
        memcpy(blk, ckpt + b * st, sizeof(double) * (size_t)st);
        for (int32_t j = 0; j < interval; ++j) {
            double* cur = blk + ((j + 1) & 1) * st;
            forward_token(q, k, v, g, beta, t0 + b * interval + j, H, h, dk, dv, blk + (j & 1) * st, cur, vec);
        }
        memcpy(ckpt + (b + 1) * st, blk + (interval & 1) * st, sizeof(double) * (size_t)st);
    }
    /* reverse */
    if (dSf) memcpy(dS, dSf, sizeof(double) * (size_t)st);
    else memset(dS, 0, sizeof(double) * (size_t)st);
    for (int64_t b = nblk - 1; b >= 0; --b) {
        const int64_t tb = t0 + b * interval;
        const int32_t n = (int32_t)((t1 - tb) < interval ? (t1 - tb) : interval);
        memcpy(blk, ckpt + b * st, sizeof(double) * (size_t)st);
        for (int32_t j = 0; j + 1 < n; ++j)
            forward_token(q, k, v, g, beta, tb + j, H, h, dk, dv, blk + j * st, blk + (j + 1) * st, vec);
        for (int32_t j = n - 1; j >= 0; --j)
            backward_token(q, k, v, g, beta, dO, tb + j, H, h, dk, dv, blk + j * st, dS, X, vec, dq, dkk, dvv, dg,
                           dbeta);
    }
    if (dS0) memcpy(dS0, dS, sizeof(double) * (size_t)st);
}

/* All sequences and heads, spread over `nthreads` OpenMP threads.  S0, dSf
 * and dS0 may be NULL (zero initial state, zero final-state gradient, initial
 * state gradient not wanted).  Returns 0, or -1 when scratch memory is
 * short. */
int gdn_oracle_backward_f64(const double* q, const double* k, const double* v, const double* g,
                            const double* beta, const int32_t* cu_seqlens, int32_t num_seqs, int32_t H, int32_t dk,
                            int32_t dv, const double* S0, const double* dO, const double* dSf, int32_t interval,
                            double* dq, double* dk_out, double* dv_out, double* dg, double* dbeta, double* dS0,
                            int32_t nthreads)
{
    const int64_t units = (int64_t)num_seqs * H;
    const int64_t st = (int64_t)dk * dv;
    int64_t maxlen = 0;
    for (int32_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] - cu_seqlens[n] > maxlen) maxlen = cu_seqlens[n + 1] - cu_seqlens[n];
    if (interval < 1) interval = 1;
    const int64_t nblk = (maxlen + interval - 1) / interval;
    const size_t words = (size_t)((nblk + interval + 3) * st + 4 * dv + dk);
    int failed = 0;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
    {
        double* mem = (double*)malloc(sizeof(double) * words);
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!mem) { failed = 1; continue; }
            const int32_t n = (int32_t)(u / H), h = (int32_t)(u % H);
            backward_head(q, k, v, g, beta, dO, cu_seqlens[n], cu_seqlens[n + 1], H, h, dk, dv, interval,
                          S0 ? S0 + u * st : NULL, dSf ? dSf + u * st : NULL, dS0 ? dS0 + u * st : NULL, dq,
                          dk_out, dv_out, dg, dbeta, mem);
        }
        free(mem);
    }
    return failed ? -1 : 0;
}
