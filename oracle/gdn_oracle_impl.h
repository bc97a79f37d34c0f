/* Sequential recurrence of the gated delta rule, written once and included by
 * gdn_oracle.c twice: with REAL = double (the parity reference) and with
 * REAL = float (the CPU baseline that the benchmark times).
 *
 * TEST INFRASTRUCTURE ONLY: see the header of gdn_oracle.c.
 *
 * What it computes, per sequence n and head h, starting from S = S0 (or 0):
 *
 *   for each token t of the sequence:
 *       alpha = exp(g_t)                 (one decay per key channel)
 *       S     = diag(alpha) S            (decay the state first)
 *       r     = S^T k_t                  (what the decayed state returns for k_t)
 *       u     = beta_t (v_t - r)         (correct-on-write: remove the old value)
 *       S     = S + k_t u^T
 *       o_t   = S^T q_t
 *   final state = S
 *
 * Sources: the state semantics (a fixed-size matrix state updated token by
 * token, where writing a key-value pair first reduces the conflicting old
 * content, under a position-dependent decay gate) are those of "How to Think
 * About Trillion-Parameter Sparse Multimodal LLMs", section 2.2 ("Incremental
 * Linear Attention: Compressing History into a Fixed State"); the decay is the
 * exponential of a per-token log-decay g ("What a Trillion-Parameter MoE Model
 * Reveals About the Next Stage of LLM Scaling", section 3.2, where the per-step
 * factor is exp(g_t)).  The order "decay, then read, then write" and the
 * per-key-channel granularity are readings of that prose; every reading is
 * listed in the design notes.
 */

#ifndef REAL
#error "define REAL before including gdn_oracle_impl.h"
#endif
#ifndef FN
#error "define FN(name) before including gdn_oracle_impl.h"
#endif

static void FN(one_head)(const REAL* q, const REAL* k, const REAL* v, const REAL* g, const REAL* beta,
                         int64_t t0, int64_t t1, int32_t H, int32_t h, int32_t dk, int32_t dv,
                         REAL* S, REAL* o, REAL* r)
{
    for (int64_t t = t0; t < t1; ++t) {
        const REAL* qt = q + (t * H + h) * (int64_t)dk;
        const REAL* kt = k + (t * H + h) * (int64_t)dk;
        const REAL* vt = v + (t * H + h) * (int64_t)dv;
        const REAL* gt = g + (t * H + h) * (int64_t)dk;
        const REAL bt = beta[t * H + h];
        /* S <- diag(exp(g_t)) S */
        for (int32_t i = 0; i < dk; ++i) {
            const REAL a = (REAL)exp((double)gt[i]);
            REAL* Si = S + (int64_t)i * dv;
            for (int32_t j = 0; j < dv; ++j) Si[j] *= a;
        }
        /* r = S^T k_t */
        for (int32_t j = 0; j < dv; ++j) r[j] = 0;
        for (int32_t i = 0; i < dk; ++i) {
            const REAL ki = kt[i];
            const REAL* Si = S + (int64_t)i * dv;
            for (int32_t j = 0; j < dv; ++j) r[j] += Si[j] * ki;
        }
        /* u = beta_t (v_t - r), stored in r */
        for (int32_t j = 0; j < dv; ++j) r[j] = bt * (vt[j] - r[j]);
        /* S <- S + k_t u^T */
        for (int32_t i = 0; i < dk; ++i) {
            const REAL ki = kt[i];
            REAL* Si = S + (int64_t)i * dv;
            for (int32_t j = 0; j < dv; ++j) Si[j] += ki * r[j];
        }
        /* o_t = S^T q_t */
        REAL* ot = o + (t * H + h) * (int64_t)dv;
        for (int32_t j = 0; j < dv; ++j) ot[j] = 0;
        for (int32_t i = 0; i < dk; ++i) {
            const REAL qi = qt[i];
            const REAL* Si = S + (int64_t)i * dv;
            for (int32_t j = 0; j < dv; ++j) ot[j] += Si[j] * qi;
        }
    }
}

/* All sequences and heads.  Units (sequence, head) are independent, so they
 * are spread over `nthreads` OpenMP threads.  S0 and S_final may be NULL;
 * S_final may alias S0.  Returns 0, or -1 when scratch memory is short. */
int FN(recurrent)(const REAL* q, const REAL* k, const REAL* v, const REAL* g, const REAL* beta,
                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                  const REAL* S0, REAL* o, REAL* S_final, int32_t nthreads)
{
    const int64_t units = (int64_t)num_seqs * H;
    const int64_t state = (int64_t)dk * dv;
    int failed = 0;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
    {
        /* every thread takes part in the work-sharing loop, even without scratch */
        REAL* S = (REAL*)malloc(sizeof(REAL) * (size_t)(state + dv));
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!S) { failed = 1; continue; }
            const int32_t n = (int32_t)(u / H), h = (int32_t)(u % H);
            if (S0) memcpy(S, S0 + u * state, sizeof(REAL) * (size_t)state);
            else memset(S, 0, sizeof(REAL) * (size_t)state);
            FN(one_head)(q, k, v, g, beta, cu_seqlens[n], cu_seqlens[n + 1], H, h, dk, dv, S, o, S + state);
            if (S_final) memcpy(S_final + u * state, S, sizeof(REAL) * (size_t)state);
        }
        free(S);
    }
    return failed ? -1 : 0;
}
