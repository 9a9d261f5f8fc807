/*
 * attn_oracle.c -- plain, slow, fp64 CPU oracle for causal scaled-dot-product
 * attention, forward and analytic backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or runs
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or helper with the HIP
 * library: it is written from the definition of attention, not from the
 * kernels.
 *
 * What it computes (per batch b and head h, Q,K,V,dO in R^{T x d}, scale s):
 *   S_ij  = s * sum_c Q_ic K_jc                       (every i, j: T x T matrix)
 *   A_i   = { j <= i } if causal else { all j }       (decoder-only masking)
 *   m_i   = max_{j in A_i} S_ij
 *   E_ij  = exp(S_ij - m_i) for j in A_i, else exactly 0
 *   l_i   = sum_j E_ij,  P_ij = E_ij / l_i
 *   O     = P V,  LSE_i = m_i + ln l_i   (natural log of the scaled scores)
 * and the gradient of L = <dO, O> by the chain rule through the softmax:
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
 *   dS_ij = P_ij (dP_ij - D_i),  dQ = s dS K,  dK = s dS^T Q.
 *
 * Sources: Forge (S.-P. Boucher, "Forge: Building an LLM Training Framework
 * from Scratch in C++ and Metal on Apple Silicon", 2026):
 *   - section "Attention kernel design": online-softmax forward whose saved
 *     logsumexp fixes the normalisation for the backward pass;
 *   - section "Ecosystem survey": the backward is D = rowsum(dO o O) followed
 *     by a dQ pass and a dK/dV pass;
 *   - section "Related work": the design follows FlashAttention-2, which
 *     computes exactly the explicit-matrix attention above, only tiled.
 * The oracle therefore writes out the plain definition (explicit T x T score
 * and probability matrices, no tiling, no online rescaling).
 *
 * The row-partitioned threading (each thread owns whole (b,h) slabs, no shared
 * write targets) follows the multithreading step of "How to train an LLM on
 * Apple Silicon without Python" (toolsonfire.com, 2026).  Every sum runs in
 * sequential index order inside one thread, so results do not depend on the
 * thread count.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -pthread (no -ffast-math, no BLAS).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    int T, d, causal;
    double s;
    const double *Q, *K, *V, *dO;       /* slabs of the whole [BH,T,d] arrays */
    double *O, *LSE, *dQ, *dK, *dV, *Dv; /* outputs (may be NULL when unused) */
    int bh_begin, bh_end;
    int backward;
    int status;
} job_t;

/* Probabilities P (T x T, row-major) and, optionally, O and LSE of one (b,h). */
static void softmax_probs(int T, int d, int causal, double s, const double *Q,
                          const double *K, double *P, double *LSE)
{
    for (int i = 0; i < T; ++i) {
        double *Pi = P + (size_t)i * T;
        const int jmax = causal ? i : T - 1; /* last visible key */
        for (int j = 0; j < T; ++j) {
            if (j > jmax) { Pi[j] = 0.0; continue; }
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += Q[(size_t)i * d + c] * K[(size_t)j * d + c];
            Pi[j] = s * acc; /* S_ij, overwritten by P_ij below */
        }
        double m = -INFINITY;
        for (int j = 0; j <= jmax; ++j) if (Pi[j] > m) m = Pi[j];
        double l = 0.0;
        for (int j = 0; j <= jmax; ++j) { Pi[j] = exp(Pi[j] - m); l += Pi[j]; }
        for (int j = 0; j <= jmax; ++j) Pi[j] /= l;
        if (LSE) LSE[i] = m + log(l);
    }
}

static void one_head(job_t *jb, size_t bh, double *P, double *dS)
{
    const int T = jb->T, d = jb->d;
    const size_t off = bh * (size_t)T * d;
    const double *Q = jb->Q + off, *K = jb->K + off, *V = jb->V + off;
    double *O_out = jb->O ? jb->O + off : NULL;
    double *LSE_out = jb->LSE ? jb->LSE + bh * (size_t)T : NULL;

    softmax_probs(T, d, jb->causal, jb->s, Q, K, P, LSE_out);

    /* O = P V (also needed by the backward for D). */
    double *O = O_out;
    double *Otmp = NULL;
    if (!O) { Otmp = (double *)malloc((size_t)T * d * sizeof(double)); O = Otmp; }
    for (int i = 0; i < T; ++i)
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int j = 0; j < T; ++j) acc += P[(size_t)i * T + j] * V[(size_t)j * d + c];
            O[(size_t)i * d + c] = acc;
        }

    if (jb->backward) {
        const double *dO = jb->dO + off;
        double *dQ = jb->dQ + off, *dK = jb->dK + off, *dV = jb->dV + off;
        double *Dv = jb->Dv ? jb->Dv + bh * (size_t)T : NULL;
        /* dV = P^T dO */
        for (int j = 0; j < T; ++j)
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int i = 0; i < T; ++i) acc += P[(size_t)i * T + j] * dO[(size_t)i * d + c];
                dV[(size_t)j * d + c] = acc;
            }
        for (int i = 0; i < T; ++i) {
            /* D_i = sum_c dO_ic O_ic */
            double Di = 0.0;
            for (int c = 0; c < d; ++c) Di += dO[(size_t)i * d + c] * O[(size_t)i * d + c];
            if (Dv) Dv[i] = Di;
            for (int j = 0; j < T; ++j) {
                /* dP_ij = sum_c dO_ic V_jc ; dS_ij = P_ij (dP_ij - D_i) */
                double dP = 0.0;
                for (int c = 0; c < d; ++c) dP += dO[(size_t)i * d + c] * V[(size_t)j * d + c];
                dS[(size_t)i * T + j] = P[(size_t)i * T + j] * (dP - Di);
            }
        }
        /* dQ = s dS K */
        for (int i = 0; i < T; ++i)
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int j = 0; j < T; ++j) acc += dS[(size_t)i * T + j] * K[(size_t)j * d + c];
                dQ[(size_t)i * d + c] = jb->s * acc;
            }
        /* dK = s dS^T Q */
        for (int j = 0; j < T; ++j)
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int i = 0; i < T; ++i) acc += dS[(size_t)i * T + j] * Q[(size_t)i * d + c];
                dK[(size_t)j * d + c] = jb->s * acc;
            }
    }
    free(Otmp);
}

static void *worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    const size_t TT = (size_t)jb->T * jb->T;
    double *P = (double *)malloc(TT * sizeof(double));
    double *dS = jb->backward ? (double *)malloc(TT * sizeof(double)) : NULL;
    if (!P || (jb->backward && !dS)) { free(P); free(dS); jb->status = 2; return NULL; }
    for (int bh = jb->bh_begin; bh < jb->bh_end; ++bh) one_head(jb, (size_t)bh, P, dS);
    free(P); free(dS);
    jb->status = 0;
    return NULL;
}

static int run(int BH, int T, int d, double s, int causal, const double *Q, const double *K,
               const double *V, const double *dO, double *O, double *LSE, double *dQ,
               double *dK, double *dV, double *Dv, int nthreads, int backward)
{
    if (BH < 1 || T < 1 || d < 1 || !Q || !K || !V) return 1;
    if (backward && (!dO || !dQ || !dK || !dV)) return 1;
    if (!backward && (!O || !LSE)) return 1;
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > BH) nthreads = BH;
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return 2; }
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        job_t *jb = &jobs[t];
        jb->T = T; jb->d = d; jb->causal = causal; jb->s = s;
        jb->Q = Q; jb->K = K; jb->V = V; jb->dO = dO;
        jb->O = O; jb->LSE = LSE; jb->dQ = dQ; jb->dK = dK; jb->dV = dV; jb->Dv = Dv;
        jb->bh_begin = (int)((long long)BH * t / nthreads);
        jb->bh_end = (int)((long long)BH * (t + 1) / nthreads);
        jb->backward = backward;
        jb->status = 3;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) { rc = 2; break; }
        started = t;
    }
    worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    for (int t = 0; t < nthreads && rc == 0; ++t) if (jobs[t].status) rc = jobs[t].status;
    free(jobs); free(th);
    return rc;
}

/* Forward: O [BH,T,d], LSE [BH,T].  Returns 0 on success, 1 bad args, 2 OOM. */
int oracle_attn_fwd(int BH, int T, int d, double scale, int causal, const double *Q,
                    const double *K, const double *V, double *O, double *LSE, int nthreads)
{
    return run(BH, T, d, scale, causal, Q, K, V, NULL, O, LSE, NULL, NULL, NULL, NULL,
               nthreads, 0);
}

/* Backward of L = <dO, O>: dQ, dK, dV [BH,T,d]; optional O [BH,T,d], LSE and
 * D = rowsum(dO o O) [BH,T] (NULL to skip).  P and O are the oracle's own. */
int oracle_attn_bwd(int BH, int T, int d, double scale, int causal, const double *Q,
                    const double *K, const double *V, const double *dO, double *dQ,
                    double *dK, double *dV, double *O, double *LSE, double *D, int nthreads)
{
    return run(BH, T, d, scale, causal, Q, K, V, dO, O, LSE, dQ, dK, dV, D, nthreads, 1);
}

int oracle_threads_default(void)
{
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}
