/*
 * Plain fp64 CPU oracle for the frame-wise Gated DeltaNet (GDN) forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the HIP library; it is deliberately slow and
 * written to be checked against the definition by eye.
 *
 * What it computes.  The SGLang-diffusion cookbook page "SANA-WM" (table
 * "Architecture & components", row "Attention") names the token mixer a
 * frame-wise Gated DeltaNet; the blog post on SANA-WM (section "core idea /
 * structure") describes it as a frame-unit GDN recurrent/linear attention
 * with a bounded state.  The pages print no formula, so the oracle takes the
 * published gated delta rule (Yang, Kautz & Hatamizadeh, "Gated Delta
 * Networks: Improving Mamba2 with Delta Rule", ICLR 2025), per (batch, head):
 *
 *     S_t = alpha_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * with S a d_v x d_k matrix (row i = value channel i), token order as given
 * (frame-major), and the readings:
 *   - q and k are L2-normalised per token and head: x / max(||x||, 1e-6),
 *     so a zero vector stays zero (skipped with ORACLE_QK_PRENORMALIZED);
 *   - beta_t = sigmoid(beta input) (taken as is with ORACLE_BETA_IS_PROB);
 *   - alpha_t = exp(g_t), g being the per-token log-decay; the frame-wise
 *     gate lives in the data (g non-zero only on a frame's first token);
 *   - the output reads the state after the token's own update (inclusive),
 *     with no 1/sqrt(d) scale.
 *
 * The product form above is expanded, row by row, as
 *     u_i   = alpha * (S[i,:] . k)
 *     S[i,:] = alpha * S[i,:] + beta * (v_i - u_i) * k^T
 *     o_i   = S[i,:] . q
 * which is the same matrix identity written without forming I - beta k k^T.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BETA_IS_PROB 1u
#define ORACLE_QK_PRENORMALIZED 2u

typedef struct {
    int B, T, H, dk, dv;
    const double *q, *k, *v, *g, *beta, *state_in;
    double *state_out, *o;
    unsigned flags;
    int first_unit, stride;
} oracle_job;

/* x / max(||x||_2, 1e-6) */
static void normalize(const double *x, int d, double *out, int skip)
{
    if (skip) {
        memcpy(out, x, sizeof(double) * (size_t)d);
        return;
    }
    double ss = 0.0;
    for (int j = 0; j < d; ++j) ss += x[j] * x[j];
    double n = sqrt(ss);
    if (n < 1e-6) n = 1e-6;
    for (int j = 0; j < d; ++j) out[j] = x[j] / n;
}

static void run_unit(const oracle_job *J, int unit, double *S, double *qh, double *kh)
{
    const int b = unit / J->H, h = unit % J->H;
    const int dk = J->dk, dv = J->dv;
    const size_t sbase = (size_t)unit * dv * dk; /* state is [B,H,dv,dk] */

    if (J->state_in)
        memcpy(S, J->state_in + sbase, sizeof(double) * (size_t)dv * dk);
    else
        memset(S, 0, sizeof(double) * (size_t)dv * dk);

    for (int t = 0; t < J->T; ++t) {
        const size_t th = ((size_t)b * J->T + t) * J->H + h; /* token-head index */
        normalize(J->q + th * dk, dk, qh, (J->flags & ORACLE_QK_PRENORMALIZED) != 0);
        normalize(J->k + th * dk, dk, kh, (J->flags & ORACLE_QK_PRENORMALIZED) != 0);
        const double bl = J->beta[th];
        const double beta = (J->flags & ORACLE_BETA_IS_PROB) ? bl : 1.0 / (1.0 + exp(-bl));
        const double alpha = exp(J->g[th]);
        const double *vt = J->v + th * dv;
        double *ot = J->o + th * dv;
        for (int i = 0; i < dv; ++i) {
            double *row = S + (size_t)i * dk;
            double sk = 0.0;
            for (int j = 0; j < dk; ++j) sk += row[j] * kh[j];
            const double w = beta * (vt[i] - alpha * sk);
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) {
                row[j] = alpha * row[j] + w * kh[j];
                acc += row[j] * qh[j];
            }
            ot[i] = acc;
        }
    }
    if (J->state_out)
        memcpy(J->state_out + sbase, S, sizeof(double) * (size_t)dv * dk);
}

static void *worker(void *arg)
{
    const oracle_job *J = (const oracle_job *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)J->dv * J->dk);
    double *qh = (double *)malloc(sizeof(double) * (size_t)J->dk);
    double *kh = (double *)malloc(sizeof(double) * (size_t)J->dk);
    if (S && qh && kh)
        for (int u = J->first_unit; u < J->B * J->H; u += J->stride) run_unit(J, u, S, qh, kh);
    free(S);
    free(qh);
    free(kh);
    return NULL;
}

/*
 * q, k: [B,T,H,dk]; v: [B,T,H,dv]; g, beta: [B,T,H]; state_in/state_out:
 * [B,H,dv,dk] (NULL = zero initial state / not written); o: [B,T,H,dv].
 * All fp64, contiguous.  The (batch, head) units are independent and are
 * spread over nthreads POSIX threads.  Returns 0, or -1 on bad arguments.
 */
int oracle_gdn_fwd(int B, int T, int H, int dk, int dv,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta,
                   const double *state_in, double *state_out, double *o,
                   unsigned flags, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (B * H == 0) return 0;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B * H) nthreads = B * H;

    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return -1;
    }
    for (int w = 0; w < nthreads; ++w) {
        oracle_job J = {B, T, H, dk, dv, q, k, v, g, beta, state_in, state_out, o, flags, w, nthreads};
        jobs[w] = J;
    }
    int spawned = 0;
    for (int w = 1; w < nthreads; ++w)
        if (pthread_create(&tid[w], NULL, worker, &jobs[w]) == 0) ++spawned;
        else break;
    worker(&jobs[0]);
    for (int w = 1; w <= spawned; ++w) pthread_join(tid[w], NULL);
    /* units of threads that could not be spawned run here */
    for (int w = spawned + 1; w < nthreads; ++w) worker(&jobs[w]);
    free(jobs);
    free(tid);
    return 0;
}
