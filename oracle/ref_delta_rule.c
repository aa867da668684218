/*
 * fp64 CPU oracle of the DeltaNet delta rule -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load or call this file.  It shares no code, header, helper or build flag
 * with the HIP library; the GPU path never links it.
 *
 * What it computes (one independent recurrence per batch row b and head h):
 *
 *   S <- S0 (or the zero matrix)                     S is d_v x d_k
 *   for t = 0 .. T-1:
 *       p   = S k_t                 prediction of the current key
 *       u   = beta_t (v_t - p)      scaled prediction error
 *       S   = S + u k_t^T           rank-1 error-correcting write
 *       o_t = S q_t                 read after the write
 *   S_T <- S
 *
 * Sources:
 *  - "Tour d'horizon des variantes d'attention lineaire de la famille
 *    DeltaNet" (hada.io digest), section "DeltaNet : ecrire l'erreur de
 *    prediction plutot que la valeur": the prediction S_{t-1} k_t, the error
 *    e_t = beta_t (v_t - S_{t-1} k_t) and the write S_t = S_{t-1} + e_t k_t^T;
 *    section "Calcul de toutes les sorties internes au chunk": a token's output
 *    includes its own write (read after write).
 *  - houmin.site "infra/delta-net", section "DeltaNet 引入 Delta Rule": the
 *    output o_t = S_t q_t, and the state as the map from key space to value
 *    space (d_v x d_k), which is the orientation used here.
 *
 * Arithmetic: IEEE fp64, each dot product summed in ascending key index, no
 * fused multiply-add (build with -ffp-contract=off), no blocking or
 * reordering.  Inputs arrive already rounded to the caller's dtype and widened
 * to fp64.
 *
 * Layouts (row-major, contiguous): q, k [B,T,H,Dk]; v, o [B,T,H,Dv];
 * beta [B,T,H]; S0, S_T [B,H,Dv,Dk].  S0 may be NULL (zero state).
 *
 * Gated variant (ref_gated_delta_rule_f64): one more input g [B,T,H], the
 * natural log of a scalar forget gate alpha_t = exp(g_t).  Each token first
 * decays the whole state, then predicts, corrects and writes:
 *
 *       S   = alpha_t S             forget (the whole matrix, one scalar)
 *       p   = S k_t                 prediction from the decayed state
 *       u   = beta_t (v_t - p)
 *       S   = S + u k_t^T
 *       o_t = S q_t
 *
 * Source: hada.io digest, section "Gated DeltaNet : oublier d'abord l'etat
 * entier" (forget, predict, correct, write, in that order, with the decayed
 * state used for the prediction); houmin.site "infra/delta-net", section
 * "Gated DeltaNet" (S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t
 * k_t^T).  alpha_t = exp(g_t) is evaluated with the C library's exp in fp64;
 * g_t = 0 gives alpha_t = 1 exactly, i.e. the ungated recurrence bit for bit.
 *
 * Per-channel variant (ref_kda_f64, Kimi Delta Attention): gk [B,T,H,Dk]
 * holds the log decay of every key channel; the forget step scales column j
 * of the state (key channel j) by exp(gk_t[j]):
 *
 *       S   = S Diag(exp(gk_t))     forget, per key channel
 *       p   = S k_t ... as above
 *
 * Source: hada.io digest, section "Kimi Delta Attention : attenuation par
 * canal" (decay S_{t-1} D_t with D_t = Diag(alpha_t), then predict, correct,
 * write, read; the key channels are the columns of the state).  The read
 * there also scales q by d_k^{-1/2}; here, as for the other rules, o = S q and
 * callers pass the scale they want.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *beta, *g, *gk, *S0;
    double *o, *S_T;
    int64_t B, T, H, Dk, Dv;
    int64_t next; /* next (b,h) pair to take; shared work counter */
    int failed;
} oracle_job;

static void one_head(const oracle_job *J, int64_t b, int64_t h, double *S, double *u)
{
    const int64_t T = J->T, H = J->H, Dk = J->Dk, Dv = J->Dv;
    const int64_t sh = (b * H + h) * Dv * Dk;

    if (J->S0)
        memcpy(S, J->S0 + sh, (size_t)(Dv * Dk) * sizeof(double));
    else
        memset(S, 0, (size_t)(Dv * Dk) * sizeof(double));

    for (int64_t t = 0; t < T; ++t) {
        const int64_t row = (b * T + t) * H + h;
        const double *qt = J->q + row * Dk;
        const double *kt = J->k + row * Dk;
        const double *vt = J->v + row * Dv;
        const double bt = J->beta[row];
        double *ot = J->o + row * Dv;

        /* forget: S = alpha_t S (gated variant only) */
        if (J->g) {
            const double at = exp(J->g[row]);
            for (int64_t i = 0; i < Dv * Dk; ++i)
                S[i] = at * S[i];
        }
        /* forget per key channel: column j of S times exp(gk_t[j]) (KDA) */
        if (J->gk) {
            const double *gt = J->gk + row * Dk;
            for (int64_t i = 0; i < Dv; ++i)
                for (int64_t j = 0; j < Dk; ++j)
                    S[i * Dk + j] = exp(gt[j]) * S[i * Dk + j];
        }

        /* u = beta_t (v_t - S k_t), with S the (decayed) state before this
         * token's write */
        for (int64_t i = 0; i < Dv; ++i) {
            double p = 0.0;
            for (int64_t j = 0; j < Dk; ++j)
                p += S[i * Dk + j] * kt[j];
            u[i] = bt * (vt[i] - p);
        }
        /* S = S + u k_t^T */
        for (int64_t i = 0; i < Dv; ++i)
            for (int64_t j = 0; j < Dk; ++j)
                S[i * Dk + j] += u[i] * kt[j];
        /* o_t = S q_t, with S the state after this token's write */
        for (int64_t i = 0; i < Dv; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < Dk; ++j)
                acc += S[i * Dk + j] * qt[j];
            ot[i] = acc;
        }
    }
    if (J->S_T)
        memcpy(J->S_T + sh, S, (size_t)(Dv * Dk) * sizeof(double));
}

static void *worker(void *arg)
{
    oracle_job *J = (oracle_job *)arg;
    double *S = (double *)malloc((size_t)(J->Dv * J->Dk) * sizeof(double));
    double *u = (double *)malloc((size_t)J->Dv * sizeof(double));
    if (!S || !u) {
        __atomic_store_n(&J->failed, 1, __ATOMIC_SEQ_CST);
        free(S);
        free(u);
        return NULL;
    }
    for (;;) {
        int64_t bh = __atomic_fetch_add(&J->next, 1, __ATOMIC_SEQ_CST);
        if (bh >= J->B * J->H)
            break;
        one_head(J, bh / J->H, bh % J->H, S, u);
    }
    free(S);
    free(u);
    return NULL;
}

static int run(const double *q, const double *k, const double *v, const double *beta,
               const double *g, const double *gk, const double *S0, double *o, double *S_T,
               int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int nthreads)
{
    if (!q || !k || !v || !beta || !o || B < 0 || T < 0 || H < 0 || Dk < 1 ||
        Dv < 1)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    oracle_job J = {q, k, v, beta, g, gk, S0, o, S_T, B, T, H, Dk, Dv, 0, 0};
    if (B * H == 0)
        return 0;
    if (nthreads > B * H)
        nthreads = (int)(B * H);

    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!tid)
        return -2;
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, &J) != 0)
            break;
        ++started;
    }
    worker(&J); /* the calling thread works too */
    for (int i = 1; i <= started; ++i)
        pthread_join(tid[i], NULL);
    free(tid);
    return J.failed ? -2 : 0;
}

/*
 * Runs the recurrence for every (b,h).  Work is split over `nthreads` POSIX
 * threads by (b,h) pair only; each pair is computed by one thread in token
 * order, so the result does not depend on the thread count.
 * Returns 0 on success, -1 on bad arguments, -2 on allocation or thread
 * failure.
 */
int ref_delta_rule_f64(const double *q, const double *k, const double *v,
                       const double *beta, const double *S0, double *o,
                       double *S_T, int64_t B, int64_t T, int64_t H,
                       int64_t Dk, int64_t Dv, int nthreads)
{
    return run(q, k, v, beta, NULL, NULL, S0, o, S_T, B, T, H, Dk, Dv, nthreads);
}

/* The gated recurrence (g = log alpha, [B,T,H], required); otherwise as above. */
int ref_gated_delta_rule_f64(const double *q, const double *k, const double *v,
                             const double *beta, const double *g, const double *S0,
                             double *o, double *S_T, int64_t B, int64_t T, int64_t H,
                             int64_t Dk, int64_t Dv, int nthreads)
{
    if (!g)
        return -1;
    return run(q, k, v, beta, g, NULL, S0, o, S_T, B, T, H, Dk, Dv, nthreads);
}

/* The per-channel (KDA) recurrence (gk = log decay per key channel,
 * [B,T,H,Dk], required); otherwise as above. */
int ref_kda_f64(const double *q, const double *k, const double *v, const double *beta,
                const double *gk, const double *S0, double *o, double *S_T, int64_t B,
                int64_t T, int64_t H, int64_t Dk, int64_t Dv, int nthreads)
{
    if (!gk)
        return -1;
    return run(q, k, v, beta, NULL, gk, S0, o, S_T, B, T, H, Dk, Dv, nthreads);
}
