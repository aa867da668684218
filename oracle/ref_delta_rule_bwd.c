/*
 * fp64 CPU oracle of the delta rule's backward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite may load or call this file.  It shares no code, header,
 * helper or build flag with the HIP library.
 *
 * The forward pass is the recurrence of ref_delta_rule.c (plain, or gated
 * when g != NULL); per (b,h), with a_t = exp(g_t) (1 for the plain rule):
 *
 *   P_t     = a_t S_{t-1}                      decayed state (S_0 = S0)
 *   u_t     = v_t - P_t k_t                    prediction error
 *   S_t     = P_t + beta_t u_t k_t^T           = P_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   o_t     = S_t q_t
 *
 * For a loss L with upstream gradients do_t = dL/do_t and dS_T = dL/dS_T, the
 * gradients follow by the chain rule through one token at a time, in reverse
 * token order.  With D the gradient of L with respect to S_t (everything that
 * S_t influences: o_t, later tokens and S_T):
 *
 *   D       <- D + do_t q_t^T                  o_t reads S_t
 *   dq_t     = S_t^T do_t
 *   w        = D k_t                            (d_v vector)
 *   dv_t     = beta_t w
 *   dbeta_t  = u_t . w
 *   dk_t     = beta_t (D^T u_t - P_t^T w)       k_t enters the write twice
 *   dP       = D - beta_t w k_t^T              = D (I - beta_t k_t k_t^T)
 *   dg_t     = <dP, P_t>                        P_t = exp(g_t) S_{t-1}
 *   D       <- a_t dP                           gradient with respect to S_{t-1}
 *
 * and finally dS0 = D.
 *
 * Per-channel decay (ref_kda_bwd_f64, Kimi Delta Attention): gk_t [d_k]
 * scales column j of the state by a_t[j] = exp(gk_t[j]) (hada.io digest,
 * section "Kimi Delta Attention : attenuation par canal": the decay S_{t-1}
 * D_t with D_t = Diag(alpha_t) comes before the prediction), so
 *
 *   P_t     = S_{t-1} Diag(a_t)
 *   dgk_t[j] = sum_i dP_ij (P_t)_ij             column j of <dP, P_t>
 *   D       <- dP Diag(a_t)
 *
 * and every other line above is unchanged.  These are derived here from the update as the pages
 * state it (the pages give the strategy of recomputing states in the
 * backward -- paperlayer summary of arXiv:2406.06484, section 3 -- but not
 * the equations); the tests pin them with central finite differences and
 * with PyTorch autograd through an independently written forward loop.
 *
 * Arithmetic: IEEE fp64, ascending-index dot products, no FMA contraction.
 * The forward states S_0 .. S_T of one head are kept in memory
 * ((T+1) d_v d_k doubles per thread), then read back in reverse.
 *
 * Layouts as the forward: q, k, dq, dk [B,T,H,Dk]; v, do_, dv [B,T,H,Dv];
 * beta, g, dbeta, dg [B,T,H]; S0, dS_T, dS0 [B,H,Dv,Dk].  S0 and dS_T may be
 * NULL (zero); g and dg may be NULL (plain rule; dg is ignored without g).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *beta, *g, *gk, *S0, *dout, *dST;
    double *dq, *dk, *dv, *dbeta, *dg, *dgk, *dS0;
    int64_t B, T, H, Dk, Dv;
    int64_t next;
    int failed;
} bwd_job;

typedef struct {
    double *S;   /* (T+1) x Dv x Dk: S_0 .. S_T */
    double *P;   /* Dv x Dk */
    double *D;   /* Dv x Dk */
    double *u, *w;
} bwd_scratch;

/* Decay of element (i, j) of the state before token `row`: exp(g) for the
 * gated rule, exp(gk[j]) per key channel, 1 for the plain rule. */
static double decay(const bwd_job *J, int64_t row, int64_t j)
{
    if (J->gk)
        return exp(J->gk[row * J->Dk + j]);
    return J->g ? exp(J->g[row]) : 1.0;
}

static void one_head_bwd(const bwd_job *J, int64_t b, int64_t h, bwd_scratch *W)
{
    const int64_t T = J->T, H = J->H, Dk = J->Dk, Dv = J->Dv, M = Dv * Dk;
    const int64_t sh = (b * H + h) * M;
    double *S = W->S, *P = W->P, *D = W->D, *u = W->u, *w = W->w;

    /* forward, keeping every state */
    if (J->S0)
        memcpy(S, J->S0 + sh, (size_t)M * sizeof(double));
    else
        memset(S, 0, (size_t)M * sizeof(double));
    for (int64_t t = 0; t < T; ++t) {
        const int64_t row = (b * T + t) * H + h;
        const double *kt = J->k + row * Dk, *vt = J->v + row * Dv;
        const double bt = J->beta[row];
        const double *Sp = S + t * M;
        double *Sn = S + (t + 1) * M;
        for (int64_t i = 0; i < Dv; ++i)
            for (int64_t j = 0; j < Dk; ++j)
                P[i * Dk + j] = decay(J, row, j) * Sp[i * Dk + j];
        for (int64_t i = 0; i < Dv; ++i) {
            double p = 0.0;
            for (int64_t j = 0; j < Dk; ++j)
                p += P[i * Dk + j] * kt[j];
            u[i] = vt[i] - p;
        }
        for (int64_t i = 0; i < Dv; ++i)
            for (int64_t j = 0; j < Dk; ++j)
                Sn[i * Dk + j] = P[i * Dk + j] + (bt * u[i]) * kt[j];
    }

    /* reverse */
    if (J->dST)
        memcpy(D, J->dST + sh, (size_t)M * sizeof(double));
    else
        memset(D, 0, (size_t)M * sizeof(double));
    for (int64_t t = T - 1; t >= 0; --t) {
        const int64_t row = (b * T + t) * H + h;
        const double *qt = J->q + row * Dk, *kt = J->k + row * Dk, *vt = J->v + row * Dv;
        const double *dot = J->dout + row * Dv;
        const double bt = J->beta[row];
        const double *Sp = S + t * M, *Sn = S + (t + 1) * M;
        double *dqt = J->dq + row * Dk, *dkt = J->dk + row * Dk, *dvt = J->dv + row * Dv;

        /* o_t = S_t q_t */
        for (int64_t i = 0; i < Dv; ++i)
            for (int64_t j = 0; j < Dk; ++j)
                D[i * Dk + j] += dot[i] * qt[j];
        for (int64_t j = 0; j < Dk; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < Dv; ++i)
                acc += Sn[i * Dk + j] * dot[i];
            dqt[j] = acc;
        }
        /* recompute P_t and u_t */
        for (int64_t i = 0; i < Dv; ++i)
            for (int64_t j = 0; j < Dk; ++j)
                P[i * Dk + j] = decay(J, row, j) * Sp[i * Dk + j];
        for (int64_t i = 0; i < Dv; ++i) {
            double p = 0.0;
            for (int64_t j = 0; j < Dk; ++j)
                p += P[i * Dk + j] * kt[j];
            u[i] = vt[i] - p;
        }
        /* w = D k_t */
        for (int64_t i = 0; i < Dv; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < Dk; ++j)
                acc += D[i * Dk + j] * kt[j];
            w[i] = acc;
        }
        double db = 0.0;
        for (int64_t i = 0; i < Dv; ++i) {
            dvt[i] = bt * w[i];
            db += u[i] * w[i];
        }
        J->dbeta[row] = db;
        for (int64_t j = 0; j < Dk; ++j) {
            double a1 = 0.0, a2 = 0.0;
            for (int64_t i = 0; i < Dv; ++i) {
                a1 += D[i * Dk + j] * u[i];
                a2 += P[i * Dk + j] * w[i];
            }
            dkt[j] = bt * (a1 - a2);
        }
        /* dP = D - beta_t w k_t^T, kept in D */
        for (int64_t i = 0; i < Dv; ++i)
            for (int64_t j = 0; j < Dk; ++j)
                D[i * Dk + j] -= (bt * w[i]) * kt[j];
        if (J->g && J->dg) {
            double acc = 0.0;
            for (int64_t i = 0; i < M; ++i)
                acc += D[i] * P[i];
            J->dg[row] = acc;
        }
        if (J->gk && J->dgk) {
            for (int64_t j = 0; j < Dk; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < Dv; ++i)
                    acc += D[i * Dk + j] * P[i * Dk + j];
                J->dgk[row * Dk + j] = acc;
            }
        }
        for (int64_t i = 0; i < Dv; ++i)
            for (int64_t j = 0; j < Dk; ++j)
                D[i * Dk + j] = decay(J, row, j) * D[i * Dk + j];
    }
    memcpy(J->dS0 + sh, D, (size_t)M * sizeof(double));
}

static void *bwd_worker(void *arg)
{
    bwd_job *J = (bwd_job *)arg;
    const int64_t M = J->Dv * J->Dk;
    bwd_scratch W;
    W.S = (double *)malloc((size_t)((J->T + 1) * M) * sizeof(double));
    W.P = (double *)malloc((size_t)M * sizeof(double));
    W.D = (double *)malloc((size_t)M * sizeof(double));
    W.u = (double *)malloc((size_t)J->Dv * sizeof(double));
    W.w = (double *)malloc((size_t)J->Dv * sizeof(double));
    if (!W.S || !W.P || !W.D || !W.u || !W.w) {
        __atomic_store_n(&J->failed, 1, __ATOMIC_SEQ_CST);
    } else {
        for (;;) {
            int64_t bh = __atomic_fetch_add(&J->next, 1, __ATOMIC_SEQ_CST);
            if (bh >= J->B * J->H)
                break;
            one_head_bwd(J, bh / J->H, bh % J->H, &W);
        }
    }
    free(W.S);
    free(W.P);
    free(W.D);
    free(W.u);
    free(W.w);
    return NULL;
}

static int run_bwd(bwd_job *J, int nthreads)
{
    if (J->B * J->H == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > J->B * J->H)
        nthreads = (int)(J->B * J->H);
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!tid)
        return -2;
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, bwd_worker, J) != 0)
            break;
        ++started;
    }
    bwd_worker(J);
    for (int i = 1; i <= started; ++i)
        pthread_join(tid[i], NULL);
    free(tid);
    return J->failed ? -2 : 0;
}

/*
 * Gradients of L = sum_t <do_t, o_t> + <dS_T, S_T> with respect to q, k, v,
 * beta, g (gated rule only) and S0.  Threads split (b,h) pairs only; the
 * result does not depend on the thread count.  Returns 0 on success, -1 on
 * bad arguments, -2 on allocation or thread failure.
 */
int ref_delta_rule_bwd_f64(const double *q, const double *k, const double *v,
                           const double *beta, const double *g, const double *S0,
                           const double *dout, const double *dST, double *dq, double *dk,
                           double *dv, double *dbeta, double *dg, double *dS0, int64_t B,
                           int64_t T, int64_t H, int64_t Dk, int64_t Dv, int nthreads)
{
    if (!q || !k || !v || !beta || !dout || !dq || !dk || !dv || !dbeta || !dS0 || B < 0 ||
        T < 0 || H < 0 || Dk < 1 || Dv < 1)
        return -1;
    bwd_job J = {q,  k,  v,     beta, g,    NULL, S0, dout, dST, dq, dk, dv,
                 dbeta, dg, NULL, dS0, B, T, H, Dk, Dv, 0, 0};
    return run_bwd(&J, nthreads);
}

/*
 * The same gradients for the per-key-channel decay (gk [B,T,H,Dk] in, dgk
 * [B,T,H,Dk] out).  Same return codes.
 */
int ref_kda_bwd_f64(const double *q, const double *k, const double *v, const double *beta,
                    const double *gk, const double *S0, const double *dout, const double *dST,
                    double *dq, double *dk, double *dv, double *dbeta, double *dgk, double *dS0,
                    int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int nthreads)
{
    if (!q || !k || !v || !beta || !gk || !dout || !dq || !dk || !dv || !dbeta || !dgk ||
        !dS0 || B < 0 || T < 0 || H < 0 || Dk < 1 || Dv < 1)
        return -1;
    bwd_job J = {q,  k,  v,     beta, NULL, gk, S0, dout, dST, dq, dk, dv,
                 dbeta, NULL, dgk, dS0, B, T, H, Dk, Dv, 0, 0};
    return run_bwd(&J, nthreads);
}
