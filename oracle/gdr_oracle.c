/*
 * gdr_oracle.c -- plain fp64 CPU oracle of the gated delta rule forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the GPU path is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it; the product library never links or calls
 * it, and it shares no code, header or constant with the GPU path.
 *
 * What it computes (token by token, no chunking, no reordering):
 *
 *   S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   o_t = S_t q_t
 *
 * with S in R^{d_v x d_k} (row i = value channel i, column c = key channel c).
 * Sources on the pages:
 *  - "FG2-GDN" page, section 1 (Introduction): Gated DeltaNet's scalar decay
 *    alpha_t in (0,1); KDA's channel-wise decay Diag(alpha_t).
 *  - same page, section 5, "Linear Attention as Recurrent Memory": the unified
 *    update S_t = A_t S_{t-1} + (write term), read-out through the state with
 *    the query; the page stores S as d_k x d_v and reads o = S^T q, which is the
 *    transpose of the orientation used here (same numbers).
 *  - same page, section 5, "Delta Rule and Online Learning": each update is one
 *    SGD step on ||S^T k_t - v_t||^2, i.e. write beta_t times the prediction
 *    error along k_t.
 *  - "Gated Delta Networks" page, abstract: gating (decay) combined with the
 *    delta update.
 * The order "decay first, then erase with the decayed read" is the reading of
 * the formula above (Diag(alpha) applied before the rank-1 erase); with a
 * scalar decay the two orders coincide.  The output reads the state after the
 * update of the same token.
 *
 * Per token, for each (b,h) pair independently:
 *   a_c   = exp(log_alpha[c])           (one value for every c if the gate is scalar)
 *   S[i][c] *= a_c                      decay
 *   p_i   = sum_c S[i][c] k_c           read the decayed memory at k
 *   u_i   = beta (v_i - p_i)            delta-rule correction
 *   S[i][c] += u_i k_c                  rank-1 write
 *   o_i   = sum_c S[i][c] q_c           read-out after the update
 *
 * Layouts (row-major, contiguous), all fp64 here:
 *   q, k       [B, T, H, dk]
 *   v, o       [B, T, H, dv]
 *   log_alpha  [B, T, H]            (scalar gate)  or [B, T, H, dk] (channel gate)
 *   beta       [B, T, H]
 *   S0, S_T    [B, H, dv, dk]       (S0 may be NULL: zero initial state;
 *                                    S_T may be NULL: not written)
 * Threads split the independent (b,h) pairs; each pair is computed by exactly
 * one thread with the sequential loop above, so the result does not depend on
 * the thread count.
 *
 * Channel-wise write rate (FG2-GDN and FG2-GDN+, "FG2-GDN" page, sections 3.2,
 * 3.4-3.6 and 6): the scalar beta_t becomes a vector beta^k_t in R^{d_k} that
 * enters through the scaled key k~_t = sqrt(beta^k_t) (elementwise) * k_t, and
 * the value is scaled the same way, v~_t = sqrt(beta^v_t) * v_t, with
 * beta^v = beta^k for FG2-GDN (d_k = d_v) and a separate beta^v in R^{d_v} for
 * FG2-GDN+.  The update keeps the tied, symmetric form with unit rate on the
 * scaled vectors:
 *
 *   S_t = S_{t-1} Diag(alpha_t) (I - k~_t k~_t^T) + v~_t k~_t^T,   o_t = S_t q_t
 *
 * The page prints neither equation; this is the reading that keeps its stated
 * properties: a tied diagonal-plus-rank-1 transition, elementwise square roots
 * and scalings only, the same chunkwise algorithm with the scaled keys, and
 * exactly KDA (Gated DeltaNet for a scalar decay) when beta^k = beta^v is the
 * same number in every channel (k~ k~^T = beta k k^T, v~ k~^T = beta v k^T).
 * Queries are not scaled.
 *
 * Decoupled erase and write gates (Gated DeltaNet-2; "Daily Papers" pages,
 * the Gated DeltaNet-2 abstract and citation notes): a channel-wise erase gate
 * b_t in R^{d_k} on the key side and a channel-wise write gate w_t in R^{d_v}
 * on the value side replace the tied scalar beta_t:
 *
 *   S_t = S_{t-1} Diag(alpha_t) (I - k_t (b_t * k_t)^T) + (w_t * v_t) k_t^T
 *
 * i.e. read the decayed memory at k, erase that read along the gated key
 * b * k (the asymmetric "erase factor"), write the gated value along k.  The
 * page prints no equation; this reading keeps what it states: the delta-rule
 * fast-weight structure, erase on the key side and write on the value side,
 * KDA (Gated DeltaNet for a scalar decay) when b_t and w_t collapse to the same
 * scalar beta_t, and an erase factor that is beta_r gamma_r^2 kbar_r in the
 * scalar-decay chunk form (kbar_r = k_r / gamma_r).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *log_alpha, *beta, *S0;
    double *o, *S_T;
    int64_t B, T, H, dk, dv;
    int channel_gate;
    int64_t next_unit;           /* work counter, guarded by mu */
    pthread_mutex_t mu;
} job_t;

/* One token of the recurrence on one state S [dv][dk] (in place). */
static void step(double *S, const double *q, const double *k, const double *v,
                 const double *log_alpha, int channel_gate, double beta,
                 double *o, double *a, int64_t dk, int64_t dv)
{
    for (int64_t c = 0; c < dk; ++c)
        a[c] = exp(channel_gate ? log_alpha[c] : log_alpha[0]);
    for (int64_t i = 0; i < dv; ++i) {
        double *row = S + i * dk;
        for (int64_t c = 0; c < dk; ++c) row[c] *= a[c];
        double p = 0.0;
        for (int64_t c = 0; c < dk; ++c) p += row[c] * k[c];
        double u = beta * (v[i] - p);
        for (int64_t c = 0; c < dk; ++c) row[c] += u * k[c];
        double acc = 0.0;
        for (int64_t c = 0; c < dk; ++c) acc += row[c] * q[c];
        o[i] = acc;
    }
}

static void run_unit(job_t *J, int64_t unit, double *S, double *a)
{
    const int64_t b = unit / J->H, h = unit % J->H;
    const int64_t dk = J->dk, dv = J->dv, T = J->T, H = J->H;
    if (J->S0)
        memcpy(S, J->S0 + unit * dv * dk, sizeof(double) * dv * dk);
    else
        memset(S, 0, sizeof(double) * dv * dk);
    for (int64_t t = 0; t < T; ++t) {
        const int64_t bth = (b * T + t) * H + h;
        const double *la = J->log_alpha + (J->channel_gate ? bth * dk : bth);
        step(S, J->q + bth * dk, J->k + bth * dk, J->v + bth * dv, la,
             J->channel_gate, J->beta[bth], J->o + bth * dv, a, dk, dv);
    }
    if (J->S_T) memcpy(J->S_T + unit * dv * dk, S, sizeof(double) * dv * dk);
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *S = (double *)malloc(sizeof(double) * J->dv * J->dk);
    double *a = (double *)malloc(sizeof(double) * J->dk);
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t u = J->next_unit++;
        pthread_mutex_unlock(&J->mu);
        if (u >= J->B * J->H) break;
        run_unit(J, u, S, a);
    }
    free(S);
    free(a);
    return NULL;
}

/* Full sequence: returns 0 on success, -1 on bad arguments. */
int gdr_oracle_chunk_fwd(const double *q, const double *k, const double *v,
                         const double *log_alpha, const double *beta,
                         const double *S0, double *o, double *S_T,
                         int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                         int channel_gate, int nthreads)
{
    if (!q || !k || !v || !log_alpha || !beta || !o) return -1;
    if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) return -1;
    job_t J = {q, k, v, log_alpha, beta, S0, o, S_T, B, T, H, dk, dv,
               channel_gate != 0, 0};
    pthread_mutex_init(&J.mu, NULL);
    int64_t units = B * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)units;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/* One decode step: S_out = step(S_in); S_out may equal S_in. */
int gdr_oracle_decode_step(const double *q, const double *k, const double *v,
                           const double *log_alpha, const double *beta,
                           const double *S_in, double *S_out, double *o,
                           int64_t B, int64_t H, int64_t dk, int64_t dv,
                           int channel_gate)
{
    if (!q || !k || !v || !log_alpha || !beta || !S_in || !S_out || !o) return -1;
    if (B < 1 || H < 1 || dk < 1 || dv < 1) return -1;
    double *a = (double *)malloc(sizeof(double) * dk);
    for (int64_t u = 0; u < B * H; ++u) {
        if (S_out != S_in)
            memcpy(S_out + u * dv * dk, S_in + u * dv * dk, sizeof(double) * dv * dk);
        const double *la = log_alpha + (channel_gate ? u * dk : u);
        step(S_out + u * dv * dk, q + u * dk, k + u * dk, v + u * dv, la,
             channel_gate != 0, beta[u], o + u * dv, a, dk, dv);
    }
    free(a);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Channel-wise write rate (FG2): the delta rule with unit rate on the scaled  */
/* key sqrt(beta^k) k and the scaled value sqrt(beta^v) v (see the header).    */
/* ------------------------------------------------------------------------ */
typedef struct {
    const double *q, *k, *v, *log_alpha, *beta_k, *beta_v, *S0;
    double *o, *S_T;
    int64_t B, T, H, dk, dv;
    int channel_gate;
    int64_t next_unit;
    pthread_mutex_t mu;
} job_fg2_t;

/* The scaled key and value of one token. */
static void scale_kv(const double *k, const double *v, const double *bk, const double *bv,
                     double *ks, double *vs, int64_t dk, int64_t dv)
{
    for (int64_t c = 0; c < dk; ++c) ks[c] = sqrt(bk[c]) * k[c];
    for (int64_t i = 0; i < dv; ++i) vs[i] = sqrt(bv[i]) * v[i];
}

static void *worker_fg2(void *arg)
{
    job_fg2_t *J = (job_fg2_t *)arg;
    const int64_t dk = J->dk, dv = J->dv, T = J->T, H = J->H;
    double *S = (double *)malloc(sizeof(double) * dv * dk);
    double *a = (double *)malloc(sizeof(double) * dk);
    double *ks = (double *)malloc(sizeof(double) * dk);
    double *vs = (double *)malloc(sizeof(double) * dv);
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t u = J->next_unit++;
        pthread_mutex_unlock(&J->mu);
        if (u >= J->B * J->H) break;
        const int64_t b = u / H, h = u % H;
        if (J->S0)
            memcpy(S, J->S0 + u * dv * dk, sizeof(double) * dv * dk);
        else
            memset(S, 0, sizeof(double) * dv * dk);
        for (int64_t t = 0; t < T; ++t) {
            const int64_t bth = (b * T + t) * H + h;
            const double *la = J->log_alpha + (J->channel_gate ? bth * dk : bth);
            const double *bk = J->beta_k + bth * dk;
            const double *bv = J->beta_v ? J->beta_v + bth * dv : bk;
            scale_kv(J->k + bth * dk, J->v + bth * dv, bk, bv, ks, vs, dk, dv);
            step(S, J->q + bth * dk, ks, vs, la, J->channel_gate, 1.0, J->o + bth * dv, a, dk, dv);
        }
        if (J->S_T) memcpy(J->S_T + u * dv * dk, S, sizeof(double) * dv * dk);
    }
    free(S);
    free(a);
    free(ks);
    free(vs);
    return NULL;
}

/* Full sequence with channel-wise write rates.  beta_k: [B,T,H,dk];
 * beta_v: [B,T,H,dv] or NULL (then beta^v = beta^k, which needs dk == dv).
 * Returns 0 on success, -1 on bad arguments. */
int gdr_oracle_fg2_chunk_fwd(const double *q, const double *k, const double *v,
                             const double *log_alpha, const double *beta_k, const double *beta_v,
                             const double *S0, double *o, double *S_T,
                             int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             int channel_gate, int nthreads)
{
    if (!q || !k || !v || !log_alpha || !beta_k || !o) return -1;
    if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) return -1;
    if (!beta_v && dk != dv) return -1;
    job_fg2_t J = {q, k, v, log_alpha, beta_k, beta_v, S0, o, S_T, B, T, H, dk, dv,
                   channel_gate != 0, 0};
    pthread_mutex_init(&J.mu, NULL);
    int64_t units = B * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)units;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker_fg2, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/* One decode step with channel-wise write rates; S_out may equal S_in. */
int gdr_oracle_fg2_decode_step(const double *q, const double *k, const double *v,
                               const double *log_alpha, const double *beta_k,
                               const double *beta_v, const double *S_in, double *S_out,
                               double *o, int64_t B, int64_t H, int64_t dk, int64_t dv,
                               int channel_gate)
{
    if (!q || !k || !v || !log_alpha || !beta_k || !S_in || !S_out || !o) return -1;
    if (B < 1 || H < 1 || dk < 1 || dv < 1) return -1;
    if (!beta_v && dk != dv) return -1;
    double *a = (double *)malloc(sizeof(double) * dk);
    double *ks = (double *)malloc(sizeof(double) * dk);
    double *vs = (double *)malloc(sizeof(double) * dv);
    for (int64_t u = 0; u < B * H; ++u) {
        if (S_out != S_in)
            memcpy(S_out + u * dv * dk, S_in + u * dv * dk, sizeof(double) * dv * dk);
        const double *la = log_alpha + (channel_gate ? u * dk : u);
        const double *bk = beta_k + u * dk;
        scale_kv(k + u * dk, v + u * dv, bk, beta_v ? beta_v + u * dv : bk, ks, vs, dk, dv);
        step(S_out + u * dv * dk, q + u * dk, ks, vs, la, channel_gate != 0, 1.0, o + u * dv, a,
             dk, dv);
    }
    free(a);
    free(ks);
    free(vs);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Decoupled erase and write gates (Gated DeltaNet-2, see the header).        */
/* ------------------------------------------------------------------------ */
static void step_gdn2(double *S, const double *q, const double *k, const double *v,
                      const double *log_alpha, int channel_gate, const double *eb,
                      const double *ww, double *o, double *a, int64_t dk, int64_t dv)
{
    for (int64_t c = 0; c < dk; ++c)
        a[c] = exp(channel_gate ? log_alpha[c] : log_alpha[0]);
    for (int64_t i = 0; i < dv; ++i) {
        double *row = S + i * dk;
        for (int64_t c = 0; c < dk; ++c) row[c] *= a[c];          /* decay            */
        double r = 0.0;
        for (int64_t c = 0; c < dk; ++c) r += row[c] * k[c];      /* read at k        */
        for (int64_t c = 0; c < dk; ++c) row[c] -= r * eb[c] * k[c]; /* erase along b*k */
        const double u = ww[i] * v[i];
        for (int64_t c = 0; c < dk; ++c) row[c] += u * k[c];      /* write w*v along k */
        double acc = 0.0;
        for (int64_t c = 0; c < dk; ++c) acc += row[c] * q[c];
        o[i] = acc;
    }
}

typedef struct {
    const double *q, *k, *v, *log_alpha, *eb, *ww, *S0;
    double *o, *S_T;
    int64_t B, T, H, dk, dv;
    int channel_gate;
    int64_t next_unit;
    pthread_mutex_t mu;
} job_gdn2_t;

static void *worker_gdn2(void *arg)
{
    job_gdn2_t *J = (job_gdn2_t *)arg;
    const int64_t dk = J->dk, dv = J->dv, T = J->T, H = J->H;
    double *S = (double *)malloc(sizeof(double) * dv * dk);
    double *a = (double *)malloc(sizeof(double) * dk);
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t u = J->next_unit++;
        pthread_mutex_unlock(&J->mu);
        if (u >= J->B * J->H) break;
        const int64_t b = u / H, h = u % H;
        if (J->S0)
            memcpy(S, J->S0 + u * dv * dk, sizeof(double) * dv * dk);
        else
            memset(S, 0, sizeof(double) * dv * dk);
        for (int64_t t = 0; t < T; ++t) {
            const int64_t bth = (b * T + t) * H + h;
            const double *la = J->log_alpha + (J->channel_gate ? bth * dk : bth);
            step_gdn2(S, J->q + bth * dk, J->k + bth * dk, J->v + bth * dv, la, J->channel_gate,
                      J->eb + bth * dk, J->ww + bth * dv, J->o + bth * dv, a, dk, dv);
        }
        if (J->S_T) memcpy(J->S_T + u * dv * dk, S, sizeof(double) * dv * dk);
    }
    free(S);
    free(a);
    return NULL;
}

/* Full sequence with decoupled gates.  erase: [B,T,H,dk]; write: [B,T,H,dv].
 * Returns 0 on success, -1 on bad arguments. */
int gdr_oracle_gdn2_chunk_fwd(const double *q, const double *k, const double *v,
                              const double *log_alpha, const double *erase, const double *write,
                              const double *S0, double *o, double *S_T,
                              int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                              int channel_gate, int nthreads)
{
    if (!q || !k || !v || !log_alpha || !erase || !write || !o) return -1;
    if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) return -1;
    job_gdn2_t J = {q, k, v, log_alpha, erase, write, S0, o, S_T, B, T, H, dk, dv,
                    channel_gate != 0, 0};
    pthread_mutex_init(&J.mu, NULL);
    int64_t units = B * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)units;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker_gdn2, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return 0;
}
