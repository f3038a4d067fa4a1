/*
 * Causal grouped-query attention oracle: plain, slow, fp64, CPU only.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU-baseline
 * leg may load this library. The product path (the HIP library) never calls it,
 * shares no code, header, table or helper with it, and must fail loudly instead of
 * falling back to it.
 *
 * What it computes is the plain definition of the method, not the method's blocked
 * algorithm. Flash attention is an exact reordering of softmax attention (page "A
 * transformer in PTX", section "Flash attention", contrasts it with naive kernels that
 * store every score of a head; both give the same result). So this file stores the
 * full score matrix of each (batch, query head), as the naive kernels do, in double
 * precision, with no blocking, no online softmax and no log2 units.
 *
 * Conventions (readings of the pages, each one stated where it is used):
 *  - Layout: q, o, dO, dq are [B][T][Hq][d]; k, v, dk, dv are [B][T][Hkv][d];
 *    lse and delta are [B][Hq][T]. Element (b,t,h,c) of a [B][T][H][d] tensor sits
 *    at ((b*T + t)*H + h)*d + c.
 *  - Grouped-query sharing ("A transformer in PTX", section "The model": the dev preset
 *    maps six query heads onto two key/value heads): query head h reads key/value head
 *    h / G, G = Hq / Hkv, i.e. contiguous groups of G query heads.
 *  - Causality (section "Flash attention": a query block only visits key blocks that
 *    are not past it): query i sees keys 0..i inclusive; queries and keys share one
 *    position index.
 *  - Scale: scores are q.k * scale (the pages apply 1/sqrt(64) a single time).
 *  - LSE is the natural-log log-sum-exp of each row's scaled scores (section "Flash
 *    attention": the forward keeps it so that the backward can rebuild the
 *    probabilities without storing them).
 *  - Backward: the vector-Jacobian product for the loss L = sum(O * dO), with
 *    D_i = sum_c dO_ic O_ic. dK and dV of a key/value head sum over the G query
 *    heads that share it (section "The same bits every time": the dK/dV kernel loops
 *    over all the query heads that share the key/value head), in ascending head
 *    order, then ascending query index, so the oracle is itself deterministic.
 *
 * Parallelism: rows of one (batch, kv-group) are independent in the first phase, key
 * rows in the second; both are split over POSIX threads. Every sum is a plain loop
 * in a fixed order, so results do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

static size_t idx4(int b, int t, int h, int c, int T, int H, int d) {
    return (((size_t)b * T + t) * H + h) * d + c;
}
static size_t idx3(int b, int h, int t, int H, int T) {
    return ((size_t)b * H + h) * T + t;
}

/* bf16 -> fp64 decode: a bf16 value is the upper half of an IEEE binary32 pattern,
 * so widening is exact. */
int oracle_bf16_to_f64(const uint16_t* src, double* dst, long n) {
    if (n < 0 || (n > 0 && (!src || !dst))) return ORACLE_EINVAL;
    for (long i = 0; i < n; ++i) {
        uint32_t bits = (uint32_t)src[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        dst[i] = (double)f;
    }
    return ORACLE_OK;
}

int oracle_default_threads(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/* ------------------------------------------------------------------------- */
/* One (batch, kv-group) problem. The score, probability and dS matrices of    */
/* all G heads of the group are materialised in full ([G][T][T] each).        */

typedef struct {
    /* inputs */
    const double *q, *k, *v, *dO;
    int B, T, Hq, Hkv, d, G;
    double scale;
    int b, g;             /* the group being processed */
    int want_bwd;
    /* outputs (full tensors) */
    double *o, *lse, *delta, *dq, *dk, *dv;
    /* per-group working set */
    double *S, *P, *dS;   /* [G][T][T] */
    /* work distribution */
    pthread_mutex_t lock;
    long next, total;
} group_job;

static long take_work(group_job* job) {
    pthread_mutex_lock(&job->lock);
    long w = job->next < job->total ? job->next++ : -1;
    pthread_mutex_unlock(&job->lock);
    return w;
}

/* Phase 1, one query row i of query head h = g*G + hh: scores, softmax, O, LSE,
 * and (backward) dP, D, dS, dQ. */
static void row_phase(group_job* j, int hh, int i) {
    const int T = j->T, d = j->d, Hq = j->Hq, Hkv = j->Hkv, b = j->b, g = j->g;
    const int h = g * j->G + hh;
    double* S = j->S + ((size_t)hh * T + i) * T;
    double* P = j->P + ((size_t)hh * T + i) * T;
    const double* qi = j->q + idx4(b, i, h, 0, T, Hq, d);

    /* S_ij = scale * q_i . k_j for j <= i; -inf above the diagonal (masked). */
    for (int jj = 0; jj < T; ++jj) {
        if (jj > i) { S[jj] = -INFINITY; continue; }
        const double* kj = j->k + idx4(b, jj, g, 0, T, Hkv, d);
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += qi[c] * kj[c];
        S[jj] = j->scale * acc;
    }
    /* LSE_i = m + ln sum_j exp(S_ij - m), m the row max (row i always has key 0..i). */
    double m = -INFINITY;
    for (int jj = 0; jj <= i; ++jj) if (S[jj] > m) m = S[jj];
    double sum = 0.0;
    for (int jj = 0; jj <= i; ++jj) sum += exp(S[jj] - m);
    const double lse = m + log(sum);
    j->lse[idx3(b, h, i, Hq, T)] = lse;
    /* P_ij = exp(S_ij - LSE_i); zero where masked. */
    for (int jj = 0; jj < T; ++jj) P[jj] = jj <= i ? exp(S[jj] - lse) : 0.0;
    /* O_i = sum_j P_ij v_j */
    double* oi = j->o + idx4(b, i, h, 0, T, Hq, d);
    for (int c = 0; c < d; ++c) oi[c] = 0.0;
    for (int jj = 0; jj <= i; ++jj) {
        const double* vj = j->v + idx4(b, jj, g, 0, T, Hkv, d);
        for (int c = 0; c < d; ++c) oi[c] += P[jj] * vj[c];
    }
    if (!j->want_bwd) return;

    const double* doi = j->dO + idx4(b, i, h, 0, T, Hq, d);
    double* dS = j->dS + ((size_t)hh * T + i) * T;
    /* D_i = dO_i . O_i */
    double D = 0.0;
    for (int c = 0; c < d; ++c) D += doi[c] * oi[c];
    j->delta[idx3(b, h, i, Hq, T)] = D;
    /* dP_ij = dO_i . v_j ; dS_ij = P_ij (dP_ij - D_i) */
    for (int jj = 0; jj < T; ++jj) {
        if (jj > i) { dS[jj] = 0.0; continue; }
        const double* vj = j->v + idx4(b, jj, g, 0, T, Hkv, d);
        double dp = 0.0;
        for (int c = 0; c < d; ++c) dp += doi[c] * vj[c];
        dS[jj] = P[jj] * (dp - D);
    }
    /* dQ_i = scale * sum_j dS_ij k_j */
    double* dqi = j->dq + idx4(b, i, h, 0, T, Hq, d);
    for (int c = 0; c < d; ++c) dqi[c] = 0.0;
    for (int jj = 0; jj <= i; ++jj) {
        const double* kj = j->k + idx4(b, jj, g, 0, T, Hkv, d);
        for (int c = 0; c < d; ++c) dqi[c] += dS[jj] * kj[c];
    }
    for (int c = 0; c < d; ++c) dqi[c] *= j->scale;
}

/* Phase 2, one key row jj of kv head g: dV_j = sum_h sum_{i>=j} P^h_ij dO^h_i,
 * dK_j = scale * sum_h sum_{i>=j} dS^h_ij q^h_i, heads ascending, then rows ascending. */
static void key_phase(group_job* j, int jj) {
    const int T = j->T, d = j->d, Hq = j->Hq, Hkv = j->Hkv, b = j->b, g = j->g;
    double* dvj = j->dv + idx4(b, jj, g, 0, T, Hkv, d);
    double* dkj = j->dk + idx4(b, jj, g, 0, T, Hkv, d);
    for (int c = 0; c < d; ++c) { dvj[c] = 0.0; dkj[c] = 0.0; }
    for (int hh = 0; hh < j->G; ++hh) {
        const int h = g * j->G + hh;
        for (int i = jj; i < T; ++i) {
            const double p = j->P[((size_t)hh * T + i) * T + jj];
            const double ds = j->dS[((size_t)hh * T + i) * T + jj];
            const double* doi = j->dO + idx4(b, i, h, 0, T, Hq, d);
            const double* qi = j->q + idx4(b, i, h, 0, T, Hq, d);
            for (int c = 0; c < d; ++c) { dvj[c] += p * doi[c]; dkj[c] += ds * qi[c]; }
        }
    }
    for (int c = 0; c < d; ++c) dkj[c] *= j->scale;
}

static void* row_worker(void* arg) {
    group_job* j = (group_job*)arg;
    for (long w; (w = take_work(j)) >= 0;) row_phase(j, (int)(w / j->T), (int)(w % j->T));
    return NULL;
}
static void* key_worker(void* arg) {
    group_job* j = (group_job*)arg;
    for (long w; (w = take_work(j)) >= 0;) key_phase(j, (int)w);
    return NULL;
}

static void run_parallel(group_job* j, void* (*fn)(void*), long total, int nthreads) {
    j->next = 0;
    j->total = total;
    if (nthreads > total) nthreads = (int)total;
    if (nthreads <= 1) { fn(j); return; }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    if (th)
        for (; started < nthreads; ++started)
            if (pthread_create(&th[started], NULL, fn, j) != 0) break;
    fn(j); /* the calling thread works too; it also finishes everything if no thread started */
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    free(th);
}

static int run_all(const double* q, const double* k, const double* v, const double* dO,
                   double* o, double* lse, double* delta, double* dq, double* dk, double* dv,
                   int B, int T, int Hq, int Hkv, int d, double scale, int nthreads, int want_bwd) {
    if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0) return ORACLE_EINVAL;
    if (!(scale > 0.0) || !isfinite(scale)) return ORACLE_EINVAL;
    if (B == 0 || T == 0) return ORACLE_OK;
    if (!q || !k || !v || !o || !lse) return ORACLE_EINVAL;
    if (want_bwd && (!dO || !delta || !dq || !dk || !dv)) return ORACLE_EINVAL;
    if (nthreads <= 0) nthreads = oracle_default_threads();
    group_job job;
    memset(&job, 0, sizeof job);
    job.q = q; job.k = k; job.v = v; job.dO = dO;
    job.o = o; job.lse = lse; job.delta = delta; job.dq = dq; job.dk = dk; job.dv = dv;
    job.B = B; job.T = T; job.Hq = Hq; job.Hkv = Hkv; job.d = d; job.G = Hq / Hkv;
    job.scale = scale; job.want_bwd = want_bwd;
    const size_t mat = (size_t)job.G * T * T;
    job.S = (double*)malloc(mat * sizeof(double));
    job.P = (double*)malloc(mat * sizeof(double));
    job.dS = want_bwd ? (double*)malloc(mat * sizeof(double)) : NULL;
    if (!job.S || !job.P || (want_bwd && !job.dS)) {
        free(job.S); free(job.P); free(job.dS);
        return ORACLE_ENOMEM;
    }
    pthread_mutex_init(&job.lock, NULL);
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            job.b = b;
            job.g = g;
            run_parallel(&job, row_worker, (long)job.G * T, nthreads);
            if (want_bwd) run_parallel(&job, key_worker, (long)T, nthreads);
        }
    }
    pthread_mutex_destroy(&job.lock);
    free(job.S); free(job.P); free(job.dS);
    return ORACLE_OK;
}

/* Forward: o [B][T][Hq][d], lse [B][Hq][T]. */
int oracle_attn_fwd(const double* q, const double* k, const double* v, double* o, double* lse,
                    int B, int T, int Hq, int Hkv, int d, double scale, int nthreads) {
    return run_all(q, k, v, NULL, o, lse, NULL, NULL, NULL, NULL, B, T, Hq, Hkv, d, scale,
                   nthreads, 0);
}

/* Forward and backward: also delta [B][Hq][T], dq [B][T][Hq][d], dk, dv [B][T][Hkv][d]. */
int oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dO,
                    double* o, double* lse, double* delta, double* dq, double* dk, double* dv,
                    int B, int T, int Hq, int Hkv, int d, double scale, int nthreads) {
    return run_all(q, k, v, dO, o, lse, delta, dq, dk, dv, B, T, Hq, Hkv, d, scale, nthreads, 1);
}
