/*
 * kda_oracle.c -- plain fp64 CPU oracle for the gated delta-rule state layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the GPU library.
 *
 * What it computes (page "The argument, in one page", section "Everything, in one
 * table", rows "Delta rule", "Gated DeltaNet" and "KDA"): a state S of shape dk x dv
 * that every token updates in place.  For token t of one (sequence, head):
 *
 *   order 0 (the table's KDA row, erase, then decay, then write):
 *       S <- Diag(a_t) (I - beta_t k_t^T k_t) S + beta_t k_t^T v_t
 *   order 1 (decay first, then erase and write):
 *       S <- (I - beta_t k_t^T k_t) Diag(a_t) S + beta_t k_t^T v_t
 *
 *   followed by the read o_t = q_t S (read after the update).
 *
 * a_t = exp(log_a_t) is per key channel (KDA: "a gate per channel; every row of the
 * state gets its own lifetime", page "The efficiency lineage", item 10) or one scalar
 * per token and head (Gated DeltaNet row).  q_t, k_t are 1 x dk row vectors, v_t is
 * 1 x dv, beta_t a scalar.  Both orderings coincide when a_t is uniform over channels.
 *
 * The read o = q S is not printed on the pages (they only say a query performs a
 * weighted read of the values); it is the plainest reading of S as an associative
 * memory from keys (rows) to values (columns).
 *
 * Everything is evaluated token by token in double precision, exactly as written:
 * no chunking, no reassociation beyond the loops below.  Sequences are packed along
 * the token axis and delimited by cu_seqlens; each starts from its own S0 (or zero).
 *
 * Layouts (all row-major, contiguous):
 *   q, k   [T, H, dk]     v, o [T, H, dv]
 *   log_a  [T, H, dk]  (scalar_decay = 0)   or  [T, H]  (scalar_decay = 1)
 *   beta   [T, H]
 *   S0, ST [N, H, dk, dv]   (S0 may be NULL: zero initial state)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t num_seqs, num_heads, dk, dv;
    const int64_t* cu;
    const double *q, *k, *v, *log_a, *beta, *S0;
    int scalar_decay, order;
    double *o, *ST;
    int64_t next_unit; /* shared work counter, guarded by mu */
    pthread_mutex_t mu;
    int failed;
} oracle_job;

/* One (sequence n, head h): the token loop. */
static int run_unit(oracle_job* J, int64_t n, int64_t h) {
    const int64_t H = J->num_heads, dk = J->dk, dv = J->dv;
    double* S = (double*)malloc(sizeof(double) * (size_t)(dk * dv));
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    double* y = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!S || !a || !y) {
        free(S); free(a); free(y);
        return 1;
    }
    const size_t state_off = (size_t)((n * H + h) * dk * dv);
    if (J->S0)
        memcpy(S, J->S0 + state_off, sizeof(double) * (size_t)(dk * dv));
    else
        memset(S, 0, sizeof(double) * (size_t)(dk * dv));

    for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
        const int64_t th = t * H + h;
        const double* qt = J->q + th * dk;
        const double* kt = J->k + th * dk;
        const double* vt = J->v + th * dv;
        const double b = J->beta[th];
        for (int64_t c = 0; c < dk; ++c)
            a[c] = exp(J->scalar_decay ? J->log_a[th] : J->log_a[th * dk + c]);

        if (J->order == 0) {
            /* y = k S : what the state currently holds along k */
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < dk; ++c) acc += kt[c] * S[c * dv + j];
                y[j] = acc;
            }
            /* erase along k, decay every row c by a_c, then write beta k^T v */
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < dv; ++j)
                    S[c * dv + j] = a[c] * (S[c * dv + j] - b * kt[c] * y[j]) + b * kt[c] * vt[j];
        } else {
            /* decay rows first */
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < dv; ++j) S[c * dv + j] = a[c] * S[c * dv + j];
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < dk; ++c) acc += kt[c] * S[c * dv + j];
                y[j] = acc;
            }
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < dv; ++j)
                    S[c * dv + j] = S[c * dv + j] - b * kt[c] * y[j] + b * kt[c] * vt[j];
        }

        /* read after the update: o_t = q_t S_t */
        double* ot = J->o + th * dv;
        for (int64_t j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < dk; ++c) acc += qt[c] * S[c * dv + j];
            ot[j] = acc;
        }
    }
    if (J->ST) memcpy(J->ST + state_off, S, sizeof(double) * (size_t)(dk * dv));
    free(S); free(a); free(y);
    return 0;
}

static void* worker(void* arg) {
    oracle_job* J = (oracle_job*)arg;
    const int64_t units = J->num_seqs * J->num_heads;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t u = J->next_unit++;
        pthread_mutex_unlock(&J->mu);
        if (u >= units) break;
        if (run_unit(J, u / J->num_heads, u % J->num_heads)) {
            pthread_mutex_lock(&J->mu);
            J->failed = 1;
            pthread_mutex_unlock(&J->mu);
        }
    }
    return NULL;
}

/*
 * Returns 0 on success; 1 for invalid sizes or cu_seqlens (not starting at 0,
 * decreasing); 2 if memory or threads could not be obtained.  o receives [T,H,dv]
 * (T = cu_seqlens[num_seqs]); ST (may be NULL) receives [N,H,dk,dv].
 */
int kda_oracle_fwd(int64_t num_seqs, const int64_t* cu_seqlens, int64_t num_heads,
                   int64_t dk, int64_t dv, const double* q, const double* k,
                   const double* v, const double* log_a, int scalar_decay,
                   const double* beta, const double* S0, int order, double* o,
                   double* ST, int num_threads) {
    if (num_seqs < 0 || num_heads <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return 1;
    if (order != 0 && order != 1) return 1;
    if (cu_seqlens[0] != 0) return 1;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return 1;
    if (num_seqs == 0) return 0;
    if (cu_seqlens[num_seqs] > 0 && (!q || !k || !v || !log_a || !beta || !o)) return 1;

    oracle_job J;
    memset(&J, 0, sizeof(J));
    J.num_seqs = num_seqs; J.num_heads = num_heads; J.dk = dk; J.dv = dv;
    J.cu = cu_seqlens; J.q = q; J.k = k; J.v = v; J.log_a = log_a; J.beta = beta;
    J.S0 = S0; J.scalar_decay = scalar_decay ? 1 : 0; J.order = order; J.o = o; J.ST = ST;
    pthread_mutex_init(&J.mu, NULL);

    const int64_t units = num_seqs * num_heads;
    int nt = num_threads > 0 ? num_threads : 1;
    if (nt > units) nt = (int)units;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th) { pthread_mutex_destroy(&J.mu); return 2; }
    int started = 0;
    for (int i = 0; i < nt; ++i) {
        if (pthread_create(&th[i], NULL, worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) worker(&J); /* could not start any thread: run inline */
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return J.failed ? 2 : 0;
}
