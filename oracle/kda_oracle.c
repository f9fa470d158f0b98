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
 *
 * kda_oracle_bwd (further below) is the gradient of the same token loop: for a
 * scalar loss whose derivatives with respect to o and S_T are dO and dS_T, it
 * returns the derivatives with respect to q, k, v, log_a, beta and S0.  It walks
 * the tokens backwards with the chain rule applied to the update above, one
 * token at a time, again in double precision.
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

/* ------------------------------------------------------------------------- */
/* Backward: reverse-mode derivative of the token loop above.                 */
/*                                                                           */
/* Write L for a scalar loss with dL/do_t = dO_t and dL/dS_T = dS_T, and      */
/* Lam for dL/dS_t, the total derivative with respect to the state after     */
/* token t (through o_t and through every later token).  Going backwards:    */
/*                                                                           */
/*   Lam <- Lam + q_t^T dO_t                 (o_t = q_t S_t)                  */
/*   dq_t = dO_t S_t^T                                                        */
/*                                                                           */
/* order 0, S_t = D (S_{t-1} - beta k^T y) + beta k^T v with y = k S_{t-1},  */
/* D = Diag(a_t):                                                             */
/*   g       = (k . a) Lam      (1 x dv; k . a is the channel-wise product)   */
/*   r       = k Lam            (1 x dv)                                      */
/*   dv_t    = beta r                                                         */
/*   dbeta_t = r . v - g . y                                                  */
/*   dk_t[c] = beta ((Lam v^T)[c] - a[c] (Lam y^T)[c] - (S_{t-1} g^T)[c])     */
/*   dlog_a_t[c] = sum_j Lam[c][j] (S_t[c][j] - beta k[c] v[j])              */
/*   Lam <- D Lam - beta k^T g  (the derivative with respect to S_{t-1})     */
/*                                                                           */
/* order 1, S_t = P - beta k^T (k P) + beta k^T v with P = D S_{t-1}:        */
/*   r       = k Lam,  y' = k P,  dP = Lam - beta k^T r                       */
/*   dv_t    = beta r                                                         */
/*   dbeta_t = r . (v - y')                                                   */
/*   dk_t[c] = beta ((Lam v^T)[c] - (Lam y'^T)[c] - a[c] (S_{t-1} r^T)[c])    */
/*   dlog_a_t[c] = sum_j dP[c][j] P[c][j]                                    */
/*   Lam <- D dP                                                              */
/*                                                                           */
/* With a scalar decay the one log_a_t of a token feeds every channel, so its */
/* derivative is the sum of the per-channel ones.  After the first token Lam  */
/* is dL/dS0.                                                                 */
/*                                                                           */
/* The states S_{t-1}, S_t are recomputed: the forward loop keeps a copy of  */
/* the state every CKPT tokens, and each stretch is replayed from its copy    */
/* before it is walked backwards.  Replaying runs the same arithmetic as the */
/* forward loop above, so the states are the ones it produces.               */
/* ------------------------------------------------------------------------- */

#define CKPT 64

typedef struct {
    int64_t num_seqs, num_heads, dk, dv;
    const int64_t* cu;
    const double *q, *k, *v, *log_a, *beta, *S0, *dO, *dST;
    int scalar_decay, order;
    double *dq, *dk_out, *dv_out, *dla, *dbeta, *dS0;
    int64_t next_unit;
    pthread_mutex_t mu;
    int failed;
} oracle_bwd_job;

/* One token of the forward loop (same arithmetic as run_unit): S <- update(S). */
static void fwd_token(const oracle_bwd_job* J, int64_t th, double* S, double* a, double* y) {
    const int64_t dk = J->dk, dv = J->dv;
    const double* kt = J->k + th * dk;
    const double* vt = J->v + th * dv;
    const double b = J->beta[th];
    for (int64_t c = 0; c < dk; ++c)
        a[c] = exp(J->scalar_decay ? J->log_a[th] : J->log_a[th * dk + c]);
    if (J->order == 0) {
        for (int64_t j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < dk; ++c) acc += kt[c] * S[c * dv + j];
            y[j] = acc;
        }
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < dv; ++j)
                S[c * dv + j] = a[c] * (S[c * dv + j] - b * kt[c] * y[j]) + b * kt[c] * vt[j];
    } else {
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
}

static int run_unit_bwd(oracle_bwd_job* J, int64_t n, int64_t h) {
    const int64_t H = J->num_heads, dk = J->dk, dv = J->dv;
    const int64_t t0 = J->cu[n], t1 = J->cu[n + 1], len = t1 - t0;
    const size_t SZ = (size_t)(dk * dv);
    const int64_t nck = len / CKPT + 1;                 /* copies at t0, t0+CKPT, ... */
    double* ck = (double*)malloc(sizeof(double) * SZ * (size_t)nck);
    double* st = (double*)malloc(sizeof(double) * SZ * (size_t)(CKPT + 1)); /* S_{s-1} .. S_{e-1} */
    double* Lam = (double*)malloc(sizeof(double) * SZ);
    double* dP = (double*)malloc(sizeof(double) * SZ);
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    double* y = (double*)malloc(sizeof(double) * (size_t)dv);
    double* g = (double*)malloc(sizeof(double) * (size_t)dv);
    double* r = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!ck || !st || !Lam || !dP || !a || !y || !g || !r) {
        free(ck); free(st); free(Lam); free(dP); free(a); free(y); free(g); free(r);
        return 1;
    }
    const size_t state_off = (size_t)((n * H + h) * dk * dv);

    /* forward loop, keeping the state before tokens t0 + m * CKPT */
    double* S = st;
    if (J->S0) memcpy(S, J->S0 + state_off, sizeof(double) * SZ);
    else memset(S, 0, sizeof(double) * SZ);
    for (int64_t t = t0; t < t1; ++t) {
        if ((t - t0) % CKPT == 0) memcpy(ck + SZ * (size_t)((t - t0) / CKPT), S, sizeof(double) * SZ);
        fwd_token(J, t * H + h, S, a, y);
    }

    if (J->dST) memcpy(Lam, J->dST + state_off, sizeof(double) * SZ);
    else memset(Lam, 0, sizeof(double) * SZ);

    for (int64_t m = (len - 1) / CKPT; len > 0 && m >= 0; --m) {
        const int64_t s = t0 + m * CKPT;
        const int64_t e = s + CKPT < t1 ? s + CKPT : t1;
        /* replay: st[i] = state before token s + i, i = 0 .. e - s */
        memcpy(st, ck + SZ * (size_t)m, sizeof(double) * SZ);
        for (int64_t t = s; t < e; ++t) {
            memcpy(st + SZ * (size_t)(t - s + 1), st + SZ * (size_t)(t - s), sizeof(double) * SZ);
            fwd_token(J, t * H + h, st + SZ * (size_t)(t - s + 1), a, y);
        }
        for (int64_t t = e - 1; t >= s; --t) {
            const int64_t th = t * H + h;
            const double* Sp = st + SZ * (size_t)(t - s);      /* S_{t-1} */
            const double* Sc = st + SZ * (size_t)(t - s + 1);  /* S_t */
            const double* qt = J->q + th * dk;
            const double* kt = J->k + th * dk;
            const double* vt = J->v + th * dv;
            const double* dot = J->dO + th * dv;
            const double b = J->beta[th];
            for (int64_t c = 0; c < dk; ++c)
                a[c] = exp(J->scalar_decay ? J->log_a[th] : J->log_a[th * dk + c]);

            /* o_t = q_t S_t */
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < dv; ++j) Lam[c * dv + j] += qt[c] * dot[j];
            for (int64_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) acc += dot[j] * Sc[c * dv + j];
                J->dq[th * dk + c] = acc;
            }

            double dla_sum = 0.0;
            if (J->order == 0) {
                for (int64_t j = 0; j < dv; ++j) {
                    double ay = 0.0, ag = 0.0, ar = 0.0;
                    for (int64_t c = 0; c < dk; ++c) {
                        ay += kt[c] * Sp[c * dv + j];
                        ag += kt[c] * a[c] * Lam[c * dv + j];
                        ar += kt[c] * Lam[c * dv + j];
                    }
                    y[j] = ay; g[j] = ag; r[j] = ar;
                }
                double db = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    J->dv_out[th * dv + j] = b * r[j];
                    db += r[j] * vt[j] - g[j] * y[j];
                }
                J->dbeta[th] = db;
                for (int64_t c = 0; c < dk; ++c) {
                    double lv = 0.0, ly = 0.0, sg = 0.0, dl = 0.0;
                    for (int64_t j = 0; j < dv; ++j) {
                        lv += Lam[c * dv + j] * vt[j];
                        ly += Lam[c * dv + j] * y[j];
                        sg += Sp[c * dv + j] * g[j];
                        dl += Lam[c * dv + j] * (Sc[c * dv + j] - b * kt[c] * vt[j]);
                    }
                    J->dk_out[th * dk + c] = b * (lv - a[c] * ly - sg);
                    if (J->scalar_decay) dla_sum += dl;
                    else J->dla[th * dk + c] = dl;
                }
                for (int64_t c = 0; c < dk; ++c)
                    for (int64_t j = 0; j < dv; ++j)
                        Lam[c * dv + j] = a[c] * Lam[c * dv + j] - b * kt[c] * g[j];
            } else {
                for (int64_t j = 0; j < dv; ++j) {
                    double ay = 0.0, ar = 0.0;
                    for (int64_t c = 0; c < dk; ++c) {
                        ay += kt[c] * a[c] * Sp[c * dv + j];
                        ar += kt[c] * Lam[c * dv + j];
                    }
                    y[j] = ay; r[j] = ar;
                }
                double db = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    J->dv_out[th * dv + j] = b * r[j];
                    db += r[j] * (vt[j] - y[j]);
                }
                J->dbeta[th] = db;
                for (int64_t c = 0; c < dk; ++c)
                    for (int64_t j = 0; j < dv; ++j) dP[c * dv + j] = Lam[c * dv + j] - b * kt[c] * r[j];
                for (int64_t c = 0; c < dk; ++c) {
                    double lv = 0.0, ly = 0.0, sr = 0.0, dl = 0.0;
                    for (int64_t j = 0; j < dv; ++j) {
                        lv += Lam[c * dv + j] * vt[j];
                        ly += Lam[c * dv + j] * y[j];
                        sr += Sp[c * dv + j] * r[j];
                        dl += dP[c * dv + j] * a[c] * Sp[c * dv + j];
                    }
                    J->dk_out[th * dk + c] = b * (lv - ly - a[c] * sr);
                    if (J->scalar_decay) dla_sum += dl;
                    else J->dla[th * dk + c] = dl;
                }
                for (int64_t c = 0; c < dk; ++c)
                    for (int64_t j = 0; j < dv; ++j) Lam[c * dv + j] = a[c] * dP[c * dv + j];
            }
            if (J->scalar_decay) J->dla[th] = dla_sum;
        }
    }
    if (J->dS0) memcpy(J->dS0 + state_off, Lam, sizeof(double) * SZ);
    free(ck); free(st); free(Lam); free(dP); free(a); free(y); free(g); free(r);
    return 0;
}

static void* worker_bwd(void* arg) {
    oracle_bwd_job* J = (oracle_bwd_job*)arg;
    const int64_t units = J->num_seqs * J->num_heads;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t u = J->next_unit++;
        pthread_mutex_unlock(&J->mu);
        if (u >= units) break;
        if (run_unit_bwd(J, u / J->num_heads, u % J->num_heads)) {
            pthread_mutex_lock(&J->mu);
            J->failed = 1;
            pthread_mutex_unlock(&J->mu);
        }
    }
    return NULL;
}

/*
 * Gradient of kda_oracle_fwd.  dO [T,H,dv] and dST [N,H,dk,dv] (NULL: zero) are the
 * loss's derivatives with respect to o and S_T.  Outputs: dq, dk [T,H,dk], dv
 * [T,H,dv], dla with the shape of log_a, dbeta [T,H], dS0 [N,H,dk,dv] (may be NULL).
 * Return codes as kda_oracle_fwd.
 */
int kda_oracle_bwd(int64_t num_seqs, const int64_t* cu_seqlens, int64_t num_heads,
                   int64_t dk, int64_t dv, const double* q, const double* k,
                   const double* v, const double* log_a, int scalar_decay,
                   const double* beta, const double* S0, int order, const double* dO,
                   const double* dST, double* dq, double* dk_out, double* dv_out,
                   double* dla, double* dbeta, double* dS0, int num_threads) {
    if (num_seqs < 0 || num_heads <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return 1;
    if (order != 0 && order != 1) return 1;
    if (cu_seqlens[0] != 0) return 1;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return 1;
    if (num_seqs == 0) return 0;
    if (cu_seqlens[num_seqs] > 0 &&
        (!q || !k || !v || !log_a || !beta || !dO || !dq || !dk_out || !dv_out || !dla || !dbeta))
        return 1;

    oracle_bwd_job J;
    memset(&J, 0, sizeof(J));
    J.num_seqs = num_seqs; J.num_heads = num_heads; J.dk = dk; J.dv = dv;
    J.cu = cu_seqlens; J.q = q; J.k = k; J.v = v; J.log_a = log_a; J.beta = beta;
    J.S0 = S0; J.dO = dO; J.dST = dST; J.scalar_decay = scalar_decay ? 1 : 0; J.order = order;
    J.dq = dq; J.dk_out = dk_out; J.dv_out = dv_out; J.dla = dla; J.dbeta = dbeta; J.dS0 = dS0;
    pthread_mutex_init(&J.mu, NULL);

    const int64_t units = num_seqs * num_heads;
    int nt = num_threads > 0 ? num_threads : 1;
    if (nt > units) nt = (int)units;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th) { pthread_mutex_destroy(&J.mu); return 2; }
    int started = 0;
    for (int i = 0; i < nt; ++i) {
        if (pthread_create(&th[i], NULL, worker_bwd, &J) != 0) break;
        ++started;
    }
    if (started == 0) worker_bwd(&J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return J.failed ? 2 : 0;
}
