/* Driver for the sanitizer build of the oracle (oracle/kda_oracle.c): runs the
 * forward and gradient token loops over ragged packed batches (empty, one-token
 * and multi-chunk sequences; both orders; scalar and per-channel decay; one and
 * several threads; with and without S0, dS_T) and the argument checks, so that
 * AddressSanitizer and UndefinedBehaviorSanitizer see every index the loops
 * compute.  Exit status 0 when every call returned what it should and every
 * output is finite.  Test infrastructure (CPU only). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kda_oracle_fwd(int64_t num_seqs, const int64_t* cu_seqlens, int64_t num_heads, int64_t dk, int64_t dv,
                   const double* q, const double* k, const double* v, const double* log_a, int scalar_decay,
                   const double* beta, const double* S0, int order, double* o, double* ST, int num_threads);
int kda_oracle_bwd(int64_t num_seqs, const int64_t* cu_seqlens, int64_t num_heads, int64_t dk, int64_t dv,
                   const double* q, const double* k, const double* v, const double* log_a, int scalar_decay,
                   const double* beta, const double* S0, int order, const double* dO, const double* dST,
                   double* dq, double* dk_out, double* dv_out, double* dla, double* dbeta, double* dS0,
                   int num_threads);

static double rnd(uint64_t* s) {
    *s = *s * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(*s >> 11) / 9007199254740992.0 - 0.5;
}

static double* filled(size_t n, uint64_t* s, double lo, double hi) {
    double* p = (double*)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * (rnd(s) + 0.5);
    return p;
}

static int all_finite(const double* p, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static int run_case(const int64_t* lens, int64_t N, int64_t H, int64_t dk, int64_t dv, int scalar, int order,
                    int with_state, int threads, uint64_t seed) {
    int64_t* cu = (int64_t*)malloc((N + 1) * sizeof(int64_t));
    cu[0] = 0;
    for (int64_t n = 0; n < N; ++n) cu[n + 1] = cu[n] + lens[n];
    const int64_t T = cu[N];
    uint64_t s = seed;
    double* q = filled(T * H * dk, &s, -1, 1);
    double* k = filled(T * H * dk, &s, -1, 1);
    double* v = filled(T * H * dv, &s, -1, 1);
    double* la = filled(T * H * (scalar ? 1 : dk), &s, -3, 0);
    double* beta = filled(T * H, &s, 0, 1);
    double* S0 = with_state ? filled(N * H * dk * dv, &s, -0.1, 0.1) : NULL;
    double* dO = filled(T * H * dv, &s, -1, 1);
    double* dST = with_state ? filled(N * H * dk * dv, &s, -1, 1) : NULL;
    double* o = filled(T * H * dv, &s, 0, 0);
    double* ST = filled(N * H * dk * dv, &s, 0, 0);
    double* dq = filled(T * H * dk, &s, 0, 0);
    double* dkk = filled(T * H * dk, &s, 0, 0);
    double* dvv = filled(T * H * dv, &s, 0, 0);
    double* dla = filled(T * H * (scalar ? 1 : dk), &s, 0, 0);
    double* db = filled(T * H, &s, 0, 0);
    double* dS0 = filled(N * H * dk * dv, &s, 0, 0);
    int bad = 0;
    if (kda_oracle_fwd(N, cu, H, dk, dv, q, k, v, la, scalar, beta, S0, order, o, ST, threads) != 0) bad = 1;
    if (kda_oracle_bwd(N, cu, H, dk, dv, q, k, v, la, scalar, beta, S0, order, dO, dST, dq, dkk, dvv, dla, db,
                       dS0, threads) != 0)
        bad = 1;
    if (!all_finite(o, T * H * dv) || !all_finite(ST, N * H * dk * dv) || !all_finite(dq, T * H * dk) ||
        !all_finite(dkk, T * H * dk) || !all_finite(dvv, T * H * dv) || !all_finite(dla, T * H * (scalar ? 1 : dk)) ||
        !all_finite(db, T * H) || !all_finite(dS0, N * H * dk * dv))
        bad = 1;
    free(cu); free(q); free(k); free(v); free(la); free(beta); free(S0); free(dO); free(dST);
    free(o); free(ST); free(dq); free(dkk); free(dvv); free(dla); free(db); free(dS0);
    return bad;
}

int main(void) {
    int bad = 0;
    const int64_t lens1[] = {37, 0, 96, 5, 1};
    const int64_t lens2[] = {70};
    const int64_t lens3[] = {0, 0};
    for (int order = 0; order < 2; ++order)
        for (int scalar = 0; scalar < 2; ++scalar) {
            bad |= run_case(lens1, 5, 2, 8, 4, scalar, order, 1, 3, 11 + order + 2 * scalar);
            bad |= run_case(lens2, 1, 1, 4, 8, scalar, order, 0, 1, 21 + order + 2 * scalar);
            bad |= run_case(lens3, 2, 3, 4, 4, scalar, order, 1, 2, 31 + order + 2 * scalar);
        }
    /* argument checks: each must refuse (return 1) without touching the buffers */
    const int64_t cu_bad[] = {0, 5, 3};
    const int64_t cu_off[] = {1, 5};
    const int64_t cu_ok[] = {0, 2};
    double x[64] = {0};
    if (kda_oracle_fwd(2, cu_bad, 1, 2, 2, x, x, x, x, 0, x, NULL, 0, x, x, 1) != 1) bad = 1;
    if (kda_oracle_fwd(1, cu_off, 1, 2, 2, x, x, x, x, 0, x, NULL, 0, x, x, 1) != 1) bad = 1;
    if (kda_oracle_fwd(1, cu_ok, 1, 2, 2, x, x, x, x, 0, x, NULL, 2, x, x, 1) != 1) bad = 1;
    if (kda_oracle_fwd(1, cu_ok, 0, 2, 2, x, x, x, x, 0, x, NULL, 0, x, x, 1) != 1) bad = 1;
    if (kda_oracle_fwd(1, NULL, 1, 2, 2, x, x, x, x, 0, x, NULL, 0, x, x, 1) != 1) bad = 1;
    if (kda_oracle_fwd(1, cu_ok, 1, 2, 2, NULL, x, x, x, 0, x, NULL, 0, x, x, 1) != 1) bad = 1;
    printf(bad ? "oracle sanitizer check FAILED\n" : "oracle sanitizer check ok\n");
    return bad;
}
