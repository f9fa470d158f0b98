// kda_bwd.hip -- gradient of the prefill (the erase-then-decay ordering of the
// table row "KDA" on page "The argument, in one page", and the decay-first one, in
// their chunkwise form, row "Chunkwise / WY" of the same table).
//
// For a loss with derivatives dO (outputs) and dS_T (final states), the call
// returns dq, dk, dv, dlog_a, dbeta and dS0.  Per (sequence, head) the tokens are
// cut into sub-chunks of 16.  With S the state at a sub-chunk start, X the
// derivative with respect to the state at its end, g the cumulative log-decay from
// the sub-chunk start (gm: exclusive, gC: at the end), b = beta:
//
//   Kb = k e^{gm}, Qb = q e^{g}, Kcc = k e^{gC-gm}, Ktc = k e^{gC-g}, gamma = e^{gC}
//   A0 = strict_lower(Kb (k e^{-gm})^T), L = strict_lower(Kb (k e^{-g})^T),
//   P1 = lower(Qb (k e^{-gm})^T), P2 = lower(Qb (k e^{-g})^T), T = (I + diag(b) A0)^-1
//   forward:  Y0 = Kb S + L bV, E = -T diag(b) Y0, Y = Y0 + A0 E,
//             S_next = gamma S + Kcc^T E + Ktc^T bV
//   backward: G = T^T (P1^T dO + Kcc X), F = -diag(b) G, R = Ktc X + P2^T dO + L^T F,
//             X_prev = gamma X + Qb^T dO + Kb^T F
//   dv = diag(b) R, dbeta = rowsum(R V) - rowsum(G Y),
//   dq   = e^{g} (dO S^T)      + e^{g-m}  [lower(dO E^T) Kc' + lower(dO bV^T) Kt']
//   gs   = e^{gm} (G S^T)      + e^{gm-m} [strict_lower(G E^T) Kc' + strict_lower(G bV^T) Kt']
//   vds  = e^{gC-g} (V X^T)    + e^{m-g}  [upper(V dO^T) Qb' + strict_upper(V F^T) Kb']
//   ayds = e^{gC-gm} (Y X^T)   + e^{m-gm} [upper(Y dO^T) Qb' + strict_upper(Y F^T) Kb']
//   dk = diag(b) (vds - ayds - gs),
//   dlog_a_i = phi_i - b_i k_i vds_i, phi_i = phi_{-1} + sum_{j<=i} (k dk + 2 b k gs)_j
//              - sum_{j<i} (q dq)_j, phi_{-1} = rowsum(X_prev * S)
// where the primed operands carry the decay relative to a per-channel reference
// m = gC / 2 (Kc' = k e^{m-gm}, Kt' = k e^{m-g}, Qb' = q e^{g-m}, Kb' = k e^{gm-m}),
// so every factor stays below e^{span/2}.  A sub-chunk whose span -gC exceeds 160
// nats in some channel takes one exponent per term instead.
//
// The decay-first ordering, S_i = (I - b_i k_i^T k_i) Diag(a_i) S_{i-1} + b_i k_i^T v_i,
// reads its token after the token's own decay and erases along the same key it
// writes: its chunk form is every line above with gm replaced by g (then A0 = L,
// P1 = P2, Kcc = Ktc), except the last step of dlog_a, which takes the step's own
// telescoping terms off phi instead of b k vds:
//   dlog_a_i = phi_i - (k dk + 2 b k gs)_i.
// The kernels read gm from the decay-sum row of the token itself (gmo = 1) instead
// of the row before it.
//
// Barriers inside the walks order LDS only (lds_barrier), so global loads fetched
// for the next step stay in flight across them; every global value a walk reads
// back is read by the lane that wrote it or reaches LDS through registers.
//
// Three kernels follow the forward prefill, which leaves the state at every 64th
// token: kda_bwd_ops (one wavefront per sub-chunk: the C x C products, the solve,
// the operators of the reverse walk), the reverse walk X <- X_prev keeping X at
// every 64-token boundary (one workgroup per (sequence, head, value slice):
// kda_bwd_walk for bf16, kda_bwd_scan for fp32) and kda_bwd_grad (one workgroup
// per 64-token chunk: its sub-chunks in reverse, each start state recomputed from
// the chunk's kept state, all products on matrix cores).
#include "kda_chunk_common.hpp"
#include "kda_launch.hpp"
#include "kda_ws.hpp"

namespace kda {
namespace {

constexpr int SC = 16;                   // sub-chunk tokens
constexpr int GW = 8;                    // wavefronts of a gradient-pass workgroup
constexpr int CHB = 64;                  // tokens between kept states
constexpr float SPAN2_MAX = 160.f * LOG2E;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float ex2n(float x) { return __builtin_amdgcn_exp2f(fminf(x, 0.f)); }

// ---------------------------------------------------------------- products
// A 16-deep contraction in bf16 runs as the 32-deep instruction with the upper
// half of k zero (lanes 32..63 supply zeros), so that every accumulation chain
// uses a single instruction type.
__device__ __forceinline__ f32x4 mma16(const bf16* ra, const bf16* rb, f32x4 acc, int lane) {
    bf16x8 a = {}, b = {};
    if (lane < 32) {
        a = *reinterpret_cast<const bf16x8*>(ra + 8 * (lane >> 4));
        b = *reinterpret_cast<const bf16x8*>(rb + 8 * (lane >> 4));
    }
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const float* ra, const float* rb, f32x4 acc, int lane) {
    return tile_mma_r<float, 16>(ra, rb, acc, lane);
}

// acc += A[16 x KD] B[KD x 16]; ra / rb: this lane's A row and B column, both
// k-contiguous in LDS (row (lane % 16) of A stored [m][k], of B stored [n][k]).
template <typename MT, int KD>
__device__ __forceinline__ f32x4 mmak(const MT* ra, const MT* rb, f32x4 acc, int lane) {
    if constexpr (sizeof(MT) == 2) {
        constexpr int N32 = KD / 32;
        static_assert(KD % 16 == 0, "contraction must be a multiple of 16");
        if constexpr (N32 > 0) acc = tile_mma_r<bf16, N32 * 32>(ra, rb, acc, lane);
        if constexpr (KD % 32 == 16) acc = mma16(ra + N32 * 32, rb + N32 * 32, acc, lane);
        return acc;
    } else {
        return tile_mma_r<float, KD>(ra, rb, acc, lane);
    }
}

// An accumulator tile holds D[m][n] with m = 4 (lane / 16) + r, n = lane % 16.
// store_nat writes it to Z[n][m] (four consecutive m per lane), store_rm to Z[m][n].
template <typename MT>
__device__ __forceinline__ void store_nat(MT* z, int ld, f32x4 d, int lane) {
    store4<MT>(z + (lane & 15) * ld + 4 * (lane >> 4), d);
}
template <typename MT>
__device__ __forceinline__ void store_rm(MT* z, int ld, f32x4 d, int lane) {
#pragma unroll
    for (int r = 0; r < 4; ++r) z[(4 * (lane >> 4) + r) * ld + (lane & 15)] = from_f32<MT>(d[r]);
}

// fp32 state tile <-> row-major global [rows][ld] (inverse of store_state_tile).
__device__ __forceinline__ f32x4 load_state_tile(const float* src, int64_t ld, int lane) {
    const int row = 4 * (lane >> 4) + (lane & 3), col = 4 * ((lane & 15) >> 2);
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + (int64_t)row * ld + col);
    return __builtin_bit_cast(f32x4, quad_transpose(__builtin_bit_cast(i32x4, v), lane));
}

// 16 bytes of MT as one vector of MT (keeps every access in the element type).
template <typename MT> struct V16;
template <> struct V16<bf16> { typedef bf16x8 type; };
template <> struct V16<float> { typedef f32x4 type; };
template <typename MT>
__device__ __forceinline__ void copy16(MT* dst, const MT* src) {
    *reinterpret_cast<typename V16<MT>::type*>(dst) = *reinterpret_cast<const typename V16<MT>::type*>(src);
}
// eight values rounded to MT, stored at dst (16 bytes for bf16, 32 for fp32)
template <typename MT>
__device__ __forceinline__ void store8(MT* dst, const float* x) {
    if constexpr (sizeof(MT) == 2) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
        *reinterpret_cast<bf16x8*>(dst) = v;
    } else {
        reinterpret_cast<f32x4*>(dst)[0] = f32x4{x[0], x[1], x[2], x[3]};
        reinterpret_cast<f32x4*>(dst)[1] = f32x4{x[4], x[5], x[6], x[7]};
    }
}

template <bool B> struct BoolC { static constexpr bool value = B; };

// ------------------------------------------------------------ sequences
struct SeqSpan {
    int64_t t0;
    int len;
};
__device__ __forceinline__ SeqSpan seq_span(const int32_t* cu, int64_t eq_len, int n) {
    if (!cu) return SeqSpan{(int64_t)n * eq_len, (int)eq_len};
    return SeqSpan{(int64_t)cu[n], cu[n + 1] - cu[n]};
}
__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
// sum over sequences m < n of ceil(len_m / div) (wavefront-wide; every lane gets it)
__device__ __forceinline__ int64_t ceil_blocks_before(const int32_t* cu, int64_t eq_len, int n, int div) {
    if (!cu) return (int64_t)n * ((eq_len + div - 1) / div);
    int64_t s = 0;
    for (int m = (int)(threadIdx.x & 63); m < n; m += 64) s += (cu[m + 1] - cu[m] + div - 1) / div;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    return s;
}

// ------------------------------------------------------- operator block
// Per (sequence, head, sub-chunk), written by kda_bwd_ops:
//   W    [16][DK]   diag(b) T^T Kcc                (reverse walk: F = -(W X + M dO))
//   M    [16][16]   diag(b) T^T P1^T
//   QK   [DK][32]   [Qb^T | Kb^T]                  (X_prev = gamma X + QK [dO; F])
//   gam  [DK]       e^{gC} (fp32)
//   mats 7 x [16][16]: T diag(b), T^T, L, L^T, A0, P1^T, P2^T (row-major)
//   flag int32: 1 if the sub-chunk needs one exponent per term
// In bf16 blocks the walk's part (W, M, QK, gam) is stored as the LDS image
// that kda_bwd_walk reads after a verbatim copy (WL below):
//   W  rows of DK channels in kperm order (kda_ws.hpp), 16-byte pieces
//      XOR-swizzled by the row (swz), so that X's accumulator tiles are its
//      B operand and 16 lanes reading one piece of 16 rows meet no conflict;
//   M  piece-major: columns 8q..8q+7 of row t at byte 16 (16 q + t);
//   QK piece-major (piece g of channel row c at byte 16 (g DK + c)) with its
//      32 columns interleaved: piece g holds Qb^T columns 4g..4g+3, then Kb^T
//      columns 4g..4g+3, matching the operand [dO; F] that a lane group g
//      holds as dO rows 4g..4g+3 and F's accumulator rows 4g..4g+3.
// fp32 blocks keep the plain row-major matrices (kda_bwd_scan).
template <typename MT, int DK>
struct OpBlock {
    static constexpr int S = (int)sizeof(MT);
    static constexpr int W = 0;
    static constexpr int M = W + 16 * DK * S;
    static constexpr int QK = M + 256 * S;
    static constexpr int GAM = QK + 32 * DK * S;
    static constexpr int MATS = GAM + 4 * DK;
    static constexpr int FLAG = MATS + 7 * 256 * S;
    static constexpr int BYTES = FLAG + 16;
    static constexpr int WALK = MATS;  // bytes the reverse walk reads
    static_assert(BYTES % 16 == 0 && WALK % 16 == 0, "16-byte pieces");
};
enum { MAT_TB = 0, MAT_TT, MAT_L, MAT_LT, MAT_A0, MAT_P1T, MAT_P2T };

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const float* log_a;
    const float* beta;
    const float* S0;
    const int32_t* cu;
    int64_t eq_len;
    const void* dO;
    const float* dST;
    void* dq;
    void* dk;
    void* dv;
    float* dla;
    float* dbeta;
    float* dS0;
    const float* snap;       // forward states, row per 64 tokens of each sequence
    int64_t snap_rows;       // rows snap holds (reads stay below it)
    uint8_t* ops;            // operator blocks
    float* xbuf;             // state derivatives at 64-token chunk ends
    void* scr;               // per chunk: start state, E and Y of its sub-chunks
    int32_t H;
    int32_t scalar;
    int32_t split;
    int32_t gmo;             // 1: decay-first order, whose operators take g where erase-first takes gm
};

// A sub-chunk's inputs for one wavefront, in two halves: fetch issues every load
// (into registers, at addresses that are always valid: rows past the sub-chunk
// repeat its first row), place writes them to LDS (those rows as zeros).  All
// loads are in flight before the first is waited for.
template <typename MT, int D>
struct RowFetch {  // 16 rows of a [T, H, D] tensor, for LDS z[16][ld]
    static constexpr int PER = 16 / (int)sizeof(MT), PR = D / PER, NPT = (16 * PR + 63) / 64;
    typedef typename V16<MT>::type VT;
    VT x[NPT];
    __device__ __forceinline__ void fetch(const MT* g, int64_t t0, int H, int h, int nrow, int lane) {
#pragma unroll
        for (int a = 0; a < NPT; ++a) {
            const int pc = min(lane + 64 * a, 16 * PR - 1), i = pc / PR, e = (pc % PR) * PER;
            x[a] = *reinterpret_cast<const VT*>(g + ((t0 + (i < nrow ? i : 0)) * H + h) * (int64_t)D + e);
        }
    }
    __device__ __forceinline__ void place(MT* z, int ld, int nrow, int lane) const {
#pragma unroll
        for (int a = 0; a < NPT; ++a) {
            const int pc = lane + 64 * a, i = pc / PR, e = (pc % PR) * PER;
            if (pc < 16 * PR) *reinterpret_cast<VT*>(z + i * ld + e) = i < nrow ? x[a] : VT{};
        }
    }
};
// The decays (log a, per channel or one per token) and beta of a sub-chunk: place
// writes log2 e * log a into rows 1..16 of G2 (rows G2L apart) and beta into bt;
// prefix (after a barrier) turns the rows into running sums, G2[i][c] =
// log2 e * sum_{j < i} log a_j for i = 0..16.
template <int DK, int G2L>
struct DecayFetch {
    static constexpr int Q = DK / 4, NPT = (16 * Q + 63) / 64;  // 16-byte pieces
    f32x4 x[NPT];
    float b, as;
    __device__ __forceinline__ void fetch(const float* la, const float* beta, int64_t t0, int H, int h, int nrow,
                                          int scalar, int lane) {
        const int64_t rb = (t0 + min(lane & (SC - 1), nrow - 1)) * H + h;
        b = beta[rb];
        as = la[scalar ? rb : rb * DK];
        if (!scalar) {
#pragma unroll
            for (int a = 0; a < NPT; ++a) {
                const int pc = min(lane + 64 * a, 16 * Q - 1), i = pc / Q, c4 = (pc % Q) * 4;
                x[a] = *reinterpret_cast<const f32x4*>(la + ((t0 + (i < nrow ? i : 0)) * H + h) * (int64_t)DK + c4);
            }
        }
    }
    __device__ __forceinline__ void place(float* G2, float* bt, int nrow, int scalar, int lane) const {
#pragma unroll
        for (int a = 0; a < NPT; ++a) {
            const int pc = lane + 64 * a, i = pc / Q, c4 = (pc % Q) * 4;
            if (pc < 16 * Q) {
                const float s1 = __shfl(as, i);  // the token's decay, scalar gate
                const f32x4 v = scalar ? f32x4{s1, s1, s1, s1} : x[a];
                *reinterpret_cast<f32x4*>(G2 + (i + 1) * G2L + c4) = i < nrow ? v * LOG2E : zero4();
            }
        }
        if (lane < SC) bt[lane] = lane < nrow ? b : 0.f;
    }
    __device__ __forceinline__ static void prefix(float* G2, int lane) {
        for (int c = lane; c < DK; c += 64) {
            float s = 0.f;
            G2[c] = 0.f;
#pragma unroll
            for (int i = 1; i <= SC; ++i) {
                s += G2[i * G2L + c];
                G2[i * G2L + c] = s;
            }
        }
    }
};

// ===================================================================== ops
// One wavefront per (sequence, head, sub-chunk).  LDS is reused as the sub-chunk's
// inputs die (19 KB at dk = 128, so that eight wavefronts share a compute unit):
// q's rows give way to Kcc^T once the Gram products are in registers, and k's
// rows and the decays to the masked products and T once Kcc^T is formed.
template <typename MT, int DK>
__global__ __launch_bounds__(64) void kda_bwd_ops_kernel(BwdParams p) {
    const int gmo = p.gmo;
    typedef OpBlock<MT, DK> OB;
    constexpr bool WL = sizeof(MT) == 2;                      // the walk's operands in its LDS layout
    constexpr int P = 16 / (int)sizeof(MT);
    constexpr int LDK = DK + P, L16 = 16 + P;
    constexpr int ROWB = 16 * LDK * (int)sizeof(MT);          // bytes of 16 padded rows
    constexpr int G2L = DK + 4;                               // decay-sum row stride (no bank conflicts)
    constexpr int G2B = (SC + 1) * G2L * 4;                   // bytes of the decay sums
    static_assert(DK * 16 * (int)sizeof(MT) <= ROWB, "Kcc^T fits in q's rows");
    constexpr int GTB = (4 * 16 * 17 + 16 * 17) * 4;          // bytes of the products and T
    constexpr int UKB = ROWB + G2B > GTB ? ROWB + G2B : GTB;
    __shared__ __attribute__((aligned(16))) uint8_t u_k[UKB];          // kr | G2, later Gf | Tf
    __shared__ __attribute__((aligned(16))) uint8_t u_q[ROWB];         // qr, later KCT
    __shared__ __attribute__((aligned(16))) MT P1rm[16 * L16];
    __shared__ __attribute__((aligned(16))) MT bTT[16 * L16];
    __shared__ float bt[SC];
    MT* kr = reinterpret_cast<MT*>(u_k);
    float* G2 = reinterpret_cast<float*>(u_k + ROWB);
    MT* qr = reinterpret_cast<MT*>(u_q);
    MT* KCT = reinterpret_cast<MT*>(u_q);                             // [DK][16], unpadded
    float (*Gf)[16][17] = reinterpret_cast<float (*)[16][17]>(u_k);  // A0, L, P1, P2 (fp32, masked)
    float (*Tf)[17] = reinterpret_cast<float (*)[17]>(u_k + 4 * 16 * 17 * 4);

    const int lane = threadIdx.x;
    const int s = blockIdx.x;
    const int64_t unit = blockIdx.y;
    const int n = (int)(unit / p.H), h = (int)(unit % p.H);
    const SeqSpan sq = seq_span(p.cu, p.eq_len, n);
    if (s * SC >= sq.len) return;
    const int nrow = min(SC, sq.len - s * SC);
    const int nsub = ceil_div(sq.len, SC);
    const int64_t t0 = sq.t0 + (int64_t)s * SC;

    uint8_t* blk;
    {
        RowFetch<MT, DK> fk, fq;
        DecayFetch<DK, G2L> fd;
        fk.fetch(static_cast<const MT*>(p.k), t0, p.H, h, nrow, lane);
        fq.fetch(static_cast<const MT*>(p.q), t0, p.H, h, nrow, lane);
        fd.fetch(p.log_a, p.beta, t0, p.H, h, nrow, p.scalar, lane);
        // the block's index (which reads the sequence lengths) while the inputs load
        const int64_t bi = ceil_blocks_before(p.cu, p.eq_len, n, SC) * p.H + (int64_t)h * nsub + s;
        blk = p.ops + bi * OB::BYTES;
        fk.place(kr, LDK, nrow, lane);
        fq.place(qr, LDK, nrow, lane);
        fd.place(G2, bt, nrow, p.scalar, lane);
        __syncthreads();
        DecayFetch<DK, G2L>::prefix(G2, lane);
    }
    __syncthreads();

    // QK [c][32] = [q_s e^{g_s} | k_s e^{gm_s}], gamma
    {
        MT* qk = reinterpret_cast<MT*>(blk + OB::QK);
        for (int pc = lane; pc < DK * 4; pc += 64) {
            const int c = pc >> 2, g = pc & 3, s0 = 8 * g;
            float out[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // WL: piece g holds the q terms of tokens 4g..4g+3, then their k terms
                const bool qt = WL ? e < 4 : s0 + e < 16;
                const int s2 = WL ? 4 * g + (e & 3) : (s0 + e) & 15;
                out[e] = qt ? to_f32(qr[s2 * LDK + c]) * ex2(G2[(s2 + 1) * G2L + c])
                            : to_f32(kr[s2 * LDK + c]) * ex2(G2[(s2 + gmo) * G2L + c]);
            }
            store8<MT>(qk + (WL ? 8 * (g * DK + c) : c * 32 + s0), out);
        }
        float* gam = reinterpret_cast<float*>(blk + OB::GAM);
        for (int c = lane; c < DK; c += 64) gam[c] = ex2(G2[SC * G2L + c]);
    }

    float span = 0.f;
    for (int c = lane; c < DK; c += 64) span = fmaxf(span, -G2[SC * G2L + c]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) span = fmaxf(span, __shfl_xor(span, off));
    const bool exact = span > SPAN2_MAX;
    if (lane == 0) *reinterpret_cast<int*>(blk + OB::FLAG) = exact ? 1 : 0;

    // C x C products, kept in registers until k's rows and the decays are dead:
    // factored, acc[g][r] is element (t = 4 (lane / 16) + r, i = lane % 16);
    // exact, ex[g][j] is element (t, i) = ((lane + 64 j) / 16, (lane + 64 j) % 16)
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
    float ex[4][4];
    if (!exact) {
        // (m = t, n = i); A rows: k (A0, L) or q (P1, P2) times e^{h_t - m}; B rows: k times e^{m - h_i}
        const int r16 = lane & 15;
        constexpr int KPL = Mma<MT>::KPL, KS = Mma<MT>::K;
#pragma unroll
        for (int kb = 0; kb < DK; kb += KS) {
            typename Mma<MT>::frag ak, aq, bm, bg;
            float fk[KPL], fq[KPL], fm[KPL], fg[KPL];
            const int c0 = kb + (lane >> 4) * KPL;
#pragma unroll
            for (int e = 0; e < KPL; ++e) {
                const int c = c0 + e;
                const float m2 = 0.5f * G2[SC * G2L + c];
                fk[e] = ex2(G2[(r16 + gmo) * G2L + c] - m2);  // e^{gm_t - m}
                fq[e] = ex2(G2[(r16 + 1) * G2L + c] - m2);    // e^{g_t - m}
                fm[e] = ex2(m2 - G2[(r16 + gmo) * G2L + c]);  // e^{m - gm_i}
                fg[e] = ex2(m2 - G2[(r16 + 1) * G2L + c]);    // e^{m - g_i}
            }
            const typename Mma<MT>::frag kx = Mma<MT>::loadr(kr + r16 * LDK + kb, lane);
            const typename Mma<MT>::frag qx = Mma<MT>::loadr(qr + r16 * LDK + kb, lane);
            ak = Mma<MT>::scale(kx, fk);
            aq = Mma<MT>::scale(qx, fq);
            bm = Mma<MT>::scale(kx, fm);
            bg = Mma<MT>::scale(kx, fg);
            acc[0] = Mma<MT>::mma(ak, bm, acc[0]);  // A0
            acc[1] = Mma<MT>::mma(ak, bg, acc[1]);  // L
            acc[2] = Mma<MT>::mma(aq, bm, acc[2]);  // P1
            acc[3] = Mma<MT>::mma(aq, bg, acc[3]);  // P2
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pi = lane + 64 * j, t = pi >> 4, i = pi & 15;
            float a0 = 0.f, l = 0.f, p1 = 0.f, p2 = 0.f;
            if (i <= t) {
                for (int c = 0; c < DK; ++c) {
                    const float kt = to_f32(kr[t * LDK + c]), qt = to_f32(qr[t * LDK + c]), ki = to_f32(kr[i * LDK + c]);
                    const float gmt = G2[(t + gmo) * G2L + c], gt = G2[(t + 1) * G2L + c];
                    const float gmi = G2[(i + gmo) * G2L + c], gi = G2[(i + 1) * G2L + c];
                    if (i < t) {
                        a0 += kt * ki * ex2(gmt - gmi);
                        l += kt * ki * ex2(gmt - gi);
                    }
                    p1 += qt * ki * ex2(gt - gmi);
                    p2 += qt * ki * ex2(gt - gi);
                }
            }
            ex[0][j] = a0; ex[1][j] = l; ex[2][j] = p1; ex[3][j] = p2;
        }
    }
    __syncthreads();  // q's rows are dead

    // Kcc^T [c][s] = k_s e^{gC - gm_s}
    for (int x = lane; x < DK * 16; x += 64) {
        const int c = x >> 4, s2 = x & 15;
        KCT[c * 16 + s2] = from_f32<MT>(to_f32(kr[s2 * LDK + c]) * ex2(G2[SC * G2L + c] - G2[(s2 + gmo) * G2L + c]));
    }
    __syncthreads();  // k's rows and the decays are dead

    if (!exact) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * (lane >> 4) + r, i = lane & 15;
                const bool keep = g < 2 ? i < t : i <= t;
                Gf[g][t][i] = keep ? acc[g][r] : 0.f;
            }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pi = lane + 64 * j, t = pi >> 4, i = pi & 15;
#pragma unroll
            for (int g = 0; g < 4; ++g) Gf[g][t][i] = ex[g][j];
        }
    }
    __syncthreads();

    // T = (I + diag(b) A0)^-1, one column per lane
    if (lane < 16) {
        const int j = lane;
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float a = i == j ? 1.f : 0.f;
            if (i > j) {
                float sdot = 0.f;
#pragma unroll
                for (int kk = 0; kk < i; ++kk) sdot += Gf[0][i][kk] * t[kk];  // t[kk] = 0 for kk < j
                a = -bt[i] * sdot;
            }
            t[i] = a;
        }
        const float bj = bt[j];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            Tf[i][j] = t[i];
            bTT[j * L16 + i] = from_f32<MT>(bj * t[i]);  // (diag(b) T^T)[j][i] = b_j T[i][j]
        }
    }
    for (int x = lane; x < 256; x += 64) P1rm[(x >> 4) * L16 + (x & 15)] = from_f32<MT>(Gf[2][x >> 4][x & 15]);
    __syncthreads();

    // the seven 16 x 16 matrices of the gradient pass, 8 elements per piece: one
    // matrix at a time (lanes 0..31), so that which matrix is the same across the
    // wavefront
    MT* mats = reinterpret_cast<MT*>(blk + OB::MATS);
    if (lane < 32) {
        const int row = lane >> 1, c0 = (lane & 1) * 8;
#pragma unroll
        for (int mi = 0; mi < 7; ++mi) {
            float out[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int col = c0 + e;
                out[e] = mi == MAT_TB ? Tf[row][col] * bt[col]
                       : mi == MAT_TT ? Tf[col][row]
                       : mi == MAT_L ? Gf[1][row][col]
                       : mi == MAT_LT ? Gf[1][col][row]
                       : mi == MAT_A0 ? Gf[0][row][col]
                       : mi == MAT_P1T ? Gf[2][col][row]
                                       : Gf[3][col][row];
            }
            store8<MT>(mats + mi * 256 + row * 16 + c0, out);
        }
    }

    // W (m = c, n = t): W^T[c][t] = sum_s Kcc^T[c][s] (b_t T[s][t]); natural store gives W[t][c]
    // (WL: lane row t = lane % 16, channels 16 cb + 4 g + r at positions
    // kperm(...) = 32 (cb / 2) + 8 g + 4 (cb % 2) + r, four consecutive ones)
    MT* Wg = reinterpret_cast<MT*>(blk + OB::W);
    for (int cb = 0; cb < DK / 16; ++cb) {
        f32x4 a = mma16(KCT + (cb * 16 + (lane & 15)) * 16, bTT + (lane & 15) * L16, zero4(), lane);
        if constexpr (WL) {
            const int p0 = 32 * (cb >> 1) + 8 * (lane >> 4) + 4 * (cb & 1);
            store4<MT>(reinterpret_cast<MT*>(blk + OB::W + swz_elem<2 * DK>(lane & 15, p0)), a);
        } else {
            store_nat<MT>(Wg + cb * 16, DK, a, lane);
        }
    }
    // M (m = i, n = t): M^T[i][t] = sum_s P1[i][s] (b_t T[s][t]); natural store gives M[t][i]
    // (WL: M[t][4g .. 4g+3] is half g % 2 of piece g / 2 of row t)
    {
        f32x4 a = mma16(P1rm + (lane & 15) * L16, bTT + (lane & 15) * L16, zero4(), lane);
        if constexpr (WL) {
            const int g = lane >> 4;
            store4<MT>(reinterpret_cast<MT*>(blk + OB::M + 16 * (16 * (g >> 1) + (lane & 15)) + 8 * (g & 1)), a);
        } else {
            store_nat<MT>(reinterpret_cast<MT*>(blk + OB::M), 16, a, lane);
        }
    }
}

// ==================================================================== scan
// Reverse walk of the state derivative for one (sequence, head, value slice).
template <typename MT, int DK, int DVS>
__global__ __launch_bounds__(256) void kda_bwd_scan_kernel(BwdParams p, int DV, int nitems) {
    typedef OpBlock<MT, DK> OB;
    constexpr int P = 16 / (int)sizeof(MT);
    constexpr int LDK = DK + P, L16 = 16 + P, L32 = 32 + P;
    constexpr int PER = 16 / (int)sizeof(MT);
    constexpr int NCB = DK / 16, NJB = DVS / 16, CBW = (NCB + 3) / 4;
    constexpr int WALKP = OB::WALK / 16;          // 16-byte pieces of the walk's operators
    constexpr int DOP = 16 * DVS / PER;           // 16-byte pieces of the dO slice
    constexpr int NB = (WALKP + 255) / 256;        // block pieces per thread
    constexpr int NP = NB + 1;                     // and one dO piece
    static_assert(DOP <= 256 && (DOP & (DOP - 1)) == 0, "dO pieces");
    __shared__ __attribute__((aligned(16))) MT Wl[2][16 * LDK];
    __shared__ __attribute__((aligned(16))) MT Ml[2][16 * L16];
    __shared__ __attribute__((aligned(16))) MT QKl[2][DK * L32];
    __shared__ __attribute__((aligned(16))) float gl[2][DK];
    __shared__ __attribute__((aligned(16))) MT DFT[2][DVS * L32];  // [j][dO^T (16) | F^T (16)]
    __shared__ __attribute__((aligned(16))) MT XT[DVS * LDK];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // Workgroups are dealt to the 8 XCDs round-robin; item = (bid % 8) * per + bid / 8
    // puts consecutive items, the value slices of one (sequence, head), on one XCD,
    // so its operator blocks come from HBM once and from that XCD's L2 after.
    const int per = (nitems + 7) / 8;
    const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (item >= nitems) return;
    const int nsl = DV / DVS;
    const int64_t unit = item / nsl;
    const int slice = item % nsl;
    const int n = (int)(unit / p.H), h = (int)(unit % p.H);
    const SeqSpan sq = seq_span(p.cu, p.eq_len, n);
    const int nsub = ceil_div(sq.len, SC), nch = ceil_div(sq.len, CHB);
    const int j0 = slice * DVS;
    const int64_t sbase = ceil_blocks_before(p.cu, p.eq_len, n, SC) * p.H + (int64_t)h * nsub;
    const int64_t cbase = ceil_blocks_before(p.cu, p.eq_len, n, CHB) * p.H + (int64_t)h * nch;
    const int64_t st_off = unit * (int64_t)DK * DV + j0;  // this slice of [N, H, DK, DV]

    f32x4 X[CBW][NJB];
#pragma unroll
    for (int a = 0; a < CBW; ++a)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            const int cb = w + 4 * a;
            X[a][jb] = zero4();
            if (cb < NCB && p.dST) X[a][jb] = load_state_tile(p.dST + st_off + (int64_t)cb * 16 * DV + jb * 16, DV, lane);
        }

    const MT* dO = static_cast<const MT*>(p.dO);
    typedef typename V16<MT>::type VT;
    // Operators and dO rows are fetched two steps ahead into one of two register
    // sets (the loop is unrolled by two so that each set is a fixed set of
    // registers) and placed in one of two LDS buffers one step ahead.
    VT pre[2][NP];
    // Every thread issues the same NP loads, at addresses that are always valid
    // (block pieces past the end repeat earlier ones, dO rows past the sub-chunk
    // repeat its first row) and without branches, so the loads stay in program
    // order and a later use waits only for its own set, not for the set issued
    // after it.  place() skips the repeats and zeroes the rows past the end.
    const int dp = tid & (DOP - 1), di = dp / (DVS / PER), de = (dp % (DVS / PER)) * PER;
    auto fetch = [&](int s, VT (&dst)[NP]) {
        const uint8_t* blk = p.ops + (sbase + s) * OB::BYTES;
        const int64_t t0 = sq.t0 + (int64_t)s * SC;
        const int nrow = min(SC, sq.len - s * SC);
#pragma unroll
        for (int a = 0; a < NB; ++a) {
            const int pc = tid + 256 * a, pcc = pc >= WALKP ? pc - WALKP : pc;
            dst[a] = *reinterpret_cast<const VT*>(blk + 16 * pcc);
        }
        const int row = di < nrow ? di : 0;
        dst[NB] = *reinterpret_cast<const VT*>(dO + ((t0 + row) * p.H + h) * (int64_t)DV + j0 + de);
    };
    // places sub-chunk s's fetched pieces in LDS buffer b
    auto place = [&](int b, const VT (&src)[NP], int s) {
#pragma unroll
        for (int a = 0; a < NB; ++a) {
            const int pc = tid + 256 * a;
            const int off = 16 * pc;
            if (pc >= WALKP) continue;
            if (off < OB::M) {
                const int row = off / (DK * (int)sizeof(MT)), col = (off % (DK * (int)sizeof(MT))) / (int)sizeof(MT);
                *reinterpret_cast<VT*>(&Wl[b][row * LDK + col]) = src[a];
            } else if (off < OB::QK) {
                const int o = (off - OB::M) / (int)sizeof(MT), row = o / 16, col = o % 16;
                *reinterpret_cast<VT*>(&Ml[b][row * L16 + col]) = src[a];
            } else if (off < OB::GAM) {
                const int o = (off - OB::QK) / (int)sizeof(MT), row = o / 32, col = o % 32;
                *reinterpret_cast<VT*>(&QKl[b][row * L32 + col]) = src[a];
            } else {
                // gamma is fp32 in the block whatever MT is
                *reinterpret_cast<f32x4*>(&gl[b][(off - OB::GAM) / 4]) = __builtin_bit_cast(f32x4, src[a]);
            }
        }
        if (tid < DOP) {
            const int nrow = min(SC, sq.len - s * SC);
            const VT x = di < nrow ? src[NB] : VT{};
#pragma unroll
            for (int u = 0; u < PER; ++u) DFT[b][(de + u) * L32 + di] = x[u];
        }
    };
    // One step of the walk, sub-chunk s: on entry LDS buffer s & 1 holds its
    // operators and register set cur holds those of s - 1 (fetched two steps ago).
    auto step = [&](int s, VT (&cur)[NP], VT (&nxt)[NP]) {
        const int b = s & 1;
        // derivative at the end of a 64-token chunk
        if (s % (CHB / SC) == CHB / SC - 1 || s == nsub - 1) {
            float* dst = p.xbuf + (cbase + s / (CHB / SC)) * (int64_t)DK * DV + j0;
#pragma unroll
            for (int a = 0; a < CBW; ++a)
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {
                    const int cb = w + 4 * a;
                    if (cb < NCB) store_state_tile(dst + (int64_t)cb * 16 * DV + jb * 16, DV, lane, X[a][jb]);
                }
        }
#pragma unroll
        for (int a = 0; a < CBW; ++a)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int cb = w + 4 * a;
                if (cb < NCB) store_nat<MT>(XT + jb * 16 * LDK + cb * 16, LDK, X[a][jb], lane);
            }
        if (s > 1) fetch(s - 2, nxt);
        lds_barrier();
        // F = -(W X + M dO)   (m = t, n = j)
        for (int jb = w; jb < NJB; jb += 4) {
            f32x4 acc = mmak<MT, DK>(&Wl[b][(lane & 15) * LDK], XT + (jb * 16 + (lane & 15)) * LDK, zero4(), lane);
            acc = mmak<MT, 16>(&Ml[b][(lane & 15) * L16], &DFT[b][(jb * 16 + (lane & 15)) * L32], acc, lane);
            store_nat<MT>(&DFT[b][jb * 16 * L32 + 16], L32, -acc, lane);
        }
        lds_barrier();
        // X <- gamma X + [Qb^T | Kb^T] [dO; F]   (m = c, n = j)
#pragma unroll
        for (int a = 0; a < CBW; ++a) {
            const int cb = w + 4 * a;
            if (cb < NCB) {
                f32x4 gmm;
#pragma unroll
                for (int r = 0; r < 4; ++r) gmm[r] = gl[b][cb * 16 + 4 * (lane >> 4) + r];
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
                    X[a][jb] = mmak<MT, 32>(&QKl[b][(cb * 16 + (lane & 15)) * L32],
                                            &DFT[b][(jb * 16 + (lane & 15)) * L32], gmm * X[a][jb], lane);
            }
        }
        if (s > 0) place((s - 1) & 1, cur, s - 1);
    };

    if (nsub > 0) {
        fetch(nsub - 1, pre[0]);
        place((nsub - 1) & 1, pre[0], nsub - 1);
    }
    if (nsub > 1) fetch(nsub - 2, pre[0]);
    // step s uses set (nsub - 1 - s) & 1 for s - 1 and fills the other with s - 2
    for (int s = nsub - 1; s >= 0; s -= 2) {
        step(s, pre[0], pre[1]);
        if (s >= 1) step(s - 1, pre[1], pre[0]);
    }
    if (p.dS0) {
#pragma unroll
        for (int a = 0; a < CBW; ++a)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int cb = w + 4 * a;
                if (cb < NCB) store_state_tile(p.dS0 + st_off + (int64_t)cb * 16 * DV + jb * 16, DV, lane, X[a][jb]);
            }
    }
}

// ==================================================================== walk
// The reverse walk for bf16 blocks, built like the prefill's state pass.  Each
// compute wavefront owns one 16-column block of X for all DK channel rows, in
// matrix-core accumulators for the whole walk, and needs no other wavefront's
// data: X's accumulator tiles become the B operand of W X by a register move
// (W's channels are stored in kperm order), and F's accumulator tile with the
// step's dO rows becomes the B operand of the update (QK's columns are
// interleaved to match).  Per step, with slot B holding the step's operators:
//   F = -(M dO + W X)       (M dO as a 32-deep product whose upper half is zero)
//   X <- Diag(gamma) X + QK [dO; F]
// Two copy wavefronts bring each step's operators (the walk's part of the
// block, stored by kda_bwd_ops as the LDS image read here) and dO rows into
// one of NBUF LDS slots with the LDS-DMA form of the global load, AHEAD steps
// ahead, and touch the block TOUCH steps further into L2 (the value slices of
// a head share it there).  One barrier per step, between F and the update,
// hands the slots over: after it the next step's operands are read while the
// update runs.  The dO rows of a slot sit in the order 4 (t % 4) + t / 4, so
// that the four rows 4g..4g+3 a lane group reads fall on distinct banks; rows
// past a sub-chunk's end repeat its last row (they meet zero operator rows and
// columns).  X at each 64-token chunk end is written by the compute
// wavefronts into an LDS staging buffer and stored by the copy wavefronts
// after the step's barrier, so that the compute wavefronts issue no global
// memory operation in the walk.
template <int DK>
struct WalkCfg {
    typedef OpBlock<bf16, DK> OB;
    static constexpr int DVS = 32, NW = DVS / 16, NL = 2;  // compute and copy wavefronts
    static constexpr int NT = 64 * (NW + NL), LT = 64 * NL;
    static constexpr int NPB = OB::WALK / 16;            // 16-byte pieces of the operators
    static constexpr int NPV = 16 * DVS * 2 / 16;        // and of the dO rows
    static constexpr int NPS = NPB + NPV;
    static constexpr int ROUNDS = (NPS + LT - 1) / LT;   // copy instructions per copy wavefront and step
    static constexpr int TOFF = ROUNDS * LT * 16;        // where the touches land (never read)
    static constexpr int SLOT = TOFF + 256 * NL;
    static constexpr int NBUF = 6, AHEAD = NBUF - 1, TOUCH = 2;
    // X at a 64-token chunk end: two staging buffers of DK rows x DVS fp32
    // (rows XP floats apart, so that the quad-transposed writes of 16 lanes
    // meet no conflict), stored to global memory by the copy wavefronts
    static constexpr int XP = DVS + 16, STG = NBUF * SLOT, XB = DK * XP * 4;
    static constexpr int XR = DK * (DVS / 4) / LT;       // 16-byte stores per copy lane
    static constexpr int LDS = STG + 2 * XB;
    static_assert(OB::WALK % 16 == 0 && DVS / 8 == 4, "pieces");
    static_assert((AHEAD - 1) * (ROUNDS + 1) < 64, "vmcnt range");
    static_assert(XR * LT == DK * (DVS / 4), "staging rounds");
    static_assert(LDS <= 160 * 1024, "LDS");
};

template <int DK>
__global__ void __launch_bounds__(WalkCfg<DK>::NT, 1) kda_bwd_walk_kernel(BwdParams p, int DV, int nitems) {
    typedef WalkCfg<DK> G;
    typedef OpBlock<bf16, DK> OB;
    constexpr int NR = DK / 16, NKS = DK / 32, ROUNDS = G::ROUNDS, LT = G::LT;
    __shared__ alignas(16) uint8_t lds[G::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    // the value slices of one (sequence, head) on one XCD (item = (bid % 8) per + bid / 8)
    const int per = (nitems + 7) / 8;
    const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (item >= nitems) return;
    const int nsl = DV / G::DVS;
    const int64_t unit = item / nsl;
    const int slice = item % nsl;
    const int n = (int)(unit / p.H), h = (int)(unit % p.H);
    const SeqSpan sq = seq_span(p.cu, p.eq_len, n);
    const int nsub = ceil_div(sq.len, SC), nch = ceil_div(sq.len, CHB);
    const int j0 = slice * G::DVS;
    const int64_t sbase = ceil_blocks_before(p.cu, p.eq_len, n, SC) * p.H + (int64_t)h * nsub;
    const int64_t cbase = ceil_blocks_before(p.cu, p.eq_len, n, CHB) * p.H + (int64_t)h * nch;
    const bf16* __restrict__ dO = static_cast<const bf16*>(p.dO);
    // walk steps that end a 64-token chunk keep X (the derivative at that end),
    // staged in buffer (chunk index) % 2: consecutive kept chunks alternate
    auto keeps = [&](int jj) {
        const int s = nsub - 1 - jj;
        return s % (CHB / SC) == CHB / SC - 1 || s == nsub - 1;
    };
    auto staging = [&](int jj) { return lds + G::STG + ((nsub - 1 - jj) / (CHB / SC) & 1) * G::XB; };

    if (wv >= G::NW) {
        // ---- copy wavefronts: walk step jj is sub-chunk nsub - 1 - jj.  Step
        // jj + AHEAD is copied during step jj and step jj + AHEAD + TOUCH touched;
        // before the barrier of step jj the copies of step jj + 1 are waited for
        // (younger: AHEAD - 1 steps of copies and touches; loads complete in order).
        const int lt = tid - 64 * G::NW, lw = wv - G::NW;
        auto copy = [&](int jj, int sl) {
            const int s = nsub - 1 - jj;
            const uint8_t* blk = p.ops + (sbase + s) * OB::BYTES;
            const int64_t t0 = sq.t0 + (int64_t)s * SC;
            const int nrow = min(SC, sq.len - s * SC);
            uint8_t* slot = lds + sl * G::SLOT + lw * 1024;
#pragma unroll
            for (int r = 0; r < ROUNDS; ++r) {
                const uint8_t* src;
                if ((r + 1) * LT <= G::NPB) {
                    src = blk + r * LT * 16 + 16 * lt;
                } else {
                    const int pc = min(r * LT + lt, G::NPS - 1);
                    const int x = max(pc - G::NPB, 0), rp = x >> 2, u = x & 3;
                    const int t = 4 * (rp & 3) + (rp >> 2);  // token held by row position rp
                    const int64_t row = (t0 + min(t, nrow - 1)) * p.H + h;
                    const uint8_t* dsrc = reinterpret_cast<const uint8_t*>(dO + row * DV + j0 + 8 * u);
                    src = pc < G::NPB ? blk + 16 * pc : dsrc;
                }
                __builtin_amdgcn_global_load_lds(src, slot + r * LT * 16, 16, 0, 0);
            }
        };
        // one dword per 128-byte line of the walk's operators, slice s taking
        // lines s, s + nsl, ...; landing past the slot's pieces
        auto touch = [&](int jj) {
            constexpr int LINES = (OB::WALK + 127) / 128;
            const int nb = (LINES - slice + nsl - 1) / nsl;
            const int line = min(lt, nb - 1) * nsl + slice;
            __builtin_amdgcn_global_load_lds(p.ops + (sbase + nsub - 1 - jj) * OB::BYTES + 128 * line,
                                             lds + lw * G::SLOT + G::TOFF + 256 * lw, 4, 0, 0);
        };
        // X staged by the compute wavefronts at walk step jj (published by that
        // step's barrier) goes to its 64-token chunk's row of xbuf
        auto store_x = [&](int jj) {
            const uint8_t* sx = staging(jj);
            float* dst = p.xbuf + (cbase + (nsub - 1 - jj) / (CHB / SC)) * (int64_t)DK * DV + j0;
#pragma unroll
            for (int r = 0; r < G::XR; ++r) {
                const int q = r * LT + lt, row = q / (G::DVS / 4), cp = q % (G::DVS / 4);
                const i32x4 x = *reinterpret_cast<const i32x4*>(sx + (row * G::XP + 4 * cp) * 4);
                *reinterpret_cast<i32x4*>(dst + (int64_t)row * DV + 4 * cp) = x;
            }
        };
        if (nsub > 0) {
#pragma unroll
            for (int c = 0; c < G::AHEAD; ++c) {
                copy(min(c, nsub - 1), c);
                touch(min(c + G::TOUCH, nsub - 1));
            }
        }
        // the vmcnt waits count copies and touches only: stores issued in between
        // are older than the copies waited for or among the younger operations
        slot_barrier<(G::AHEAD - 1) * (ROUNDS + 1)>();
        for (int jj = 0; jj < nsub; ++jj) {
            if (jj > 0 && keeps(jj - 1)) store_x(jj - 1);
            copy(min(jj + G::AHEAD, nsub - 1), (jj + G::AHEAD) % G::NBUF);
            touch(min(jj + G::AHEAD + G::TOUCH, nsub - 1));
            slot_barrier<(G::AHEAD - 1) * (ROUNDS + 1)>();
        }
        if (nsub > 0 && keeps(nsub - 1)) store_x(nsub - 1);
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): no copy outlives the workgroup
        return;
    }

    // ---- X: columns jw .. jw + 15 of the slice, tile r rows 16 r + 4 lg + i
    const int jw = j0 + 16 * wv;
    const int64_t xo = unit * (int64_t)DK * DV + jw;
    f32x4 X[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
        X[r] = p.dST ? load_state_tile(p.dST + xo + (int64_t)16 * r * DV, DV, lane) : zero4();
    bf16x8 xfr[NKS];
    auto make_xfr = [&]() {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xfr[ks][i] = (bf16)X[2 * ks][i];
                xfr[ks][4 + i] = (bf16)X[2 * ks + 1][i];
            }
    };
    make_xfr();

    // lane parts of the operand addresses in a slot
    uint32_t oW[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) oW[ks] = OB::W + swz<2 * DK>(lr, 4 * ks + lg);
    const uint32_t oM = OB::M + 16 * (16 * (lg >> 1) + lr) + 8 * (lg & 1);
    const uint32_t oQ = OB::QK + 16 * (lg * DK + lr);   // + 256 r: channel rows 16 r ..
    const uint32_t oG = OB::GAM + 16 * lg;              // + 64 r
    const uint32_t oD = G::NPB * 16 + 64 * lg + 2 * (16 * wv + lr);  // + 256 i: dO row 4 lg + i

    // A step's operands, read right after the barrier that publishes its slot
    // (while the previous step's update runs): W's fragments, M's half row and
    // the four dO values of this lane, and the update's QK fragments and gamma.
    // The loop is unrolled by two so that the QK / gamma registers of the step
    // and of the next one are fixed sets.
    bf16x8 wf[NKS];
    bf16x4 mh;
    bf16 dv4[4];
    bf16x8 qf[2][NR];
    f32x4 gm[2][NR];
    auto read_ops = [&](const uint8_t* B, bf16x8 (&q)[NR], f32x4 (&g)[NR]) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) wf[ks] = *reinterpret_cast<const bf16x8*>(B + oW[ks]);
        mh = *reinterpret_cast<const bf16x4*>(B + oM);
#pragma unroll
        for (int i = 0; i < 4; ++i) dv4[i] = *reinterpret_cast<const bf16*>(B + oD + 256 * i);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            q[r] = *reinterpret_cast<const bf16x8*>(B + oQ + 256 * r);
            g[r] = *reinterpret_cast<const f32x4*>(B + oG + 64 * r);
        }
    };

    // step jj with its update operands in (q, g); the next step's go to (qn, gn)
    auto step = [&](int jj, bf16x8 (&q)[NR], f32x4 (&g)[NR], bf16x8 (&qn)[NR], f32x4 (&gn)[NR]) {
        // derivative at the end of a 64-token chunk: staged rows, each lane four
        // consecutive columns of one row (quad transpose), for the copy wavefronts
        if (keeps(jj)) {
            uint8_t* sx = staging(jj) + ((4 * lg + (lane & 3)) * G::XP + 16 * wv + 4 * ((lane & 15) >> 2)) * 4;
#pragma unroll
            for (int r = 0; r < NR; ++r)
                *reinterpret_cast<i32x4*>(sx + 16 * r * G::XP * 4) =
                    quad_transpose(__builtin_bit_cast(i32x4, X[r]), lane);
        }
        // F = -(M dO + W X): rows t = 4 lg + i of this lane, column jw + lr, as two
        // independent accumulation chains
        bf16x8 ma = {}, db = {};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ma[i] = mh[i];
            db[i] = dv4[i];
        }
        constexpr int KH = (NKS + 1) / 2;
        f32x4 fa = Mma<bf16>::mma(ma, db, zero4()), fb = zero4();
#pragma unroll
        for (int ks = 0; ks < KH; ++ks) fa = Mma<bf16>::mma(wf[ks], xfr[ks], fa);
#pragma unroll
        for (int ks = KH; ks < NKS; ++ks) fb = Mma<bf16>::mma(wf[ks], xfr[ks], fb);
        const f32x4 f = fa + fb;
#pragma unroll
        for (int i = 0; i < 4; ++i) db[4 + i] = (bf16)(-f[i]);
        __builtin_amdgcn_sched_barrier(0);

        // this step's LDS reads are done: the barrier hands its slot to the copy
        // wavefronts and publishes step jj + 1 (after the last step: a harmless
        // read of a stale slot)
        slot_barrier<63>();
        read_ops(lds + ((jj + 1) % G::NBUF) * G::SLOT, qn, gn);
        __builtin_amdgcn_sched_barrier(0);

        // X <- Diag(gamma) X + QK [dO; F]
#pragma unroll
        for (int r = 0; r < NR; ++r) X[r] = Mma<bf16>::mma(q[r], db, X[r] * g[r]);
        __builtin_amdgcn_sched_barrier(0);
        make_xfr();
    };

    slot_barrier<63>();
    if (nsub > 0) read_ops(lds, qf[0], gm[0]);
    for (int jj = 0; jj < nsub; jj += 2) {
        step(jj, qf[0], gm[0], qf[1], gm[1]);
        if (jj + 1 < nsub) step(jj + 1, qf[1], gm[1], qf[0], gm[0]);
    }
    if (p.dS0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) store_state_tile(p.dS0 + xo + (int64_t)16 * r * DV, DV, lane, X[r]);
    }
}

// ==================================================================== grad
template <typename MT, int DK, int DV>
struct GradSmem {
    static constexpr int P = 16 / (int)sizeof(MT);
    // dk- and dv-long rows are padded by 32 bytes (288-byte rows at d = 128 bf16):
    // with 16 bytes of pad, fragment reads of 16 such rows collide in pairs on
    // gfx950's LDS banks (measured); the gradient kernels run 0.6 % faster
    static constexpr int PR = 32 / (int)sizeof(MT);
    static constexpr int LDK = DK + PR, LDV = DV + PR, L16 = 16 + P, L32 = 32 + P;
    static constexpr int DMX = DK > DV ? DK : DV;
    static constexpr int LMX = (DK > DV ? DK : DV) + PR;
    MT kr[16 * LDK], qr[16 * LDK], vr[16 * LDV], dor[16 * LDV];
    MT mats[7][16 * L16];
    MT SB[DMX * LMX];         // S^T / X^T [j][c], or X / S row-major [c][j]
    MT GA[16 * LDK], GB[16 * LDK];
    MT CT[DK * L32];          // [Kcc^T | Ktc^T], [Qb^T | Kb^T], [Kc'^T | Kt'^T], [Qb'^T | Kb'^T]
    MT EBVT[DV * L32];        // [E^T | (bV)^T]
    MT DFT[DV * L32];         // [dO^T | F^T]
    MT Y0T[DV * L16];         // Y0^T, then dE^T
    MT Erm[16 * LDV], Yrm[16 * LDV], Grm[16 * LDV];
    MT MQ[16 * L32], MG[16 * L32], MV[16 * L32], MY[16 * L32];
    // decay sums, rows padded by 4 so that 16 lanes reading one channel of 16
    // tokens hit 16 different banks
    static constexpr int G2L = DK + 4;
    float G2[(SC + 1) * G2L];
    float bt[SC];
    float phi0[DK];
    float red[3][GW][16];     // per-wave partials: R.V, G.Y, dlog_a (scalar gate)
    int exact;
};

// The four masked products of a sub-chunk whose decay spans too much for the
// factor split, one exponent per term: out[t][c] = sum_i M[t][i] y_ic e^{+-(h_tc - h'_ic)}
// for this lane's rows t = 4 g4 + r and channel c.  Masked-out pairs hold 0;
// clamping their exponents at 0 keeps them finite.
// (returned by value: the out-of-line call then keeps the caller's products in
// registers instead of stack slots that every step would store and reload)
struct ExactTerms { f32x4 q, g, v, y; };
template <typename MT, int DK, typename SM>
__device__ __attribute__((noinline)) ExactTerms exact_terms(const SM& sm, int c, int g4, int gmo) {
    constexpr int LDK = SM::LDK, L32 = SM::L32;
    f32x4 mq, mg, mv, my;
    for (int r = 0; r < 4; ++r) {
        const int t = 4 * g4 + r;
        float aq = 0.f, ag = 0.f, av = 0.f, ay = 0.f;
        const float gmt = sm.G2[(t + gmo) * SM::G2L + c], gt = sm.G2[(t + 1) * SM::G2L + c];
        for (int i = 0; i < 16; ++i) {
            const float ki = to_f32(sm.kr[i * LDK + c]), qi = to_f32(sm.qr[i * LDK + c]);
            const float gmi = sm.G2[(i + gmo) * SM::G2L + c], gi = sm.G2[(i + 1) * SM::G2L + c];
            aq += to_f32(sm.MQ[t * L32 + i]) * ki * ex2n(gt - gmi) + to_f32(sm.MQ[t * L32 + 16 + i]) * ki * ex2n(gt - gi);
            ag += to_f32(sm.MG[t * L32 + i]) * ki * ex2n(gmt - gmi) + to_f32(sm.MG[t * L32 + 16 + i]) * ki * ex2n(gmt - gi);
            av += to_f32(sm.MV[t * L32 + i]) * qi * ex2n(gi - gt) + to_f32(sm.MV[t * L32 + 16 + i]) * ki * ex2n(gmi - gt);
            ay += to_f32(sm.MY[t * L32 + i]) * qi * ex2n(gi - gmt) + to_f32(sm.MY[t * L32 + 16 + i]) * ki * ex2n(gmi - gmt);
        }
        mq[r] = aq; mg[r] = ag; mv[r] = av; my[r] = ay;
    }
    return ExactTerms{mq, mg, mv, my};
}

template <typename MT, int DK, int DV>
__global__ __launch_bounds__(64 * GW) void kda_bwd_grad_kernel(BwdParams p) {
    const int gmo = p.gmo;
    typedef GradSmem<MT, DK, DV> SM;
    typedef OpBlock<MT, DK> OB;
    constexpr int LDK = SM::LDK, LDV = SM::LDV, L16 = SM::L16, L32 = SM::L32;
    constexpr int NCB = DK / 16, NJB = DV / 16, CBW = (NCB + GW - 1) / GW, JBW = (NJB + GW - 1) / GW;
    constexpr int NT = 64 * GW;
    constexpr int SUBE = DK * DV + 2 * 16 * DV;  // kept per sub-chunk: start state, E, Y (elements of MT)
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int jc = blockIdx.x;
    const int64_t unit = blockIdx.y;
    const int n = (int)(unit / p.H), h = (int)(unit % p.H);
    const SeqSpan sq = seq_span(p.cu, p.eq_len, n);
    if (jc * CHB >= sq.len) return;
    const int nsub = ceil_div(sq.len, SC), nch = ceil_div(sq.len, CHB);
    const int clen = min(CHB, sq.len - jc * CHB);
    const int ns = ceil_div(clen, SC);
    const int64_t sbase = ceil_blocks_before(p.cu, p.eq_len, n, SC) * p.H + (int64_t)h * nsub + jc * (CHB / SC);
    const int64_t xrow = ceil_blocks_before(p.cu, p.eq_len, n, CHB) * p.H + (int64_t)h * nch + jc;
    // forward state at the chunk start: S0, or the kept state after jc chunks
    const float* s_start = nullptr;
    if (jc == 0) {
        if (p.S0) s_start = p.S0 + unit * (int64_t)DK * DV;
    } else {
        int64_t before;
        if (!p.cu) before = (int64_t)n * (p.eq_len / CHB);
        else before = snapshots_before(p.cu, p.eq_len, n, CHB);
        if (before + jc - 1 < p.snap_rows) s_start = p.snap + ((before + jc - 1) * p.H + h) * (int64_t)DK * DV;
    }
    const MT* Kg = static_cast<const MT*>(p.k);
    const MT* Qg = static_cast<const MT*>(p.q);
    const MT* Vg = static_cast<const MT*>(p.v);
    const MT* Og = static_cast<const MT*>(p.dO);
    // this chunk's scratch: per sub-chunk its start state, E and Y, each tile as the
    // owning lanes hold it (4 consecutive values per lane)
    MT* scr = static_cast<MT*>(p.scr) + xrow * (int64_t)(CHB / SC) * SUBE;
    auto kS = [&](int s2, int cb, int jb) { return scr + (int64_t)s2 * SUBE + ((cb * NJB + jb) * 64 + lane) * 4; };
    auto kE = [&](int s2, int jb) { return scr + (int64_t)s2 * SUBE + DK * DV + (jb * 64 + lane) * 4; };
    auto kY = [&](int s2, int jb) { return scr + (int64_t)s2 * SUBE + DK * DV + 16 * DV + (jb * 64 + lane) * 4; };

    auto load_state = [&](f32x4 (&Z)[CBW][NJB], const float* src) {
#pragma unroll
        for (int a = 0; a < CBW; ++a)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int cb = w + GW * a;
                Z[a][jb] = zero4();
                if (cb < NCB && src) Z[a][jb] = load_state_tile(src + (int64_t)cb * 16 * DV + jb * 16, DV, lane);
            }
    };
    // A step's inputs (rows of k, v and, walking backwards, q and dO; the decays;
    // the step's 16 x 16 matrices) are fetched into registers one step ahead and
    // placed in LDS at the start of the step (walking backwards: at the end of the
    // step before, after its last LDS read).  Pieces of 16 bytes, numbered
    // [k | v | q | dO | decays | matrices], thread tid holding tid + NT a.
    typedef typename V16<MT>::type VT;
    constexpr int PER = 16 / (int)sizeof(MT);
    constexpr int PRK = DK / PER, PRV = DV / PER, PLA = DK / 4, PM = 256 / PER;
    constexpr int NPF = (16 * (2 * PRK + 2 * PRV + PLA) + 4 * PM + NT - 1) / NT;
    VT pf[NPF];
    float pfb = 0.f;
    auto mat_of = [](bool bwd, int idx) {
        return bwd ? (idx == 0 ? MAT_TT : idx == 1 ? MAT_LT : idx == 2 ? MAT_P1T : MAT_P2T)
                   : (idx == 0 ? MAT_TB : idx == 1 ? MAT_L : MAT_A0);
    };
    // piece pc of a step: which tensor, row i and offset e (elements) within it
    struct Piece { int kind, i, e; };
    auto decode = [&](int pc, bool bwd) -> Piece {
        const int B0 = 16 * PRK, B1 = B0 + 16 * PRV, B2 = bwd ? B1 + 16 * PRK : B1, B3 = bwd ? B2 + 16 * PRV : B1;
        const int B4 = B3 + 16 * PLA, B5 = B4 + (bwd ? 4 : 3) * PM;
        if (pc < B0) return Piece{0, pc / PRK, (pc % PRK) * PER};
        if (pc < B1) return Piece{1, (pc - B0) / PRV, ((pc - B0) % PRV) * PER};
        if (pc < B2) return Piece{2, (pc - B1) / PRK, ((pc - B1) % PRK) * PER};
        if (pc < B3) return Piece{3, (pc - B2) / PRV, ((pc - B2) % PRV) * PER};
        if (pc < B4) return Piece{4, (pc - B3) / PLA, ((pc - B3) % PLA) * 4};
        if (pc < B5) return Piece{5, (pc - B4) / PM, ((pc - B4) % PM) * PER};
        return Piece{6, 0, 0};
    };
    // A thread's pieces are the same at every step, so they are decoded once and
    // packed, 16 bits per walk direction (kind << 11 | row << 6 | offset / 4), and
    // unpacked where used behind an empty asm statement: the compiler then keeps
    // one register per piece, and every address is a wave-uniform base of the step
    // plus a small lane offset.  (Addresses hoisted per piece and tensor had spilled,
    // and each reload waited for every load issued before it.)
    uint32_t pdesc[NPF];
#pragma unroll
    for (int a = 0; a < NPF; ++a) {
        const Piece f = decode(tid + NT * a, false), b = decode(tid + NT * a, true);
        pdesc[a] = (uint32_t)(f.kind << 11 | f.i << 6 | f.e >> 2) | (uint32_t)(b.kind << 11 | b.i << 6 | b.e >> 2) << 16;
    }
    auto piece_of = [&](int a, bool bwd) -> Piece {
        uint32_t d = pdesc[a];
        asm volatile("" : "+v"(d));
        d = bwd ? d >> 16 : d & 0xFFFFu;
        return Piece{(int)(d >> 11), (int)((d >> 6) & 31), (int)((d & 63) << 2)};
    };
    auto issue = [&](int s2, bool bwd) {
        const int64_t t0 = sq.t0 + (int64_t)jc * CHB + s2 * SC;
        const int nrow = min(SC, clen - s2 * SC);
        const int64_t rb = t0 * p.H + h;  // the step's first row (wave-uniform)
        const MT* kb = Kg + rb * DK;
        const MT* vb = Vg + rb * DV;
        const MT* qb = Qg + rb * DK;
        const MT* ob = Og + rb * DV;
        const float* lb = p.log_a + rb * (p.scalar ? 1 : DK);
        const MT* mats = reinterpret_cast<const MT*>(p.ops + (sbase + s2) * OB::BYTES + OB::MATS);
#pragma unroll
        for (int a = 0; a < NPF; ++a) {
            const Piece pc = piece_of(a, bwd);
            VT x = {};
            const int ro = pc.i * p.H;  // the piece's row, counted from the step's first
            if (pc.kind <= 4 && pc.i >= nrow) {
            } else if (pc.kind == 0) {
                x = *reinterpret_cast<const VT*>(kb + (ro * DK + pc.e));
            } else if (pc.kind == 1) {
                x = *reinterpret_cast<const VT*>(vb + (ro * DV + pc.e));
            } else if (pc.kind == 2) {
                x = *reinterpret_cast<const VT*>(qb + (ro * DK + pc.e));
            } else if (pc.kind == 3) {
                x = *reinterpret_cast<const VT*>(ob + (ro * DV + pc.e));
            } else if (pc.kind == 4) {
                f32x4 d;
                if (p.scalar) {
                    const float a1 = lb[ro];
                    d = f32x4{a1, a1, a1, a1};
                } else {
                    d = *reinterpret_cast<const f32x4*>(lb + (ro * DK + pc.e));
                }
                x = __builtin_bit_cast(VT, d);
            } else if (pc.kind == 5) {
                x = *reinterpret_cast<const VT*>(mats + mat_of(bwd, pc.i) * 256 + pc.e);
            }
            pf[a] = x;
        }
        pfb = tid < nrow && tid < SC ? p.beta[(t0 + tid) * p.H + h] : 0.f;
    };
    // places the fetched pieces in LDS; the decays as log2 e * log a in rows 1..16 of G2
    auto commit = [&](bool bwd) {
#pragma unroll
        for (int a = 0; a < NPF; ++a) {
            const Piece pc = piece_of(a, bwd);
            if (pc.kind == 0) *reinterpret_cast<VT*>(sm.kr + pc.i * LDK + pc.e) = pf[a];
            else if (pc.kind == 1) *reinterpret_cast<VT*>(sm.vr + pc.i * LDV + pc.e) = pf[a];
            else if (pc.kind == 2) *reinterpret_cast<VT*>(sm.qr + pc.i * LDK + pc.e) = pf[a];
            else if (pc.kind == 3) *reinterpret_cast<VT*>(sm.dor + pc.i * LDV + pc.e) = pf[a];
            else if (pc.kind == 4)
                *reinterpret_cast<f32x4*>(sm.G2 + (pc.i + 1) * SM::G2L + pc.e) = __builtin_bit_cast(f32x4, pf[a]) * LOG2E;
            else if (pc.kind == 5)
                *reinterpret_cast<VT*>(&sm.mats[mat_of(bwd, pc.i)][(pc.e / 16) * L16 + pc.e % 16]) = pf[a];
        }
        if (tid < SC) sm.bt[tid] = pfb;
    };
    // G2[i][c] = running sum over the first i tokens (after commit and a barrier)
    auto prefix_decay = [&]() {
        for (int c = tid; c < DK; c += NT) {
            float s2 = 0.f;
            sm.G2[c] = 0.f;
#pragma unroll
            for (int i = 1; i <= SC; ++i) {
                s2 += sm.G2[i * SM::G2L + c];
                sm.G2[i * SM::G2L + c] = s2;
            }
        }
    };

    // The kept E, Y and start state S of a sub-chunk, as stored (MT).  The forward
    // walk's last step leaves those of the last sub-chunk here; the others are
    // loaded at the end of the backward step before, ahead of its output stores,
    // so that waiting for them does not also wait for the stores (the counter of
    // outstanding memory operations drains in order).
    typedef typename Vec4<MT>::type V4;
    V4 Sk[CBW][NJB], Ek[JBW], Yk[JBW];

    // The state derivative at the chunk end: its loads go out during the forward
    // walk's last step (peeled, so that they take the registers of the state, which
    // that step no longer updates) and it is brought into tile order after the walk,
    // as load_state_tile does.
    f32x4 X[CBW][NJB];
    // Elementwise fills of the step's operands.  A thread takes four consecutive
    // channels (or value columns) of one token row, so that its LDS reads are
    // vectors; the transposed fills (dst[c][off + i], rows L32 apart) give 16 lanes
    // 16 consecutive rows i of one column, so that their 2- or 4-byte writes meet
    // no bank conflict either.
    typedef typename Vec4<MT>::type VX4;
    auto rd4 = [&](const MT* src) { return Vec4<MT>::to_f32(*reinterpret_cast<const VX4*>(src)); };
    auto gsum = [&](int row, int c0) { return *reinterpret_cast<const f32x4*>(sm.G2 + row * SM::G2L + c0); };
    auto ex2v = [](f32x4 x) { return f32x4{ex2(x[0]), ex2(x[1]), ex2(x[2]), ex2(x[3])}; };
    // row-major: f(t, c0) for t < 16, c0 = 0, 4, .. < N
    auto fill_rows = [&](int N, auto&& f) {
        for (int x = tid; x < 4 * N; x += NT) f(x / (N / 4), 4 * (x % (N / 4)));
    };
    // transposed: dst[(c0 + u) L32 + off + i] = f(i, c0)[u], and with a second part at off2
    auto fill_cols = [&](MT* dst, int N, int off, auto&& f) {
        for (int x = tid; x < 4 * N; x += NT) {
            const int i = x & 15, c0 = 4 * (x >> 4);
            const f32x4 v = f(i, c0);
#pragma unroll
            for (int u = 0; u < 4; ++u) dst[(c0 + u) * L32 + off + i] = from_f32<MT>(v[u]);
        }
    };
    auto fill_cols2 = [&](MT* dst, int N, auto&& f) {
        for (int x = tid; x < 4 * N; x += NT) {
            const int i = x & 15, c0 = 4 * (x >> 4);
            f32x4 a, b;
            f(i, c0, a, b);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                dst[(c0 + u) * L32 + i] = from_f32<MT>(a[u]);
                dst[(c0 + u) * L32 + 16 + i] = from_f32<MT>(b[u]);
            }
        }
    };

    // ================= forward walk: start state, E and Y of every sub-chunk
    {
        f32x4 S[CBW][NJB];
        issue(0, false);
        load_state(S, s_start);
        auto fwd_step = [&](int sf, auto lastc) {
            constexpr bool last = decltype(lastc)::value;
            lds_barrier();
            commit(false);
            if constexpr (!last) issue(sf + 1, false);
            else issue(ns - 1, true);  // the backward walk starts at the last sub-chunk
#pragma unroll
            for (int a = 0; a < CBW; ++a)
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {
                    const int cb = w + GW * a;
                    if (cb < NCB) {
                        store_nat<MT>(sm.SB + jb * 16 * LDK + cb * 16, LDK, S[a][jb], lane);
                        if constexpr (last) Sk[a][jb] = Vec4<MT>::from_f32(S[a][jb]);
                        else store4<MT>(kS(sf, cb, jb), S[a][jb]);
                    }
                }
            if constexpr (last) {
                const float* xsrc = p.xbuf + xrow * (int64_t)DK * DV;
                const int row = 4 * (lane >> 4) + (lane & 3), col = 4 * ((lane & 15) >> 2);
#pragma unroll
                for (int a = 0; a < CBW; ++a)
#pragma unroll
                    for (int jb = 0; jb < NJB; ++jb) {
                        const int cb = w + GW * a;
                        X[a][jb] = zero4();
                        if (cb < NCB)
                            X[a][jb] = *reinterpret_cast<const f32x4*>(xsrc + (int64_t)(cb * 16 + row) * DV + jb * 16 + col);
                    }
            }
            lds_barrier();
            prefix_decay();
            lds_barrier();
            // ---- Kb rows, (bV)^T, [Kcc^T | Ktc^T]
            fill_rows(DK, [&](int t, int c0) {
                store4<MT>(sm.GA + t * LDK + c0, rd4(sm.kr + t * LDK + c0) * ex2v(gsum(t + gmo, c0)));
            });
            fill_cols(sm.EBVT, DV, 16, [&](int i, int j0) { return sm.bt[i] * rd4(sm.vr + i * LDV + j0); });
            if constexpr (!last) {
                fill_cols2(sm.CT, DK, [&](int i, int c0, f32x4& a, f32x4& b) {
                    const f32x4 kv = rd4(sm.kr + i * LDK + c0), gc = gsum(SC, c0);
                    a = kv * ex2v(gc - gsum(i + gmo, c0));
                    b = kv * ex2v(gc - gsum(i + 1, c0));
                });
            }
            lds_barrier();
            // ---- Y0 = Kb S + L bV   (m = t, n = j)
            f32x4 Y0[JBW];
#pragma unroll
            for (int a = 0; a < JBW; ++a) {
                const int jb = w + GW * a;
                Y0[a] = zero4();
                if (jb < NJB) {
                    Y0[a] = mmak<MT, DK>(sm.GA + r16 * LDK, sm.SB + (jb * 16 + r16) * LDK, zero4(), lane);
                    Y0[a] = mmak<MT, 16>(sm.mats[MAT_L] + r16 * L16, sm.EBVT + (jb * 16 + r16) * L32 + 16, Y0[a], lane);
                    store_nat<MT>(sm.Y0T + jb * 16 * L16, L16, Y0[a], lane);
                }
            }
            lds_barrier();
            // ---- E = -T diag(b) Y0
#pragma unroll
            for (int a = 0; a < JBW; ++a) {
                const int jb = w + GW * a;
                if (jb < NJB) {
                    const f32x4 e = -mmak<MT, 16>(sm.mats[MAT_TB] + r16 * L16, sm.Y0T + (jb * 16 + r16) * L16, zero4(), lane);
                    store_nat<MT>(sm.EBVT + jb * 16 * L32, L32, e, lane);
                    if constexpr (last) Ek[a] = Vec4<MT>::from_f32(e);
                    else store4<MT>(kE(sf, jb), e);
                }
            }
            lds_barrier();
            // ---- Y = Y0 + A0 E; S <- gamma S + [Kcc^T | Ktc^T] [E; bV]
#pragma unroll
            for (int a = 0; a < JBW; ++a) {
                const int jb = w + GW * a;
                if (jb < NJB) {
                    const f32x4 y = mmak<MT, 16>(sm.mats[MAT_A0] + r16 * L16, sm.EBVT + (jb * 16 + r16) * L32, Y0[a], lane);
                    if constexpr (last) Yk[a] = Vec4<MT>::from_f32(y);
                    else store4<MT>(kY(sf, jb), y);
                }
            }
            if constexpr (!last) {
#pragma unroll
                for (int a = 0; a < CBW; ++a) {
                    const int cb = w + GW * a;
                    if (cb < NCB) {
                        f32x4 gmm;
#pragma unroll
                        for (int r = 0; r < 4; ++r) gmm[r] = ex2(sm.G2[SC * SM::G2L + cb * 16 + 4 * g4 + r]);
#pragma unroll
                        for (int jb = 0; jb < NJB; ++jb)
                            S[a][jb] = mmak<MT, 32>(sm.CT + (cb * 16 + r16) * L32, sm.EBVT + (jb * 16 + r16) * L32,
                                                    gmm * S[a][jb], lane);
                    }
                }
            }
        };
        for (int sf = 0; sf < ns - 1; ++sf) fwd_step(sf, BoolC<false>{});
        fwd_step(ns - 1, BoolC<true>{});
    }

    // ================= backward walk over the sub-chunks
#pragma unroll
    for (int a = 0; a < CBW; ++a)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
            X[a][jb] = __builtin_bit_cast(f32x4, quad_transpose(__builtin_bit_cast(i32x4, X[a][jb]), lane));
    int kflag = *reinterpret_cast<const int*>(p.ops + (sbase + ns - 1) * OB::BYTES + OB::FLAG);
    auto load_kept = [&](int s2) {
        kflag = *reinterpret_cast<const int*>(p.ops + (sbase + s2) * OB::BYTES + OB::FLAG);
#pragma unroll
        for (int a = 0; a < JBW; ++a) {
            const int jb = w + GW * a;
            if (jb < NJB) {
                Ek[a] = *reinterpret_cast<const V4*>(kE(s2, jb));
                Yk[a] = *reinterpret_cast<const V4*>(kY(s2, jb));
            }
        }
#pragma unroll
        for (int a = 0; a < CBW; ++a)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int cb = w + GW * a;
                if (cb < NCB) Sk[a][jb] = *reinterpret_cast<const V4*>(kS(s2, cb, jb));
            }
    };
    // a step's inputs are placed in LDS at the end of the step before (here for the
    // first), after that step's last LDS read and before its output stores
    lds_barrier();
    commit(true);
    if (ns > 1) issue(ns - 2, true);
    for (int sg = ns - 1; sg >= 0; --sg) {
        const int64_t t0 = sq.t0 + (int64_t)jc * CHB + sg * SC;
        const int nrow = min(SC, clen - sg * SC);
        lds_barrier();
        prefix_decay();
        if (tid == 0) sm.exact = kflag;
#pragma unroll
        for (int a = 0; a < JBW; ++a) {
            const int jb = w + GW * a;
            if (jb < NJB) {
                store_rm<MT>(sm.Erm + jb * 16, LDV, Vec4<MT>::to_f32(Ek[a]), lane);
                store_rm<MT>(sm.Yrm + jb * 16, LDV, Vec4<MT>::to_f32(Yk[a]), lane);
            }
        }
        lds_barrier();
        // ================= gradient of sub-chunk sg (start state S, end derivative X)
        // ---- X^T; dO^T; Kcc, Ktc rows; [Qb^T | Kb^T]
#pragma unroll
        for (int a = 0; a < CBW; ++a)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int cb = w + GW * a;
                if (cb < NCB) store_nat<MT>(sm.SB + jb * 16 * LDK + cb * 16, LDK, X[a][jb], lane);
            }
        fill_cols(sm.DFT, DV, 0, [&](int i, int j0) { return rd4(sm.dor + i * LDV + j0); });
        fill_rows(DK, [&](int t, int c0) {
            const f32x4 kv = rd4(sm.kr + t * LDK + c0), gc = gsum(SC, c0);
            store4<MT>(sm.GA + t * LDK + c0, kv * ex2v(gc - gsum(t + gmo, c0)));
            store4<MT>(sm.GB + t * LDK + c0, kv * ex2v(gc - gsum(t + 1, c0)));
        });
        fill_cols2(sm.CT, DK, [&](int i, int c0, f32x4& a, f32x4& b) {
            a = rd4(sm.qr + i * LDK + c0) * ex2v(gsum(i + 1, c0));
            b = rd4(sm.kr + i * LDK + c0) * ex2v(gsum(i + gmo, c0));
        });
        lds_barrier();
        // ---- dE = Kcc X + P1^T dO  (m = t, n = j) -> dE^T
#pragma unroll
        for (int a = 0; a < JBW; ++a) {
            const int jb = w + GW * a;
            if (jb < NJB) {
                f32x4 d = mmak<MT, DK>(sm.GA + r16 * LDK, sm.SB + (jb * 16 + r16) * LDK, zero4(), lane);
                d = mmak<MT, 16>(sm.mats[MAT_P1T] + r16 * L16, sm.DFT + (jb * 16 + r16) * L32, d, lane);
                store_nat<MT>(sm.Y0T + jb * 16 * L16, L16, d, lane);
            }
        }
        lds_barrier();
        // ---- G^T = dE^T T  (m = j, n = t): G row-major, F^T = -b G^T, partial G.Y
        {
            float gy[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int a = 0; a < JBW; ++a) {
                const int jb = w + GW * a;
                if (jb < NJB) {
                    const f32x4 gt = mmak<MT, 16>(sm.Y0T + (jb * 16 + r16) * L16, sm.mats[MAT_TT] + r16 * L16, zero4(), lane);
                    store_nat<MT>(sm.Grm + jb * 16, LDV, gt, lane);
                    const float bneg = -sm.bt[r16];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = jb * 16 + 4 * g4 + r;
                        sm.DFT[j * L32 + 16 + r16] = from_f32<MT>(bneg * gt[r]);
                        gy[0] += gt[r] * to_f32(sm.Yrm[r16 * LDV + j]);
                    }
                }
            }
            float v0 = gy[0];
            v0 += __shfl_xor(v0, 16);
            v0 += __shfl_xor(v0, 32);
            if (g4 == 0) sm.red[1][w][r16] = v0;
        }
        lds_barrier();
        // ---- R = Ktc X + P2^T dO + L^T F  (m = t, n = j): dv, partial R.V
        {
            float rv[4] = {0.f, 0.f, 0.f, 0.f};
            MT* dvg = static_cast<MT*>(p.dv);
#pragma unroll
            for (int a = 0; a < JBW; ++a) {
                const int jb = w + GW * a;
                if (jb < NJB) {
                    f32x4 rr = mmak<MT, DK>(sm.GB + r16 * LDK, sm.SB + (jb * 16 + r16) * LDK, zero4(), lane);
                    rr = mmak<MT, 16>(sm.mats[MAT_P2T] + r16 * L16, sm.DFT + (jb * 16 + r16) * L32, rr, lane);
                    rr = mmak<MT, 16>(sm.mats[MAT_LT] + r16 * L16, sm.DFT + (jb * 16 + r16) * L32 + 16, rr, lane);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 4 * g4 + r, j = jb * 16 + r16;
                        rv[r] += rr[r] * to_f32(sm.vr[t * LDV + j]);
                        if (t < nrow) dvg[((t0 + t) * p.H + h) * (int64_t)DV + j] = from_f32<MT>(sm.bt[t] * rr[r]);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) rv[r] = row_sum16(rv[r]);
            if (r16 == 0)
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.red[0][w][4 * g4 + r] = rv[r];
        }
        lds_barrier();
        // ---- X row-major; dbeta
#pragma unroll
        for (int a = 0; a < CBW; ++a)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int cb = w + GW * a;
                if (cb < NCB) store_rm<MT>(sm.SB + cb * 16 * LDV + jb * 16, LDV, X[a][jb], lane);
            }
        if (tid < 16 && tid < nrow) {
            float db = 0.f;
#pragma unroll
            for (int u = 0; u < GW; ++u) db += sm.red[0][u][tid] - sm.red[1][u][tid];
            p.dbeta[(t0 + tid) * p.H + h] = db;
        }
        lds_barrier();
        // ---- state parts with X: vds_s = V X^T, ayds_s = Y X^T  (m = t, n = c)
        f32x4 vds[CBW], ayds[CBW], dqs[CBW], gss[CBW];
#pragma unroll
        for (int a = 0; a < CBW; ++a) {
            const int cb = w + GW * a;
            vds[a] = ayds[a] = zero4();
            if (cb < NCB) {
                vds[a] = mmak<MT, DV>(sm.vr + r16 * LDV, sm.SB + (cb * 16 + r16) * LDV, zero4(), lane);
                ayds[a] = mmak<MT, DV>(sm.Yrm + r16 * LDV, sm.SB + (cb * 16 + r16) * LDV, zero4(), lane);
            }
        }
        // ---- the eight 16 x 16 products (m = i, n = t), stored row-major [t][i] with their masks
        for (int mi = w; mi < 8; mi += GW) {
            const MT *A, *B;
            switch (mi) {
                case 0: A = sm.Erm; B = sm.dor; break;  // lower(dO E^T)
                case 1: A = sm.vr; B = sm.dor; break;   // lower(dO bV^T)
                case 2: A = sm.Erm; B = sm.Grm; break;  // strict_lower(G E^T)
                case 3: A = sm.vr; B = sm.Grm; break;   // strict_lower(G bV^T)
                case 4: A = sm.dor; B = sm.vr; break;   // upper(V dO^T)
                case 5: A = sm.Grm; B = sm.vr; break;   // strict_upper(V F^T)
                case 6: A = sm.dor; B = sm.Yrm; break;  // upper(Y dO^T)
                default: A = sm.Grm; B = sm.Yrm; break; // strict_upper(Y F^T)
            }
            f32x4 d = mmak<MT, DV>(A + r16 * LDV, B + r16 * LDV, zero4(), lane);
            MT* dst = mi < 2 ? sm.MQ : mi < 4 ? sm.MG : mi < 6 ? sm.MV : sm.MY;
            const int coff = (mi & 1) * 16;
            // the lane's four rows i = 4 g4 .. 4 g4 + 3 of column t are consecutive in [t][i]
            const f32x4 bq = *reinterpret_cast<const f32x4*>(sm.bt + 4 * g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * g4 + r, t = r16;
                float x = d[r];
                if (mi == 1 || mi == 3) x *= bq[r];
                if (mi == 5 || mi == 7) x *= -bq[r];
                const bool keep = mi < 2 ? i <= t : mi < 4 ? i < t : (mi & 1) ? i > t : i >= t;
                d[r] = keep ? x : 0.f;
            }
            store4<MT>(dst + r16 * L32 + coff + 4 * g4, d);
        }
        // ---- X <- gamma X + [Qb^T | Kb^T] [dO; F]; phi_{-1} = rowsum(X_prev * S)
#pragma unroll
        for (int a = 0; a < CBW; ++a) {
            const int cb = w + GW * a;
            if (cb < NCB) {
                f32x4 gmm;
#pragma unroll
                for (int r = 0; r < 4; ++r) gmm[r] = ex2(sm.G2[SC * SM::G2L + cb * 16 + 4 * g4 + r]);
                f32x4 ph = zero4();
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {
                    X[a][jb] = mmak<MT, 32>(sm.CT + (cb * 16 + r16) * L32, sm.DFT + (jb * 16 + r16) * L32,
                                            gmm * X[a][jb], lane);
                    ph += X[a][jb] * Vec4<MT>::to_f32(Sk[a][jb]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) ph[r] = row_sum16(ph[r]);
                if (r16 == 0)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sm.phi0[cb * 16 + 4 * g4 + r] = ph[r];
            }
        }
        lds_barrier();
        // ---- S row-major; [Kc'^T | Kt'^T]
#pragma unroll
        for (int a = 0; a < CBW; ++a)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int cb = w + GW * a;
                if (cb < NCB) store_rm<MT>(sm.SB + cb * 16 * LDV + jb * 16, LDV, Vec4<MT>::to_f32(Sk[a][jb]), lane);
            }
        fill_cols2(sm.CT, DK, [&](int i, int c0, f32x4& a, f32x4& b) {
            const f32x4 kv = rd4(sm.kr + i * LDK + c0), m2 = 0.5f * gsum(SC, c0);
            a = kv * ex2v(m2 - gsum(i + gmo, c0));
            b = kv * ex2v(m2 - gsum(i + 1, c0));
        });
        lds_barrier();
        const bool exact = sm.exact != 0;
        f32x4 mq[CBW], mg[CBW], mv[CBW], my[CBW];
#pragma unroll
        for (int a = 0; a < CBW; ++a) {
            const int cb = w + GW * a;
            dqs[a] = gss[a] = mq[a] = mg[a] = zero4();
            if (cb < NCB) {
                dqs[a] = mmak<MT, DV>(sm.dor + r16 * LDV, sm.SB + (cb * 16 + r16) * LDV, zero4(), lane);
                gss[a] = mmak<MT, DV>(sm.Grm + r16 * LDV, sm.SB + (cb * 16 + r16) * LDV, zero4(), lane);
                if (!exact) {
                    mq[a] = mmak<MT, 32>(sm.MQ + r16 * L32, sm.CT + (cb * 16 + r16) * L32, zero4(), lane);
                    mg[a] = mmak<MT, 32>(sm.MG + r16 * L32, sm.CT + (cb * 16 + r16) * L32, zero4(), lane);
                }
            }
        }
        lds_barrier();
        fill_cols2(sm.CT, DK, [&](int i, int c0, f32x4& a, f32x4& b) {
            const f32x4 m2 = 0.5f * gsum(SC, c0);
            a = rd4(sm.qr + i * LDK + c0) * ex2v(gsum(i + 1, c0) - m2);
            b = rd4(sm.kr + i * LDK + c0) * ex2v(gsum(i + gmo, c0) - m2);
        });
        lds_barrier();
        // ---- masked products, combination, outputs  (m = t, n = c)
        MT* dqg = static_cast<MT*>(p.dq);
        MT* dkg = static_cast<MT*>(p.dk);
        float dla_s[4] = {0.f, 0.f, 0.f, 0.f};
        float oq[CBW][4], ok[CBW][4], od[CBW][4];
#pragma unroll
        for (int a = 0; a < CBW; ++a) {
            const int cb = w + GW * a;
            if (cb >= NCB) continue;
            const int c = cb * 16 + r16;
            if (!exact) {
                mv[a] = mmak<MT, 32>(sm.MV + r16 * L32, sm.CT + c * L32, zero4(), lane);
                my[a] = mmak<MT, 32>(sm.MY + r16 * L32, sm.CT + c * L32, zero4(), lane);
            } else {
                const ExactTerms x = exact_terms<MT, DK>(sm, c, g4, gmo);
                mq[a] = x.q; mg[a] = x.g; mv[a] = x.v; my[a] = x.y;
            }
            const float gc = sm.G2[SC * SM::G2L + c], m2 = 0.5f * gc, em = ex2(m2);
            float av[4], au[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g4 + r;
                const float gmt = sm.G2[(t + gmo) * SM::G2L + c], gt = sm.G2[(t + 1) * SM::G2L + c];
                // factored: the state parts' factors e^{g}, e^{gm}, e^{gC-g}, e^{gC-gm} are e^{m}
                // times the masked parts' ones (each within e^{+-span/2}, no overflow); exact:
                // one exponent each
                float dq, gs, vd, ay;
                if (!exact) {
                    const float fq = ex2(gt - m2), fg = ex2(gmt - m2), fv = ex2(m2 - gt), fy = ex2(m2 - gmt);
                    dq = (em * fq) * dqs[a][r] + fq * mq[a][r];
                    gs = (em * fg) * gss[a][r] + fg * mg[a][r];
                    vd = (em * fv) * vds[a][r] + fv * mv[a][r];
                    ay = (em * fy) * ayds[a][r] + fy * my[a][r];
                } else {
                    dq = ex2(gt) * dqs[a][r] + mq[a][r];
                    gs = ex2(gmt) * gss[a][r] + mg[a][r];
                    vd = ex2(gc - gt) * vds[a][r] + mv[a][r];
                    ay = ex2(gc - gmt) * ayds[a][r] + my[a][r];
                }
                const float b = sm.bt[t];
                const float kt = to_f32(sm.kr[t * LDK + c]), qt = to_f32(sm.qr[t * LDK + c]);
                const float dk = b * (vd - ay - gs);
                av[r] = kt * dk + 2.f * b * kt * gs;
                au[r] = qt * dq;
                // reuse: the term dlog a takes off phi (erase-first b k vds; decay-first the
                // step's own k dk + 2 b k gs)
                mv[a][r] = gmo ? av[r] : b * kt * vd;
                oq[a][r] = dq;
                ok[a][r] = dk;
            }
            // phi_t = phi_{-1} + sum_{j<=t} av_j - sum_{j<t} au_j, over the 16 tokens of column c
            float ia[4], eu[4];
            float sa = 0.f, su = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                eu[r] = su;
                sa += av[r]; su += au[r];
                ia[r] = sa;
            }
            // exclusive prefix over the four lane groups (t blocks of 4)
            float pa = 0.f, pu = 0.f;
            {
                const float a1 = __shfl(sa, (lane - 16) & 63), u1 = __shfl(su, (lane - 16) & 63);
                const float a2 = __shfl(sa, (lane - 32) & 63), u2 = __shfl(su, (lane - 32) & 63);
                const float a3 = __shfl(sa, (lane - 48) & 63), u3 = __shfl(su, (lane - 48) & 63);
                if (g4 >= 1) { pa += a1; pu += u1; }
                if (g4 >= 2) { pa += a2; pu += u2; }
                if (g4 >= 3) { pa += a3; pu += u3; }
            }
            const float ph0 = sm.phi0[c];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float dl = ph0 + pa + ia[r] - (pu + eu[r]) - mv[a][r];
                if (p.scalar) dla_s[r] += dl;
                od[a][r] = dl;
            }
        }
        if (p.scalar) {
#pragma unroll
            for (int r = 0; r < 4; ++r) dla_s[r] = row_sum16(dla_s[r]);
            if (r16 == 0)
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.red[2][w][4 * g4 + r] = dla_s[r];
            lds_barrier();
            if (tid < 16 && tid < nrow) {
                float dl = 0.f;
#pragma unroll
                for (int u = 0; u < GW; ++u) dl += sm.red[2][u][tid];
                p.dla[(t0 + tid) * p.H + h] = dl;
            }
        }
        // this step's dead kept slot takes the stores of rows past the end, so that
        // every path issues the same stores (and a later wait can count them)
        MT* dummy = kS(sg, 0, 0);
        if (sg > 0) {
            lds_barrier();
            commit(true);
            if (sg > 1) issue(sg - 2, true);
            load_kept(sg - 1);
        }
#pragma unroll
        for (int a = 0; a < CBW; ++a) {
            const int cb = w + GW * a;
            if (cb >= NCB) continue;
            const int c = cb * 16 + r16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g4 + r;
                const bool live = t < nrow;
                const int64_t o = ((t0 + (live ? t : 0)) * p.H + h) * (int64_t)DK + c;
                *(live ? dqg + o : dummy) = from_f32<MT>(oq[a][r]);
                *(live ? dkg + o : dummy) = from_f32<MT>(ok[a][r]);
                *(live && !p.scalar ? p.dla + o : reinterpret_cast<float*>(dummy)) = od[a][r];
            }
        }
    }
}

template <typename MT, int DK>
hipError_t ops_dispatch(const BwdParams& p, int64_t units, int nsub_max, hipStream_t st) {
    hipLaunchKernelGGL((kda_bwd_ops_kernel<MT, DK>), dim3((unsigned)nsub_max, (unsigned)units), dim3(64), 0, st, p);
    return hipGetLastError();
}
template <typename MT, int DK, int DVS>
hipError_t scan_dispatch(const BwdParams& p, int64_t units, int dv, hipStream_t st) {
    const int64_t nitems = (int64_t)(dv / DVS) * units;
    const int64_t nblk = (nitems + 7) / 8 * 8;
    hipLaunchKernelGGL((kda_bwd_scan_kernel<MT, DK, DVS>), dim3((unsigned)nblk), dim3(256), 0, st, p, dv, (int)nitems);
    return hipGetLastError();
}
template <int DK>
hipError_t walk_dispatch(const BwdParams& p, int64_t units, int dv, hipStream_t st) {
    const int64_t nitems = (int64_t)(dv / WalkCfg<DK>::DVS) * units;
    const int64_t nblk = (nitems + 7) / 8 * 8;
    hipLaunchKernelGGL((kda_bwd_walk_kernel<DK>), dim3((unsigned)nblk), dim3(WalkCfg<DK>::NT), 0, st, p, dv,
                       (int)nitems);
    return hipGetLastError();
}
template <typename MT, int DK, int DV>
hipError_t grad_dispatch(const BwdParams& p, int64_t units, int nch_max, hipStream_t st) {
    const size_t sm = sizeof(GradSmem<MT, DK, DV>);
    static_assert(sizeof(GradSmem<MT, DK, DV>) <= 160 * 1024, "gradient pass LDS");
    auto kern = kda_bwd_grad_kernel<MT, DK, DV>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nch_max, (unsigned)units), dim3(64 * GW), sm, st, p);
    return hipGetLastError();
}

template <typename MT, int DK, int DV>
hipError_t run_all(const BwdLaunch& a, const BwdParams& p, hipStream_t st) {
    hipError_t e = hipSuccess;
    if (a.nsub_max > 0) e = ops_dispatch<MT, DK>(p, a.units, a.nsub_max, st);
    if (e != hipSuccess) return e;
    // the reverse walk (also writes dS0 of empty sequences)
    if constexpr (sizeof(MT) == 2) {
        static_assert(DV % WalkCfg<DK>::DVS == 0, "bf16 value widths are multiples of 32");
        e = walk_dispatch<DK>(p, a.units, DV, st);
    } else {
        constexpr int DVS = DV >= 32 ? 32 : DV;
        e = scan_dispatch<MT, DK, DVS>(p, a.units, DV, st);
    }
    if (e != hipSuccess || a.nch_max == 0) return e;
    return grad_dispatch<MT, DK, DV>(p, a.units, a.nch_max, st);
}

}  // namespace

int bwd_block_bytes(int dtype, int dk) {
    if (dtype == 1) {
        if (dk == 32) return OpBlock<bf16, 32>::BYTES;
        if (dk == 64) return OpBlock<bf16, 64>::BYTES;
        if (dk == 128) return OpBlock<bf16, 128>::BYTES;
    } else if (dtype == 0) {
        if (dk == 16) return OpBlock<float, 16>::BYTES;
        if (dk == 32) return OpBlock<float, 32>::BYTES;
        if (dk == 64) return OpBlock<float, 64>::BYTES;
    }
    return 0;
}

int64_t bwd_scratch_bytes(int dtype, int dk, int dv) {
    const int64_t s = dtype == 1 ? 2 : 4;
    return (int64_t)(CHB / SC) * ((int64_t)dk * dv + 2 * 16 * dv) * s;
}

// Compiled (dk, dv): bf16 with dk, dv in {32, 64, 128} and dk, dv at most a
// factor 2 apart; fp32 with dk, dv in {16, 32, 64}, likewise.
bool bwd_supported(int dtype, int dk, int dv) {
    const bool near = dk == dv || dk == 2 * dv || dv == 2 * dk;
    if (dtype == 1) return (dk == 32 || dk == 64 || dk == 128) && (dv == 32 || dv == 64 || dv == 128) && near;
    if (dtype == 0) return (dk == 16 || dk == 32 || dk == 64) && (dv == 16 || dv == 32 || dv == 64) && near;
    return false;
}

hipError_t launch_bwd(const BwdLaunch& a, hipStream_t st) {
    BwdParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.log_a = a.log_a; p.beta = a.beta; p.S0 = a.S0;
    p.cu = a.cu_seqlens; p.eq_len = a.eq_len; p.dO = a.dO; p.dST = a.dST;
    p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dla = a.dlog_a; p.dbeta = a.dbeta; p.dS0 = a.dS0;
    p.snap = a.snap; p.snap_rows = a.snap_rows; p.ops = static_cast<uint8_t*>(a.ops); p.xbuf = a.xbuf; p.scr = a.scr;
    p.H = a.num_heads; p.scalar = a.scalar; p.split = 0; p.gmo = a.order ? 1 : 0;
    if (a.dtype == 1) {
        if (a.kdim == 128 && a.vdim == 128) return run_all<bf16, 128, 128>(a, p, st);
        if (a.kdim == 128 && a.vdim == 64) return run_all<bf16, 128, 64>(a, p, st);
        if (a.kdim == 64 && a.vdim == 128) return run_all<bf16, 64, 128>(a, p, st);
        if (a.kdim == 64 && a.vdim == 64) return run_all<bf16, 64, 64>(a, p, st);
        if (a.kdim == 64 && a.vdim == 32) return run_all<bf16, 64, 32>(a, p, st);
        if (a.kdim == 32 && a.vdim == 64) return run_all<bf16, 32, 64>(a, p, st);
        if (a.kdim == 32 && a.vdim == 32) return run_all<bf16, 32, 32>(a, p, st);
    } else {
        if (a.kdim == 64 && a.vdim == 64) return run_all<float, 64, 64>(a, p, st);
        if (a.kdim == 64 && a.vdim == 32) return run_all<float, 64, 32>(a, p, st);
        if (a.kdim == 32 && a.vdim == 64) return run_all<float, 32, 64>(a, p, st);
        if (a.kdim == 32 && a.vdim == 32) return run_all<float, 32, 32>(a, p, st);
        if (a.kdim == 32 && a.vdim == 16) return run_all<float, 32, 16>(a, p, st);
        if (a.kdim == 16 && a.vdim == 32) return run_all<float, 16, 32>(a, p, st);
        if (a.kdim == 16 && a.vdim == 16) return run_all<float, 16, 16>(a, p, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
