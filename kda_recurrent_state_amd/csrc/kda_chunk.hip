// kda_chunk.hip -- chunkwise (WY) prefill of the KDA state layer on gfx950.
//
// Same map as the token recurrence of the KDA row of the table on page "The
// argument, in one page" ("Everything, in one table"), reorganised as that
// table's "Chunkwise / WY" row describes: chunks of C tokens, one C x C
// triangular solve per chunk, everything else dense products on the matrix
// cores.  Per chunk, with g_t the running sum of log a inside the chunk, the
// state normalised by Diag(e^{-g}) gives (k_t, q_t rows; b = beta):
//
//   Kb = K e^{g_{t-1}}, Kc = K e^{-g_{t-1}}, Kt = K e^{-g_t}, Qb = Q e^{g_t}
//   A  = strict_lower(diag(b) Kb Kc^T),  L = strict_lower(Kb Kt^T)
//   P1 = lower(Qb Kc^T),                 P2 = lower(Qb Kt^T)
//   T  = (I + A)^-1,  Tb = T diag(b)
//   E  = -Tb (Kb S + L (b V))             (the chunk's erase coefficients)
//   O  = Qb S + P2 (b V) + P1 E
//   S <- Diag(e^{g_C}) S + (Kt e^{g_C})^T (b V) + (Kc e^{g_C})^T E
//
// Only the solve and the E-dependent terms wait for T; Z = Kb S + L (b V), the
// first two terms of O and of the state update are formed while one wavefront
// inverts (I + A).
//
// The per-channel decay ("a gate per channel", page "The efficiency lineage",
// item 10) spans hundreds of nats over a chunk, which is the numerical-range
// problem the KDA row of the table mentions.  Factors are therefore split
// around references placed per 16-token sub-block: blocks on the diagonal of
// a C x C product use the sub-block's mid-point (row and column factors stay
// within e^{+-8 max|log a|}, upper-triangle overflow is discarded by select),
// and a block pair (bt > bi) additionally scales the row factor by
// e^{mu_bt - mu_bi} <= 1.  The state-side operands are referenced to the chunk
// start or end, where every factor is <= 1.  This split is exact to ~2^-30 while
// every valid token of the chunk has log2 a >= STEEP_LOG2 (kda_chunk_common.hpp);
// a chunk with a steeper token forms the chunk-referenced operands with one
// exponential each and its Gram products by exact_gram, which is exact for any
// decay (phases P2 and P3 below).
//
// The decay-first ordering (ORD1: S <- (I - b k^T k) Diag(a) S + b k^T v,
// per-channel decay only) has the same structure with Kb = K e^{g_t} and no
// write outside the erase term:
//   A  = strict_lower(diag(b) Kb Kt^T),  P2 = lower(Qb Kt^T),  Tb as above
//   E  = -Tb (Kb S - V)   (= the chunk's new values, T diag(b) (V - Kb S))
//   O  = Qb S + P2 E
//   S <- Diag(e^{g_C}) S + (Kt e^{g_C})^T E
// so L, P1, Kc and the (b V) terms drop out.
//
// Work decomposition: one workgroup (8 wavefronts) per (sequence, head,
// dv-slice of width DVS).  The workgroup walks its sequence chunk by chunk,
// loading the next chunk's inputs into registers while it computes the
// current one; the fp32 state slice [DK x DVS] lives in matrix-core
// accumulators across the walk.  Inputs are read from HBM once per slice
// (slices of one head are placed on one XCD so they share its L2) and o is
// written once.  Per chunk there are six phases separated by LDS-only
// barriers:
//   P1  prefetched inputs -> decay sums per 4-token group, (b V)^T; prefetch next
//   P2  decay factors and all eight gated operands
//   P3  the four Gram products
//   P4  wavefront 0: (I + A)^-1;  the others: Z, first O terms, Gamma S + Kt^T bV
//   P5  E = -Tb Z
//   P6  O += P1 E, S += Kc^T E
#include "kda_chunk_common.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename T, int DK, int DVS, int C>
struct ChunkCfg {
    static constexpr int NT = 512, NW = NT / WAVE;     // 8 wavefronts, 2 per SIMD
    static constexpr int NB = C / 16;                  // 16-token sub-blocks
    static constexpr int NPAIR = NB * (NB - 1) / 2;    // off-diagonal block pairs
    static constexpr int NBP = NB * (NB + 1) / 2;      // block pairs incl. diagonal
    static constexpr int PAD = 16 / sizeof(T);         // one 16-byte pad per row
    static constexpr int LDK = DK + PAD;               // rows with dk contiguous
    static constexpr int LDC = C + PAD;                // rows with tokens contiguous
    static constexpr int LDA = C + 4;                  // fp32 C x C matrices
    static constexpr int NCP = DK / 2;                 // channel pairs
    static constexpr int NU = NCP * (C / 4);           // 4 tokens x 2 channels units
    static constexpr int UPT = (NU + NT - 1) / NT;     // units per thread
    static constexpr int NUV = (DVS / 4) * (C / 4);    // 4 tokens x 4 value columns units
    static constexpr int UVPT = (NUV + NT - 1) / NT;
    static constexpr int NST = (DK / 16) * (DVS / 16); // state tiles
    static constexpr int STPW = (NST + NW - 1) / NW;   // state tiles per wavefront
    static constexpr int NOT = (DVS / 16) * (C / 16);  // output (and Z, E) tiles
    static constexpr int OTPW = (NOT + NW - 1) / NW;
    static constexpr int OTPWX = (NOT + NW - 2) / (NW - 1);  // per wavefront 1..NW-1
};

// LDS bytes of a configuration with Kbar and Qbar in rows of their own.
template <typename T, int DK, int DVS, int C>
constexpr size_t chunk_lds_full() {
    typedef ChunkCfg<T, DK, DVS, C> G;
    auto a16 = [](size_t n) { return (n + 15) / 16 * 16; };
    return a16(6 * C * G::LDK * sizeof(T)) + a16(DVS * G::LDK * sizeof(T)) +
           a16(2 * (size_t)prows<DK>() * G::LDC * sizeof(T)) + a16((size_t)prows<DVS>() * G::LDC * sizeof(T)) +
           a16(2 * DVS * G::LDC * sizeof(T)) + a16(4 * C * G::LDC * sizeof(T)) + 4 * C * G::LDA + 4 * 2 * G::NB * 256 +
           4 * (C / 4) * DK + 4 * (G::NPAIR > 0 ? G::NPAIR : 1) * DK + 4 * DK + 4 * C + 4 * G::NW;
}
// Configurations that would not fit a compute unit (fp32 at dk = 128) keep Kbar
// and Qbar over the Gram columns Kce and Kci instead: they are formed with the
// other gated operands but held in registers until the Gram products have read
// the columns, and written there before the state products read them.
template <typename T, int DK, int DVS, int C>
constexpr bool chunk_alias_bar() { return chunk_lds_full<T, DK, DVS, C>() > 160 * 1024; }

template <typename T, int DK, int DVS, int C>
struct ChunkLds {
    typedef ChunkCfg<T, DK, DVS, C> G;
    static constexpr bool AB = chunk_alias_bar<T, DK, DVS, C>();
    static constexpr int NBAR = AB ? 16 / (int)sizeof(T) : C * G::LDK;  // own rows of Kbar, Qbar
    alignas(16) T Kr[C * G::LDK];    // K e^{g_{t-1} - mid}   Gram rows (A, L)
    alignas(16) T Qr[C * G::LDK];    // Q e^{g_t - mid}       Gram rows (P1, P2)
    alignas(16) T Kce[C * G::LDK];   // K e^{mid - g_{t-1}}   Gram columns (A, P1); Kbar when AB
    alignas(16) T Kci[C * G::LDK];   // K e^{mid - g_t}       Gram columns (L, P2); Qbar when AB
    alignas(16) T Kbar_own[NBAR];    // K e^{g_{t-1}}
    alignas(16) T Qbar_own[NBAR];    // Q e^{g_t}
    __device__ T* Kbar() { return AB ? Kce : Kbar_own; }
    __device__ T* Qbar() { return AB ? Kci : Qbar_own; }
    alignas(16) T ST[DVS * G::LDK];  // state slice at the chunk start, [j][c]
    alignas(16) T KccT[prows<DK>() * G::LDC];  // (K e^{g_C - g_{t-1}})^T, plane rows
    alignas(16) T KtcT[prows<DK>() * G::LDC];  // (K e^{g_C - g_t})^T, plane rows
    alignas(16) T VT[prows<DVS>() * G::LDC];   // (b V)^T, plane rows
    alignas(16) T ZT[DVS * G::LDC];  // (Kbar S + L b V)^T
    alignas(16) T ET[DVS * G::LDC];  // E^T
    alignas(16) T L[C * G::LDC];
    alignas(16) T P1[C * G::LDC];
    alignas(16) T P2[C * G::LDC];
    alignas(16) T Tb[C * G::LDC];
    alignas(16) float A[C * G::LDA];           // diag(b) strict_lower(Kb Kc^T), fp32
    alignas(16) float X[2 * G::NB * 256];      // panel exchange of the blocked solve
    alignas(16) float grp[(C / 4) * DK];       // per 4-token group: summed log2 decay
    alignas(16) float F[(G::NPAIR > 0 ? G::NPAIR : 1) * DK];  // e^{mu_bt - mu_bi}
    alignas(16) float gam[DK];                 // e^{g_C}
    alignas(16) float beta[C];
    int steep[G::NW];                          // per wavefront: a token below STEEP_LOG2
};

template <typename T, int DK, int DVS, int C>
constexpr size_t chunk_lds_bytes() { return sizeof(ChunkLds<T, DK, DVS, C>); }

struct ChunkParams {
    const void* q;
    const void* k;
    const void* v;
    const float* log_a;
    const float* beta;
    const float* S0;
    const int32_t* cu;
    void* o;
    float* ST;
    int H, DV, split, xcd_group;
    int64_t eq_len;  // used when cu is null
    float* snap;     // state snapshots [rows][H][DK][DV], or null
    int64_t snap_rows;
    int snap_every;  // tokens between snapshots (a multiple of C)
};

// Input prologue switches (read by the PRO instances only) and its clip of log2 a.
struct ChunkPro {
    int nk, bl, la;
    float lo2;
};

// Raw inputs of one 4-token x 2-channel unit, held in registers one chunk ahead.
template <typename T>
struct UnitIn {
    typename Vec2<T>::type q[4], k[4];
    f32x2 la[4];
};
template <typename T>
struct ValIn {
    typename Vec4<T>::type v[4];
    float b[4];
};

// Value units are spread over the wavefronts (v is narrower than k).
template <int NW>
__device__ __forceinline__ int value_unit(int tid, int u, int nt) { return (tid & 63) * NW + (tid >> 6) + nt * u; }

template <typename T, int DK, int DVS, int C, bool SCALAR>
__device__ __forceinline__ void load_chunk(const ChunkParams& p, const T* gq, const T* gk, const T* gv,
                                           int64_t t0, int Lc, int h, int dv0, int tid,
                                           UnitIn<T> (&ui)[ChunkCfg<T, DK, DVS, C>::UPT],
                                           ValIn<T> (&vi)[ChunkCfg<T, DK, DVS, C>::UVPT]) {
    typedef ChunkCfg<T, DK, DVS, C> G;
    const int H = p.H, DV = p.DV;
    const int64_t r0 = t0 * H + h;  // row of the chunk's first token
#pragma unroll
    for (int u = 0; u < G::UPT; ++u) {
        const int uu = tid + G::NT * u;
        if (uu < G::NU) {
            int c, tg;
            unit_of<G::NCP>(uu, c, tg);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // rows past the chunk's end re-read its last row; beta and log_a are
                // masked at use, which makes the other values irrelevant
                const int64_t row = r0 + (int64_t)min(4 * tg + i, Lc - 1) * H;
                ui[u].q[i] = *reinterpret_cast<const typename Vec2<T>::type*>(gq + row * DK + c);
                ui[u].k[i] = *reinterpret_cast<const typename Vec2<T>::type*>(gk + row * DK + c);
                if (SCALAR) {
                    const float x = p.log_a[row];
                    ui[u].la[i] = f32x2{x, x};
                } else {
                    ui[u].la[i] = *reinterpret_cast<const f32x2*>(p.log_a + row * DK + c);
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < G::UVPT; ++u) {
        const int uv = value_unit<G::NW>(tid, u, G::NT);
        if (uv < G::NUV) {
            const int j = 4 * (uv % (DVS / 4)), tg = uv / (DVS / 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = r0 + (int64_t)min(4 * tg + i, Lc - 1) * H;
                vi[u].v[i] = *reinterpret_cast<const typename Vec4<T>::type*>(gv + row * DV + dv0 + j);
                vi[u].b[i] = p.beta[row];
            }
        }
    }
}

// Input prologue: the sum of x over the lanes that hold one token's key row
// (32 lanes for dk >= 64, whose rows a half-wavefront covers in one or two
// pieces; dk / 2 consecutive lanes below), in a fixed order.  Every lane of a
// wavefront runs it.
template <int NCP>
__device__ __forceinline__ float key_row_sum(float x) {
    constexpr int GS = NCP >= 32 ? 32 : NCP;
#pragma unroll
    for (int m = 1; m < GS; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// log2 a of a unit's two channels as loaded (x: log a, or with the prologue's
// log_a_raw the pre-activation of log a = max(-softplus(x), lo))
// (used by the PRO instances; the others scale by log2 e in place)
__device__ __forceinline__ f32x2 unit_log2_a(const ChunkPro& pr, f32x2 x) {
    if (pr.la) return f32x2{prologue_log2_a(x[0], pr.lo2), prologue_log2_a(x[1], pr.lo2)};
    return x * LOG2E;
}

// Prologue scale of token t's key, 1 / sqrt(|k_t|^2 + eps), from the squared
// norms P1 left in knrm (two row pieces at dk = 128), or 1 without normalisation
template <int C, int DK>
__device__ __forceinline__ float key_scale(const ChunkPro& pr, const float* knrm, int t) {
    if (!pr.nk) return 1.f;
    float x = knrm[t];
    if (DK >= 128) x += knrm[C + t];
    return rsqrtf(x + PROLOGUE_EPS);
}

// P2 of a chunk with a token below STEEP_LOG2: the chunk-referenced operands
// Kbar, Qbar, Kcc^T, Ktc^T with one exponential each, from running sums of log2 a
// referenced to the chunk start (prefixes: group sums before the unit's group,
// then its own decays) or end (suffixes), every exponent a run of consecutive
// decays; the raw rows go to Kr, Qr and the log2 decays ([C][DK] fp32) over Kce
// and Kci for exact_gram.  e^{g_C} comes from the block loop after it, as in the
// factored path.  The unit's decays are read again from memory (rare path; the
// walk does not keep them in registers).
template <typename T, int DK, int DVS, int C, bool SCALAR, bool ORD1, bool PRO>
__device__ __forceinline__ void chunk_steep_operands(const ChunkParams& p, const ChunkPro& pr,
                                                     ChunkLds<T, DK, DVS, C>& s, int64_t t0,
                                                     int Lc, int h, int tid,
                                                     const typename Vec2<T>::type (&qraw)[ChunkCfg<T, DK, DVS, C>::UPT][4],
                                                     const typename Vec2<T>::type (&kraw)[ChunkCfg<T, DK, DVS, C>::UPT][4],
                                                     f32x2 (&kbk)[ChunkCfg<T, DK, DVS, C>::UPT][4],
                                                     f32x2 (&qbk)[ChunkCfg<T, DK, DVS, C>::UPT][4]) {
    typedef ChunkCfg<T, DK, DVS, C> G;
    constexpr int NT = G::NT, LDK = G::LDK, LDC = G::LDC;
    constexpr bool AB = ChunkLds<T, DK, DVS, C>::AB;
    float* LA = reinterpret_cast<float*>(s.Kce);
    static_assert(sizeof(s.Kce) + sizeof(s.Kci) >= C * DK * sizeof(float), "log2 decays fit over Kce, Kci");
    auto ex2v = [](f32x2 x) { return f32x2{__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1])}; };
#pragma unroll
    for (int u = 0; u < G::UPT; ++u) {
        const int uu = tid + NT * u;
        if (uu < G::NU) {
            int c, tg;
            unit_of<G::NCP>(uu, c, tg);
            f32x2 l2[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = (t0 + min(4 * tg + i, Lc - 1)) * p.H + h;
                const f32x2 x = SCALAR ? f32x2{p.log_a[row], p.log_a[row]}
                                       : *reinterpret_cast<const f32x2*>(p.log_a + row * DK + c);
                l2[i] = 4 * tg + i < Lc ? (PRO ? unit_log2_a(pr, x) : x * LOG2E) : f32x2{0.f, 0.f};
            }
            f32x2 pre = {0.f, 0.f}, suf = {0.f, 0.f};
#pragma unroll
            for (int g = 0; g < C / 4; ++g) {
                const f32x2 x = *reinterpret_cast<const f32x2*>(&s.grp[g * DK + c]);
                if (g < tg) pre += x;
                if (g > tg) suf += x;
            }
            f32x2 sx[4];  // g_C - g_t
            {
                f32x2 run = suf;
#pragma unroll
                for (int i = 3; i >= 0; --i) {
                    sx[i] = run;
                    run += l2[i];
                }
            }
            f32x2 kc[4], kt[4];
            f32x2 gp = pre;  // g_{t-1}
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * tg + i;
                f32x2 k = f32x2{Vec2<T>::lo(kraw[u][i]), Vec2<T>::hi(kraw[u][i])};
                if constexpr (PRO) k = k * key_scale<C, DK>(pr, s.X, t);
                const f32x2 q = f32x2{Vec2<T>::lo(qraw[u][i]), Vec2<T>::hi(qraw[u][i])};
                const f32x2 g = gp + l2[i];
                const f32x2 kb = k * ex2v(ORD1 ? g : gp), qb = q * ex2v(g);
                kc[i] = k * ex2v(sx[i] + l2[i]);
                kt[i] = k * ex2v(sx[i]);
                if (AB) {
                    kbk[u][i] = kb;
                    qbk[u][i] = qb;
                } else {
                    store2(&s.Kbar()[t * LDK + c], kb[0], kb[1]);
                    store2(&s.Qbar()[t * LDK + c], qb[0], qb[1]);
                }
                store2(&s.Kr[t * LDK + c], k[0], k[1]);
                store2(&s.Qr[t * LDK + c], q[0], q[1]);
                *reinterpret_cast<f32x2*>(&LA[t * DK + c]) = l2[i];
                gp = g;
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                if (!ORD1)
                    store4(&s.KccT[prow<DK>(c + e) * LDC + 4 * tg], f32x4{kc[0][e], kc[1][e], kc[2][e], kc[3][e]});
                store4(&s.KtcT[prow<DK>(c + e) * LDC + 4 * tg], f32x4{kt[0][e], kt[1][e], kt[2][e], kt[3][e]});
            }
        }
    }
}

// SNAP: the call asks for state snapshots (a separate instantiation: the
// snapshot stores would otherwise cost the plain walk registers).  PRO: the
// call has an input prologue (also separate; its switches are read at run time):
// beta and log a are transformed as P1 takes them from the prefetch registers,
// and each token's key row is scaled by 1 / sqrt(|k|^2 + eps) where P2 forms the
// gated operands, the squared norm summed over the lanes of the row and, at
// dk = 128, over the two wavefronts that share it (through LDS).
template <typename T, int DK, int DVS, int C, bool SCALAR, bool ORD1, bool SNAP, bool PRO>
__global__ void __launch_bounds__(512) kda_chunk_kernel(ChunkParams p, ChunkPro pr) {
    typedef ChunkCfg<T, DK, DVS, C> G;
    typedef Mma<T> M;
    constexpr int NT = G::NT, NW = G::NW, NB = G::NB, LDK = G::LDK, LDC = G::LDC, LDA = G::LDA;
    typedef ChunkLds<T, DK, DVS, C> SL;
    __shared__ SL s;

    const T* __restrict__ gq = static_cast<const T*>(p.q);
    const T* __restrict__ gk = static_cast<const T*>(p.k);
    const T* __restrict__ gv = static_cast<const T*>(p.v);
    T* __restrict__ go = static_cast<T*>(p.o);
    const int H = p.H, DV = p.DV;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lrow = lane & 15, lgrp = lane >> 4;

    // workgroup -> (sequence, head, slice); slices of one head on one XCD
    int item = blockIdx.x;
    if (p.xcd_group) {
        const int per = gridDim.x / 8;
        item = (blockIdx.x % 8) * per + blockIdx.x / 8;
    }
    const int unit = item / p.split, slice = item % p.split;
    const int n = unit / H, h = unit % H;
    const int dv0 = slice * DVS;
    int64_t tb, te;
    if (p.cu) { tb = p.cu[n]; te = p.cu[n + 1]; }
    else { tb = (int64_t)n * p.eq_len; te = tb + p.eq_len; }

    // upper blocks of the masked C x C products are never written: zero once
    for (int e = tid; e < C * LDC; e += NT) {
        s.L[e] = from_f32<T>(0.f); s.P1[e] = from_f32<T>(0.f); s.P2[e] = from_f32<T>(0.f);
        s.Tb[e] = from_f32<T>(0.f);
    }

    // state slice in accumulators: tile ix = wv + NW * i -> (mi, ni); copy in LDS
    f32x4 acc[G::STPW];
    const int64_t sbase = ((int64_t)n * H + h) * DK * DV + dv0;
#pragma unroll
    for (int i = 0; i < G::STPW; ++i) {
        const int ix = wv + NW * i;
        acc[i] = zero4();
        if (ix < G::NST) {
            const int mi = ix / (DVS / 16), ni = ix % (DVS / 16);
            if (p.S0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[i][r] = p.S0[sbase + (int64_t)(16 * mi + 4 * lgrp + r) * DV + 16 * ni + lrow];
            }
            store4(&s.ST[(16 * ni + lrow) * LDK + 16 * mi + 4 * lgrp], acc[i]);
        }
    }

    // snapshots: the state after every snap_every tokens goes to row
    // snap0 + (tokens / snap_every) - 1; snap_cd counts the chunks to the next
    int64_t snap0 = 0;
    int snap_ec = 1, snap_cd = 0;
    if (SNAP) {
        snap0 = snapshots_before(p.cu, p.eq_len, n, p.snap_every);
        snap_ec = p.snap_every / C;
        snap_cd = snap_ec;
    }

    UnitIn<T> ui[G::UPT];
    ValIn<T> vi[G::UVPT];
    if (tb < te)
        load_chunk<T, DK, DVS, C, SCALAR>(p, gq, gk, gv, tb, (int)((te - tb) < C ? (te - tb) : C), h, dv0,
                                          tid, ui, vi);

    // outputs of a chunk are stored at the start of the next iteration, after
    // the wait for the prefetched inputs (stores share the vector-memory counter)
    f32x4 opend[G::OTPWX];
    int64_t t0_prev = tb;
    int Lc_prev = 0;
    auto store_o = [&]() {
        if (wv == 0) return;
#pragma unroll
        for (int i = 0; i < G::OTPWX; ++i) {
            const int w = (wv - 1) + (NW - 1) * i;
            if (w < G::NOT) {
                const int mj = w / (C / 16), nt = w % (C / 16);
                const int t = 16 * nt + lrow;
                if (t < Lc_prev) store4(go + ((t0_prev + t) * H + h) * DV + dv0 + 16 * mj + 4 * lgrp, opend[i]);
            }
        }
    };

    for (int64_t t0 = tb; t0 < te; t0 += C) {
        const int Lc = (int)((te - t0) < C ? (te - t0) : C);

        // ---- P1: decay sums per 4-token group, (b V)^T, beta; prefetch next chunk ---
        f32x2 lam[G::UPT][4];
        typename Vec2<T>::type qraw[G::UPT][4], kraw[G::UPT][4];
        bool steep = false;
#pragma unroll
        for (int u = 0; u < G::UPT; ++u) {
            const int uu = tid + NT * u;
            if (uu < G::NU) {
                int c, tg;
                unit_of<G::NCP>(uu, c, tg);
                f32x2 run = f32x2{0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x2 l2 = (4 * tg + i < Lc) ? (PRO ? unit_log2_a(pr, ui[u].la[i]) : ui[u].la[i] * LOG2E) : f32x2{0.f, 0.f};
                    steep |= l2[0] < STEEP_LOG2 || l2[1] < STEEP_LOG2;
                    run += l2;
                    lam[u][i] = run;
                    qraw[u][i] = ui[u].q[i];
                    kraw[u][i] = ui[u].k[i];
                }
                *reinterpret_cast<f32x2*>(&s.grp[tg * DK + c]) = run;
            }
        }
        if (PRO && pr.nk) {
            // squared key norms: per token, the sum over its row's lanes, stored
            // by the row piece's first lane (a piece per wavefront half at dk = 128)
            float* knrm = s.X;  // the solve's exchange buffer is free until P4
#pragma unroll
            for (int u = 0; u < G::UPT; ++u) {
                const int uu = tid + NT * u;
                int c = 0, tg = 0;
                if (uu < G::NU) unit_of<G::NCP>(uu, c, tg);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = 0.f;
                    if (uu < G::NU) {
                        const float k0 = Vec2<T>::lo(kraw[u][i]), k1 = Vec2<T>::hi(kraw[u][i]);
                        x = k0 * k0 + k1 * k1;
                    }
                    x = key_row_sum<G::NCP>(x);
                    constexpr int GS = G::NCP >= 32 ? 32 : G::NCP;
                    if (uu < G::NU && (uu % GS) == 0) {
                        const int half = G::NCP >= 32 ? (uu >> 6) % (G::NCP / 32) : 0;
                        knrm[half * C + 4 * tg + i] = x;
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < G::UVPT; ++u) {
            const int uv = value_unit<NW>(tid, u, NT);
            if (uv < G::NUV) {
                const int j = 4 * (uv % (DVS / 4)), tg = uv / (DVS / 4);
                f32x4 vals[4], bb;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bb[i] = 4 * tg + i < Lc ? (PRO && pr.bl ? prologue_beta(vi[u].b[i]) : vi[u].b[i]) : 0.f;
                    // (b V)^T; ORD1: V^T, padded rows zero
                    vals[i] = (ORD1 ? (4 * tg + i < Lc ? 1.f : 0.f) : bb[i]) * Vec4<T>::to_f32(vi[u].v[i]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    store4(&s.VT[prow<DVS>(j + e) * LDC + 4 * tg], f32x4{vals[0][e], vals[1][e], vals[2][e], vals[3][e]});
                if (j == 0) *reinterpret_cast<f32x4*>(&s.beta[4 * tg]) = bb;
            }
        }
        {
            const bool ws = wave_any(steep);
            if (lane == 0) s.steep[wv] = ws;
        }
        if (Lc_prev > 0) store_o();
        t0_prev = t0;
        Lc_prev = Lc;
        {
            const int64_t t1 = t0 + C;
            if (t1 < te)
                load_chunk<T, DK, DVS, C, SCALAR>(p, gq, gk, gv, t1, (int)((te - t1) < C ? (te - t1) : C), h,
                                                  dv0, tid, ui, vi);
        }
        lds_barrier();

        // ---- P2: decay factors and all gated operands ------------------------------
        // rin = e^{g_t - mid}, rex = e^{g_{t-1} - mid}, cin, cex their reciprocals,
        // em = e^{mu_b}, ec = e^{g_C - mu_b} (mu_b the mid-point of the sub-block).
        // Exponents are clamped to the fp32 range so no factor is inf or zero.
        int steep_any = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) steep_any |= s.steep[w];
        const bool steep_chunk = __builtin_amdgcn_readfirstlane(steep_any) != 0;
        // Kbar, Qbar of this thread's units, when they wait for the Gram columns' rows
        f32x2 kbk[SL::AB ? G::UPT : 1][4], qbk[SL::AB ? G::UPT : 1][4];
        if (steep_chunk) {
            chunk_steep_operands<T, DK, DVS, C, SCALAR, ORD1, PRO>(p, pr, s, t0, Lc, h, tid, qraw, kraw, kbk, qbk);
        } else {
#pragma unroll
        for (int u = 0; u < G::UPT; ++u) {
            const int uu = tid + NT * u;
            if (uu < G::NU) {
                int c, tg;
                unit_of<G::NCP>(uu, c, tg);
                const int b = tg / 4, gib = tg % 4;
                f32x2 off = {0.f, 0.f}, rho = {0.f, 0.f}, tot = {0.f, 0.f}, mid = {0.f, 0.f};
#pragma unroll
                for (int g = 0; g < C / 4; ++g) {
                    const f32x2 x = *reinterpret_cast<const f32x2*>(&s.grp[g * DK + c]);
                    tot += x;
                    if (g < 4 * b) rho += x;
                    if (g >= 4 * b && g < 4 * b + gib) off += x;
                    if (g == 4 * b || g == 4 * b + 1) mid += x;
                }
                f32x2 em, ec, prev, prevc;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    em[e] = __builtin_amdgcn_exp2f(__builtin_amdgcn_fmed3f(rho[e] + mid[e], -126.f, 0.f));
                    ec[e] = __builtin_amdgcn_exp2f(__builtin_amdgcn_fmed3f(tot[e] - rho[e] - mid[e], -126.f, 0.f));
                    prev[e] = __builtin_amdgcn_exp2f(__builtin_amdgcn_fmed3f(off[e] - mid[e], -126.f, 126.f));
                    prevc[e] = __builtin_amdgcn_rcpf(prev[e]);
                }
                f32x2 kc[4], kt[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 4 * tg + i;
                    f32x2 ri, ci;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        ri[e] = __builtin_amdgcn_exp2f(
                            __builtin_amdgcn_fmed3f(off[e] + lam[u][i][e] - mid[e], -126.f, 126.f));
                        ci[e] = __builtin_amdgcn_rcpf(ri[e]);
                    }
                    f32x2 k = f32x2{Vec2<T>::lo(kraw[u][i]), Vec2<T>::hi(kraw[u][i])};
                    if constexpr (PRO) k = k * key_scale<C, DK>(pr, s.X, t);
                    const f32x2 q = f32x2{Vec2<T>::lo(qraw[u][i]), Vec2<T>::hi(qraw[u][i])};
                    const f32x2 kr = ORD1 ? k * ri : k * prev, qr = q * ri, kce = k * prevc, kci = k * ci;
                    store2(&s.Kr[t * LDK + c], kr[0], kr[1]);
                    store2(&s.Qr[t * LDK + c], qr[0], qr[1]);
                    if (!ORD1) store2(&s.Kce[t * LDK + c], kce[0], kce[1]);
                    store2(&s.Kci[t * LDK + c], kci[0], kci[1]);
                    if (SL::AB) {
                        kbk[u][i] = kr * em;
                        qbk[u][i] = qr * em;
                    } else {
                        store2(&s.Kbar()[t * LDK + c], kr[0] * em[0], kr[1] * em[1]);
                        store2(&s.Qbar()[t * LDK + c], qr[0] * em[0], qr[1] * em[1]);
                    }
                    kc[i] = kce * ec;
                    kt[i] = kci * ec;
                    prev = ri;
                    prevc = ci;
                }
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    if (!ORD1)
                        store4(&s.KccT[prow<DK>(c + e) * LDC + 4 * tg], f32x4{kc[0][e], kc[1][e], kc[2][e], kc[3][e]});
                    store4(&s.KtcT[prow<DK>(c + e) * LDC + 4 * tg], f32x4{kt[0][e], kt[1][e], kt[2][e], kt[3][e]});
                }
            }
        }
        }
        // per (sub-block, channel): e^{mu_bt - mu_bi} for block pairs, e^{g_C}
        for (int e = tid; e < NB * DK; e += NT) {
            const int b = e / DK, c = e % DK;
            float rho[NB + 1], mu[NB];
            rho[0] = 0.f;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                const float g0 = s.grp[(4 * bb) * DK + c], g1 = s.grp[(4 * bb + 1) * DK + c];
                const float g2 = s.grp[(4 * bb + 2) * DK + c], g3 = s.grp[(4 * bb + 3) * DK + c];
                mu[bb] = rho[bb] + g0 + g1;
                rho[bb + 1] = rho[bb] + ((g0 + g1) + (g2 + g3));
            }
            if (b == 0) s.gam[c] = exp2f(rho[NB]);
            for (int bi = 0; bi < b; ++bi) s.F[(b * (b - 1) / 2 + bi) * DK + c] = exp2f(mu[b] - mu[bi]);
        }
        lds_barrier();

        // ---- P3: Gram products: tile w is product w % 4 (0 A, 1 L, 2 P1, 3 P2) of
        //      block pair w / 4, transposed (G^T) so it lands row-major in LDS;
        //      ORD1: A (w even, columns Kt) or P2 (w odd) of block pair w / 2 --------
        constexpr int NG = ORD1 ? 2 : 4;
        if (steep_chunk) {
            exact_gram<T, DK, C, NW, ORD1>(s.Kr, s.Qr, LDK, reinterpret_cast<const float*>(s.Kce), DK, wv, lane,
                                           [&](int t, int i, float av, float lv, float p1v, float p2v) {
                s.A[t * LDA + i] = s.beta[t] * av;
                s.P2[t * LDC + i] = from_f32<T>(p2v);
                if (!ORD1) {
                    s.L[t * LDC + i] = from_f32<T>(lv);
                    s.P1[t * LDC + i] = from_f32<T>(p1v);
                }
            });
        } else
        for (int w = wv; w < NG * G::NBP; w += NW) {
            const int g = ORD1 ? ((w & 1) ? 3 : 0) : w % 4, pr = w / NG;
            int bt = 0;
            while ((bt + 1) * (bt + 2) / 2 <= pr) ++bt;
            const int bi = pr - bt * (bt + 1) / 2;
            const T* rows = (g < 2 ? s.Kr : s.Qr) + (16 * bt + lrow) * LDK;
            const T* cols = ((g & 1) == 0 && !ORD1 ? s.Kce : s.Kci) + (16 * bi + lrow) * LDK;
            constexpr int NK = DK / M::K;
            typename M::frag fr[NK], fc[NK];
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                fr[k] = M::loadr(rows + k * M::K, lane);
                fc[k] = M::loadr(cols + k * M::K, lane);
            }
            if (bt != bi) {
                const float* F = s.F + (bt * (bt - 1) / 2 + bi) * DK + lgrp * M::KPL;
#pragma unroll
                for (int k = 0; k < NK; ++k) fr[k] = M::scale(fr[k], F + k * M::K);
            }
            f32x4 acc_g = zero4();
#pragma unroll
            for (int k = 0; k < NK; ++k) acc_g = M::mma(fc[k], fr[k], acc_g);
            const int t = 16 * bt + lrow, i0 = 16 * bi + 4 * lgrp;
            f32x4 m;
#pragma unroll
            for (int r = 0; r < 4; ++r) m[r] = (g < 2 ? i0 + r < t : i0 + r <= t) ? acc_g[r] : 0.f;
            if (g == 0) *reinterpret_cast<f32x4*>(&s.A[t * LDA + i0]) = s.beta[t] * m;
            else store4(&(g == 1 ? s.L : (g == 2 ? s.P1 : s.P2))[t * LDC + i0], m);
        }
        lds_barrier();
        if constexpr (SL::AB) {
            // the Gram columns are read: Kbar and Qbar take their rows
#pragma unroll
            for (int u = 0; u < G::UPT; ++u) {
                const int uu = tid + NT * u;
                if (uu < G::NU) {
                    int c, tg;
                    unit_of<G::NCP>(uu, c, tg);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 4 * tg + i;
                        store2(&s.Kbar()[t * LDK + c], kbk[u][i][0], kbk[u][i][1]);
                        store2(&s.Qbar()[t * LDK + c], qbk[u][i][0], qbk[u][i][1]);
                    }
                }
            }
            lds_barrier();
        }

        // ---- P4: wavefront 0 inverts (I + A); the others form Z = Kbar S + L (bV),
        //      O^T = S^T Qbar^T + (bV)^T P2^T and Gamma S + Kt^T bV for their tiles ---
        f32x4 oacc[G::OTPWX];
        if (wv == 0) {
            block_inverse<T, C, LDA, LDC>(s.A, s.beta, s.X, s.Tb, lane);
        } else {
#pragma unroll
            for (int i = 0; i < G::OTPWX; ++i) {
                const int w = (wv - 1) + (NW - 1) * i;
                oacc[i] = zero4();
                if (w < G::NOT) {
                    const int mt = w / (DVS / 16), nj = w % (DVS / 16);
                    f32x4 z = tile_mma<T, DK>(s.Kbar() + 16 * mt * LDK, LDK, s.ST + 16 * nj * LDK, LDK, zero4(), lane);
                    if (ORD1)  // Z = Kbar S - V
                        z -= load4(&s.VT[prow<DVS>(16 * nj + lrow) * LDC + 16 * mt + 4 * lgrp]);
                    else
                        z = tile_mma_r<T, C>(s.L + (16 * mt + lrow) * LDC, s.VT + prow<DVS>(16 * nj + lrow) * LDC, z,
                                             lane);
                    store4(&s.ZT[(16 * nj + lrow) * LDC + 16 * mt + 4 * lgrp], z);
                    const int mj = w / (C / 16), nt = w % (C / 16);
                    f32x4 x = tile_mma<T, DK>(s.ST + 16 * mj * LDK, LDK, s.Qbar() + 16 * nt * LDK, LDK, zero4(), lane);
                    oacc[i] = ORD1 ? x
                                   : tile_mma_r<T, C>(s.VT + prow<DVS>(16 * mj + lrow) * LDC,
                                                      s.P2 + (16 * nt + lrow) * LDC, x, lane);
                }
            }
#pragma unroll
            for (int i = 0; i < G::STPW; ++i) {
                const int ix = wv + NW * i;
                if (ix < G::NST) {
                    const int mi = ix / (DVS / 16), ni = ix % (DVS / 16);
                    const f32x4 gm = *reinterpret_cast<const f32x4*>(&s.gam[16 * mi + 4 * lgrp]);
                    acc[i] = ORD1 ? acc[i] * gm
                                  : tile_mma_r<T, C>(s.KtcT + prow<DK>(16 * mi + lrow) * LDC,
                                                     s.VT + prow<DVS>(16 * ni + lrow) * LDC, acc[i] * gm, lane);
                }
            }
        }
        lds_barrier();

        // ---- P5: E = -Tb Z; wavefront 0 applies Gamma S + Kt^T bV to its state tiles --
#pragma unroll
        for (int i = 0; i < G::OTPW; ++i) {
            const int w = wv + NW * i;
            if (w < G::NOT) {
                const int mt = w / (DVS / 16), nj = w % (DVS / 16);
                f32x4 x = tile_mma<T, C>(s.Tb + 16 * mt * LDC, LDC, s.ZT + 16 * nj * LDC, LDC, zero4(), lane);
                store4(&s.ET[(16 * nj + lrow) * LDC + 16 * mt + 4 * lgrp], -x);
            }
        }
        if (wv == 0) {
#pragma unroll
            for (int i = 0; i < G::STPW; ++i) {
                const int ix = wv + NW * i;
                if (ix < G::NST) {
                    const int mi = ix / (DVS / 16), ni = ix % (DVS / 16);
                    const f32x4 gm = *reinterpret_cast<const f32x4*>(&s.gam[16 * mi + 4 * lgrp]);
                    acc[i] = ORD1 ? acc[i] * gm
                                  : tile_mma_r<T, C>(s.KtcT + prow<DK>(16 * mi + lrow) * LDC,
                                                     s.VT + prow<DVS>(16 * ni + lrow) * LDC, acc[i] * gm, lane);
                }
            }
        }
        lds_barrier();

        // ---- P6: O^T += E^T P1^T (stored next iteration); S += Kc^T E; state -> LDS ---
        if (wv != 0) {
#pragma unroll
            for (int i = 0; i < G::OTPWX; ++i) {
                const int w = (wv - 1) + (NW - 1) * i;
                if (w < G::NOT) {
                    const int mj = w / (C / 16), nt = w % (C / 16);
                    opend[i] = tile_mma<T, C>(s.ET + 16 * mj * LDC, LDC, (ORD1 ? s.P2 : s.P1) + 16 * nt * LDC, LDC,
                                              oacc[i], lane);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < G::STPW; ++i) {
            const int ix = wv + NW * i;
            if (ix < G::NST) {
                const int mi = ix / (DVS / 16), ni = ix % (DVS / 16);
                acc[i] = tile_mma_r<T, C>((ORD1 ? s.KtcT : s.KccT) + prow<DK>(16 * mi + lrow) * LDC,
                                          s.ET + (16 * ni + lrow) * LDC, acc[i], lane);
                store4(&s.ST[(16 * ni + lrow) * LDK + 16 * mi + 4 * lgrp], acc[i]);
            }
        }
        if (SNAP && --snap_cd == 0) {
            snap_cd = snap_ec;
            const int64_t done = t0 + C - tb;  // tokens of the sequence behind this state
            const int64_t row = snap0 + done / p.snap_every - 1;
            if (done <= te - tb && row < p.snap_rows) {
                float* dst = p.snap + (row * H + h) * DK * DV + dv0;
#pragma unroll
                for (int i = 0; i < G::STPW; ++i) {
                    const int ix = wv + NW * i;
                    if (ix < G::NST) {
                        const int mi = ix / (DVS / 16), ni = ix % (DVS / 16);
                        store_state_tile(dst + (int64_t)16 * mi * DV + 16 * ni, DV, lane, acc[i]);
                    }
                }
            }
        }
        lds_barrier();
    }

    if (Lc_prev > 0) store_o();
    if (p.ST) {
#pragma unroll
        for (int i = 0; i < G::STPW; ++i) {
            const int ix = wv + NW * i;
            if (ix < G::NST) {
                const int mi = ix / (DVS / 16), ni = ix % (DVS / 16);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p.ST[sbase + (int64_t)(16 * mi + 4 * lgrp + r) * DV + 16 * ni + lrow] = acc[i][r];
            }
        }
    }
}

// ------------------------------------------------------------------------------------
// Instantiation table.  A configuration exists when its LDS image fits a CU.
template <typename T, int DK, int DVS, int C>
constexpr bool chunk_fits() { return chunk_lds_bytes<T, DK, DVS, C>() <= 160 * 1024; }

template <typename T, int DK, int DVS, int C, bool SC, bool ORD1>
static hipError_t launch_cfg(const ChunkArgs& a, hipStream_t stream) {
    constexpr int NT = ChunkCfg<T, DK, DVS, C>::NT;
    ChunkParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.log_a = a.log_a; p.beta = a.beta; p.S0 = a.S0;
    p.cu = a.cu_seqlens; p.o = a.o; p.ST = a.S_T;
    p.H = a.num_heads; p.DV = a.dv; p.split = a.split;
    p.eq_len = a.cu_seqlens ? 0 : a.total_tokens / (a.num_seqs > 0 ? a.num_seqs : 1);
    p.snap = a.snap; p.snap_rows = a.snap_rows; p.snap_every = a.snap_every;
    const ChunkPro pr{a.pro.normalize_k, a.pro.beta_logits, a.pro.log_a_raw, a.pro.log_a_min * LOG2E};
    const int64_t blocks = (int64_t)a.num_seqs * a.num_heads * a.split;
    p.xcd_group = (blocks % 8 == 0 && (blocks / 8) % a.split == 0) ? 1 : 0;
    const dim3 grid((unsigned)blocks), block(NT);
    if (a.pro.any()) {
        if (a.snap) hipLaunchKernelGGL((kda_chunk_kernel<T, DK, DVS, C, SC, ORD1, true, true>), grid, block, 0, stream, p, pr);
        else hipLaunchKernelGGL((kda_chunk_kernel<T, DK, DVS, C, SC, ORD1, false, true>), grid, block, 0, stream, p, pr);
    } else {
        if (a.snap) hipLaunchKernelGGL((kda_chunk_kernel<T, DK, DVS, C, SC, ORD1, true, false>), grid, block, 0, stream, p, pr);
        else hipLaunchKernelGGL((kda_chunk_kernel<T, DK, DVS, C, SC, ORD1, false, false>), grid, block, 0, stream, p, pr);
    }
    return hipGetLastError();
}

template <typename T, int DK, int DVS, int C>
static bool try_cfg(int scalar, bool launch, const ChunkArgs* a, hipStream_t stream, hipError_t* err) {
    if constexpr (chunk_fits<T, DK, DVS, C>()) {
        // order 1 comes with per-channel decay only (the host maps scalar decay to order 0)
        if (launch) *err = scalar     ? launch_cfg<T, DK, DVS, C, true, false>(*a, stream)
                           : a->order ? launch_cfg<T, DK, DVS, C, false, true>(*a, stream)
                                      : launch_cfg<T, DK, DVS, C, false, false>(*a, stream);
        return true;
    } else {
        return false;
    }
}

#define KDA_CHUNK_CASE(T, DK_, DVS_, C_) \
    if (dk == DK_ && dvs == DVS_ && chunk == C_) return try_cfg<T, DK_, DVS_, C_>(scalar, launch, a, stream, err);

// Returns whether the configuration exists; launches it when `launch`.
static bool chunk_dispatch(int dtype, int dk, int dvs, int chunk, int scalar, bool launch,
                           const ChunkArgs* a, hipStream_t stream, hipError_t* err) {
    if (dtype == 1) {
        KDA_CHUNK_CASE(bf16, 32, 16, 32) KDA_CHUNK_CASE(bf16, 32, 32, 32)
        KDA_CHUNK_CASE(bf16, 64, 16, 32) KDA_CHUNK_CASE(bf16, 64, 32, 32) KDA_CHUNK_CASE(bf16, 64, 64, 32)
        KDA_CHUNK_CASE(bf16, 128, 16, 32) KDA_CHUNK_CASE(bf16, 128, 32, 32) KDA_CHUNK_CASE(bf16, 128, 64, 32)
        KDA_CHUNK_CASE(bf16, 32, 32, 64) KDA_CHUNK_CASE(bf16, 64, 32, 64)
    } else if (dtype == 0) {
        KDA_CHUNK_CASE(float, 16, 16, 32) KDA_CHUNK_CASE(float, 32, 16, 32) KDA_CHUNK_CASE(float, 32, 32, 32)
        KDA_CHUNK_CASE(float, 64, 16, 32) KDA_CHUNK_CASE(float, 64, 32, 32) KDA_CHUNK_CASE(float, 128, 16, 32)
        KDA_CHUNK_CASE(float, 16, 16, 64) KDA_CHUNK_CASE(float, 32, 32, 64)
    }
    return false;
}

bool chunk_supported(int dtype, int dk, int dvs, int chunk, int scalar) {
    return chunk_dispatch(dtype, dk, dvs, chunk, scalar, false, nullptr, nullptr, nullptr);
}

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t stream) {
    hipError_t err = hipErrorInvalidValue;
    if (!chunk_dispatch(a.dtype, a.dk, a.dv / a.split, a.chunk, a.scalar_decay, true, &a, stream, &err))
        return hipErrorInvalidValue;
    return err;
}

}  // namespace kda
