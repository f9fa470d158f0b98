// kda_prep.hip -- chunk-parallel pass of the two-pass KDA prefill on gfx950.
//
// The chunkwise (WY) form (page "The argument, in one page", section
// "Everything, in one table", row "Chunkwise / WY") splits each chunk's work
// into a part that does not depend on the state -- decay sums, gated
// operands, the four C x C Gram products, the triangular solve and every
// product of those -- and a short state-dependent recurrence.  This kernel
// does the first part for every chunk of every (sequence, head) at once, so
// the whole GPU is busy with it, and writes one operator block per chunk
// (layout in kda_ws.hpp).  The sequential pass (kda_scan.hip) then only
// applies the blocks to the running state.
//
// Per chunk (g_t the running sum of log a, b = beta, mid-point references
// per 16-token sub-block as in the single-pass kernel):
//   A  = strict_lower(diag(b) Kb Kc^T)   L = strict_lower(Kb Kt^T)
//   P1 = lower(Qb Kc^T)                  P2 = lower(Qb Kt^T)
//   Tb = (I + A)^-1 diag(b)
//   W  = Tb Kb,  M1 = Tb L diag(b),  QP = Qb - P1 W,  M2 = P2 diag(b) - P1 M1
//   KC = (K e^{g_C - g_{t-1}})^T,  KT = (diag(b) K e^{g_C - g_t})^T,  GAM = e^{g_C}
// where Kb, Qb in W and QP are referenced to the chunk start (factors <= 1).
// The decay-first ordering (ORD1) takes Kb = K e^{g_t}, Kc = Kt and needs only
// A and P2 (unscaled, in place of P1); with L diag(b) = -I and P2 diag(b) = 0
// the same phases 5 and 6 then give M1 = -Tb and M2 = P2 Tb (kda_ws.hpp), and
// KC = (K e^{g_C - g_t})^T; no KT.
//
// Decay range: the factor split (phase 2) is exact to ~2^-30 while every valid
// token of a chunk has log2 a >= STEEP_LOG2 (kda_chunk_common.hpp).  A chunk with
// a steeper token is marked (GAM[0] = -1; a true GAM lies in [0, 1]) and its
// whole block is formed again by kda_prep_exact_kernel with every decay factor
// one exponential of a run of consecutive log2 decays, which is exact for any
// decay.
//
// Persistent workgroups of 8 wavefronts, each walking a strided list of
// chunks; the next chunk's inputs are loaded while the current one is in
// phases 3-6.  Phases, separated by LDS barriers:
//   1 decay sums per 4-token group              2 factors, gated operands, KC/KT/GAM out
//   3 Gram products                             4 (I + A)^-1 diag(b) (C = 32: two wavefronts)
//   5 W, M1 (to the block and, transposed, to LDS)   6 QP, M2 out
#include "kda_chunk_common.hpp"
#include "kda_launch.hpp"
#include "kda_ws.hpp"

namespace kda {

template <int DK, int C>
struct PrepCfg {
    static constexpr int NT = 512, NW = NT / WAVE;
    static constexpr int NB = C / 16;
    static constexpr int NPAIR = NB * (NB - 1) / 2;
    static constexpr int NBP = NB * (NB + 1) / 2;
    static constexpr int LDK = DK + 8;  // bf16 rows over channels (+16 bytes)
    static constexpr int LDC = C + 8;   // bf16 rows over tokens (+16 bytes)
    static constexpr int LDA = C + 4;   // fp32 rows over tokens
    static constexpr int NCP = DK / 2;
    static constexpr int NU = NCP * (C / 4);
    static_assert(NU <= NT, "one 4-token x 2-channel unit per thread");
    static constexpr bool SPLIT_SOLVE = (C == 32);  // two wavefronts invert the diagonal blocks
};

template <int DK, int C>
struct PrepLds {
    typedef PrepCfg<DK, C> G;
    union {
        struct {  // phases 2-3: Gram operands (mid-point references)
            bf16 Kr[C * G::LDK], Qr[C * G::LDK], Kce[C * G::LDK], Kci[C * G::LDK];
        } g;
        struct {  // phase 4: the solve's working set
            float Tf[C * G::LDA];       // (I + A)^-1, fp32, unscaled (split solve)
            float Xs[16 * 17];          // one 16 x 16 product, fp32
            float X[2 * G::NB * 256];   // panel exchange
        } v;
        struct {  // phases 5-6
            bf16 WT[DK * G::LDC];  // W^T  [channel][token]
            bf16 M1T[C * G::LDC];  // M1^T [i][t]
        } w;
        struct {  // exact kernel, phases 2-3: raw rows and log2 decays for exact_gram
            bf16 K[C * G::LDK], Q[C * G::LDK];
            float LA[C * DK];
        } x;
    } u;
    union {
        float grp[(C / 4) * DK];   // phases 1-2: summed log2 decay per 4-token group
        float A[C * G::LDA];       // phases 3-4: diag(b) strict_lower(Kb Kc^T)
    } u2;
    alignas(16) bf16 KbT[DK * G::LDC];  // (K e^{g_{t-1}})^T [channel][token]
    alignas(16) bf16 Qb[C * G::LDK];    // Q e^{g_t} [token][channel]
    alignas(16) bf16 LbT[C * G::LDC];   // (L diag(b))^T [i][t]
    alignas(16) bf16 P1[C * G::LDC];    // [t][i]
    alignas(16) bf16 Tb[C * G::LDC];    // (I + A)^-1 diag(b) [t][s]
    alignas(16) float P2[C * G::LDA];   // P2 diag(b) [t][i]
    alignas(16) float F[(G::NPAIR > 0 ? G::NPAIR : 1) * DK];
    alignas(16) float beta[C];
    alignas(16) float ones[16];  // unit column scale of the split solve (outside the unions)
    int steep[G::NW];            // per wavefront: a token below STEEP_LOG2
    int list[G::NT];             // exact kernel: marked items of one round
};

struct PrepParams {
    const void* q;
    const void* k;
    const float* log_a;
    const float* beta;
    const int32_t* cu;
    int64_t eq_len;   // sequence length when cu is null
    uint8_t* ws;      // operator blocks [unit][m]
    int H;
    int m;            // chunks per unit in this segment (block stride)
    int items;        // units * m
    int64_t chunk0;   // first chunk index of the segment
    Prologue pro;     // input prologue (instantiations with PRO only)
};

// Raw inputs of one chunk for one thread: its 4-token x 2-channel unit, and
// beta of token `tid` (threads below C).
struct PrepIn {
    Vec2<bf16>::type q[4], k[4];
    f32x2 la[4];
    float b;
};

template <int DK, int C, bool SCALAR>
__device__ __forceinline__ bool prep_locate(const PrepParams& p, int item, int64_t& t0, int& Lc, int& h) {
    const int unit = item / p.m, j = item % p.m;
    const int n = unit / p.H;
    h = unit % p.H;
    int64_t tb, te;
    if (p.cu) { tb = p.cu[n]; te = p.cu[n + 1]; }
    else { tb = (int64_t)n * p.eq_len; te = tb + p.eq_len; }
    t0 = tb + (p.chunk0 + j) * C;
    Lc = (int)((te - t0) < C ? (te - t0) : C);
    return t0 < te;
}

template <int DK, int C, bool SCALAR>
__device__ __forceinline__ void prep_load(const PrepParams& p, int64_t t0, int Lc, int h, int tid, int c, int tg,
                                          PrepIn& in) {
    typedef Vec2<bf16>::type b2;
    const bf16* __restrict__ gq = static_cast<const bf16*>(p.q);
    const bf16* __restrict__ gk = static_cast<const bf16*>(p.k);
    const int H = p.H;
    const int64_t r0 = t0 * H + h;
    if (tid < PrepCfg<DK, C>::NU) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // rows past the chunk's end repeat its last row; b and log a are masked there
            const int64_t row = r0 + (int64_t)min(4 * tg + i, Lc - 1) * H;
            in.q[i] = *reinterpret_cast<const b2*>(gq + row * DK + c);
            in.k[i] = *reinterpret_cast<const b2*>(gk + row * DK + c);
            if (SCALAR) { const float x = p.log_a[row]; in.la[i] = f32x2{x, x}; }
            else in.la[i] = *reinterpret_cast<const f32x2*>(p.log_a + row * DK + c);
        }
    }
    in.b = (tid < Lc) ? p.beta[r0 + (int64_t)tid * H] : 0.f;
}

// Unit-lower (I + A)^-1 diag(b) for C = 32 on two wavefronts: each inverts one
// 16 x 16 diagonal block (fp32), then wavefront 0 forms the off-diagonal block
// T21 = -T22 A21 T11 with two fp32 matrix-core products.  Ends with Tb written.
template <int DK, int C>
__device__ __forceinline__ void split_solve(PrepLds<DK, C>& s, int wv, int lane, int tid) {
    typedef PrepCfg<DK, C> G;
    constexpr int LDA = G::LDA, LDC = G::LDC;
    const int l16 = lane & 15, lg = lane >> 4;
    if (wv < 2)
        block_inverse<float, 16, LDA, LDA>(s.u2.A + 16 * wv * LDA + 16 * wv, s.ones, s.u.v.X + wv * 512,
                                           s.u.v.Tf + 16 * wv * LDA + 16 * wv, lane);
    lds_barrier();
    if (wv == 0) {
        // X = A21 T11 (rows i of block 1, columns n of block 0)
        f32x4 x = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kk = 4 * ks + lg;
            const float a = s.u2.A[(16 + l16) * LDA + kk];
            const float b = s.u.v.Tf[kk * LDA + l16];
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, x, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) s.u.v.Xs[(4 * lg + r) * 17 + l16] = x[r];
        wave_sync();
        // T21 = -T22 X
        f32x4 t = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kk = 4 * ks + lg;
            const float a = s.u.v.Tf[(16 + l16) * LDA + 16 + kk];
            const float b = s.u.v.Xs[kk * 17 + l16];
            t = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, t, 0, 0, 0);
        }
        const float bn = s.beta[l16];
#pragma unroll
        for (int r = 0; r < 4; ++r) s.Tb[(16 + 4 * lg + r) * LDC + l16] = (bf16)(-t[r] * bn);
    }
    // diagonal blocks
    for (int e = tid; e < 512; e += G::NT) {
        const int w = e >> 8, i = (e >> 4) & 15, jj = e & 15;
        const int row = 16 * w + i, col = 16 * w + jj;
        s.Tb[row * LDC + col] = (bf16)(s.u.v.Tf[row * LDA + col] * s.beta[col]);
    }
}

// Phases 4-6 of one chunk (after the Gram products): Tb = (I + A)^-1 diag(b), then
// W, M1, QP and M2 to the block.  Shared by both kernels.
template <int DK, int C, bool ORD1>
__device__ __forceinline__ void prep_solve_store(PrepLds<DK, C>& s, uint8_t* __restrict__ blk, int tid, int lane,
                                                 int wv) {
    typedef PrepCfg<DK, C> G;
    typedef WsBlock<DK, C, ORD1> WS;
    typedef Mma<bf16> M;
    constexpr int NW = G::NW, LDK = G::LDK, LDC = G::LDC, LDA = G::LDA;
    const int lrow = lane & 15, lgrp = lane >> 4;
    // ---- 4: Tb = (I + A)^-1 diag(b) ---------------------------------------------
    if constexpr (G::SPLIT_SOLVE) {
        split_solve<DK, C>(s, wv, lane, tid);
    } else {
        if (wv == 0) block_inverse<bf16, C, LDA, LDC>(s.u2.A, s.beta, s.u.v.X, s.Tb, lane);
    }
    lds_barrier();

    // ---- 5: W = Tb Kb and M1 = Tb L diag(b).  Each tile is formed in both
    //      orientations from the same fragments: W^T (rows: channels) goes to the
    //      block, W (rows: tokens) to LDS as [channel][token] for phase 6 --------
    constexpr int NWT = (DK / 16) * (C / 16), NMT = (C / 16) * (C / 16);
    for (int w = wv; w < NWT + NMT; w += NW) {
        const bool isw = w < NWT;
        const int x = isw ? w : w - NWT;
        const int ra = x / (C / 16), tt = x % (C / 16);  // row tile of KbT (or LbT), token tile
        const bf16* pa = (isw ? s.KbT : s.LbT) + (16 * ra + lrow) * LDC;
        const bf16* pb = s.Tb + (16 * tt + lrow) * LDC;
        constexpr int NK = C / M::K;
        M::frag fa[NK], fb[NK];
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            fa[k] = M::loadr(pa + k * M::K, lane);
            fb[k] = M::loadr(pb + k * M::K, lane);
        }
        f32x4 xt = zero4(), xn = zero4();
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            xt = M::mma(fa[k], fb[k], xt);  // rows: channel (or i), column: token t
            xn = M::mma(fb[k], fa[k], xn);  // rows: token t, column: channel (or i)
        }
        const int t = 16 * tt + lrow, a0 = 16 * ra + 4 * lgrp;
        const int an = 16 * ra + lrow, t0n = 16 * tt + 4 * lgrp;
        if (isw) {
            store4(reinterpret_cast<bf16*>(blk + WS::W + swz_elem<2 * DK>(kinv(t), kperm(a0))), xt);
            store4(&s.u.w.WT[an * LDC + t0n], xn);
        } else {
            store4(reinterpret_cast<bf16*>(blk + WS::M1 + piece<C>(kinv(t), a0 >> 3) + 2 * (a0 & 7)), xt);
            store4(&s.u.w.M1T[an * LDC + t0n], xn);
        }
    }
    lds_barrier();

    // ---- 6: QP = Qb - P1 W and M2 = P2 diag(b) - P1 M1, as their transposes -----
    for (int w = wv; w < NWT + NMT; w += NW) {
        const bool isq = w < NWT;
        const int x = isq ? w : w - NWT;
        const int ra = x / (C / 16), tt = x % (C / 16);
        const bf16* pa = (isq ? s.u.w.WT : s.u.w.M1T) + (16 * ra + lrow) * LDC;
        const bf16* pb = s.P1 + (16 * tt + lrow) * LDC;
        const f32x4 pw = tile_mma_r<bf16, C>(pa, pb, zero4(), lane);
        const int t = 16 * tt + lrow, a0 = 16 * ra + 4 * lgrp;
        if (isq) {
            const f32x4 qb = load4(&s.Qb[t * LDK + a0]);
            store4(reinterpret_cast<bf16*>(blk + WS::QP + swz_elem<2 * DK>(t, kperm(a0))), qb - pw);
        } else {
            const f32x4 p2 = *reinterpret_cast<const f32x4*>(&s.P2[t * LDA + a0]);
            store4(reinterpret_cast<bf16*>(blk + WS::M2 + piece<C>(t, a0 >> 3) + 2 * (a0 & 7)), p2 - pw);
        }
    }
}

// Phases 1-2 of a marked chunk in kda_prep_exact_kernel.  Kb, Qb, KC, KT and GAM
// are formed with one exponential each from running sums of log2 a referenced to
// the chunk start (prefixes) or end (suffixes), every exponent a run of
// consecutive decays; the raw rows (k after the prologue's scaling) and the
// log2 decays go to LDS for exact_gram.  Thread unit (c, tg) as in phase 1 of
// kda_prep_kernel; two LDS barriers.
template <int DK, int C, bool ORD1, bool PRO>
__device__ __forceinline__ void prep_steep_operands(const PrepParams& p, PrepLds<DK, C>& s, const PrepIn& in,
                                                    uint8_t* blk, int tid, int c, int tg, int Lc) {
    typedef PrepCfg<DK, C> G;
    typedef WsBlock<DK, C, ORD1> WS;
    constexpr int LDK = G::LDK, LDC = G::LDC;
    f32x2 l2[4];
    float kscale[4] = {1.f, 1.f, 1.f, 1.f};
    if (tid < G::NU) {
        f32x2 run = {0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            l2[i] = in.la[i] * LOG2E;
            if (PRO && p.pro.log_a_raw) {
                const float lo2 = p.pro.log_a_min * LOG2E;
                l2[i] = f32x2{prologue_log2_a(in.la[i][0], lo2), prologue_log2_a(in.la[i][1], lo2)};
            }
            if (4 * tg + i >= Lc) l2[i] = f32x2{0.f, 0.f};
            run += l2[i];
        }
        *reinterpret_cast<f32x2*>(&s.u2.grp[tg * DK + c]) = run;
        if (PRO && p.pro.normalize_k) {
            const bool hi = (tid & 63) >= 32;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float k0 = Vec2<bf16>::lo(in.k[i]), k1 = Vec2<bf16>::hi(in.k[i]);
                const float x = row_sum16(k0 * k0 + k1 * k1);
                const float lo2 = readlanef(x, 0) + readlanef(x, 16), hi2 = readlanef(x, 32) + readlanef(x, 48);
                kscale[i] = rsqrtf((hi ? hi2 : lo2) + PROLOGUE_EPS);
            }
        }
    }
    if (tid < C) s.beta[tid] = (PRO && p.pro.beta_logits && tid < Lc) ? prologue_beta(in.b) : in.b;
    lds_barrier();
    if (tid < G::NU) {
        f32x2 pre = {0.f, 0.f}, suf = {0.f, 0.f}, tot = {0.f, 0.f};
#pragma unroll
        for (int g = 0; g < C / 4; ++g) {
            const f32x2 x = *reinterpret_cast<const f32x2*>(&s.u2.grp[g * DK + c]);
            tot += x;
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
        auto ex2v = [](f32x2 x) { return f32x2{__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1])}; };
        f32x2 kb[4], kc[4], kt[4];
        f32x2 gp = pre;  // g_{t-1}
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * tg + i;
            const f32x2 k = f32x2{Vec2<bf16>::lo(in.k[i]), Vec2<bf16>::hi(in.k[i])} * kscale[i];
            const f32x2 q = f32x2{Vec2<bf16>::lo(in.q[i]), Vec2<bf16>::hi(in.q[i])};
            const f32x2 g = gp + l2[i];
            kb[i] = k * ex2v(ORD1 ? g : gp);
            kc[i] = k * ex2v(ORD1 ? sx[i] : sx[i] + l2[i]);
            kt[i] = k * ex2v(sx[i]) * s.beta[t];
            const f32x2 qb = q * ex2v(g);
            store2(&s.Qb[t * LDK + c], qb[0], qb[1]);
            store2(&s.u.x.K[t * LDK + c], k[0], k[1]);
            store2(&s.u.x.Q[t * LDK + c], q[0], q[1]);
            *reinterpret_cast<f32x2*>(&s.u.x.LA[t * DK + c]) = l2[i];
            gp = g;
        }
        if (tg == 0) *reinterpret_cast<f32x2*>(blk + WS::GAM + 4 * c) = ex2v(tot);
        const int half = 8 * (tg & 1);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            store4(&s.KbT[(c + e) * LDC + 4 * tg], f32x4{kb[0][e], kb[1][e], kb[2][e], kb[3][e]});
            store4(reinterpret_cast<bf16*>(blk + WS::KC + piece<DK>(c + e, tg >> 1) + half),
                   f32x4{kc[0][e], kc[1][e], kc[2][e], kc[3][e]});
            if (!ORD1)
                store4(reinterpret_cast<bf16*>(blk + WS::KT + piece<DK>(c + e, tg >> 1) + half),
                       f32x4{kt[0][e], kt[1][e], kt[2][e], kt[3][e]});
        }
    }
    lds_barrier();
}

// Phase 3 of a marked chunk: the masked Gram products by exact_gram, stored as
// phase 3 of kda_prep_kernel stores the factored ones (ORD1: A and P2, P2 in P1's
// slot; L diag(b) = -I and P2 diag(b) = 0 left as set up).
template <int DK, int C, bool ORD1>
__device__ __forceinline__ void prep_steep_gram(PrepLds<DK, C>& s, int wv, int lane) {
    typedef PrepCfg<DK, C> G;
    constexpr int LDC = G::LDC, LDA = G::LDA;
    exact_gram<bf16, DK, C, G::NW, ORD1>(s.u.x.K, s.u.x.Q, G::LDK, s.u.x.LA, DK, wv, lane,
                                         [&](int t, int i, float av, float lv, float p1v, float p2v) {
        s.u2.A[t * LDA + i] = s.beta[t] * av;
        if (ORD1) {
            s.P1[t * LDC + i] = (bf16)p2v;
        } else {
            s.LbT[i * LDC + t] = (bf16)(lv * s.beta[i]);
            s.P1[t * LDC + i] = (bf16)p1v;
            s.P2[t * LDA + i] = p2v * s.beta[i];
        }
    });
}

// The masked matrices are never written outside their lower triangle: they start
// at zero; ORD1 sets L diag(b) = -I.
template <int DK, int C>
__device__ __forceinline__ void prep_init_lds(PrepLds<DK, C>& s, int tid, bool ord1) {
    typedef PrepCfg<DK, C> G;
    constexpr int NT = G::NT, LDC = G::LDC, LDA = G::LDA;
    for (int e = tid; e < C * LDC; e += NT) {
        s.LbT[e] = (bf16)0.f; s.P1[e] = (bf16)0.f; s.Tb[e] = (bf16)0.f;
    }
    for (int e = tid; e < C * LDA; e += NT) s.P2[e] = 0.f;
    if (tid < 16) s.ones[tid] = 1.f;
    if (ord1) {
        lds_barrier();
        if (tid < C) s.LbT[tid * LDC + tid] = (bf16)-1.f;
    }
}

// PRO: the call has an input prologue (k scaled per token by (|k|^2 + eps)^{-1/2},
// each token's channels being one half-wavefront; beta and log a transformed
// where they are loaded).
template <int DK, int C, bool SCALAR, bool ORD1, bool PRO>
__global__ void __launch_bounds__(512, 2) kda_prep_kernel(PrepParams p) {
    typedef PrepCfg<DK, C> G;
    typedef WsBlock<DK, C, ORD1> WS;
    typedef Mma<bf16> M;
    constexpr int NT = G::NT, NW = G::NW, NB = G::NB, LDK = G::LDK, LDC = G::LDC, LDA = G::LDA;
    __shared__ PrepLds<DK, C> s;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lrow = lane & 15, lgrp = lane >> 4;
    int c = 0, tg = 0;
    if (tid < G::NU) unit_of<G::NCP>(tid, c, tg);

    // upper blocks of the masked products are never written: zero them once
    prep_init_lds<DK, C>(s, tid, ORD1);

    // this workgroup's chunks: item = blockIdx.x + k gridDim.x, empty ones skipped,
    // 64 candidates at a time per wavefront (one per lane), as in kda_prep2.hip
    auto next_item = [&](int it, int64_t& t0, int& Lc, int& h) {
        const int64_t G = gridDim.x;
        const int ln = tid & 63;
        for (int64_t at = it; at < p.items; at += 64 * G) {
            const int64_t cand = at + ln * G;
            int64_t ct0;
            int cLc, ch;
            const bool live = cand < p.items && prep_locate<DK, C, SCALAR>(p, (int)cand, ct0, cLc, ch);
            const uint64_t m = __ballot(live);
            if (m) {
                const int first = (int)(at + (__ffsll((unsigned long long)m) - 1) * G);
                prep_locate<DK, C, SCALAR>(p, first, t0, Lc, h);
                return first;
            }
        }
        return p.items;
    };
    int64_t t0 = 0;
    int Lc = 0, h = 0;
    int item = next_item(blockIdx.x, t0, Lc, h);
    PrepIn in;
    if (item < p.items) prep_load<DK, C, SCALAR>(p, t0, Lc, h, tid, c, tg, in);

    while (item < p.items) {
        uint8_t* __restrict__ blk = p.ws + (size_t)item * WS::BYTES;

        // ---- 1: decay sums per 4-token group in the log2 domain ------------------
        f32x2 lam[4];
        float kscale[4] = {1.f, 1.f, 1.f, 1.f};
        bool steep = false;
        if (tid < G::NU) {
            f32x2 run = f32x2{0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x2 l2 = in.la[i] * LOG2E;
                if (PRO && p.pro.log_a_raw) {
                    const float lo2 = p.pro.log_a_min * LOG2E;
                    l2 = f32x2{prologue_log2_a(in.la[i][0], lo2), prologue_log2_a(in.la[i][1], lo2)};
                }
                if (4 * tg + i >= Lc) l2 = f32x2{0.f, 0.f};
                steep |= l2[0] < STEEP_LOG2 || l2[1] < STEEP_LOG2;
                run += l2;
                lam[i] = run;
            }
            *reinterpret_cast<f32x2*>(&s.u2.grp[tg * DK + c]) = run;
            if (PRO && p.pro.normalize_k) {
                static_assert(G::NCP == 32, "a token's channels are one half-wavefront");
                const bool hi = (tid & 63) >= 32;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float k0 = Vec2<bf16>::lo(in.k[i]), k1 = Vec2<bf16>::hi(in.k[i]);
                    const float x = row_sum16(k0 * k0 + k1 * k1);
                    const float lo2 = readlanef(x, 0) + readlanef(x, 16), hi2 = readlanef(x, 32) + readlanef(x, 48);
                    kscale[i] = rsqrtf((hi ? hi2 : lo2) + PROLOGUE_EPS);
                }
            }
        }
        if (tid < C) s.beta[tid] = (PRO && p.pro.beta_logits && tid < Lc) ? prologue_beta(in.b) : in.b;
        {
            const bool ws = wave_any(steep);
            if (lane == 0) s.steep[wv] = ws;
        }
        lds_barrier();

        // ---- 2: factors (exponents clamped to the fp32 range) and gated operands ---
        //   rin = e^{g_t - mid}, rex = e^{g_{t-1} - mid}, em = e^{mu_b}, ec = e^{g_C - mu_b}
        if (tid < G::NU) {
            const int b = tg / 4, gib = tg % 4;
            f32x2 off = {0.f, 0.f}, rho = {0.f, 0.f}, tot = {0.f, 0.f}, mid = {0.f, 0.f};
#pragma unroll
            for (int g = 0; g < C / 4; ++g) {
                const f32x2 x = *reinterpret_cast<const f32x2*>(&s.u2.grp[g * DK + c]);
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
            f32x2 kb[4], kc[4], kt[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * tg + i;
                f32x2 ri, ci;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    ri[e] = __builtin_amdgcn_exp2f(
                        __builtin_amdgcn_fmed3f(off[e] + lam[i][e] - mid[e], -126.f, 126.f));
                    ci[e] = __builtin_amdgcn_rcpf(ri[e]);
                }
                const f32x2 k = f32x2{Vec2<bf16>::lo(in.k[i]), Vec2<bf16>::hi(in.k[i])} * kscale[i];
                const f32x2 q = f32x2{Vec2<bf16>::lo(in.q[i]), Vec2<bf16>::hi(in.q[i])};
                const f32x2 kr = ORD1 ? k * ri : k * prev, qr = q * ri, kce = k * prevc, kci = k * ci;
                store2(&s.u.g.Kr[t * LDK + c], kr[0], kr[1]);
                store2(&s.u.g.Qr[t * LDK + c], qr[0], qr[1]);
                if (!ORD1) store2(&s.u.g.Kce[t * LDK + c], kce[0], kce[1]);
                store2(&s.u.g.Kci[t * LDK + c], kci[0], kci[1]);
                store2(&s.Qb[t * LDK + c], qr[0] * em[0], qr[1] * em[1]);
                kb[i] = kr * em;
                kc[i] = ORD1 ? kci * ec : kce * ec;
                kt[i] = kci * ec * s.beta[t];
                prev = ri;
                prevc = ci;
            }
            // KC, KT: tokens 4 tg .. 4 tg + 3 are half of piece tg / 2 of channel row c + e
            const int half = 8 * (tg & 1);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                store4(&s.KbT[(c + e) * LDC + 4 * tg], f32x4{kb[0][e], kb[1][e], kb[2][e], kb[3][e]});
                store4(reinterpret_cast<bf16*>(blk + WS::KC + piece<DK>(c + e, tg >> 1) + half),
                       f32x4{kc[0][e], kc[1][e], kc[2][e], kc[3][e]});
                if (!ORD1)
                    store4(reinterpret_cast<bf16*>(blk + WS::KT + piece<DK>(c + e, tg >> 1) + half),
                           f32x4{kt[0][e], kt[1][e], kt[2][e], kt[3][e]});
            }
        }
        // per (sub-block, channel): e^{mu_bt - mu_bi} for block pairs; e^{g_C} to the block
        for (int e = tid; e < NB * DK; e += NT) {
            const int b = e / DK, ch = e % DK;
            float rho[NB + 1], mu[NB];
            rho[0] = 0.f;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                const float g0 = s.u2.grp[(4 * bb) * DK + ch], g1 = s.u2.grp[(4 * bb + 1) * DK + ch];
                const float g2 = s.u2.grp[(4 * bb + 2) * DK + ch], g3 = s.u2.grp[(4 * bb + 3) * DK + ch];
                mu[bb] = rho[bb] + g0 + g1;
                rho[bb + 1] = rho[bb] + ((g0 + g1) + (g2 + g3));
            }
            if (b == 0) {  // a steep chunk is marked for kda_prep_exact_kernel instead
                int st = 0;
#pragma unroll
                for (int w = 0; w < NW; ++w) st |= s.steep[w];
                reinterpret_cast<float*>(blk + WS::GAM)[ch] = st ? -1.f : exp2f(rho[NB]);
            }
            for (int bi = 0; bi < b; ++bi) s.F[(b * (b - 1) / 2 + bi) * DK + ch] = exp2f(mu[b] - mu[bi]);
        }
        lds_barrier();

        // next chunk's inputs: in flight during phases 3-6
        int64_t nt0 = 0;
        int nLc = 0, nh = 0;
        const int nitem = next_item(item + gridDim.x, nt0, nLc, nh);
        if (nitem < p.items) prep_load<DK, C, SCALAR>(p, nt0, nLc, nh, tid, c, tg, in);

        // ---- 3: Gram products; tile w is product w % 4 (0 A, 1 L, 2 P1, 3 P2) of block
        //      pair w / 4.  A, P1, P2 land row-major [t][i], L transposed [i][t].
        //      ORD1: tile w is A (w even) or P2 (w odd, unscaled, into P1) of pair w / 2
        constexpr int NG = ORD1 ? 2 : 4;
        for (int w = wv; w < NG * G::NBP; w += NW) {
            const int g = ORD1 ? ((w & 1) ? 3 : 0) : w % 4, pr = w / NG;
            int bt = 0;
            while ((bt + 1) * (bt + 2) / 2 <= pr) ++bt;
            const int bi = pr - bt * (bt + 1) / 2;
            const bf16* rows = (g < 2 ? s.u.g.Kr : s.u.g.Qr) + (16 * bt + lrow) * LDK;
            const bf16* cols = ((g & 1) == 0 && !ORD1 ? s.u.g.Kce : s.u.g.Kci) + (16 * bi + lrow) * LDK;
            constexpr int NK = DK / M::K;
            M::frag fr[NK], fc[NK];
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
            f32x4 acc = zero4();
            if (g == 1) {
#pragma unroll
                for (int k = 0; k < NK; ++k) acc = M::mma(fr[k], fc[k], acc);
                // rows t = 16 bt + 4 lgrp + r, column i = 16 bi + lrow
                const int i = 16 * bi + lrow, tt = 16 * bt + 4 * lgrp;
                const float bi_ = s.beta[i];
                f32x4 m;
#pragma unroll
                for (int r = 0; r < 4; ++r) m[r] = (i < tt + r) ? acc[r] * bi_ : 0.f;
                store4(&s.LbT[i * LDC + tt], m);
            } else {
#pragma unroll
                for (int k = 0; k < NK; ++k) acc = M::mma(fc[k], fr[k], acc);
                // column t = 16 bt + lrow, rows i = 16 bi + 4 lgrp + r
                const int t = 16 * bt + lrow, i0 = 16 * bi + 4 * lgrp;
                f32x4 m;
#pragma unroll
                for (int r = 0; r < 4; ++r) m[r] = (g == 0 ? i0 + r < t : i0 + r <= t) ? acc[r] : 0.f;
                if (g == 0) *reinterpret_cast<f32x4*>(&s.u2.A[t * LDA + i0]) = s.beta[t] * m;
                else if (g == 2 || ORD1) store4(&s.P1[t * LDC + i0], m);
                else *reinterpret_cast<f32x4*>(&s.P2[t * LDA + i0]) =
                         m * *reinterpret_cast<const f32x4*>(&s.beta[i0]);
            }
        }
        lds_barrier();

        prep_solve_store<DK, C, ORD1>(s, blk, tid, lane, wv);
        lds_barrier();  // LDS of this chunk is reused by the next

        item = nitem; t0 = nt0; Lc = nLc; h = nh;
    }
}

// Marked chunks of one segment, run after kda_prep_kernel on the same items: every
// non-empty item whose block carries the mark (GAM[0] == -1) is formed again,
// all of it, with every decay factor one exponential (prep_steep_operands,
// exact_gram); phases 4-6 are those of kda_prep_kernel.  Workgroup b checks its
// items b, b + G, ... (G = gridDim.x) NT at a time, one per thread, and forms the
// marked ones of each round; unmarked blocks are not touched.
template <int DK, int C, bool SCALAR, bool ORD1, bool PRO>
__global__ void __launch_bounds__(512, 2) kda_prep_exact_kernel(PrepParams p) {
    typedef PrepCfg<DK, C> G;
    typedef WsBlock<DK, C, ORD1> WS;
    constexpr int NT = G::NT, NW = G::NW;
    __shared__ PrepLds<DK, C> s;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    int c = 0, tg = 0;
    if (tid < G::NU) unit_of<G::NCP>(tid, c, tg);
    bool init = false;
    for (int64_t base = 0; (int64_t)blockIdx.x + base * gridDim.x < p.items; base += NT) {
        const int64_t it = (int64_t)blockIdx.x + (base + tid) * gridDim.x;
        bool marked = false;
        if (it < p.items) {
            int64_t t0;
            int Lc, h;
            if (prep_locate<DK, C, SCALAR>(p, (int)it, t0, Lc, h))
                marked = *reinterpret_cast<const float*>(p.ws + (size_t)it * WS::BYTES + WS::GAM) == -1.f;
        }
        const uint64_t m = __ballot(marked);
        if (lane == 0) s.steep[wv] = __popcll(m);
        lds_barrier();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int cnt = s.steep[w];
            before += w < wv ? cnt : 0;
            total += cnt;
        }
        if (marked) s.list[before + __popcll(m & ((1ull << lane) - 1))] = (int)it;
        lds_barrier();
        if (total > 0 && !init) {
            prep_init_lds<DK, C>(s, tid, ORD1);
            init = true;
            lds_barrier();
        }
        for (int x = 0; x < total; ++x) {
            const int item = __builtin_amdgcn_readfirstlane(s.list[x]);
            int64_t t0;
            int Lc, h;
            prep_locate<DK, C, SCALAR>(p, item, t0, Lc, h);
            uint8_t* __restrict__ blk = p.ws + (size_t)item * WS::BYTES;
            PrepIn in;
            prep_load<DK, C, SCALAR>(p, t0, Lc, h, tid, c, tg, in);
            prep_steep_operands<DK, C, ORD1, PRO>(p, s, in, blk, tid, c, tg, Lc);
            prep_steep_gram<DK, C, ORD1>(s, wv, lane);
            lds_barrier();
            prep_solve_store<DK, C, ORD1>(s, blk, tid, lane, wv);
            lds_barrier();
        }
    }
}

// ------------------------------------------------------------------------------------
template <int DK, int C, bool SC, bool ORD1, bool PRO>
static hipError_t prep_cfg(const PrepLaunch& a, hipStream_t stream) {
    PrepParams p;
    p.q = a.q; p.k = a.k; p.log_a = a.log_a; p.beta = a.beta; p.cu = a.cu_seqlens;
    p.eq_len = a.eq_len; p.ws = static_cast<uint8_t*>(a.ws); p.H = a.num_heads; p.m = a.m;
    p.chunk0 = a.chunk0;
    p.items = (int)(a.units * a.m);
    p.pro = a.pro;
    // persistent workgroups: as many as fit at once (two per compute unit when the
    // LDS image allows), each walking items blockIdx.x, + gridDim.x, ...
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int per_cu = sizeof(PrepLds<DK, C>) <= 80 * 1024 ? 2 : 1;
    int64_t blocks = (int64_t)cus * per_cu;
    if (blocks > p.items) blocks = p.items;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((kda_prep_kernel<DK, C, SC, ORD1, PRO>), dim3((unsigned)blocks), dim3(PrepCfg<DK, C>::NT), 0,
                       stream, p);
    hipLaunchKernelGGL((kda_prep_exact_kernel<DK, C, SC, ORD1, PRO>), dim3((unsigned)blocks),
                       dim3(PrepCfg<DK, C>::NT), 0, stream, p);
    return hipGetLastError();
}

int prep_block_bytes(int dk, int chunk, int order) {
    const bool o1 = order != 0;
    if (dk == 64 && chunk == 32) return o1 ? WsBlock<64, 32, true>::BYTES : WsBlock<64, 32>::BYTES;
    if (dk == 128 && chunk == 32) return o1 ? WsBlock<128, 32, true>::BYTES : WsBlock<128, 32>::BYTES;
    if (dk == 64 && chunk == 64) return o1 ? WsBlock<64, 64, true>::BYTES : WsBlock<64, 64>::BYTES;
    return 0;
}

// a scalar decay comes with the decay-first order (the host's choice for the two-pass method)
template <int DK, int C>
static hipError_t prep_dispatch(const PrepLaunch& a, hipStream_t stream) {
    if (a.pro.any()) {
        if (a.scalar) return prep_cfg<DK, C, true, true, true>(a, stream);
        return a.order ? prep_cfg<DK, C, false, true, true>(a, stream) : prep_cfg<DK, C, false, false, true>(a, stream);
    }
    if (a.scalar) return prep_cfg<DK, C, true, true, false>(a, stream);
    return a.order ? prep_cfg<DK, C, false, true, false>(a, stream) : prep_cfg<DK, C, false, false, false>(a, stream);
}

hipError_t launch_prep(const PrepLaunch& a, hipStream_t stream) {
    if (a.dk == 128 && a.chunk == 32) return launch_prep2(a, stream);
    if (a.dk == 64 && a.chunk == 32) return prep_dispatch<64, 32>(a, stream);
    if (a.dk == 64 && a.chunk == 64) return prep_dispatch<64, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
