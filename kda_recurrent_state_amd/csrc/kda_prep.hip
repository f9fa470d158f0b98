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
//
// One workgroup (4 wavefronts) per chunk.  Phases, separated by LDS barriers:
//   1 load, decay sums per 4-token group        2 factors, gated operands, KC/KT/GAM out
//   3 Gram products                             4 wavefront 0: (I + A)^-1 diag(b)
//   5 W, M1 (to the block and, transposed, to LDS)   6 QP, M2 out
#include "kda_chunk_common.hpp"
#include "kda_launch.hpp"
#include "kda_ws.hpp"

namespace kda {

template <int DK, int C>
struct PrepCfg {
    static constexpr int NT = 256, NW = NT / WAVE;
    static constexpr int NB = C / 16;
    static constexpr int NPAIR = NB * (NB - 1) / 2;
    static constexpr int NBP = NB * (NB + 1) / 2;
    static constexpr int LDK = DK + 8;  // bf16 rows over channels (+16 bytes)
    static constexpr int LDC = C + 8;   // bf16 rows over tokens (+16 bytes)
    static constexpr int LDA = C + 4;   // fp32 rows over tokens
    static constexpr int NCP = DK / 2;
    static constexpr int NU = NCP * (C / 4);
    static constexpr int UPT = (NU + NT - 1) / NT;
};

template <int DK, int C>
struct PrepLds {
    typedef PrepCfg<DK, C> G;
    union {
        struct {  // Gram operands (mid-point references), dead after phase 3
            bf16 Kr[C * G::LDK], Qr[C * G::LDK], Kce[C * G::LDK], Kci[C * G::LDK];
        } g;
        struct {  // phase 5 results read in phase 6
            bf16 WT[DK * G::LDC];  // W^T  [channel][token]
            bf16 M1T[C * G::LDC];  // M1^T [i][t]
        } w;
    } u;
    alignas(16) bf16 KbT[DK * G::LDC];  // (K e^{g_{t-1}})^T [channel][token]
    alignas(16) bf16 Qb[C * G::LDK];    // Q e^{g_t} [token][channel]
    alignas(16) bf16 LbT[C * G::LDC];   // (L diag(b))^T [i][t]
    alignas(16) bf16 P1[C * G::LDC];    // [t][i]
    alignas(16) bf16 Tb[C * G::LDC];    // (I + A)^-1 diag(b) [t][s]
    alignas(16) float A[C * G::LDA];    // diag(b) strict_lower(Kb Kc^T)
    alignas(16) float P2[C * G::LDA];   // P2 diag(b) [t][i]
    alignas(16) float X[2 * G::NB * 256];
    alignas(16) float grp[(C / 4) * DK];
    alignas(16) float F[(G::NPAIR > 0 ? G::NPAIR : 1) * DK];
    alignas(16) float beta[C];
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
    int64_t chunk0;   // first chunk index of the segment
};

template <int DK, int C, bool SCALAR>
__global__ void __launch_bounds__(256) kda_prep_kernel(PrepParams p) {
    typedef PrepCfg<DK, C> G;
    typedef WsBlock<DK, C> WS;
    typedef Mma<bf16> M;
    constexpr int NT = G::NT, NW = G::NW, NB = G::NB, LDK = G::LDK, LDC = G::LDC, LDA = G::LDA;
    __shared__ PrepLds<DK, C> s;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int H = p.H;
    const int item = blockIdx.x;
    const int unit = item / p.m, j = item % p.m;
    const int n = unit / H, h = unit % H;
    int64_t tb, te;
    if (p.cu) { tb = p.cu[n]; te = p.cu[n + 1]; }
    else { tb = (int64_t)n * p.eq_len; te = tb + p.eq_len; }
    const int64_t t0 = tb + (p.chunk0 + j) * C;
    if (t0 >= te) return;  // the whole workgroup leaves together
    const int Lc = (int)((te - t0) < C ? (te - t0) : C);
    uint8_t* __restrict__ blk = p.ws + (size_t)item * WS::BYTES;
    const bf16* __restrict__ gq = static_cast<const bf16*>(p.q);
    const bf16* __restrict__ gk = static_cast<const bf16*>(p.k);

    // upper blocks of the masked products are never written
    for (int e = tid; e < C * LDC; e += NT) {
        s.LbT[e] = (bf16)0.f; s.P1[e] = (bf16)0.f; s.Tb[e] = (bf16)0.f;
    }
    for (int e = tid; e < C * LDA; e += NT) s.P2[e] = 0.f;

    // ---- 1: inputs (rows past the chunk's end repeat its last row; b and log a are
    //      masked there), decay sums per 4-token group in the log2 domain ----------
    typedef Vec2<bf16>::type b2;
    b2 qv[G::UPT][4], kv[G::UPT][4];
    f32x2 lam[G::UPT][4];
    const int64_t r0 = t0 * H + h;
#pragma unroll
    for (int u = 0; u < G::UPT; ++u) {
        const int uu = tid + NT * u;
        if (uu < G::NU) {
            int c, tg;
            unit_of<G::NCP>(uu, c, tg);
            f32x2 run = f32x2{0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = r0 + (int64_t)min(4 * tg + i, Lc - 1) * H;
                qv[u][i] = *reinterpret_cast<const b2*>(gq + row * DK + c);
                kv[u][i] = *reinterpret_cast<const b2*>(gk + row * DK + c);
                f32x2 la;
                if (SCALAR) { const float x = p.log_a[row]; la = f32x2{x, x}; }
                else la = *reinterpret_cast<const f32x2*>(p.log_a + row * DK + c);
                run += (4 * tg + i < Lc) ? la * LOG2E : f32x2{0.f, 0.f};
                lam[u][i] = run;
            }
            *reinterpret_cast<f32x2*>(&s.grp[tg * DK + c]) = run;
        }
    }
    for (int t = tid; t < C; t += NT) s.beta[t] = t < Lc ? p.beta[r0 + (int64_t)t * H] : 0.f;
    lds_barrier();

    // ---- 2: factors (exponents clamped to the fp32 range) and gated operands -------
    //   rin = e^{g_t - mid}, rex = e^{g_{t-1} - mid}, em = e^{mu_b}, ec = e^{g_C - mu_b}
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
            f32x2 kb[4], kc[4], kt[4];
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
                const f32x2 k = f32x2{Vec2<bf16>::lo(kv[u][i]), Vec2<bf16>::hi(kv[u][i])};
                const f32x2 q = f32x2{Vec2<bf16>::lo(qv[u][i]), Vec2<bf16>::hi(qv[u][i])};
                const f32x2 kr = k * prev, qr = q * ri, kce = k * prevc, kci = k * ci;
                store2(&s.u.g.Kr[t * LDK + c], kr[0], kr[1]);
                store2(&s.u.g.Qr[t * LDK + c], qr[0], qr[1]);
                store2(&s.u.g.Kce[t * LDK + c], kce[0], kce[1]);
                store2(&s.u.g.Kci[t * LDK + c], kci[0], kci[1]);
                store2(&s.Qb[t * LDK + c], qr[0] * em[0], qr[1] * em[1]);
                kb[i] = kr * em;
                kc[i] = kce * ec;
                kt[i] = kci * ec * s.beta[t];
                prev = ri;
                prevc = ci;
            }
            const int pos = kperm(4 * tg);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                store4(&s.KbT[(c + e) * LDC + 4 * tg], f32x4{kb[0][e], kb[1][e], kb[2][e], kb[3][e]});
                store4(reinterpret_cast<bf16*>(blk + WS::KC + swz_elem<2 * C>(c + e, pos)),
                       f32x4{kc[0][e], kc[1][e], kc[2][e], kc[3][e]});
                store4(reinterpret_cast<bf16*>(blk + WS::KT + swz_elem<2 * C>(c + e, pos)),
                       f32x4{kt[0][e], kt[1][e], kt[2][e], kt[3][e]});
            }
        }
    }
    // per (sub-block, channel): e^{mu_bt - mu_bi} for block pairs; e^{g_C} to the block
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
        if (b == 0) reinterpret_cast<float*>(blk + WS::GAM)[c] = exp2f(rho[NB]);
        for (int bi = 0; bi < b; ++bi) s.F[(b * (b - 1) / 2 + bi) * DK + c] = exp2f(mu[b] - mu[bi]);
    }
    lds_barrier();

    // ---- 3: Gram products; tile w is product w % 4 (0 A, 1 L, 2 P1, 3 P2) of block
    //      pair w / 4.  A, P1, P2 land row-major [t][i], L transposed [i][t] --------
    for (int w = wv; w < 4 * G::NBP; w += NW) {
        const int g = w % 4, pr = w / 4;
        int bt = 0;
        while ((bt + 1) * (bt + 2) / 2 <= pr) ++bt;
        const int bi = pr - bt * (bt + 1) / 2;
        const bf16* rows = (g < 2 ? s.u.g.Kr : s.u.g.Qr) + (16 * bt + lrow) * LDK;
        const bf16* cols = ((g & 1) == 0 ? s.u.g.Kce : s.u.g.Kci) + (16 * bi + lrow) * LDK;
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
            if (g == 0) *reinterpret_cast<f32x4*>(&s.A[t * LDA + i0]) = s.beta[t] * m;
            else if (g == 2) store4(&s.P1[t * LDC + i0], m);
            else *reinterpret_cast<f32x4*>(&s.P2[t * LDA + i0]) =
                     m * *reinterpret_cast<const f32x4*>(&s.beta[i0]);
        }
    }
    lds_barrier();

    // ---- 4: Tb = (I + A)^-1 diag(b) ----------------------------------------------
    if (wv == 0) block_inverse<bf16, C, LDA, LDC>(s.A, s.beta, s.X, s.Tb, lane);
    lds_barrier();

    // ---- 5: W = Tb Kb and M1 = Tb L diag(b).  Each tile is formed in both
    //      orientations from the same fragments: W^T (rows: channels) goes to the
    //      block, W (rows: tokens) to LDS as [channel][token] for phase 6 ----------
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
            store4(reinterpret_cast<bf16*>(blk + WS::W + swz_elem<2 * DK>(t, kperm(a0))), xt);
            store4(&s.u.w.WT[an * LDC + t0n], xn);
        } else {
            store4(reinterpret_cast<bf16*>(blk + WS::M1 + swz_elem<2 * C>(t, kperm(a0))), xt);
            store4(&s.u.w.M1T[an * LDC + t0n], xn);
        }
    }
    lds_barrier();

    // ---- 6: QP = Qb - P1 W and M2 = P2 diag(b) - P1 M1, as their transposes -------
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
            store4(reinterpret_cast<bf16*>(blk + WS::M2 + swz_elem<2 * C>(t, kperm(a0))), p2 - pw);
        }
    }
}

// ------------------------------------------------------------------------------------
template <int DK, int C, bool SC>
static hipError_t prep_cfg(const PrepLaunch& a, hipStream_t stream) {
    PrepParams p;
    p.q = a.q; p.k = a.k; p.log_a = a.log_a; p.beta = a.beta; p.cu = a.cu_seqlens;
    p.eq_len = a.eq_len; p.ws = static_cast<uint8_t*>(a.ws); p.H = a.num_heads; p.m = a.m;
    p.chunk0 = a.chunk0;
    const int64_t blocks = (int64_t)a.units * a.m;
    hipLaunchKernelGGL((kda_prep_kernel<DK, C, SC>), dim3((unsigned)blocks), dim3(PrepCfg<DK, C>::NT), 0,
                       stream, p);
    return hipGetLastError();
}

int prep_block_bytes(int dk, int chunk) {
    if (dk == 64 && chunk == 32) return WsBlock<64, 32>::BYTES;
    if (dk == 128 && chunk == 32) return WsBlock<128, 32>::BYTES;
    if (dk == 64 && chunk == 64) return WsBlock<64, 64>::BYTES;
    return 0;
}

hipError_t launch_prep(const PrepLaunch& a, hipStream_t stream) {
    if (a.dk == 128 && a.chunk == 32) return a.scalar ? prep_cfg<128, 32, true>(a, stream) : prep_cfg<128, 32, false>(a, stream);
    if (a.dk == 64 && a.chunk == 32) return a.scalar ? prep_cfg<64, 32, true>(a, stream) : prep_cfg<64, 32, false>(a, stream);
    if (a.dk == 64 && a.chunk == 64) return a.scalar ? prep_cfg<64, 64, true>(a, stream) : prep_cfg<64, 64, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
