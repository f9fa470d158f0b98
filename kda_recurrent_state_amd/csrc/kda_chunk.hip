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
//   T  = (I + A)^-1,  Tb = T diag(b),  W = Tb Kb,  U = Tb L (b V)
//   E  = -(W S + U)
//   O  = Qb S + P1 E + P2 (b V)
//   S <- Diag(e^{g_C}) S + (Kc e^{g_C})^T E + (Kt e^{g_C})^T (b V)
//
// The per-channel decay ("a gate per channel", page "The efficiency lineage",
// item 10) spans hundreds of nats over a chunk, which is the numerical-range
// problem the KDA row of the table mentions.  Factors are therefore split
// around references placed per 16-token sub-block: blocks on the diagonal of
// a C x C product use the sub-block's mid-point (row and column factors stay
// within e^{+-8 max|log a|}, upper-triangle overflow is discarded by select),
// and a block pair (bt > bi) additionally scales the row factor by
// e^{mu_bt - mu_bi} <= 1.  The state-side operands are referenced to the chunk
// start or end, where every factor is <= 1.
//
// Work decomposition: one workgroup (4 wavefronts) per (sequence, head,
// dv-slice of width DVS).  The workgroup walks its sequence chunk by chunk;
// the fp32 state slice [DK x DVS] lives in matrix-core accumulators across the
// walk.  Inputs are read from HBM once per slice (slices of one head are
// placed on one XCD so they share its L2) and o is written once.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr float LOG2E = 1.4426950408889634f;

template <typename T, int DK, int DVS, int C>
struct ChunkCfg {
    static constexpr int NT = 256, NW = NT / WAVE;
    static constexpr int NB = C / 16;                  // 16-token sub-blocks
    static constexpr int NPAIR = NB * (NB - 1) / 2;    // off-diagonal block pairs
    static constexpr int PAD = 16 / sizeof(T);         // one 16-byte pad per row
    static constexpr int LDK = DK + PAD;               // rows with dk contiguous
    static constexpr int LDC = C + PAD;                // rows with tokens contiguous
    static constexpr int LDA = C + 4;                  // fp32 C x C matrices
    static constexpr int NU = (DK / 4) * (C / 4);      // 4 tokens x 4 channels units
    static constexpr int UPT = (NU + NT - 1) / NT;     // units per thread
    static constexpr int NUV = (DVS / 4) * (C / 4);    // value units
    static constexpr int NST = (DK / 16) * (DVS / 16); // state tiles
    static constexpr int STPW = (NST + NW - 1) / NW;   // state tiles per wavefront
};

template <typename T, int DK, int DVS, int C>
struct ChunkLds {
    typedef ChunkCfg<T, DK, DVS, C> G;
    alignas(16) T Kr[C * G::LDK];    // K e^{g_{t-1} - mid}   Gram rows (A, L)
    alignas(16) T Qr[C * G::LDK];    // Q e^{g_t - mid}       Gram rows (P1, P2)
    alignas(16) T Kce[C * G::LDK];   // K e^{mid - g_{t-1}}   Gram columns (A, P1)
    alignas(16) T Kci[C * G::LDK];   // K e^{mid - g_t}       Gram columns (L, P2)
    alignas(16) T Qbar[C * G::LDK];  // Q e^{g_t}
    alignas(16) T W[C * G::LDK];     // Tb Kbar
    alignas(16) T ST[DVS * G::LDK];  // state slice, transposed [j][c]
    alignas(16) T KbarT[DK * G::LDC];  // (K e^{g_{t-1}})^T
    alignas(16) T KccT[DK * G::LDC];   // (K e^{g_C - g_{t-1}})^T
    alignas(16) T KtcT[DK * G::LDC];   // (K e^{g_C - g_t})^T
    alignas(16) T VT[DVS * G::LDC];    // (b V)^T
    alignas(16) T YT[DVS * G::LDC];    // (L b V)^T
    alignas(16) T ET[DVS * G::LDC];    // E^T
    alignas(16) T L[C * G::LDC];
    alignas(16) T P1[C * G::LDC];
    alignas(16) T P2[C * G::LDC];
    alignas(16) T Tb[C * G::LDC];
    alignas(16) float A[C * G::LDA];   // diag(b) strict_lower(Kb Kc^T), fp32
    alignas(16) float Tm[C * G::LDA];  // (I + A)^-1, fp32
    alignas(16) float X[(G::NB > 1 ? G::NB - 1 : 1) * 256];
    alignas(16) float grp[(C / 4) * DK];  // per 4-token group: summed log2 decay
    alignas(16) float emu[G::NB * DK];    // e^{mu_b}
    alignas(16) float ecmu[G::NB * DK];   // e^{g_C - mu_b}
    alignas(16) float F[(G::NPAIR > 0 ? G::NPAIR : 1) * DK];  // e^{mu_bt - mu_bi}
    alignas(16) float gam[DK];            // e^{g_C}
    alignas(16) float beta[C];
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
};

template <typename T, int DK, int DVS, int C, bool SCALAR>
__global__ void __launch_bounds__(256) kda_chunk_kernel(ChunkParams p) {
    typedef ChunkCfg<T, DK, DVS, C> G;
    typedef Mma<T> M;
    constexpr int NT = G::NT, NW = G::NW, NB = G::NB, LDK = G::LDK, LDC = G::LDC, LDA = G::LDA;
    __shared__ ChunkLds<T, DK, DVS, C> s;

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
    }

    // state slice in accumulators: tile ix = wv + NW * i -> (mi, ni)
    f32x4 acc[G::STPW];
    const int64_t sbase = ((int64_t)n * H + h) * DK * DV + dv0;
#pragma unroll
    for (int i = 0; i < G::STPW; ++i) {
        const int ix = wv + NW * i;
        acc[i] = zero4();
        if (ix < G::NST && p.S0) {
            const int mi = ix / (DVS / 16), ni = ix % (DVS / 16);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[i][r] = p.S0[sbase + (int64_t)(16 * mi + 4 * lgrp + r) * DV + 16 * ni + lrow];
        }
    }

    for (int64_t t0 = tb; t0 < te; t0 += C) {
        const int Lc = (int)((te - t0) < C ? (te - t0) : C);

        // ---- I1: loads, decay sums per 4-token group, b V ----------------------------
        f32x4 lam[G::UPT][4], qv[G::UPT][4], kv[G::UPT][4];
#pragma unroll
        for (int u = 0; u < G::UPT; ++u) {
            const int uu = tid + NT * u;
            if (uu < G::NU) {
                const int c = 4 * (uu % (DK / 4)), tg = uu / (DK / 4);
                f32x4 run = zero4();
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 4 * tg + i;
                    const int64_t row = (t0 + t) * H + h;
                    f32x4 la4 = zero4(), q4 = zero4(), k4 = zero4();
                    if (t < Lc) {
                        if (SCALAR) {
                            const float x = p.log_a[row];
                            la4 = f32x4{x, x, x, x};
                        } else {
                            la4 = *reinterpret_cast<const f32x4*>(p.log_a + row * DK + c);
                        }
                        q4 = load4(gq + row * DK + c);
                        k4 = load4(gk + row * DK + c);
                    }
                    run += la4 * LOG2E;
                    lam[u][i] = run;
                    qv[u][i] = q4;
                    kv[u][i] = k4;
                }
                *reinterpret_cast<f32x4*>(&s.grp[tg * DK + c]) = run;
            }
        }
        for (int t = tid; t < C; t += NT) s.beta[t] = t < Lc ? p.beta[(t0 + t) * H + h] : 0.f;
        for (int uv = tid; uv < G::NUV; uv += NT) {
            const int j = 4 * (uv % (DVS / 4)), tg = uv / (DVS / 4);
            f32x4 vals[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * tg + i;
                vals[i] = zero4();
                if (t < Lc) {
                    const int64_t row = (t0 + t) * H + h;
                    vals[i] = p.beta[row] * load4(gv + row * DV + dv0 + j);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                store4(&s.VT[(j + e) * LDC + 4 * tg],
                       f32x4{vals[0][e], vals[1][e], vals[2][e], vals[3][e]});
        }
        __syncthreads();

        // ---- I2: decay factors, Gram operands, per-block constants -------------------
        // rin = e^{g_t - mid}, rex = e^{g_{t-1} - mid}; cin, cex their reciprocals.
        // Exponents are clamped to the fp32 range so no factor is inf or zero.
        f32x4 rin[G::UPT][4], rex[G::UPT][4], cin[G::UPT][4], cex[G::UPT][4];
#pragma unroll
        for (int u = 0; u < G::UPT; ++u) {
            const int uu = tid + NT * u;
            if (uu < G::NU) {
                const int c = 4 * (uu % (DK / 4)), tg = uu / (DK / 4);
                const int b = tg / 4, gib = tg % 4;
                f32x4 off = zero4();
                for (int g = 0; g < gib; ++g) off += *reinterpret_cast<const f32x4*>(&s.grp[(4 * b + g) * DK + c]);
                const f32x4 mid = *reinterpret_cast<const f32x4*>(&s.grp[(4 * b) * DK + c]) +
                                  *reinterpret_cast<const f32x4*>(&s.grp[(4 * b + 1) * DK + c]);
                f32x4 prev, prevc;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    prev[e] = __builtin_amdgcn_exp2f(__builtin_amdgcn_fmed3f(off[e] - mid[e], -126.f, 126.f));
                    prevc[e] = __builtin_amdgcn_rcpf(prev[e]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 4 * tg + i;
                    f32x4 ri, ci;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ri[e] = __builtin_amdgcn_exp2f(
                            __builtin_amdgcn_fmed3f(off[e] + lam[u][i][e] - mid[e], -126.f, 126.f));
                        ci[e] = __builtin_amdgcn_rcpf(ri[e]);
                    }
                    rin[u][i] = ri; cin[u][i] = ci;
                    rex[u][i] = prev; cex[u][i] = prevc;
                    prev = ri; prevc = ci;
                    store4(&s.Kr[t * LDK + c], kv[u][i] * rex[u][i]);
                    store4(&s.Qr[t * LDK + c], qv[u][i] * ri);
                    store4(&s.Kce[t * LDK + c], kv[u][i] * cex[u][i]);
                    store4(&s.Kci[t * LDK + c], kv[u][i] * ci);
                }
            }
        }
        // per (sub-block, channel) constants
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
            const float gC = rho[NB];
            s.emu[b * DK + c] = exp2f(mu[b]);
            s.ecmu[b * DK + c] = exp2f(gC - mu[b]);
            if (b == 0) s.gam[c] = exp2f(gC);
            for (int bi = 0; bi < b; ++bi) s.F[(b * (b - 1) / 2 + bi) * DK + c] = exp2f(mu[b] - mu[bi]);
        }
        __syncthreads();

        // ---- I3: Gram products (matrix cores) and state-side operands ----------------
        for (int w = wv; w < NB * (NB + 1); w += NW) {
            const int pr = w >> 1, rt = w & 1;  // block pair, row type (0: K rows, 1: Q rows)
            int bt = 0;
            while ((bt + 1) * (bt + 2) / 2 <= pr) ++bt;
            const int bi = pr - bt * (bt + 1) / 2;
            const T* rows = (rt ? s.Qr : s.Kr) + 16 * bt * LDK;
            const T* cols_e = s.Kce + 16 * bi * LDK;
            const T* cols_i = s.Kci + 16 * bi * LDK;
            const float* F = s.F + (bt * (bt - 1) / 2 + bi) * DK;
            f32x4 ge = zero4(), gi = zero4();
#pragma unroll
            for (int kk = 0; kk < DK; kk += M::K) {
                typename M::frag rb = M::load(rows + kk, LDK, lane);
                if (bt != bi) rb = M::scale(rb, F + kk + lgrp * M::KPL);
                ge = M::mma(M::load(cols_e + kk, LDK, lane), rb, ge);
                gi = M::mma(M::load(cols_i + kk, LDK, lane), rb, gi);
            }
            // tile holds G^T: lane column t, rows i = 16 bi + 4 lgrp + r
            const int t = 16 * bt + lrow, i0 = 16 * bi + 4 * lgrp;
            f32x4 me, mi;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + r;
                me[r] = (rt ? i <= t : i < t) ? ge[r] : 0.f;
                mi[r] = (rt ? i <= t : i < t) ? gi[r] : 0.f;
            }
            if (rt == 0) {
                *reinterpret_cast<f32x4*>(&s.A[t * LDA + i0]) = s.beta[t] * me;
                store4(&s.L[t * LDC + i0], mi);
            } else {
                store4(&s.P1[t * LDC + i0], me);
                store4(&s.P2[t * LDC + i0], mi);
            }
        }
#pragma unroll
        for (int u = 0; u < G::UPT; ++u) {
            const int uu = tid + NT * u;
            if (uu < G::NU) {
                const int c = 4 * (uu % (DK / 4)), tg = uu / (DK / 4);
                const int b = tg / 4;
                const f32x4 em = *reinterpret_cast<const f32x4*>(&s.emu[b * DK + c]);
                const f32x4 ec = *reinterpret_cast<const f32x4*>(&s.ecmu[b * DK + c]);
                f32x4 kb[4], kc[4], kt[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 4 * tg + i;
                    store4(&s.Qbar[t * LDK + c], qv[u][i] * rin[u][i] * em);
                    kb[i] = kv[u][i] * rex[u][i] * em;
                    kc[i] = kv[u][i] * cex[u][i] * ec;
                    kt[i] = kv[u][i] * cin[u][i] * ec;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    store4(&s.KbarT[(c + e) * LDC + 4 * tg], f32x4{kb[0][e], kb[1][e], kb[2][e], kb[3][e]});
                    store4(&s.KccT[(c + e) * LDC + 4 * tg], f32x4{kc[0][e], kc[1][e], kc[2][e], kc[3][e]});
                    store4(&s.KtcT[(c + e) * LDC + 4 * tg], f32x4{kt[0][e], kt[1][e], kt[2][e], kt[3][e]});
                }
            }
        }
        __syncthreads();

        // ---- I4: diagonal blocks of (I + A)^-1; Y = L (b V); state -> LDS -------------
        if (wv < NB) {
            const int b = wv;
            if (lane < 16) {
                const int j = lane;
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float* arow = &s.A[(16 * b + r) * LDA + 16 * b];
                    float a = (r == j) ? 1.f : 0.f;
#pragma unroll
                    for (int m = 0; m < r; ++m) a -= arow[m] * x[m];
                    x[r] = a;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) s.Tm[(16 * b + r) * LDA + 16 * b + j] = x[r];
            }
        }
        {
            constexpr int NY = (C / 16) * (DVS / 16);
            for (int w = (wv + NW - NB) % NW; w < NY; w += NW) {
                const int mt = w / (DVS / 16), nj = w % (DVS / 16);
                f32x4 y = tile_mma<T, C>(s.L + 16 * mt * LDC, LDC, s.VT + 16 * nj * LDC, LDC, zero4(), lane);
                store4(&s.YT[(16 * nj + lrow) * LDC + 16 * mt + 4 * lgrp], y);
            }
        }
#pragma unroll
        for (int i = 0; i < G::STPW; ++i) {
            const int ix = wv + NW * i;
            if (ix < G::NST) {
                const int mi = ix / (DVS / 16), ni = ix % (DVS / 16);
                store4(&s.ST[(16 * ni + lrow) * LDK + 16 * mi + 4 * lgrp], acc[i]);
            }
        }
        __syncthreads();

        // ---- I5: off-diagonal blocks of (I + A)^-1, level by level ------------------
        for (int bi = 1; bi < NB; ++bi) {
            for (int e = tid; e < bi * 256; e += NT) {
                const int bj = e / 256, r = (e / 16) % 16, jj = e % 16;
                float a = 0.f;
                for (int kb = bj; kb < bi; ++kb)
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        a += s.A[(16 * bi + r) * LDA + 16 * kb + m] * s.Tm[(16 * kb + m) * LDA + 16 * bj + jj];
                s.X[e] = a;
            }
            __syncthreads();
            for (int e = tid; e < bi * 256; e += NT) {
                const int bj = e / 256, r = (e / 16) % 16, jj = e % 16;
                float a = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    if (m <= r) a -= s.Tm[(16 * bi + r) * LDA + 16 * bi + m] * s.X[bj * 256 + m * 16 + jj];
                s.Tm[(16 * bi + r) * LDA + 16 * bj + jj] = a;
            }
            __syncthreads();
        }
        for (int e = tid; e < C * C; e += NT) {
            const int t = e / C, i = e % C;
            s.Tb[t * LDC + i] = from_f32<T>(i <= t ? s.Tm[t * LDA + i] * s.beta[i] : 0.f);
        }
        __syncthreads();

        // ---- I6: W = Tb Kbar, computed as W^T = Kbar^T Tb^T ------------------------
        {
            constexpr int NWT = (DK / 16) * (C / 16);
            for (int w = wv; w < NWT; w += NW) {
                const int mc = w / (C / 16), nt = w % (C / 16);
                f32x4 x = tile_mma<T, C>(s.KbarT + 16 * mc * LDC, LDC, s.Tb + 16 * nt * LDC, LDC, zero4(), lane);
                store4(&s.W[(16 * nt + lrow) * LDK + 16 * mc + 4 * lgrp], x);
            }
        }
        __syncthreads();

        // ---- I7: E = -(Tb Y + W S) ------------------------------------------------
        {
            constexpr int NE = (C / 16) * (DVS / 16);
            for (int w = wv; w < NE; w += NW) {
                const int mt = w / (DVS / 16), nj = w % (DVS / 16);
                f32x4 x = tile_mma<T, C>(s.Tb + 16 * mt * LDC, LDC, s.YT + 16 * nj * LDC, LDC, zero4(), lane);
                x = tile_mma<T, DK>(s.W + 16 * mt * LDK, LDK, s.ST + 16 * nj * LDK, LDK, x, lane);
                store4(&s.ET[(16 * nj + lrow) * LDC + 16 * mt + 4 * lgrp], -x);
            }
        }
        __syncthreads();

        // ---- I8: outputs O^T = S^T Qbar^T + E^T P1^T + (bV)^T P2^T; state update ------
        {
            constexpr int NO = (DVS / 16) * (C / 16);
            for (int w = wv; w < NO; w += NW) {
                const int mj = w / (C / 16), nt = w % (C / 16);
                f32x4 x = tile_mma<T, DK>(s.ST + 16 * mj * LDK, LDK, s.Qbar + 16 * nt * LDK, LDK, zero4(), lane);
                x = tile_mma<T, C>(s.ET + 16 * mj * LDC, LDC, s.P1 + 16 * nt * LDC, LDC, x, lane);
                x = tile_mma<T, C>(s.VT + 16 * mj * LDC, LDC, s.P2 + 16 * nt * LDC, LDC, x, lane);
                const int t = 16 * nt + lrow;
                if (t < Lc) store4(go + ((t0 + t) * H + h) * DV + dv0 + 16 * mj + 4 * lgrp, x);
            }
        }
#pragma unroll
        for (int i = 0; i < G::STPW; ++i) {
            const int ix = wv + NW * i;
            if (ix < G::NST) {
                const int mi = ix / (DVS / 16), ni = ix % (DVS / 16);
                const f32x4 gm = *reinterpret_cast<const f32x4*>(&s.gam[16 * mi + 4 * lgrp]);
                f32x4 x = acc[i] * gm;
                x = tile_mma<T, C>(s.KccT + 16 * mi * LDC, LDC, s.ET + 16 * ni * LDC, LDC, x, lane);
                x = tile_mma<T, C>(s.KtcT + 16 * mi * LDC, LDC, s.VT + 16 * ni * LDC, LDC, x, lane);
                acc[i] = x;
            }
        }
        __syncthreads();
    }

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

template <typename T, int DK, int DVS, int C, bool SC>
static hipError_t launch_cfg(const ChunkArgs& a, hipStream_t stream) {
    ChunkParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.log_a = a.log_a; p.beta = a.beta; p.S0 = a.S0;
    p.cu = a.cu_seqlens; p.o = a.o; p.ST = a.S_T;
    p.H = a.num_heads; p.DV = a.dv; p.split = a.split;
    p.eq_len = a.cu_seqlens ? 0 : a.total_tokens / (a.num_seqs > 0 ? a.num_seqs : 1);
    const int64_t blocks = (int64_t)a.num_seqs * a.num_heads * a.split;
    p.xcd_group = (blocks % 8 == 0 && (blocks / 8) % a.split == 0) ? 1 : 0;
    hipLaunchKernelGGL((kda_chunk_kernel<T, DK, DVS, C, SC>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

template <typename T, int DK, int DVS, int C>
static bool try_cfg(int scalar, bool launch, const ChunkArgs* a, hipStream_t stream, hipError_t* err) {
    if constexpr (chunk_fits<T, DK, DVS, C>()) {
        if (launch) *err = scalar ? launch_cfg<T, DK, DVS, C, true>(*a, stream)
                                  : launch_cfg<T, DK, DVS, C, false>(*a, stream);
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
        KDA_CHUNK_CASE(float, 64, 16, 32) KDA_CHUNK_CASE(float, 64, 32, 32)
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
