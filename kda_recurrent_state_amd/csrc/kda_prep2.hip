// kda_prep2.hip -- chunk-parallel pass of the two-pass KDA prefill for dk = 128
// on gfx950 (the operator blocks of kda_ws.hpp, same math as kda_prep.hip).
//
// The chunkwise (WY) form (page "The argument, in one page", section
// "Everything, in one table", row "Chunkwise / WY") separates each chunk's
// state-independent work from the short state recurrence.  Per chunk of 32
// tokens (g_t the running sum of log a, b = beta, mid-point reference mu_b of
// each 16-token block, F = e^{mu_1 - mu_0}):
//   A  = strict_lower(diag(b) Kb Kc^T)   L = strict_lower(Kb Kt^T)
//   P1 = lower(Qb Kc^T)                  P2 = lower(Qb Kt^T)
//   Tb = (I + A)^-1 diag(b),  R = P1 Tb
//   W  = Tb Kb,  QP = Qb - R Kb,  M1 = Tb L diag(b),  M2 = P2 diag(b) - R L diag(b)
//   KC = (K e^{g_C - g_{t-1}})^T,  KT = (diag(b) K e^{g_C - g_t})^T,  GAM = e^{g_C}
//
// The decay-first ordering (ORD1, blocks of kda_ws.hpp without KT) takes
// Kb = K e^{g_t} and Kc = Kt, forms only A and P2 (unscaled, in place of P1),
// and runs phase D unchanged with L diag(b) = -I and P2 diag(b) = 0, which
// gives M1 = -Tb and M2 = R; KC = (K e^{g_C - g_t})^T.
//
// Work decomposition: one workgroup of four wavefronts per chunk (persistent
// workgroups walk a strided list of chunks, two per compute unit).  In the
// elementwise phase thread (c2, o) owns the channel pair 2 c2, 2 c2 + 1 and
// the token octet o (tokens 8 o .. 8 o + 7; octets 0 and 2 end at their
// block's mid-point, octets 1 and 3 start right after it).  Its decay factors
// relative to the mid-point are running products of a = 2^{log2e log a} and
// 1 / a along its eight tokens, so each token costs two exponentials and no
// cross-thread scan; the octet totals, exchanged through LDS, give e^{mu_b},
// e^{g_C - mu_b}, F and e^{g_C}.  This factor split is exact to ~2^-30 while
// every valid token of the chunk has log2 a >= STEEP_LOG2 (kda_chunk_common.hpp).
// A chunk with a steeper token is marked (GAM[0] = -1; a true GAM lies in
// [0, 1]) and its whole block is formed again by kda_prep2_exact_kernel, which
// takes every decay factor as one exponential of a run of consecutive log2
// decays; the clamp of log2 a at -15 below only keeps the discarded values of
// such a chunk finite.
//
// Phases (LDS barriers between them):
//   A1 inputs -> factors -> mid-referenced Gram operands, octet products
//   A2 chunk-referenced operands: KbT, Qb to LDS; KC, KT, GAM to the block
//   B  the four Gram products on bf16 matrix cores (wavefront g: product g)
//   C  (I + A)^-1 by blocked forward substitution; Tb and Tb^T to LDS
//   D  R, W, QP, M1, M2 on matrix cores, each output lane writing 16 bytes
// The next chunk's inputs are loaded into registers during phases B-D.
#include "kda_chunk_common.hpp"
#include "kda_launch.hpp"
#include "kda_ws.hpp"

namespace kda {

namespace p2 {
constexpr int DK = 128, C = 32, NT = 256;
// Row pitches.  Channel rows are 288 bytes: measured on gfx950 (one access
// pattern at a time over the whole chip), the Gram fragment reads of phase B
// (16 rows x 16 bytes per lane group) take 4 LDS cycles with this pitch and 8
// with 272-byte rows.
constexpr int LDK = DK + 16; // bf16 rows over channels
constexpr int LDC = C + 8;   // bf16 rows over tokens
constexpr int LDA = C + 4;   // fp32 rows over tokens
constexpr float LA_MIN = -15.f;  // log2 clamp inside the factor split (never reached in its range)
}  // namespace p2

struct Prep2Lds {
    union {
        struct {  // phases A1-B: mid-referenced Gram operands [token][channel]
            bf16 Kr[p2::C * p2::LDK], Qr[p2::C * p2::LDK], Kce[p2::C * p2::LDK], Kci[p2::C * p2::LDK];
        } g;
        struct {  // phase C
            float Tf[p2::C * p2::LDA];  // (I + A)^-1, fp32, lower triangle
            float Xs[16 * 17];
            float X[2 * 512];
        } v;
        struct {  // exact kernel, phases A2-B: raw rows and log2 decays for exact_gram
            bf16 K[p2::C * p2::LDK], Q[p2::C * p2::LDK];
            float LA[p2::C * p2::DK];
        } x;
    } u;
    alignas(16) bf16 KbT[p2::DK * p2::LDC];  // (K e^{g_{t-1}})^T [channel][permuted token]
    alignas(16) bf16 Qb[p2::C * p2::LDK];    // Q e^{g_t} [token][channel]
    alignas(16) float A[p2::C * p2::LDA];    // diag(b) strict_lower(Kb Kc^T) [t][i]
    alignas(16) float P2b[p2::C * p2::LDA];  // lower(Qb Kt^T) diag(b) [t][i]
    alignas(16) bf16 P1[p2::C * p2::LDC];    // lower(Qb Kc^T) [t][i]
    alignas(16) bf16 LbT[p2::C * p2::LDC];   // (L diag(b))^T [i][permuted t]
    alignas(16) bf16 Tb[p2::C * p2::LDC];    // (I + A)^-1 diag(b) [t][permuted s]
    alignas(16) bf16 TbT[p2::C * p2::LDC];   // its transpose [s][t]
    alignas(16) float F[p2::DK];             // e^{mu_1 - mu_0}
    alignas(16) float Pq[4 * p2::DK];        // product of a over each token octet (exact kernel:
                                             // sum of log2 a)
    int steep[4];                            // per wavefront: a token below STEEP_LOG2
    float ltok[p2::C];                       // scalar decay: log2 a of each token
    float gtok[p2::C];                       // scalar decay: running sum of log2 a to each token
    int list[p2::NT];                        // exact kernel: marked items of one round
    alignas(16) float beta[p2::C];
    alignas(16) float ones[16];
};

struct Prep2Params {
    const void* q;
    const void* k;
    const float* log_a;
    const float* beta;
    const int32_t* cu;
    int64_t eq_len;
    uint8_t* ws;      // operator blocks [unit][m]
    int H;
    int m;            // chunks per unit in this segment (block stride)
    int items;        // units * m
    int64_t chunk0;   // first chunk index of the segment
    Prologue pro;     // input prologue (instantiations with PRO only)
};

// Raw inputs of one thread as loaded: 16 bytes per lane and row, so each vector
// memory instruction moves 1 KB.  lq/lk[g]: 8 channels (8 (lane >> 2) ..) of
// token 8 o + 4 g + (lane & 3); la[p]: 4 channels (4 (lane >> 1) ..) of token
// 8 o + 2 p + (lane & 1) (per-channel decay), or log a of token 8 o + j in
// element j % 4 of la[j / 4] (scalar decay).  b: beta of token `tid` (threads
// below C).
struct Prep2Raw {
    i32x4 lq[2], lk[2];
    f32x4 la[4];
    float b;
};

// The thread's own inputs after redistribution inside lane quads: channels
// 2 lane, 2 lane + 1 of tokens 8 o + j.
struct Prep2In {
    uint32_t q[8], k[8];  // bf16 pairs
    f32x2 la[8];
};

__device__ __forceinline__ float dppf_swap1(float x) {
    return __builtin_bit_cast(float, dpp<0xB1>(__builtin_bit_cast(int, x)));  // quad_perm [1, 0, 3, 2]
}

template <bool SCALAR>
__device__ __forceinline__ void prep2_unpack(const Prep2Raw& r, int lane, Prep2In& in) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const i32x4 tq = quad_transpose(r.lq[g], lane), tk = quad_transpose(r.lk[g], lane);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            in.q[4 * g + d] = (uint32_t)tq[d];
            in.k[4 * g + d] = (uint32_t)tk[d];
        }
    }
    if (SCALAR) {
#pragma unroll
        for (int j = 0; j < 8; ++j) in.la[j] = f32x2{r.la[j >> 2][j & 3], r.la[j >> 2][j & 3]};
    } else {
        // lane 2 m + u holds token 2 p + u, channels 4 m .. 4 m + 3; it keeps channels
        // 4 m + 2 u, + 1 of both tokens, swapping the other half with its neighbour
        const bool u = lane & 1;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const f32x4 v = r.la[p];
            const float s0 = u ? v[0] : v[2], s1 = u ? v[1] : v[3];
            const float r0 = dppf_swap1(s0), r1 = dppf_swap1(s1);
            in.la[2 * p] = u ? f32x2{r0, r1} : f32x2{v[0], v[1]};
            in.la[2 * p + 1] = u ? f32x2{v[2], v[3]} : f32x2{r0, r1};
        }
    }
}

__device__ __forceinline__ bool prep2_locate(const Prep2Params& p, int item, int64_t& t0, int& Lc, int& h) {
    const int unit = item / p.m, j = item % p.m;
    const int n = unit / p.H;
    h = unit % p.H;
    int64_t tb, te;
    if (p.cu) { tb = p.cu[n]; te = p.cu[n + 1]; }
    else { tb = (int64_t)n * p.eq_len; te = tb + p.eq_len; }
    t0 = tb + (p.chunk0 + j) * p2::C;
    Lc = (int)((te - t0) < p2::C ? (te - t0) : p2::C);
    return t0 < te;
}

template <bool SCALAR>
__device__ __forceinline__ void prep2_load(const Prep2Params& p, int64_t t0, int Lc, int h, int tid, int lane, int o,
                                           Prep2Raw& in) {
    const bf16* __restrict__ gq = static_cast<const bf16*>(p.q);
    const bf16* __restrict__ gk = static_cast<const bf16*>(p.k);
    const int64_t r0 = t0 * p.H + h;
    // rows past the chunk's end repeat its last row; b and log a are masked there
    auto row = [&](int t) { return r0 + (int64_t)min(t, Lc - 1) * p.H; };
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int64_t rw = row(8 * o + 4 * g + (lane & 3));
        in.lq[g] = *reinterpret_cast<const i32x4*>(gq + rw * p2::DK + 8 * (lane >> 2));
        in.lk[g] = *reinterpret_cast<const i32x4*>(gk + rw * p2::DK + 8 * (lane >> 2));
    }
    if (SCALAR) {
#pragma unroll
        for (int j = 0; j < 8; ++j) in.la[j >> 2][j & 3] = p.log_a[row(8 * o + j)];
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            in.la[q] = *reinterpret_cast<const f32x4*>(p.log_a + row(8 * o + 2 * q + (lane & 1)) * p2::DK +
                                                       4 * (lane >> 1));
    }
    in.b = (tid < Lc) ? p.beta[r0 + (int64_t)tid * p.H] : 0.f;
}

// Phases C and D of one chunk (after B): T = (I + A)^-1 and the block's W, QP, M1
// and M2.  Reads A, P1, P2b, LbT, KbT, Qb and beta from LDS; shared by both kernels.
template <bool ORD1>
__device__ __forceinline__ void prep2_solve_store(Prep2Lds& s, uint8_t* __restrict__ blk, int tid, int lane,
                                                  int wv) {
    using namespace p2;
    typedef WsBlock<DK, C, ORD1> WS;
    typedef Mma<bf16> M;
    const int lr = lane & 15, lg = lane >> 4;
    // ---- C: T = (I + A)^-1: diagonal blocks on wavefronts 0 and 1, then
    //      T21 = -T22 A21 T11 on wavefront 0 ---------------------------------------------
    if (wv < 2)
        block_inverse<float, 16, LDA, LDA>(s.A + 16 * wv * LDA + 16 * wv, s.ones, s.u.v.X + wv * 512,
                                           s.u.v.Tf + 16 * wv * LDA + 16 * wv, lane);
    lds_barrier();
    if (wv == 0) {
        f32x4 x = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kk = 4 * ks + lg;
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(s.A[(16 + lr) * LDA + kk], s.u.v.Tf[kk * LDA + lr], x, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) s.u.v.Xs[(4 * lg + r) * 17 + lr] = x[r];
        wave_sync();
        f32x4 t = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kk = 4 * ks + lg;
            t = __builtin_amdgcn_mfma_f32_16x16x4f32(s.u.v.Tf[(16 + lr) * LDA + 16 + kk], s.u.v.Xs[kk * 17 + lr], t,
                                                     0, 0, 0);
        }
        // T21 = -t: rows 16 + 4 lg + r, column lr.  Tb = T diag(b) at permuted
        // columns; Tb^T rows are columns of T (four consecutive rows here)
        const float bcol = s.beta[lr];
        f32x4 tb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            tb[r] = -t[r] * bcol;
            s.Tb[(16 + 4 * lg + r) * LDC + kperm(lr)] = (bf16)tb[r];
        }
        store4(&s.TbT[lr * LDC + 16 + 4 * lg], tb);
    } else {
        // diagonal blocks on wavefronts 1-3: (block, row t, column run 4 u .. 4 u + 3)
        for (int e = tid - 64; e < 128; e += 192) {
            const int bb = e >> 6, t = (e >> 2) & 15, u = e & 3;
            const int row = 16 * bb + t, col = 16 * bb + 4 * u;
            const f32x4 x = *reinterpret_cast<const f32x4*>(&s.u.v.Tf[row * LDA + col]) *
                            *reinterpret_cast<const f32x4*>(&s.beta[col]);
            store4(&s.Tb[row * LDC + kperm(col)], x);
#pragma unroll
            for (int r = 0; r < 4; ++r) s.TbT[(col + r) * LDC + row] = (bf16)x[r];
        }
    }
    lds_barrier();

    // ---- D: wavefront w: token tile tt = w & 1; channel pairs 2 (w >> 1) and
    //      2 (w >> 1) + 1 of W and QP; M1 (w < 2) or M2 (w >= 2) --------------------------
    {
        const int tt = wv & 1, half = wv >> 1;
        const int t = 16 * tt + lr;
        // R = P1 Tb as a B-operand fragment: out[s][t] = sum_i TbT[s][i] P1[t][i]
        const M::frag p1f = M::loadr(s.P1 + t * LDC, lane);
        const f32x4 r0 = M::mma(M::loadr(s.TbT + lr * LDC, lane), p1f, zero4());
        const f32x4 r1 = M::mma(M::loadr(s.TbT + (16 + lr) * LDC, lane), p1f, zero4());
        M::frag rfr;
#pragma unroll
        for (int i = 0; i < 4; ++i) { rfr[i] = (bf16)r0[i]; rfr[4 + i] = (bf16)r1[i]; }
        const M::frag tbf = M::loadr(s.Tb + t * LDC, lane);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int cp = 2 * half + cc;  // 32-channel block
            const M::frag kb0 = M::loadr(s.KbT + (32 * cp + lr) * LDC, lane);
            const M::frag kb1 = M::loadr(s.KbT + (32 * cp + 16 + lr) * LDC, lane);
            const f32x4 w0 = M::mma(kb0, tbf, zero4()), w1 = M::mma(kb1, tbf, zero4());
            const f32x4 x0 = M::mma(kb0, rfr, zero4()), x1 = M::mma(kb1, rfr, zero4());
            const f32x4 q0 = load4(&s.Qb[t * LDK + 32 * cp + 4 * lg]);
            const f32x4 q1 = load4(&s.Qb[t * LDK + 32 * cp + 16 + 4 * lg]);
            bf16x8 wo, qo;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                wo[r] = (bf16)w0[r]; wo[4 + r] = (bf16)w1[r];
                qo[r] = (bf16)(q0[r] - x0[r]); qo[4 + r] = (bf16)(q1[r] - x1[r]);
            }
            *reinterpret_cast<bf16x8*>(blk + WS::W + swz<2 * DK>(kinv(t), 4 * cp + lg)) = wo;
            *reinterpret_cast<bf16x8*>(blk + WS::QP + swz<2 * DK>(t, 4 * cp + lg)) = qo;
        }
        // rows i of (L diag(b))^T taken so that lane group lg ends with columns
        // 8 lg .. 8 lg + 7 of M1 or M2 (tile 0: i = 8 lg + r, tile 1: 8 lg + 4 + r)
        const int li = 8 * (lr >> 2) + (lr & 3);
        const M::frag lb0 = M::loadr(s.LbT + li * LDC, lane);
        const M::frag lb1 = M::loadr(s.LbT + (li + 4) * LDC, lane);
        bf16x8 mo;
        if (half == 0) {  // M1 = Tb (L diag(b)): out[i][t], row t of M1 at W's row for t
            const f32x4 m0 = M::mma(lb0, tbf, zero4()), m1 = M::mma(lb1, tbf, zero4());
#pragma unroll
            for (int r = 0; r < 4; ++r) { mo[r] = (bf16)m0[r]; mo[4 + r] = (bf16)m1[r]; }
            *reinterpret_cast<bf16x8*>(blk + WS::M1 + piece<C>(kinv(t), lg)) = mo;
        } else {  // M2 = P2 diag(b) - R (L diag(b))
            const f32x4 m0 = M::mma(lb0, rfr, zero4()), m1 = M::mma(lb1, rfr, zero4());
            const f32x4 pa = *reinterpret_cast<const f32x4*>(&s.P2b[t * LDA + 8 * lg]);
            const f32x4 pb = *reinterpret_cast<const f32x4*>(&s.P2b[t * LDA + 8 * lg + 4]);
#pragma unroll
            for (int r = 0; r < 4; ++r) { mo[r] = (bf16)(pa[r] - m0[r]); mo[4 + r] = (bf16)(pb[r] - m1[r]); }
            *reinterpret_cast<bf16x8*>(blk + WS::M2 + piece<C>(t, lg)) = mo;
        }
    }
}

// Phases A1-A2 of a marked chunk in kda_prep2_exact_kernel.  Kb, Qb, KC, KT and
// GAM are formed with one exponential each from running sums of log2 a
// referenced to the chunk start (prefixes) or end (suffixes): every exponent is
// a run of consecutive decays, so each factor is exact for any decay.  The raw
// rows (k after the prologue's scaling) and the log2 decays go to LDS for
// exact_gram.  Thread (c2, o) as in A1 of kda_prep2_kernel; two LDS barriers.
template <bool SCALAR, bool ORD1, bool PRO>
__device__ __forceinline__ void prep2_steep_operands(const Prep2Params& p, Prep2Lds& s, const Prep2Raw& raw,
                                                     uint8_t* blk, int tid, int lane, int c2, int o, int Lc) {
    using namespace p2;
    typedef WsBlock<DK, C, ORD1> WS;
    Prep2In in;
    prep2_unpack<SCALAR>(raw, lane, in);
    float kscale[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kscale[j] = 1.f;
    if (PRO && p.pro.normalize_k) {
        float ss[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const Vec2<bf16>::type kv = __builtin_bit_cast(Vec2<bf16>::type, in.k[j]);
            const float k0 = Vec2<bf16>::lo(kv), k1 = Vec2<bf16>::hi(kv);
            ss[j] = row_sum16(k0 * k0 + k1 * k1);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            kscale[j] = rsqrtf(readlanef(ss[j], 0) + readlanef(ss[j], 16) + readlanef(ss[j], 32) +
                               readlanef(ss[j], 48) + PROLOGUE_EPS);
    }
    f32x2 l2[8];
    f32x2 lsum = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        l2[j] = in.la[j] * LOG2E;
        if (PRO && p.pro.log_a_raw) {
            const float lo2 = p.pro.log_a_min * LOG2E;
            l2[j] = f32x2{prologue_log2_a(in.la[j][0], lo2), prologue_log2_a(in.la[j][1], lo2)};
        }
        if (8 * o + j >= Lc) l2[j] = f32x2{0.f, 0.f};
        lsum += l2[j];
    }
    *reinterpret_cast<f32x2*>(&s.Pq[o * DK + 2 * c2]) = lsum;
    if (tid < C) s.beta[tid] = (PRO && p.pro.beta_logits && tid < Lc) ? prologue_beta(raw.b) : raw.b;
    lds_barrier();
    // sums of the octets before and after this one, and the chunk total
    f32x2 pre = {0.f, 0.f}, suf = {0.f, 0.f}, tot = {0.f, 0.f};
#pragma unroll
    for (int oo = 0; oo < 4; ++oo) {
        const f32x2 x = *reinterpret_cast<const f32x2*>(&s.Pq[oo * DK + 2 * c2]);
        tot += x;
        if (oo < o) pre += x;
        if (oo > o) suf += x;
    }
    f32x2 sx[8];  // g_C - g_t
    {
        f32x2 run = suf;
#pragma unroll
        for (int j = 7; j >= 0; --j) {
            sx[j] = run;
            run += l2[j];
        }
    }
    auto ex2v = [](f32x2 x) { return f32x2{__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1])}; };
    f32x2 kb[8], kc[8], kt[8];
    f32x2 gp = pre;  // g_{t-1}
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int t = 8 * o + j;
        const Vec2<bf16>::type kv = __builtin_bit_cast(Vec2<bf16>::type, in.k[j]);
        const Vec2<bf16>::type qv = __builtin_bit_cast(Vec2<bf16>::type, in.q[j]);
        const f32x2 k = f32x2{Vec2<bf16>::lo(kv), Vec2<bf16>::hi(kv)} * kscale[j];
        const f32x2 q = f32x2{Vec2<bf16>::lo(qv), Vec2<bf16>::hi(qv)};
        const f32x2 g = gp + l2[j];
        kb[j] = k * ex2v(ORD1 ? g : gp);
        kc[j] = k * ex2v(ORD1 ? sx[j] : sx[j] + l2[j]);
        kt[j] = k * ex2v(sx[j]) * s.beta[t];
        const f32x2 qb = q * ex2v(g);
        store2(&s.Qb[t * LDK + 2 * c2], qb[0], qb[1]);
        store2(&s.u.x.K[t * LDK + 2 * c2], k[0], k[1]);
        store2(&s.u.x.Q[t * LDK + 2 * c2], q[0], q[1]);
        *reinterpret_cast<f32x2*>(&s.u.x.LA[t * DK + 2 * c2]) = l2[j];
        gp = g;
    }
    if (o == 0) *reinterpret_cast<f32x2*>(blk + WS::GAM + 8 * c2) = ex2v(tot);
    const int pos0 = kperm(8 * o), pos1 = kperm(8 * o + 4);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int c = 2 * c2 + e;
        store4(&s.KbT[c * LDC + pos0], f32x4{kb[0][e], kb[1][e], kb[2][e], kb[3][e]});
        store4(&s.KbT[c * LDC + pos1], f32x4{kb[4][e], kb[5][e], kb[6][e], kb[7][e]});
        bf16x8 kcv, ktv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            kcv[j] = (bf16)kc[j][e];
            ktv[j] = (bf16)kt[j][e];
        }
        *reinterpret_cast<bf16x8*>(blk + WS::KC + piece<DK>(c, o)) = kcv;
        if (!ORD1) *reinterpret_cast<bf16x8*>(blk + WS::KT + piece<DK>(c, o)) = ktv;
    }
    lds_barrier();
}

// Phase B of a marked chunk: the masked Gram products by exact_gram, stored as
// phase B of kda_prep2_kernel stores the factored ones (ORD1: A and P2, P2 in
// P1's slot, L diag(b) = -I and P2 diag(b) = 0 left as set up).
template <bool ORD1>
__device__ __forceinline__ void prep2_steep_gram(Prep2Lds& s, int wv, int lane) {
    using namespace p2;
    exact_gram<bf16, DK, C, 4, ORD1>(s.u.x.K, s.u.x.Q, LDK, s.u.x.LA, DK, wv, lane,
                                     [&](int t, int i, float av, float lv, float p1v, float p2v) {
        s.A[t * LDA + i] = s.beta[t] * av;
        if (ORD1) {
            s.P1[t * LDC + i] = (bf16)p2v;
        } else {
            s.LbT[i * LDC + kperm(t)] = (bf16)(lv * s.beta[i]);
            s.P1[t * LDC + i] = (bf16)p1v;
            s.P2b[t * LDA + i] = p2v * s.beta[i];
        }
    });
}

// The masked matrices that are never written outside their lower triangle start
// at zero (upper blocks stay zero for the whole walk); ORD1 sets L diag(b) = -I.
__device__ __forceinline__ void prep2_init_lds(Prep2Lds& s, int tid, bool ord1) {
    using namespace p2;
    for (int e = tid; e < C * LDC; e += NT) {
        s.LbT[e] = (bf16)0.f; s.P1[e] = (bf16)0.f; s.Tb[e] = (bf16)0.f; s.TbT[e] = (bf16)0.f;
    }
    for (int e = tid; e < C * LDA; e += NT) s.P2b[e] = 0.f;
    if (tid < 16) s.ones[tid] = 1.f;
    if (ord1) {
        lds_barrier();
        if (tid < C) s.LbT[tid * LDC + kperm(tid)] = (bf16)-1.f;
    }
}

// A2 of a scalar-decay chunk (after A1 has put log2 a of every token in ltok):
// running sums referenced to the chunk start (G_t = la_0 + .. + la_t) and end
// (X_t = la_{t+1} + .. + la_{C-1}), each summed in token order, give per-token
// factors, so every channel of a token takes the same two exponentials:
// Kd = k 2^G (KbT), Qb = q 2^G, KC = (k 2^X)^T, GAM = 2^{G_{C-1}}; G goes to gtok
// for the Gram masks.  A chunk with a token below STEEP_LOG2 is marked instead
// (GAM[0] = -1), as in the per-channel path.
template <bool ORD1>
__device__ __forceinline__ void prep2_scalar_operands(Prep2Lds& s, uint8_t* __restrict__ blk, const Prep2In& in,
                                                      const float (&kscale)[8], int lane, int c2, int o) {
    using namespace p2;
    typedef WsBlock<DK, C, ORD1> WS;
    float pre = 0.f, suf = 0.f, tot = 0.f;
    for (int t = 0; t < 8 * o; ++t) pre += s.ltok[t];
    for (int t = C - 1; t >= 8 * o + 8; --t) suf += s.ltok[t];
    for (int t = 0; t < C; ++t) tot += s.ltok[t];
    float G[8], X[8];
    {
        float run = pre;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            run += s.ltok[8 * o + j];
            G[j] = run;
        }
        run = suf;
#pragma unroll
        for (int j = 7; j >= 0; --j) {
            X[j] = run;
            run += s.ltok[8 * o + j];
        }
    }
    float mine = G[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mine = lane == j ? G[j] : mine;
    if (lane < 8) s.gtok[8 * o + lane] = mine;
    if (o == 0) {
        const bool steep_chunk = (s.steep[0] | s.steep[1] | s.steep[2] | s.steep[3]) != 0;
        const float gam = steep_chunk ? -1.f : __builtin_amdgcn_exp2f(tot);
        *reinterpret_cast<f32x2*>(blk + WS::GAM + 8 * c2) = f32x2{gam, gam};
    }
    float fg[8], fx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        fg[j] = __builtin_amdgcn_exp2f(G[j]);
        fx[j] = __builtin_amdgcn_exp2f(X[j]);
    }
    const int pos0 = kperm(8 * o), pos1 = kperm(8 * o + 4);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        float k[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const Vec2<bf16>::type kv = __builtin_bit_cast(Vec2<bf16>::type, in.k[j]);
            k[j] = (e ? Vec2<bf16>::hi(kv) : Vec2<bf16>::lo(kv)) * kscale[j];
        }
        const int c = 2 * c2 + e;
        store4(&s.KbT[c * LDC + pos0], f32x4{k[0] * fg[0], k[1] * fg[1], k[2] * fg[2], k[3] * fg[3]});
        store4(&s.KbT[c * LDC + pos1], f32x4{k[4] * fg[4], k[5] * fg[5], k[6] * fg[6], k[7] * fg[7]});
        bf16x8 kc;
#pragma unroll
        for (int j = 0; j < 8; ++j) kc[j] = (bf16)(k[j] * fx[j]);
        *reinterpret_cast<bf16x8*>(blk + WS::KC + piece<DK>(c, o)) = kc;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const Vec2<bf16>::type qv = __builtin_bit_cast(Vec2<bf16>::type, in.q[j]);
        store2(&s.Qb[(8 * o + j) * LDK + 2 * c2], Vec2<bf16>::lo(qv) * fg[j], Vec2<bf16>::hi(qv) * fg[j]);
    }
}

// Phase B of a scalar-decay chunk (decay-first form): wavefront 0 forms
// A = strict_lower(diag(b) (K K^T) o [2^{G_t - G_i}]), wavefront 3
// P2 = lower((Q K^T) o [2^{G_t - G_i}]) (in P1's slot), each from the raw rows with
// the decay applied to the fp32 result: for i <= t the exponent is <= 0.
__device__ __forceinline__ void prep2_scalar_gram(Prep2Lds& s, int wv, int lane) {
    using namespace p2;
    typedef Mma<bf16> M;
    constexpr int NK = DK / M::K;
    const int lr = lane & 15, lg = lane >> 4;
    const bf16* rows = wv == 0 ? s.u.g.Kr : s.u.g.Qr;
    const bf16* cols = s.u.g.Kr;
    M::frag r0[NK], r1[NK], c0[NK], c1[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        r0[kk] = M::loadr(rows + lr * LDK + kk * M::K, lane);
        r1[kk] = M::loadr(rows + (16 + lr) * LDK + kk * M::K, lane);
        c0[kk] = M::loadr(cols + lr * LDK + kk * M::K, lane);
        c1[kk] = M::loadr(cols + (16 + lr) * LDK + kk * M::K, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int pr = 0; pr < 3; ++pr) {
        const int bt = pr == 0 ? 0 : 1, bi = pr == 2 ? 1 : 0;
        const M::frag* fr = bt == 0 ? r0 : r1;
        const M::frag* fc = bi == 0 ? c0 : c1;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) acc = M::mma(fc[kk], fr[kk], acc);
        // column t = 16 bt + lr, rows i = 16 bi + 4 lg + r
        const int t = 16 * bt + lr, i0 = 16 * bi + 4 * lg;
        const float gt = s.gtok[t];
        f32x4 m;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool keep = wv == 0 ? i0 + r < t : i0 + r <= t;
            m[r] = keep ? acc[r] * __builtin_amdgcn_exp2f(fminf(gt - s.gtok[i0 + r], 0.f)) : 0.f;
        }
        if (wv == 0) *reinterpret_cast<f32x4*>(&s.A[t * LDA + i0]) = s.beta[t] * m;
        else store4(&s.P1[t * LDC + i0], m);
    }
}

// PRO: the call has an input prologue; k is scaled per token by
// (|k|^2 + eps)^{-1/2} (each token's row is one wavefront: 64 lanes x 2 channels),
// beta and log a are transformed where they are loaded.
template <bool SCALAR, bool ORD1, bool PRO>
__global__ void __launch_bounds__(p2::NT, 2) kda_prep2_kernel(Prep2Params p) {
    using namespace p2;
    typedef WsBlock<DK, C, ORD1> WS;
    typedef Mma<bf16> M;
    __shared__ Prep2Lds s;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int c2 = lane, o = wv;  // elementwise phase: channel pair, token octet
    const int blk_b = o >> 1;     // 16-token block of the octet

    // upper blocks of the masked products are never written: zero them once
    prep2_init_lds(s, tid, ORD1);

    // this workgroup's chunks: item = blockIdx.x + k gridDim.x, empty ones skipped.
    // Packed batches leave many items past their sequence's end, so each
    // wavefront tests 64 candidates at once (one per lane) and then locates the
    // first non-empty one: one round trip to the sequence bounds per 64 items
    // instead of one per item.
    auto next_item = [&](int it, int64_t& t0, int& Lc, int& h) {
        const int64_t G = gridDim.x;
        for (int64_t at = it; at < p.items; at += 64 * G) {
            const int64_t cand = at + lane * G;
            int64_t ct0;
            int cLc, ch;
            const bool live = cand < p.items && prep2_locate(p, (int)cand, ct0, cLc, ch);
            const uint64_t m = __ballot(live);
            if (m) {
                const int first = (int)(at + (__ffsll((unsigned long long)m) - 1) * G);
                prep2_locate(p, first, t0, Lc, h);
                return first;
            }
        }
        return p.items;
    };
    int64_t t0 = 0;
    int Lc = 0, h = 0;
    int item = next_item(blockIdx.x, t0, Lc, h);
    Prep2Raw raw;
    if (item < p.items) prep2_load<SCALAR>(p, t0, Lc, h, tid, lane, o, raw);

    while (item < p.items) {
        uint8_t* __restrict__ blk = p.ws + (size_t)item * WS::BYTES;
        // bounds of the next item in this workgroup's list, read now and used in
        // phase B, so the scalar loads are not waited for on the spot
        const int g_item = item + gridDim.x;
        int64_t g_tb = 0, g_te = 0;
        int g_h = 0, g_j = 0;
        if (g_item < p.items) {
            const int unit = g_item / p.m, n = unit / p.H;
            g_h = unit % p.H;
            g_j = g_item % p.m;
            if (p.cu) { g_tb = p.cu[n]; g_te = p.cu[n + 1]; }
            else { g_tb = (int64_t)n * p.eq_len; g_te = g_tb + p.eq_len; }
        }

        // ---- A1: factors relative to the block mid-point, Gram operands ---------------
        Prep2In in;
        prep2_unpack<SCALAR>(raw, lane, in);
        float kscale[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) kscale[j] = 1.f;
        if (PRO && p.pro.normalize_k) {
            float ss[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const Vec2<bf16>::type kv = __builtin_bit_cast(Vec2<bf16>::type, in.k[j]);
                const float k0 = Vec2<bf16>::lo(kv), k1 = Vec2<bf16>::hi(kv);
                ss[j] = row_sum16(k0 * k0 + k1 * k1);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                kscale[j] = rsqrtf(readlanef(ss[j], 0) + readlanef(ss[j], 16) + readlanef(ss[j], 32) +
                                   readlanef(ss[j], 48) + PROLOGUE_EPS);
        }
        if constexpr (SCALAR) {
            // scalar decay (Gated DeltaNet): one log2 decay per token, the same in every
            // lane; the Gram products take the raw rows and the decay as a scalar mask
            static_assert(ORD1, "a scalar decay runs the decay-first form");
            float l2[8];
            bool steep = false;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float x = in.la[j][0] * LOG2E;
                if (PRO && p.pro.log_a_raw) x = prologue_log2_a(in.la[j][0], p.pro.log_a_min * LOG2E);
                if (8 * o + j >= Lc) x = 0.f;
                steep |= x < STEEP_LOG2;
                l2[j] = x;
            }
            float mine = l2[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) mine = lane == j ? l2[j] : mine;
            if (lane < 8) s.ltok[8 * o + lane] = mine;
            if (lane == 0) s.steep[wv] = steep;
            if (tid < C) s.beta[tid] = (PRO && p.pro.beta_logits && tid < Lc) ? prologue_beta(raw.b) : raw.b;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int t = 8 * o + j;
                const Vec2<bf16>::type kv = __builtin_bit_cast(Vec2<bf16>::type, in.k[j]);
                const f32x2 k = f32x2{Vec2<bf16>::lo(kv), Vec2<bf16>::hi(kv)} * kscale[j];
                store2(&s.u.g.Kr[t * LDK + 2 * c2], k[0], k[1]);
                *reinterpret_cast<uint32_t*>(&s.u.g.Qr[t * LDK + 2 * c2]) = in.q[j];
            }
            lds_barrier();
            prep2_scalar_operands<ORD1>(s, blk, in, kscale, lane, c2, o);
        } else {
        f32x2 a[8], ai[8], E[8], Ei[8];
        bool steep = false;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool valid = 8 * o + j < Lc;
            f32x2 la2 = in.la[j] * LOG2E;
            if (PRO && p.pro.log_a_raw) {
                const float lo2 = p.pro.log_a_min * LOG2E;
                la2 = f32x2{prologue_log2_a(in.la[j][0], lo2), prologue_log2_a(in.la[j][1], lo2)};
            }
            if (!valid) la2 = f32x2{0.f, 0.f};
            steep |= la2[0] < STEEP_LOG2 || la2[1] < STEEP_LOG2;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float x = fmaxf(la2[e], LA_MIN);
                a[j][e] = __builtin_amdgcn_exp2f(x);
                ai[j][e] = __builtin_amdgcn_exp2f(-x);
            }
        }
        f32x2 P;
        if ((o & 1) == 0) {  // tokens up to the mid-point: backward from it
            E[7] = f32x2{1.f, 1.f};
            Ei[7] = f32x2{1.f, 1.f};
#pragma unroll
            for (int j = 6; j >= 0; --j) {
                E[j] = E[j + 1] * ai[j + 1];
                Ei[j] = Ei[j + 1] * a[j + 1];
            }
            P = Ei[0] * a[0];
        } else {  // tokens after it: forward
            E[0] = a[0];
            Ei[0] = ai[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) {
                E[j] = E[j - 1] * a[j];
                Ei[j] = Ei[j - 1] * ai[j];
            }
            P = E[7];
        }
        *reinterpret_cast<f32x2*>(&s.Pq[o * DK + 2 * c2]) = P;
        {
            const bool ws = wave_any(steep);
            if (lane == 0) s.steep[wv] = ws;
        }
        if (tid < C) s.beta[tid] = (PRO && p.pro.beta_logits && tid < Lc) ? prologue_beta(raw.b) : raw.b;

        f32x2 kr[8], qr[8], kce[8], kci[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = 8 * o + j;
            const Vec2<bf16>::type kv = __builtin_bit_cast(Vec2<bf16>::type, in.k[j]);
            const Vec2<bf16>::type qv = __builtin_bit_cast(Vec2<bf16>::type, in.q[j]);
            const f32x2 k = f32x2{Vec2<bf16>::lo(kv), Vec2<bf16>::hi(kv)} * kscale[j];
            const f32x2 q = f32x2{Vec2<bf16>::lo(qv), Vec2<bf16>::hi(qv)};
            kr[j] = ORD1 ? k * E[j] : k * (E[j] * ai[j]);  // k e^{g_{t-1} - mu} (ORD1: g_t)
            qr[j] = q * E[j];             // q e^{g_t - mu}
            kce[j] = k * (Ei[j] * a[j]);  // k e^{mu - g_{t-1}}
            kci[j] = k * Ei[j];           // k e^{mu - g_t}
            store2(&s.u.g.Kr[t * LDK + 2 * c2], kr[j][0], kr[j][1]);
            store2(&s.u.g.Qr[t * LDK + 2 * c2], qr[j][0], qr[j][1]);
            if (!ORD1) store2(&s.u.g.Kce[t * LDK + 2 * c2], kce[j][0], kce[j][1]);
            store2(&s.u.g.Kci[t * LDK + 2 * c2], kci[j][0], kci[j][1]);
        }
        lds_barrier();

        // ---- A2: chunk-referenced operands ---------------------------------------------
        {
            const f32x2 P0 = *reinterpret_cast<const f32x2*>(&s.Pq[0 * DK + 2 * c2]);
            const f32x2 P1 = *reinterpret_cast<const f32x2*>(&s.Pq[1 * DK + 2 * c2]);
            const f32x2 P2 = *reinterpret_cast<const f32x2*>(&s.Pq[2 * DK + 2 * c2]);
            const f32x2 P3 = *reinterpret_cast<const f32x2*>(&s.Pq[3 * DK + 2 * c2]);
            const f32x2 F = P1 * P2;         // e^{mu_1 - mu_0}
            const f32x2 em0 = P0;            // e^{mu_0}
            const f32x2 ec1 = P3;            // e^{g_C - mu_1}
            const f32x2 em = blk_b ? em0 * F : em0;
            const f32x2 ec = blk_b ? ec1 : F * ec1;
            if (o == 0) {
                *reinterpret_cast<f32x2*>(&s.F[2 * c2]) = F;
                // a steep chunk is marked for kda_prep2_exact_kernel instead
                const bool steep_chunk = (s.steep[0] | s.steep[1] | s.steep[2] | s.steep[3]) != 0;
                *reinterpret_cast<f32x2*>(blk + WS::GAM + 8 * c2) =
                    steep_chunk ? f32x2{-1.f, -1.f} : (em0 * F) * ec1;
            }
            // KbT rows (channels), tokens at their permuted positions: tokens 8 o .. 8 o + 3
            // and 8 o + 4 .. 8 o + 7 land at two 4-element runs
            const int pos0 = kperm(8 * o), pos1 = kperm(8 * o + 4);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                f32x4 kb0, kb1;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    kb0[j] = kr[j][e] * em[e];
                    kb1[j] = kr[4 + j][e] * em[e];
                }
                const int c = 2 * c2 + e;
                store4(&s.KbT[c * LDC + pos0], kb0);
                store4(&s.KbT[c * LDC + pos1], kb1);
                // KC, KT: the octet's 8 tokens are piece o of channel row c
                bf16x8 kc, kt;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    kc[j] = (bf16)((ORD1 ? kci[j][e] : kce[j][e]) * ec[e]);
                    kt[j] = (bf16)(kci[j][e] * ec[e] * s.beta[8 * o + j]);
                }
                *reinterpret_cast<bf16x8*>(blk + WS::KC + piece<DK>(c, o)) = kc;
                if (!ORD1) *reinterpret_cast<bf16x8*>(blk + WS::KT + piece<DK>(c, o)) = kt;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const f32x2 qb = qr[j] * em;
                store2(&s.Qb[(8 * o + j) * LDK + 2 * c2], qb[0], qb[1]);
            }
        }
        }  // per-channel decay
        lds_barrier();

        // next chunk's inputs: in flight during phases B-D
        int64_t nt0 = 0;
        int nLc = 0, nh = 0;
        int nitem = g_item;
        if (g_item < p.items) {
            nt0 = g_tb + (p.chunk0 + g_j) * C;
            nh = g_h;
            nLc = (int)((g_te - nt0) < C ? (g_te - nt0) : C);
            if (nt0 >= g_te) nitem = next_item(g_item + gridDim.x, nt0, nLc, nh);  // empty: look further
        }
        if (nitem < p.items) prep2_load<SCALAR>(p, nt0, nLc, nh, tid, lane, o, raw);

        // ---- B: Gram products.  Wavefront g forms product g (0 A, 1 L, 2 P1, 3 P2) for
        //      the block pairs (0,0), (1,0) and (1,1) from 16 fragments read at once; rows
        //      of block 1 are scaled by F for the off-diagonal pair -------------------------
        //      ORD1: only A (wavefront 0, columns Kt) and P2 (wavefront 3, unscaled, into P1)
        if (SCALAR) {
            if (wv == 0 || wv == 3) prep2_scalar_gram(s, wv, lane);
        } else if (!ORD1 || wv == 0 || wv == 3) {
            const int g = wv;
            constexpr int NK = DK / M::K;
            const bf16* rows = g < 2 ? s.u.g.Kr : s.u.g.Qr;
            const bf16* cols = (g & 1) == 0 && !ORD1 ? s.u.g.Kce : s.u.g.Kci;
            M::frag r0[NK], r1[NK], c0[NK], c1[NK], r1f[NK];
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                r0[kk] = M::loadr(rows + lr * LDK + kk * M::K, lane);
                r1[kk] = M::loadr(rows + (16 + lr) * LDK + kk * M::K, lane);
                c0[kk] = M::loadr(cols + lr * LDK + kk * M::K, lane);
                c1[kk] = M::loadr(cols + (16 + lr) * LDK + kk * M::K, lane);
            }
            const float* Fp = s.F + lg * M::KPL;
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) r1f[kk] = M::scale(r1[kk], Fp + kk * M::K);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int pr = 0; pr < 3; ++pr) {
                const int bt = pr == 0 ? 0 : 1, bi = pr == 2 ? 1 : 0;
                const M::frag* fr = pr == 0 ? r0 : (pr == 1 ? r1f : r1);
                const M::frag* fc = bi == 0 ? c0 : c1;
                f32x4 acc = zero4();
                if (g == 1) {
#pragma unroll
                    for (int kk = 0; kk < NK; ++kk) acc = M::mma(fr[kk], fc[kk], acc);
                    // rows t = 16 bt + 4 lg + r, column i = 16 bi + lr; LbT[i] at permuted t
                    const int i = 16 * bi + lr, tt = 16 * bt + 4 * lg;
                    const float bi_ = s.beta[i];
                    f32x4 m;
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[r] = (i < tt + r) ? acc[r] * bi_ : 0.f;
                    store4(&s.LbT[i * LDC + kperm(tt)], m);
                } else {
#pragma unroll
                    for (int kk = 0; kk < NK; ++kk) acc = M::mma(fc[kk], fr[kk], acc);
                    // column t = 16 bt + lr, rows i = 16 bi + 4 lg + r
                    const int t = 16 * bt + lr, i0 = 16 * bi + 4 * lg;
                    f32x4 m;
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[r] = (g == 0 ? i0 + r < t : i0 + r <= t) ? acc[r] : 0.f;
                    if (g == 0) *reinterpret_cast<f32x4*>(&s.A[t * LDA + i0]) = s.beta[t] * m;
                    else if (g == 2 || ORD1) store4(&s.P1[t * LDC + i0], m);
                    else *reinterpret_cast<f32x4*>(&s.P2b[t * LDA + i0]) =
                             m * *reinterpret_cast<const f32x4*>(&s.beta[i0]);
                }
            }
        }
        lds_barrier();

        prep2_solve_store<ORD1>(s, blk, tid, lane, wv);
        lds_barrier();  // LDS of this chunk is reused by the next

        item = nitem; t0 = nt0; Lc = nLc; h = nh;
    }
}

// Marked chunks of one segment, run after kda_prep2_kernel on the same items:
// every non-empty item whose block carries the mark (GAM[0] == -1) is formed
// again, all of it, with the decay factors of the chunk-referenced operands and
// of the Gram products taken one exponential each (prep2_steep_operands,
// exact_gram); phases C-D are those of kda_prep2_kernel.  Workgroup b checks its
// items b, b + G, b + 2 G, ... (G = gridDim.x) NT at a time, one per thread, and
// forms the marked ones of each round; unmarked blocks are not touched.
template <bool SCALAR, bool ORD1, bool PRO>
__global__ void __launch_bounds__(p2::NT, 2) kda_prep2_exact_kernel(Prep2Params p) {
    using namespace p2;
    typedef WsBlock<DK, C, ORD1> WS;
    __shared__ Prep2Lds s;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    bool init = false;
    for (int64_t base = 0; (int64_t)blockIdx.x + base * gridDim.x < p.items; base += NT) {
        const int64_t it = (int64_t)blockIdx.x + (base + tid) * gridDim.x;
        bool marked = false;
        if (it < p.items) {
            int64_t t0;
            int Lc, h;
            if (prep2_locate(p, (int)it, t0, Lc, h))
                marked = *reinterpret_cast<const float*>(p.ws + (size_t)it * WS::BYTES + WS::GAM) == -1.f;
        }
        // marked items of this round, in order, to s.list
        const uint64_t m = __ballot(marked);
        if (lane == 0) s.steep[wv] = __popcll(m);
        lds_barrier();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < NT / WAVE; ++w) {
            const int c = s.steep[w];
            before += w < wv ? c : 0;
            total += c;
        }
        if (marked) s.list[before + __popcll(m & ((1ull << lane) - 1))] = (int)it;
        lds_barrier();
        if (total > 0 && !init) {
            prep2_init_lds(s, tid, ORD1);
            init = true;
            lds_barrier();
        }
        for (int x = 0; x < total; ++x) {
            const int item = __builtin_amdgcn_readfirstlane(s.list[x]);
            int64_t t0;
            int Lc, h;
            prep2_locate(p, item, t0, Lc, h);
            uint8_t* __restrict__ blk = p.ws + (size_t)item * WS::BYTES;
            Prep2Raw raw;
            prep2_load<SCALAR>(p, t0, Lc, h, tid, lane, wv, raw);
            prep2_steep_operands<SCALAR, ORD1, PRO>(p, s, raw, blk, tid, lane, lane, wv, Lc);
            prep2_steep_gram<ORD1>(s, wv, lane);
            lds_barrier();
            prep2_solve_store<ORD1>(s, blk, tid, lane, wv);
            lds_barrier();
        }
    }
}

hipError_t launch_prep2(const PrepLaunch& a, hipStream_t stream) {
    Prep2Params p;
    p.q = a.q; p.k = a.k; p.log_a = a.log_a; p.beta = a.beta; p.cu = a.cu_seqlens;
    p.eq_len = a.eq_len; p.ws = static_cast<uint8_t*>(a.ws); p.H = a.num_heads; p.m = a.m;
    p.chunk0 = a.chunk0;
    p.items = (int)(a.units * a.m);
    p.pro = a.pro;
    // persistent workgroups, two per compute unit, walking items blockIdx.x, + gridDim.x, ...
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    int64_t blocks = (int64_t)cus * 2;
    if (blocks > p.items) blocks = p.items;
    if (blocks < 1) blocks = 1;
    const dim3 grid((unsigned)blocks), block(p2::NT);
#define KDA_PREP2_LAUNCH(SC, O1, PR)                                                                  \
    do {                                                                                              \
        hipLaunchKernelGGL((kda_prep2_kernel<SC, O1, PR>), grid, block, 0, stream, p);                \
        hipLaunchKernelGGL((kda_prep2_exact_kernel<SC, O1, PR>), grid, block, 0, stream, p);          \
    } while (0)
    // a scalar decay comes with the decay-first order (the host's choice for the two-pass method)
    if (a.pro.any()) {
        if (a.scalar) KDA_PREP2_LAUNCH(true, true, true);
        else if (a.order) KDA_PREP2_LAUNCH(false, true, true);
        else KDA_PREP2_LAUNCH(false, false, true);
    } else {
        if (a.scalar) KDA_PREP2_LAUNCH(true, true, false);
        else if (a.order) KDA_PREP2_LAUNCH(false, true, false);
        else KDA_PREP2_LAUNCH(false, false, false);
    }
#undef KDA_PREP2_LAUNCH
    return hipGetLastError();
}

}  // namespace kda
