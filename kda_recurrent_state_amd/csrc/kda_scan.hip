// kda_scan.hip -- sequential pass of the two-pass KDA prefill on gfx950.
//
// Applies the per-chunk operator blocks written by kda_prep.hip to the running
// state, chunk after chunk.  This is the part of the chunkwise form that the
// recurrence makes sequential (the "sequential dependency" of the delta rule,
// page "The argument, in one page", section "Everything, in one table", row
// "Delta rule"; the chunk form leaves one dependent step per chunk).  Per chunk
// and 16-column block of the value dimension, with V the chunk's values:
//   E = -(W S + M1 V)
//   O = QP S + M2 V                      (read after the update, per token)
//   S <- Diag(GAM) S + KC E + KT V
// Each column block of S evolves on its own: the operators are shared, the
// columns never mix.  So one wavefront owns one 16-column block of the state
// (dk x 16 fp32 in matrix-core accumulators) for the whole walk, and the
// accumulator tiles of S and E are fed straight back as bf16 operands (the
// block layout's permuted contraction order makes that a register move).
//
// Workgroup: NS compute wavefronts (the slice's column blocks) plus four loader
// wavefronts that keep the operator blocks and value tiles of the next three
// chunks in flight and copy the next one into the other half of a double
// buffer in LDS while the current chunk is being applied.  One barrier per chunk.  Slices of one (sequence, head) are placed
// on one XCD so that they read each operator block through the same L2.
#include "kda_device.hpp"
#include "kda_chunk_common.hpp"
#include "kda_launch.hpp"
#include "kda_ws.hpp"

namespace kda {

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

template <int DK, int DVS, int C>
struct ScanCfg {
    static constexpr int NS = DVS / 16;         // compute wavefronts
    static constexpr int NL = 4;                // loader wavefronts
    static constexpr int PD = 3;                // chunks in flight in the loaders' registers
    static constexpr int NT = WAVE * (NS + NL);
    static constexpr int LT = WAVE * NL;        // loader threads
    static constexpr int BYTES = WsBlock<DK, C>::BYTES;
    static constexpr int NPC = BYTES / 16;      // 16-byte pieces per block
    static constexpr int LPT = (NPC + LT - 1) / LT;
    static constexpr int VTB = DVS * 2 * C;     // value tile bytes: [column][token]
    static constexpr int NVP = C * DVS / 8;     // 16-byte value pieces per chunk
    static constexpr int VPT = (NVP + LT - 1) / LT;
};

struct ScanParams {
    const void* v;
    void* o;
    const int32_t* cu;
    int64_t eq_len;
    const uint8_t* ws;    // operator blocks [unit][m]
    const float* S_in;    // null: zero state
    float* S_out;
    int H, DV, split, m, xcd_group;
    int64_t chunk0;
};

// Register-staged copy of operator blocks and value tiles into LDS.
template <int DK, int DVS, int C>
struct ScanLoader {
    typedef ScanCfg<DK, DVS, C> G;
    i32x4 pc[G::PD][G::LPT];
    bf16x8 vv[G::PD][G::VPT];
    int ltid, H, DV, dv0, h;
    const uint8_t* src;
    const bf16* gv;
    int64_t tb, te, chunk0;

    // Every thread issues the same number of loads on every path (indices past the
    // end are clamped to a valid piece or chunk and their data is never stored),
    // so the compiler can wait for exactly the oldest register set.
    template <int S>
    __device__ __forceinline__ void fetch(int jj, int nch) {
        jj = min(jj, nch - 1);
        const i32x4* b = reinterpret_cast<const i32x4*>(src + (size_t)jj * G::BYTES);
#pragma unroll
        for (int i = 0; i < G::LPT; ++i) pc[S][i] = b[min(ltid + G::LT * i, G::NPC - 1)];
        const int64_t t0 = tb + (chunk0 + jj) * C;
        const int Lc = (int)((te - t0) < C ? (te - t0) : C);
#pragma unroll
        for (int i = 0; i < G::VPT; ++i) {
            const int idx = (ltid + G::LT * i) % G::NVP;
            const int t = idx / (DVS / 8), j0 = 8 * (idx % (DVS / 8));
            // rows past the chunk's end repeat its last row: they meet zero operator columns
            const int64_t row = (t0 + min(t, Lc - 1)) * H + h;
            vv[S][i] = *reinterpret_cast<const bf16x8*>(gv + row * DV + dv0 + j0);
        }
    }

    template <int S>
    __device__ __forceinline__ void put(int jj, uint8_t* bdst, uint8_t* vdst) {
        (void)jj;
        i32x4* dst = reinterpret_cast<i32x4*>(bdst);
#pragma unroll
        for (int i = 0; i < G::LPT; ++i) {
            const int idx = ltid + G::LT * i;
            if (idx < G::NPC) dst[idx] = pc[S][i];
        }
#pragma unroll
        for (int i = 0; i < G::VPT; ++i) {
            const int idx = ltid + G::LT * i;
            if (idx < G::NVP) {
                const int t = idx / (DVS / 8), j0 = 8 * (idx % (DVS / 8));
                const int pos = kperm(t);
#pragma unroll
                for (int e = 0; e < 8; ++e) *reinterpret_cast<bf16*>(vdst + swz_elem<2 * C>(j0 + e, pos)) = vv[S][i][e];
            }
        }
    }
};

template <int DK, int DVS, int C>
__global__ void __launch_bounds__((ScanCfg<DK, DVS, C>::NT)) kda_scan_kernel(ScanParams p) {
    typedef ScanCfg<DK, DVS, C> G;
    typedef WsBlock<DK, C> WS;
    constexpr int NS = G::NS, LT = G::LT, BYTES = G::BYTES;
    __shared__ alignas(16) uint8_t buf[2][BYTES];
    __shared__ alignas(16) uint8_t vt[2][G::VTB];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int H = p.H, DV = p.DV;
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
    const int64_t nch_all = (te - tb + C - 1) / C;
    const int64_t c_end = min(nch_all, p.chunk0 + p.m);
    const int nch = c_end > p.chunk0 ? (int)(c_end - p.chunk0) : 0;
    const uint8_t* __restrict__ wsu = p.ws + (size_t)unit * p.m * BYTES;

    if (wv >= NS) {
        // ---------------- loader wavefronts ----------------
        // Chunk c's block is fetched into register set c % PD at step c - PD and
        // written to LDS buffer c % 2 at step c - 1, so PD - 1 steps of compute
        // cover its memory latency.  Step i (one per chunk, ending in the
        // barrier) writes chunk i + 1 and fetches chunk i + PD.
        ScanLoader<DK, DVS, C> L;
        L.ltid = tid - WAVE * NS;
        L.src = wsu; L.gv = static_cast<const bf16*>(p.v);
        L.tb = tb; L.te = te; L.chunk0 = p.chunk0; L.H = H; L.DV = DV; L.dv0 = dv0; L.h = h;
        static_assert(G::PD == 3, "the loader loop is unrolled for three register sets");
        if (nch > 0) {
            L.template fetch<0>(0, nch);
            L.template fetch<1>(1, nch);
            L.template fetch<2>(2, nch);
            L.template put<0>(0, buf[0], vt[0]);
        }
        lds_barrier();
        for (int i = 0; i < nch; i += 3) {
            if (i + 1 < nch) L.template put<1>(i + 1, buf[(i + 1) & 1], vt[(i + 1) & 1]);
            L.template fetch<0>(i + 3, nch);
            lds_barrier();
            if (i + 1 < nch) {
                if (i + 2 < nch) L.template put<2>(i + 2, buf[(i + 2) & 1], vt[(i + 2) & 1]);
                L.template fetch<1>(i + 4, nch);
                lds_barrier();
            }
            if (i + 2 < nch) {
                if (i + 3 < nch) L.template put<0>(i + 3, buf[(i + 3) & 1], vt[(i + 3) & 1]);
                L.template fetch<2>(i + 5, nch);
                lds_barrier();
            }
        }
        return;
    }

    // ---------------- compute wavefronts: columns dv0 + 16 wv .. + 15 ----------------
    bf16* __restrict__ go = static_cast<bf16*>(p.o);
    constexpr int NR = DK / 16, NKS = DK / 32, NTT = C / 16, NKC = C / 32;
    f32x4 acc[NR];  // state rows 16 r + 4 lg + i, column lr of the block
    const int64_t sb = (int64_t)unit * DK * DV + dv0 + 16 * wv + lr;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[r][i] = p.S_in ? p.S_in[sb + (int64_t)(16 * r + 4 * lg + i) * DV] : 0.f;
    bf16x8 sfr[NKS];
    auto make_sfr = [&]() {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sfr[ks][i] = (bf16)acc[2 * ks][i];
                sfr[ks][4 + i] = (bf16)acc[2 * ks + 1][i];
            }
    };
    make_sfr();
    lds_barrier();

    for (int jj = 0; jj < nch; ++jj) {
        const uint8_t* B = buf[jj & 1];
        const uint8_t* Vt = vt[jj & 1];
        // operand fragment of a matrix with 2 DK-byte rows (fk) or 2 C-byte rows (fc)
        auto fk = [&](int off, int row, int piece) -> bf16x8 {
            return *reinterpret_cast<const bf16x8*>(B + off + swz<2 * DK>(row, piece));
        };
        auto fc = [&](int off, int row, int piece) -> bf16x8 {
            return *reinterpret_cast<const bf16x8*>(B + off + swz<2 * C>(row, piece));
        };

        bf16x8 vfr[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
            vfr[kc] = *reinterpret_cast<const bf16x8*>(Vt + swz<2 * C>(16 * wv + lr, 4 * kc + lg));

        // E = -(W S + M1 V), token tiles tt
        f32x4 z[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            bf16x8 a[NKS + NKC];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) a[ks] = fk(WS::W, 16 * tt + lr, 4 * ks + lg);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) a[NKS + kc] = fc(WS::M1, 16 * tt + lr, 4 * kc + lg);
            f32x4 x = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) x = Mma<bf16>::mma(a[ks], sfr[ks], x);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) x = Mma<bf16>::mma(a[NKS + kc], vfr[kc], x);
            z[tt] = x;
        }
        bf16x8 efr[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                efr[kc][i] = (bf16)(-z[2 * kc][i]);
                efr[kc][4 + i] = (bf16)(-z[2 * kc + 1][i]);
            }

        // O^T = S^T QP^T + V^T M2^T (state at the chunk start), token tiles tt
        f32x4 ot[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            bf16x8 b[NKS + NKC];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) b[ks] = fk(WS::QP, 16 * tt + lr, 4 * ks + lg);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) b[NKS + kc] = fc(WS::M2, 16 * tt + lr, 4 * kc + lg);
            f32x4 x = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) x = Mma<bf16>::mma(sfr[ks], b[ks], x);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) x = Mma<bf16>::mma(vfr[kc], b[NKS + kc], x);
            ot[tt] = x;
        }

        // S <- Diag(GAM) S + KT V + KC E
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const f32x4 gm = *reinterpret_cast<const f32x4*>(B + WS::GAM + 4 * (16 * r + 4 * lg));
            bf16x8 kt[NKC], kc_[NKC];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                kt[kc] = fc(WS::KT, 16 * r + lr, 4 * kc + lg);
                kc_[kc] = fc(WS::KC, 16 * r + lr, 4 * kc + lg);
            }
            f32x4 x = acc[r] * gm;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) x = Mma<bf16>::mma(kt[kc], vfr[kc], x);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) x = Mma<bf16>::mma(kc_[kc], efr[kc], x);
            acc[r] = x;
        }
        make_sfr();

        // outputs: lane holds columns 4 lg .. 4 lg + 3 of token 16 tt + lr
        const int64_t t0 = tb + (p.chunk0 + jj) * C;
        const int Lc = (int)((te - t0) < C ? (te - t0) : C);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const int t = 16 * tt + lr;
            if (t < Lc) store4(go + ((t0 + t) * H + h) * DV + dv0 + 16 * wv + 4 * lg, ot[tt]);
        }
        lds_barrier();
    }

#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) p.S_out[sb + (int64_t)(16 * r + 4 * lg + i) * DV] = acc[r][i];
}

// ------------------------------------------------------------------------------------
template <int DK, int DVS, int C>
static hipError_t scan_cfg(const ScanLaunch& a, hipStream_t stream) {
    ScanParams p;
    p.v = a.v; p.o = a.o; p.cu = a.cu_seqlens; p.eq_len = a.eq_len;
    p.ws = static_cast<const uint8_t*>(a.ws); p.S_in = a.S_in; p.S_out = a.S_out;
    p.H = a.num_heads; p.DV = a.dv; p.split = a.split; p.m = a.m; p.chunk0 = a.chunk0;
    const int64_t blocks = (int64_t)a.units * a.split;
    p.xcd_group = (blocks % 8 == 0 && (blocks / 8) % a.split == 0) ? 1 : 0;
    hipLaunchKernelGGL((kda_scan_kernel<DK, DVS, C>), dim3((unsigned)blocks), dim3(ScanCfg<DK, DVS, C>::NT), 0,
                       stream, p);
    return hipGetLastError();
}

#define KDA_SCAN_CASE(DK_, DVS_, C_) \
    if (dk == DK_ && dvs == DVS_ && chunk == C_) { if (a) *err = scan_cfg<DK_, DVS_, C_>(*a, stream); return true; }

static bool scan_dispatch(int dk, int dvs, int chunk, const ScanLaunch* a, hipStream_t stream, hipError_t* err) {
    KDA_SCAN_CASE(128, 16, 32) KDA_SCAN_CASE(128, 32, 32) KDA_SCAN_CASE(128, 64, 32)
    KDA_SCAN_CASE(64, 16, 32) KDA_SCAN_CASE(64, 32, 32) KDA_SCAN_CASE(64, 64, 32)
    KDA_SCAN_CASE(64, 16, 64) KDA_SCAN_CASE(64, 32, 64) KDA_SCAN_CASE(64, 64, 64)
    return false;
}

bool two_pass_supported(int dtype, int dk, int dvs, int chunk) {
    return dtype == 1 && prep_block_bytes(dk, chunk) > 0 && scan_dispatch(dk, dvs, chunk, nullptr, nullptr, nullptr);
}

hipError_t launch_scan(const ScanLaunch& a, hipStream_t stream) {
    hipError_t err = hipErrorInvalidValue;
    if (!scan_dispatch(a.dk, a.dv / a.split, a.chunk, &a, stream, &err)) return hipErrorInvalidValue;
    return err;
}

}  // namespace kda
