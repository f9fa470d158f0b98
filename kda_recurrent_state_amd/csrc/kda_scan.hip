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
// columns never mix.  One wavefront owns CB column blocks of the state
// (dk x 16 fp32 each, in matrix-core accumulators) for the whole walk, and the
// accumulator tiles of S and E are fed straight back as bf16 operands (the
// block layout's permuted contraction order makes that a register move).  Two
// column blocks per wavefront let every operator fragment read from LDS serve
// two products and give the matrix cores two independent chains.
//
// Memory path: the operator block and the value tile of a chunk are copied
// verbatim from global memory into one of three or four LDS slots by the
// LDS-DMA form of the global load (each lane's 16 bytes land at slot base +
// 16 * lane, no registers involved).  The copy of chunk j + AHEAD is issued
// while chunk j is computed; each wavefront waits for its own copies of chunk
// j + 1 with a vector-memory counter wait, and the workgroup barrier in the
// middle of chunk j makes them visible to all wavefronts and frees chunk j's
// slot.  The next chunk's first operands are read right after that barrier,
// so their LDS latency is hidden behind the state update of chunk j.  The
// compute wavefronts issue no global memory operations in the walk: they leave
// each chunk's outputs in its slot's value tile (already read by then), and the
// copy wavefronts store them, 16 bytes per lane, before they refill the slot.
#include "kda_device.hpp"
#include "kda_chunk_common.hpp"
#include "kda_launch.hpp"
#include "kda_ws.hpp"

namespace kda {

template <int DK, int DVS, int CB, bool ORD1 = false>
struct ScanCfg {
    static constexpr int C = 32;
    static constexpr int NW = DVS / (16 * CB);       // compute wavefronts
    static constexpr int NL = 2;                     // copy wavefronts
    static constexpr int NT = WAVE * (NW + NL);
    static constexpr int LT = WAVE * NL;             // copy threads
    static constexpr int BYTES = WsBlock<DK, C, ORD1>::BYTES;
    static constexpr int NPB = BYTES / 16;           // 16-byte pieces of an operator block
    static constexpr int VPR = DVS / 8;              // pieces per value row of the slice
    static constexpr int NPV = C * VPR;              // pieces of a chunk's value tile
    static constexpr int NPS = NPB + NPV;
    static constexpr int ROUNDS = (NPS + LT - 1) / LT;  // copy instructions per copy wavefront and chunk
    static constexpr int SLOT = ROUNDS * LT * 16;    // LDS bytes per slot (copies past NPS land in the pad)
    // slots: four (copies three chunks ahead) where they fit in LDS and the
    // counter wait can express them, else three
    static constexpr int NBUF = (4 * SLOT <= 160 * 1024 && 2 * ROUNDS + 3 < 64) ? 4 : 3;
    static constexpr int AHEAD = NBUF - 1;
    static constexpr int TOUCH = 2;                  // L2 touches run this many chunks past AHEAD
    static constexpr int PAD = SLOT - NPS * 16;      // unread tail of every slot
    static_assert(BYTES % 16 == 0, "operator blocks are whole 16-byte pieces");
    static_assert(NW >= 1 && NW * 16 * CB == DVS, "slice = wavefronts x column blocks x 16");
    static_assert(PAD >= 4 * WAVE && NL <= NBUF, "each copy wavefront's touches land in a slot's pad");
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
    float* snap;          // state snapshots [rows][H][DK][DV], or null
    int64_t snap_rows;
    int snap_every;       // tokens between snapshots (a multiple of C)
    const int32_t* ord;   // sequences longest first (kda_seq_rank_kernel), or null
};

// Place of the value tile's 16-byte piece u of token row t (VPR pieces per
// row) among the tile's pieces in LDS.  The copy puts each piece there (the
// LDS-DMA lands lane l's 16 bytes at slot piece l, so the permutation is in
// the choice of source), so that both LDS accesses of the tile are free of
// bank conflicts at every slice width: the column reads of the value
// fragment (16 lanes on 16 columns of a row, 4 row groups 8 rows apart) and
// the output writes (16 rows, 8 bytes per lane).  Rows are XOR-permuted in
// groups of four by bits 3-4 of t (an involution) and pieces within a row by
// bits of t and t / 4.  Slices of 128 columns keep the plain row-major order:
// there the lanes' extra read addresses would not fit in registers.
template <int VPR>
__device__ __forceinline__ int vpiece(int t, int u) {
    if constexpr (VPR > 8) return VPR * t + u;
    return VPR * (t ^ ((t >> 3) & 3)) + (u ^ ((t ^ (t >> 2)) & (VPR - 1)));
}
template <int VPR>
__device__ __forceinline__ void vpiece_source(int q, int& t, int& u) {
    const int r = q / VPR;
    if constexpr (VPR > 8) {
        t = r;
        u = q % VPR;
        return;
    }
    t = r ^ ((r >> 3) & 3);
    u = (q % VPR) ^ ((t ^ (t >> 2)) & (VPR - 1));
}

// SNAP: the call asks for state snapshots (a separate instantiation, so that
// the plain walk carries no snapshot code).  ORD1: decay-first blocks (no KT V
// term in the state update).
template <int DK, int DVS, int CB, bool SNAP, bool ORD1>
__global__ void __launch_bounds__((ScanCfg<DK, DVS, CB, ORD1>::NT), 1) kda_scan_kernel(ScanParams p) {
    typedef ScanCfg<DK, DVS, CB, ORD1> G;
    typedef WsBlock<DK, G::C, ORD1> WS;
    constexpr int C = G::C, LT = G::LT, ROUNDS = G::ROUNDS;
    constexpr int NR = DK / 16, NKS = DK / 32, NTT = C / 16;
    constexpr int RBK = 2 * DK;  // row bytes of W and QP
    __shared__ alignas(16) uint8_t lds[G::NBUF * G::SLOT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
    const int lr = lane & 15, lg = lane >> 4;
    const int H = p.H, DV = p.DV;
    int unit, slice;
    if (p.ord) {
        // Longest sequences first.  Workgroups reach an XCD's compute units in
        // the order of their index, and XCD x receives the indices x, x + 8, ...,
        // so the units of rank x, x + 8, ... are dealt to it in that order, the
        // slices of one unit next to each other (one L2 serves all of them).
        const int b = blockIdx.x;
        int rank;
        if (p.xcd_group) { rank = (b / 8 / p.split) * 8 + b % 8; slice = (b / 8) % p.split; }
        else { rank = b / p.split; slice = b % p.split; }
        unit = p.ord[rank / H] * H + rank % H;
    } else {
        int item = blockIdx.x;
        if (p.xcd_group) {
            const int per = gridDim.x / 8;
            item = (blockIdx.x % 8) * per + blockIdx.x / 8;
        }
        unit = item / p.split;
        slice = item % p.split;
    }
    const int n = unit / H, h = unit % H;
    const int dv0 = slice * DVS;
    int64_t tb, te;
    if (p.cu) { tb = p.cu[n]; te = p.cu[n + 1]; }
    else { tb = (int64_t)n * p.eq_len; te = tb + p.eq_len; }
    const int64_t nch_all = (te - tb + C - 1) / C;
    const int64_t c_end = min(nch_all, p.chunk0 + p.m);
    const int nch = c_end > p.chunk0 ? (int)(c_end - p.chunk0) : 0;
    const uint8_t* __restrict__ wsu = p.ws + (size_t)unit * p.m * G::BYTES;
    const bf16* __restrict__ gv = static_cast<const bf16*>(p.v);
    bf16* __restrict__ go = static_cast<bf16*>(p.o);

    // Lane parts of every LDS address, fixed for the whole walk.  The swizzle of
    // a row depends only on the row's position inside its 16-row tile, so tile
    // and matrix offsets are compile-time immediates on top of these.
    uint32_t oW[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) oW[ks] = swz<RBK>(lr, 4 * ks + lg);  // W, QP fragments
    const uint32_t oM = piece<C>(lr, lg);                                   // M1, M2 fragments
    const uint32_t oK = piece<DK>(lr, lg);                                  // KC, KT fragments
    const uint32_t oG = WS::GAM + 16 * lg;                                  // GAM rows 4 lg .. 4 lg + 3

    // Copy chunk jj's operator block and value tile into slot sl: piece
    // r * NT + tid of the slot comes from the block (below NPB), from the value
    // tile (below NPS), or repeats the last piece (the pad past NPS).
    // (run by the copy wavefronts only: lt = tid - 64 NW, lw = wv - NW)
    const int lt = tid - WAVE * G::NW, lw = wv - G::NW;
    auto copy = [&](int jj, int sl) {
        const uint8_t* blk = wsu + (size_t)jj * G::BYTES;
        const int64_t t0 = tb + (p.chunk0 + jj) * C;
        const int Lc = (int)((te - t0) < C ? (te - t0) : C);
        uint8_t* slot = lds + sl * G::SLOT + lw * (WAVE * 16);
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            const uint8_t* src;
            if ((r + 1) * LT <= G::NPB) {
                src = (blk + r * LT * 16) + (uint32_t)(16 * lt);
            } else {
                const int pc = min(r * LT + lt, G::NPS - 1);
                int t, u;
                vpiece_source<G::VPR>(max(pc - G::NPB, 0), t, u);
                // rows past the chunk's end repeat its last row: they meet zero operator columns
                const int64_t row = (t0 + min(t, Lc - 1)) * H + h;
                const uint8_t* vsrc = reinterpret_cast<const uint8_t*>(gv + row * DV + dv0 + 8 * u);
                src = pc < G::NPB ? blk + 16 * pc : vsrc;
            }
            __builtin_amdgcn_global_load_lds(src, slot + r * LT * 16, 16, 0, 0);
        }
    };
    // Touch the operator block of chunk jj into L2 (HBM latency is what limits
    // the copies otherwise): one dword per 128-byte line, slice s taking lines
    // s, s + split, ... (the slices of a head share the block through L2), one
    // instruction per copy wavefront.  The dwords land in the pad of slot lw.
    auto touch = [&](int jj) {
        constexpr int LINES = (G::BYTES + 127) / 128;
        const int nb = (LINES - slice + p.split - 1) / p.split;  // this slice's lines (>= 1)
        const int line = min(lt, nb - 1) * p.split + slice;
        __builtin_amdgcn_global_load_lds(wsu + (size_t)jj * G::BYTES + 128 * line, lds + lw * G::SLOT + G::NPS * 16,
                                         4, 0, 0);
    };
    // Store chunk jj's outputs, which the compute wavefronts left in the value
    // tile of its slot sl: each lane stores the 16-byte pieces that its own copy
    // into that slot will overwrite next, so it reads them before it issues the
    // copy (rows past the chunk's end are skipped).
    auto store_out = [&](int jj, int sl) {
        const int64_t t0 = tb + (p.chunk0 + jj) * C;
        const int Lc = (int)((te - t0) < C ? (te - t0) : C);
        const uint8_t* slot = lds + sl * G::SLOT;
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            if ((r + 1) * LT <= G::NPB || r * LT >= G::NPS) continue;  // rounds without output pieces
            const int pc = r * LT + lt;
            int t, u;
            vpiece_source<G::VPR>(max(pc - G::NPB, 0), t, u);
            if (pc >= G::NPB && pc < G::NPS && t < Lc) {
                const i32x4 x = *reinterpret_cast<const i32x4*>(slot + 16 * pc);
                *reinterpret_cast<i32x4*>(go + ((t0 + t) * H + h) * DV + dv0 + 8 * u) = x;
            }
        }
        __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8) | 0xF);  // lgkmcnt(0): pieces read before the copy lands
        asm volatile("" ::: "memory");
    };

    if (wv >= G::NW) {
        // ---- copy wavefronts: chunk jj + AHEAD is copied during chunk jj and chunk
        // jj + AHEAD + TOUCH touched; before the barrier of chunk jj, chunk jj + 1's
        // copies are waited for: younger are the copies of AHEAD - 1 chunks and AHEAD
        // touches (one follows every copy), and loads complete in order.  One barrier
        // before the walk and one per chunk, like the compute wavefronts.
        if (nch > 0) {
#pragma unroll
            for (int c = 0; c < G::AHEAD; ++c) {
                copy(min(c, nch - 1), c);
                touch(min(c + G::TOUCH, nch - 1));
            }
        }
        slot_barrier<(G::AHEAD - 1) * ROUNDS + G::AHEAD>();
        for (int jj = 0; jj < nch; ++jj) {
            // the slot refilled now is chunk jj - 1's: its outputs leave first
            if (jj > 0) store_out(jj - 1, (jj - 1) % G::NBUF);
            copy(min(jj + G::AHEAD, nch - 1), (jj + G::AHEAD) % G::NBUF);
            touch(min(jj + G::AHEAD + G::TOUCH, nch - 1));
            slot_barrier<(G::AHEAD - 1) * ROUNDS + G::AHEAD>();
        }
        if (nch > 0) store_out(nch - 1, (nch - 1) % G::NBUF);
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): no copy outlives the workgroup
        return;
    }

    // ---- state: column blocks cb of this wavefront, rows 16 r + 4 lg + i ------------
    f32x4 acc[CB][NR];
    const int64_t sb = (int64_t)unit * DK * DV + dv0 + 16 * wv * CB + lr;
    if (p.S_in) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[cb][r][i] = p.S_in[sb + 16 * cb + (int64_t)(16 * r + 4 * lg + i) * DV];
    } else {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[cb][r] = zero4();
    }
    bf16x8 sfr[CB][NKS];
    auto make_sfr = [&]() {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sfr[cb][ks][i] = (bf16)acc[cb][2 * ks][i];
                    sfr[cb][ks][4 + i] = (bf16)acc[cb][2 * ks + 1][i];
                }
    };
    make_sfr();

    // snapshots: the state after every snap_every tokens of the sequence goes to
    // row snap0 + (tokens / snap_every) - 1; snap_cd counts the chunks to the next
    int64_t snap0 = 0;
    int snap_ec = 1, snap_cd = 0;
    if (SNAP) {
        snap0 = snapshots_before(p.cu, p.eq_len, n, p.snap_every);
        snap_ec = p.snap_every / C;
        snap_cd = snap_ec - (int)(p.chunk0 % snap_ec);
    }

    slot_barrier<0>();

    // outputs of a chunk go (bf16) into the value tile of its slot, which the
    // value fragments have left by then; the copy wavefronts store them
    f32x4 ot[CB][NTT];
    // this lane's output piece offsets (token 16 tt + lr, columns 16 (wv CB + cb) + 4 lg ..)
    uint32_t oO[CB][NTT];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
            oO[cb][tt] = G::NPB * 16 + 16 * vpiece<G::VPR>(16 * tt + lr, 2 * (wv * CB + cb) + (lg >> 1)) +
                         8 * (lg & 1);

    auto frag = [](const uint8_t* a) { return *reinterpret_cast<const bf16x8*>(a); };
    // Group 1 of a chunk: the E operands and the value fragment (column j of the
    // value tile, tokens 8 lg .. 8 lg + 7).  It is read right after
    // the barrier that publishes the chunk, while the previous chunk's state
    // update runs on the matrix cores.  The O operands are read with group 2,
    // which keeps the registers live across the state update within the
    // register file (no accumulator-register round trips).
    bf16x8 wf[NTT][NKS], m1f[NTT], vfr[CB];
    bf16 vraw[CB][8];  // value elements as read; packed into vfr where first used
    auto read_group1 = [&](const uint8_t* B) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int u = 2 * (wv * CB + cb) + (lr >> 3);
                vraw[cb][e] = *reinterpret_cast<const bf16*>(
                    B + G::NPB * 16 + 16 * vpiece<G::VPR>(8 * lg + e, u) + 2 * (lr & 7));
            }
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            m1f[tt] = frag(B + oM + WS::M1 + 16 * 16 * tt);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) wf[tt][ks] = frag(B + oW[ks] + WS::W + 16 * tt * RBK);
        }
    };
    if (nch > 0) read_group1(lds);

    // Chunks run in stretches that end at the snapshot points (one stretch of all
    // chunks without snapshots), so the snapshot store sits outside the chunk loop.
    int jj = 0;
    while (jj < nch) {
        const int jend = SNAP ? min(nch, jj + snap_cd) : nch;
        for (; jj < jend; ++jj) {
            uint8_t* B = lds + (jj % G::NBUF) * G::SLOT;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int e = 0; e < 8; ++e) vfr[cb][e] = vraw[cb][e];
            __builtin_amdgcn_sched_barrier(0);

            // E = -(W S + M1 V): rows in W's row order, so that each lane's two
            // accumulator quads are tokens 8 lg .. 8 lg + 7, column j (lane)
            f32x4 z[CB][NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    f32x4 x = Mma<bf16>::mma(m1f[tt], vfr[cb], zero4());
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) x = Mma<bf16>::mma(wf[tt][ks], sfr[cb][ks], x);
                    z[cb][tt] = x;
                }
            __builtin_amdgcn_sched_barrier(0);

            // group 2: the O operands, then the state-update operands (in flight
            // during the O products)
            bf16x8 qpf[NTT][NKS], m2f[NTT], ktf[NR], kcf[NR];
            f32x4 gmv[NR];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                m2f[tt] = frag(B + oM + WS::M2 + 16 * 16 * tt);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) qpf[tt][ks] = frag(B + oW[ks] + WS::QP + 16 * tt * RBK);
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                if (!ORD1) ktf[r] = frag(B + oK + WS::KT + 16 * 16 * r);
                kcf[r] = frag(B + oK + WS::KC + 16 * 16 * r);
                gmv[r] = *reinterpret_cast<const f32x4*>(B + oG + 64 * r);
            }
            __builtin_amdgcn_sched_barrier(0);

            // O^T = S^T QP^T + V^T M2^T with the state at the chunk start
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    f32x4 x = Mma<bf16>::mma(vfr[cb], m2f[tt], zero4());
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) x = Mma<bf16>::mma(sfr[cb][ks], qpf[tt][ks], x);
                    ot[cb][tt] = x;
                }
            bf16x8 efr[CB], vkeep[CB];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                vkeep[cb] = vfr[cb];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    efr[cb][i] = (bf16)(-z[cb][0][i]);
                    efr[cb][4 + i] = (bf16)(-z[cb][1][i]);
                }
            }
            // outputs into this slot's value tile, stored by the copy wavefronts
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt)
                    store4(reinterpret_cast<bf16*>(B + oO[cb][tt]), ot[cb][tt]);
            __builtin_amdgcn_sched_barrier(0);

            // This chunk's LDS reads and output writes are done; the barrier hands
            // its slot to the copy wavefronts and publishes chunk jj + 1.
            slot_barrier<63>();
            // next chunk's group 1 (after the last chunk: a harmless read of a stale slot)
            read_group1(lds + ((jj + 1) % G::NBUF) * G::SLOT);
            __builtin_amdgcn_sched_barrier(0);

            // S <- Diag(GAM) S + KT V + KC E   (decay-first blocks: no KT V)
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    f32x4 x = acc[cb][r] * gmv[r];
                    if (!ORD1) x = Mma<bf16>::mma(ktf[r], vkeep[cb], x);
                    acc[cb][r] = Mma<bf16>::mma(kcf[r], efr[cb], x);
                }
            __builtin_amdgcn_sched_barrier(0);
            make_sfr();
        }
        if (SNAP) {
            // jj chunks done: a snapshot point unless the walk ended first
            if ((p.chunk0 + jj) % snap_ec == 0) {
                const int64_t done = (p.chunk0 + jj) * C;  // tokens of the sequence behind this state
                const int64_t row = snap0 + done / p.snap_every - 1;
                if (done <= te - tb && row < p.snap_rows) {
                    float* dst = p.snap + (row * H + h) * DK * DV + dv0 + 16 * wv * CB;
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                        for (int r = 0; r < NR; ++r)
                            store_state_tile(dst + 16 * cb + (int64_t)16 * r * DV, DV, lane, acc[cb][r]);
                }
            }
            snap_cd = snap_ec;
        }
    }

#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) p.S_out[sb + 16 * cb + (int64_t)(16 * r + 4 * lg + i) * DV] = acc[cb][r][i];
}

// ------------------------------------------------------------------------------------
template <int DK, int DVS, int CB, bool ORD1>
static hipError_t scan_cfg(const ScanLaunch& a, hipStream_t stream) {
    ScanParams p;
    p.v = a.v; p.o = a.o; p.cu = a.cu_seqlens; p.eq_len = a.eq_len;
    p.ws = static_cast<const uint8_t*>(a.ws); p.S_in = a.S_in; p.S_out = a.S_out;
    p.H = a.num_heads; p.DV = a.dv; p.split = a.split; p.m = a.m; p.chunk0 = a.chunk0;
    p.snap = a.snap; p.snap_rows = a.snap_rows; p.snap_every = a.snap_every;
    p.ord = a.ord;
    const int64_t blocks = (int64_t)a.units * a.split;
    if (p.ord)  // the rank mapping deals whole units to the XCDs: it needs a multiple of 8 units
        p.xcd_group = a.units % 8 == 0 ? 1 : 0;
    else
        p.xcd_group = (a.split > 1 && blocks % 8 == 0 && (blocks / 8) % a.split == 0) ? 1 : 0;
    constexpr int NT = ScanCfg<DK, DVS, CB, ORD1>::NT;
    if (a.snap)
        hipLaunchKernelGGL((kda_scan_kernel<DK, DVS, CB, true, ORD1>), dim3((unsigned)blocks), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((kda_scan_kernel<DK, DVS, CB, false, ORD1>), dim3((unsigned)blocks), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

// Compiled slices: 16-column slices use one block per wavefront; wider ones two.
#define KDA_SCAN_CASE(DK_, DVS_, CB_)                                                                 \
    if (dk == DK_ && dvs == DVS_) {                                                                   \
        if (a) *err = a->order ? scan_cfg<DK_, DVS_, CB_, true>(*a, stream)                         \
                               : scan_cfg<DK_, DVS_, CB_, false>(*a, stream);                       \
        return true;                                                                                  \
    }

static bool scan_dispatch(int dk, int dvs, int chunk, const ScanLaunch* a, hipStream_t stream, hipError_t* err) {
    if (chunk != 32) return false;
    KDA_SCAN_CASE(128, 16, 1) KDA_SCAN_CASE(128, 32, 1) KDA_SCAN_CASE(128, 64, 2) KDA_SCAN_CASE(128, 128, 2)
    KDA_SCAN_CASE(64, 16, 1) KDA_SCAN_CASE(64, 32, 1) KDA_SCAN_CASE(64, 64, 2) KDA_SCAN_CASE(64, 128, 2)
    return false;
}

// ord[r] = the sequence of rank r when sequences are ordered by decreasing
// length, equal lengths by index.  Thread i counts the sequences that come
// before sequence i, reading the lengths through LDS in tiles.
__global__ void __launch_bounds__(256) kda_seq_rank_kernel(const int32_t* __restrict__ cu, int N,
                                                             int32_t* __restrict__ ord) {
    constexpr int TILE = 1024;
    __shared__ int32_t len_s[TILE];
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int32_t li = i < N ? cu[i + 1] - cu[i] : 0;
    int rank = 0;
    for (int base = 0; base < N; base += TILE) {
        const int cnt = min(TILE, N - base);
        __syncthreads();
        for (int t = threadIdx.x; t < cnt; t += 256) len_s[t] = cu[base + t + 1] - cu[base + t];
        __syncthreads();
        for (int t = 0; t < cnt; ++t) {
            const int32_t lj = len_s[t];
            rank += (lj > li) || (lj == li && base + t < i);
        }
    }
    if (i < N) ord[rank] = i;
}

hipError_t launch_seq_rank(const int32_t* cu_seqlens, int num_seqs, int32_t* ord, hipStream_t stream) {
    hipLaunchKernelGGL(kda_seq_rank_kernel, dim3((num_seqs + 255) / 256), dim3(256), 0, stream, cu_seqlens, num_seqs,
                       ord);
    return hipGetLastError();
}

bool two_pass_supported(int dtype, int dk, int dvs, int chunk) {
    return dtype == 1 && prep_block_bytes(dk, chunk, 0) > 0 && scan_dispatch(dk, dvs, chunk, nullptr, nullptr, nullptr);
}

hipError_t launch_scan(const ScanLaunch& a, hipStream_t stream) {
    hipError_t err = hipErrorInvalidValue;
    if (!scan_dispatch(a.dk, a.dv / a.split, a.chunk, &a, stream, &err)) return hipErrorInvalidValue;
    return err;
}

}  // namespace kda
