// kda_ws.hpp -- layout of the per-chunk operator blocks that the two-pass
// prefill hands from its chunk-parallel pass (kda_prep.hip) to its sequential
// pass (kda_scan.hip).
//
// For one chunk of one (sequence, head) the block holds, in bf16 unless noted:
//   W   [C][DK]   T diag(b) Kb                      (rows: tokens)
//   QP  [C][DK]   Qb - P1 W                         (rows: tokens)
//   KC  [DK][C]   (Kc Diag(e^{g_C}))^T              (rows: key channels)
//   KT  [DK][C]   (diag(b) Kt Diag(e^{g_C}))^T      (rows: key channels)
//   M1  [C][C]    T diag(b) L diag(b)               (rows: tokens)
//   M2  [C][C]    P2 diag(b) - P1 M1                (rows: tokens)
//   GAM [DK]      e^{g_C}, fp32
// so that the sequential pass computes, per chunk and value column block,
//   E = -(W S + M1 V),  O = QP S + M2 V,  S <- Diag(GAM) S + KC E + KT V.
//
// The decay-first ordering (S <- (I - b k^T k) Diag(a) S + b k^T v) has no
// write term outside E, and its blocks (ORD1) hold no KT:
//   W   T diag(b) Kd           with Kd = K e^{g_t}
//   QP  Qb - R Kd              with R = lower(Qb Kx^T) T diag(b), Kx = K e^{-g_t}
//   KC  (Kx Diag(e^{g_C}))^T
//   M1  -T diag(b)
//   M2  R
// so that E = T diag(b) (V - Kd S) and S <- Diag(GAM) S + KC E.
//
// Every matrix is stored as the matrix-core operand it becomes.  A lane
// group g of a 16 x 16 accumulator holds rows 4g..4g+3 of each 16-row tile,
// and an operand lane group g wants 8 consecutive contraction positions
// 8g..8g+7, so a tile pair fed back as an operand reads its rows in the order
//   kperm(x) = 8 * ((x % 16) / 4) + 4 * (x / 16) + x % 4      (x = index % 32)
// and the blocks are laid out to match:
//   - W, QP: 32-channel blocks of their columns (the contraction with S) in
//     kperm order; rows are 256-byte lines of 16-byte pieces XOR-swizzled by
//     the row, so that 16 lanes reading one piece of 16 rows hit distinct LDS
//     banks after a verbatim copy.  QP row t is token t; W row w is token
//     kperm(w), so that the products W S come out with E's rows in that order
//     and E feeds the state update with tokens in natural order.
//   - M1, M2, KC, KT: token contraction in natural order, stored piece-major:
//     the 16-byte piece holding columns 8g..8g+7 of row r sits at byte
//     16 * (g * ROWS + r).  Rows of M1 follow W, rows of M2 follow QP; rows of
//     KC and KT are key channels.  Operand reads of 16 consecutive rows are
//     then 256 contiguous bytes, and the chunk-parallel pass writes whole
//     pieces of 8 consecutive tokens.
#pragma once

#include <stdint.h>

namespace kda {

template <int DK, int C, bool ORD1 = false>
struct WsBlock {
    static constexpr int W = 0;
    static constexpr int QP = W + C * DK * 2;
    static constexpr int KC = QP + C * DK * 2;
    static constexpr int KT = KC + DK * C * 2;   // absent (zero bytes) in ORD1 blocks
    static constexpr int M1 = KT + (ORD1 ? 0 : DK * C * 2);
    static constexpr int M2 = M1 + C * C * 2;
    static constexpr int GAM = M2 + C * C * 2;
    static constexpr int BYTES = (GAM + DK * 4 + 255) / 256 * 256;  // 256-byte aligned blocks
};

// permuted position of contraction index x
__host__ __device__ constexpr int kperm(int x) {
    return (x & ~31) + 8 * ((x & 15) >> 2) + 4 * ((x & 31) >> 4) + (x & 3);
}
// its inverse: the index held at position p (kperm(kinv(p)) == p)
__host__ __device__ constexpr int kinv(int p) {
    return (p & ~31) + 16 * ((p >> 2) & 1) + 4 * ((p & 31) >> 3) + (p & 3);
}
static_assert(kperm(kinv(5)) == 5 && kperm(kinv(22)) == 22 && kinv(kperm(13)) == 13, "kinv inverts kperm");

// byte offset of the 16-byte piece g of row r in a piece-major matrix of ROWS rows
template <int ROWS>
__host__ __device__ constexpr int piece(int r, int g) { return 16 * (g * ROWS + r); }

// byte offset of the 16-byte piece `piece` of row `row` in a matrix whose rows
// are RB bytes long (RB = 64, 128 or 256)
template <int RB>
__host__ __device__ constexpr int swz(int row, int piece) {
    constexpr int NP = RB / 16;                  // pieces per row
    constexpr int RPW = NP >= 16 ? 1 : 16 / NP;  // rows per 256-byte window
    return row * RB + 16 * (piece ^ ((row / RPW) % NP));
}

// byte offset of element (row, position p) of a bf16 matrix with RB-byte rows
template <int RB>
__host__ __device__ constexpr int swz_elem(int row, int p) {
    return swz<RB>(row, p >> 3) + 2 * (p & 7);
}

}  // namespace kda
