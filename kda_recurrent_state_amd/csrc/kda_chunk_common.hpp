// kda_chunk_common.hpp -- device helpers shared by the chunked-prefill kernels:
// thread-to-element maps, LDS-only barriers, 2-element vectors and the
// triangular solve of one chunk.
#pragma once

#include "kda_device.hpp"

namespace kda {

constexpr float LOG2E = 1.4426950408889634f;

// Unit (4 tokens x 2 channels) of thread slot uu: a wavefront covers 32
// consecutive channel pairs of two token groups, so its row-major stores are
// contiguous and its transposed stores use every LDS bank.
template <int NCP>
__device__ __forceinline__ void unit_of(int uu, int& c, int& tg) {
    if constexpr (NCP >= 32) {
        const int w = uu >> 6, l = uu & 63;
        constexpr int HALVES = NCP / 32;  // 32-pair groups of the channel pairs
        c = 2 * ((l & 31) + 32 * (w % HALVES));
        tg = (l >> 5) + 2 * (w / HALVES);
    } else {
        c = 2 * (uu % NCP);
        tg = uu / NCP;
    }
}

// Transposed operands ([channel][token]) are written four channels at a time
// by one thread.  Their rows are stored in four planes, channel c at row
// (c & 3) * (N/4 + 4) + (c >> 2), so neither those writes nor the matrix-core
// fragment reads of 16 consecutive channels collide on LDS banks.
template <int N>
__device__ __forceinline__ int prow(int c) { return (c & 3) * (N / 4 + 4) + (c >> 2); }
template <int N>
constexpr int prows() { return N + 16; }

// Workgroup barrier that orders LDS only: global loads issued before it stay in
// flight (the next chunk's inputs are prefetched across it).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders LDS traffic between lanes of one wavefront (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Snapshot rows of the sequences before sequence n: the sum over m < n of
// floor(len_m / every).  Called by whole wavefronts (lanes stride over the
// sequences, then a butterfly sum); the result is the same in every lane.
// cu null: every sequence has eq_len tokens.
__device__ inline int64_t snapshots_before(const int32_t* cu, int64_t eq_len, int n, int every) {
    if (!cu) return (int64_t)n * (eq_len / every);
    int64_t s = 0;
    for (int m = (int)(threadIdx.x & 63); m < n; m += 64) s += (cu[m + 1] - cu[m]) / every;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    return s;
}

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

template <int CTRL>
__device__ __forceinline__ int dpp(int x) { return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false); }

// 4 x 4 transpose of dwords inside each lane quad: lane v of a quad ends with
// dword v of every lane w of its quad (as its dword w).
__device__ __forceinline__ i32x4 quad_transpose(i32x4 m, int lane) {
    const int v = lane & 3;
    i32x4 n1, n2;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int t = dpp<0xB1>(m[d ^ 1]);  // quad_perm [1, 0, 3, 2]: lane v ^ 1's dword d ^ 1
        n1[d] = ((v ^ d) & 1) ? t : m[d];
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int t = dpp<0x4E>(n1[d ^ 2]);  // quad_perm [2, 3, 0, 1]: lane v ^ 2's dword d ^ 2
        n2[d] = ((v ^ d) & 2) ? t : n1[d];
    }
    return n2;
}

template <int CTRL>
__device__ __forceinline__ float dppf(float x) { return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(int, x))); }
__device__ __forceinline__ float readlanef(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// Sum of x over each row of 16 lanes, left in every lane of the row (quad
// swaps, then rotations of the row by 4 and by 8).
__device__ __forceinline__ float row_sum16(float x) {
    x += dppf<0xB1>(x);
    x += dppf<0x4E>(x);
    x += dppf<0x124>(x);
    x += dppf<0x128>(x);
    return x;
}

// Input prologue (kda_prologue_t).  log a = max(-softplus(x), lo) is formed in
// the log2 domain from the hardware exp2 and log2, in the form that cannot
// overflow: softplus2(y) = max(y, 0) + log2(1 + 2^{-|y|}) with y = x log2 e, so
// the result is finite for every finite x (and -x log2 e for large x), then
// clipped at lo2 = lo log2 e.  beta = 1 / (1 + e^{-x}).
__device__ __forceinline__ float prologue_log2_a(float x, float lo2) {
    const float y = x * LOG2E;
    return fmaxf(-(fmaxf(y, 0.f) + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(y)))), lo2);
}
__device__ __forceinline__ float prologue_beta(float x) { return 1.f / (1.f + __expf(-x)); }

// Decay range of the factored chunk products.  Inside a 16-token block the
// Gram operands carry decay factors relative to the block's mid-point, each a
// product of at most 8 per-token decays, so while every valid token of a chunk
// has log2 a >= STEEP_LOG2 every such factor lies in [2^-96, 2^96].  A factor
// referenced to the chunk start or end that would fall below the fp32 range
// (2^-126) then changes the product it enters by at most 2^{96 - 126}.  A chunk
// with a steeper token (log a < -8.3) takes exact_gram and chunk-referenced
// operands formed with one exponential each instead.
constexpr float STEEP_LOG2 = -12.f;

// True in every lane when some lane's `steep` is set (one wavefront).
__device__ __forceinline__ bool wave_any(bool steep) { return __ballot(steep) != 0; }

// Masked C x C Gram products of one chunk with one exponential per term, for
// chunks whose decay is too steep for the factor split.  With la_j the log2
// decay of token j (0 on padded rows) and a sum over key channels c,
//   A  (t, i) = sum_c k_t k_i 2^{la_i + ... + la_{t-1}}       i <  t
//   L  (t, i) = sum_c k_t k_i 2^{la_{i+1} + ... + la_{t-1}}   i <  t
//   P1 (t, i) = sum_c q_t k_i 2^{la_i + ... + la_t}           i <= t
//   P2 (t, i) = sum_c q_t k_i 2^{la_{i+1} + ... + la_t}       i <= t
// and for the decay-first order (ORD1) only
//   A  (t, i) = sum_c k_t k_i 2^{la_{i+1} + ... + la_t}       i <  t,   with P2 as above.
// Each exponent is a running sum of consecutive log2 decays (all <= 0), so no
// factor leaves the fp32 range and none is the difference of two large sums.
// Work: wavefront w takes key rows i = 4 qd + r (qd = w, w + NW, ...; r the
// lane's 16-lane group, which covers DK / 16 channels per lane), sweeps t
// upward keeping its running exponents, and sums each entry over the 16 lanes
// of the group.  emit(t, i, a, l, p1, p2) runs in lane 16 r for every i <= t
// (a = l = 0 at i == t; l = p1 = 0 for ORD1).  K, Q: raw rows [C][ldk] (16-byte
// aligned); LA: log2 decays [C][ldl].
template <typename T, int DK, int C, int NW, bool ORD1, typename Emit>
__device__ __forceinline__ void exact_gram(const T* K, const T* Q, int ldk, const float* LA, int ldl, int wv,
                                           int lane, Emit emit) {
    constexpr int CPL = DK / 16;
    const int r = lane >> 4, c0 = (lane & 15) * CPL;
#pragma unroll 1
    for (int qd = wv; qd < C / 4; qd += NW) {
        const int i = 4 * qd + r;
        float ki[CPL], lai[CPL], s[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            ki[e] = to_f32(K[i * ldk + c0 + e]);
            lai[e] = LA[i * ldl + c0 + e];
            s[e] = 0.f;  // la_{i+1} + ... + la_{t-1}
        }
#pragma unroll 1
        for (int t = 4 * qd; t < C; ++t) {
            const bool below = t > i;
            float a = 0.f, l = 0.f, p1 = 0.f, p2 = 0.f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                const float kt = to_f32(K[t * ldk + c0 + e]), qt = to_f32(Q[t * ldk + c0 + e]);
                const float lt = LA[t * ldl + c0 + e];
                const float kk = kt * ki[e], qk = qt * ki[e];
                const float e2 = below ? s[e] + lt : 0.f;  // la_{i+1} + ... + la_t
                const float f2 = __builtin_amdgcn_exp2f(e2);
                p2 += qk * f2;
                if (ORD1) {
                    a += kk * f2;
                } else {
                    const float e1 = below ? e2 + lai[e] : lt;  // la_i + ... + la_t
                    a += kk * __builtin_amdgcn_exp2f(s[e] + lai[e]);
                    l += kk * __builtin_amdgcn_exp2f(s[e]);
                    p1 += qk * __builtin_amdgcn_exp2f(e1);
                }
                if (below) s[e] += lt;
            }
            a = row_sum16(a);
            p2 = row_sum16(p2);
            if (!ORD1) {
                l = row_sum16(l);
                p1 = row_sum16(p1);
            }
            if (t >= i && (lane & 15) == 0) emit(t, i, below ? a : 0.f, below ? l : 0.f, p1, p2);
        }
    }
}

// Stores one 16 x 16 fp32 accumulator tile (lane: column lane % 16, rows
// 4 (lane / 16) .. + 3) into a row-major state with row stride DV; dst points at
// the tile's element (0, 0).  After a transpose inside lane quads each lane
// holds four consecutive columns of one row and writes them with one 16-byte
// store (whole wavefront: 16 rows x 64 bytes).
__device__ __forceinline__ void store_state_tile(float* dst, int64_t DV, int lane, f32x4 t) {
    const i32x4 x = quad_transpose(__builtin_bit_cast(i32x4, t), lane);
    const int row = 4 * (lane >> 4) + (lane & 3), col = 4 * ((lane & 15) >> 2);
    *reinterpret_cast<f32x4*>(dst + (int64_t)row * DV + col) = __builtin_bit_cast(f32x4, x);
}

__device__ __forceinline__ float uniform(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

template <typename T> struct Vec2;
template <> struct Vec2<bf16> {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 type;
    static __device__ __forceinline__ float lo(type v) { return (float)v[0]; }
    static __device__ __forceinline__ float hi(type v) { return (float)v[1]; }
    static __device__ __forceinline__ type make(float a, float b) { type r; r[0] = (bf16)a; r[1] = (bf16)b; return r; }
};
template <> struct Vec2<float> {
    typedef __attribute__((__vector_size__(2 * sizeof(float)))) float type;
    static __device__ __forceinline__ float lo(type v) { return v[0]; }
    static __device__ __forceinline__ float hi(type v) { return v[1]; }
    static __device__ __forceinline__ type make(float a, float b) { type r; r[0] = a; r[1] = b; return r; }
};
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

template <typename T>
__device__ __forceinline__ void store2(T* p, float a, float b) {
    *reinterpret_cast<typename Vec2<T>::type*>(p) = Vec2<T>::make(a, b);
}

// (I + A)^-1 diag(b) for a strictly lower C x C matrix A (fp32, row-major, ld
// LDA), on one wavefront, written as Tb (row-major, ld LDC, upper blocks left
// untouched).  Blocked right-looking forward substitution on fp32 matrix
// cores: the right-hand sides (identity columns of one 16-column block) live
// in 16 x 16 accumulator tiles, where lane group g holds rows 4g..4g+3; each
// 4-row panel is solved inside the lanes that hold it, passed to all lanes
// through LDS (X, double-buffered), and every tile below is updated with one
// 16x16x4 product.  Block columns are independent chains.  All coefficients
// are read before the chain starts (the uniform ones into scalar registers);
// the code has no lane-dependent branches.
template <typename T, int C, int LDA, int LDC>
__device__ __forceinline__ void block_inverse(const float* A, const float* beta, float* X, T* Tb, int lane) {
    constexpr int NB = C / 16, NP = 4 * NB;
    const int l16 = lane & 15, lg = lane >> 4;
    float cf[NP][6];
    float aop[NP][NB];
#pragma unroll
    for (int sp = 0; sp < NP; ++sp) {
        const int r0 = 4 * sp;
        cf[sp][0] = uniform(A[(r0 + 1) * LDA + r0]);
        cf[sp][1] = uniform(A[(r0 + 2) * LDA + r0]);
        cf[sp][2] = uniform(A[(r0 + 2) * LDA + r0 + 1]);
        cf[sp][3] = uniform(A[(r0 + 3) * LDA + r0]);
        cf[sp][4] = uniform(A[(r0 + 3) * LDA + r0 + 1]);
        cf[sp][5] = uniform(A[(r0 + 3) * LDA + r0 + 2]);
#pragma unroll
        for (int tr = 0; tr < NB; ++tr) {
            const int row = 16 * tr + l16;
            const float x = (tr >= sp / 4) ? A[row * LDA + r0 + lg] : 0.f;
            aop[sp][tr] = (row > r0 + 3) ? -x : 0.f;
        }
    }
    f32x4 R[NB][NB];  // R[bc][tr]: rows of tile tr, columns of block column bc
#pragma unroll
    for (int bc = 0; bc < NB; ++bc)
#pragma unroll
        for (int tr = 0; tr < NB; ++tr)
#pragma unroll
            for (int r = 0; r < 4; ++r) R[bc][tr][r] = (tr == bc && 4 * lg + r == l16) ? 1.f : 0.f;
#pragma unroll
    for (int sp = 0; sp < NP; ++sp) {  // panel: rows 4 sp .. 4 sp + 3
        const int ts = sp / 4, g = sp % 4;
        float* Xb = X + (sp & 1) * (NB * 256);
#pragma unroll
        for (int bc = 0; bc <= ts; ++bc) {
            f32x4 x = R[bc][ts];
            x[1] -= cf[sp][0] * x[0];
            x[2] -= cf[sp][1] * x[0] + cf[sp][2] * x[1];
            x[3] -= cf[sp][3] * x[0] + cf[sp][4] * x[1] + cf[sp][5] * x[2];
            R[bc][ts] = (lg == g) ? x : R[bc][ts];
            // every lane group writes its own slot; group g's slot is the panel
            *reinterpret_cast<f32x4*>(&Xb[bc * 256 + lg * 64 + 4 * l16]) = x;
        }
        wave_sync();
#pragma unroll
        for (int bc = 0; bc <= ts; ++bc) {
            const float bk = Xb[bc * 256 + g * 64 + 4 * l16 + lg];  // B[k = lg][n = l16]
#pragma unroll
            for (int tr = ts; tr < NB; ++tr)
                R[bc][tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop[sp][tr], bk, R[bc][tr], 0, 0, 0);
        }
    }
    // Tb = T diag(b): lane holds column 16 bc + l16, rows 16 tr + 4 lg + r
#pragma unroll
    for (int bc = 0; bc < NB; ++bc) {
        const float bcol = beta[16 * bc + l16];
#pragma unroll
        for (int tr = bc; tr < NB; ++tr)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Tb[(16 * tr + 4 * lg + r) * LDC + 16 * bc + l16] = from_f32<T>(R[bc][tr][r] * bcol);
    }
}

// Ends a step of a walk fed through LDS slots: waits until at most N
// vector-memory operations of this wavefront are outstanding and all its LDS
// reads have returned, then joins the workgroup barrier.  A release fence is
// not used here: on LDS it would also wait for the copies still in flight into
// the other slots.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void slot_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));  // vmcnt(N) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace kda
