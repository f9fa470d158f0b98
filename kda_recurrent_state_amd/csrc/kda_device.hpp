// kda_device.hpp -- device-side building blocks for the gfx950 kernels.
//
// Matrix-core tiles are 16 x 16 with fp32 accumulators (v_mfma_f32_16x16x32_bf16
// for bf16 operands, v_mfma_f32_16x16x4_f32 for fp32 operands).  For both, lane
// l of a 64-wide wavefront holds
//   A operand (16 x K):  row (l % 16), K-slice starting at (l / 16) * KPL
//   B operand (K x 16):  column (l % 16), same K-slice
//   accumulator:         column (l % 16), rows 4 * (l / 16) + r, r = 0..3
// where KPL (elements per lane) is 8 for bf16 and 1 for fp32.  Every operand
// is therefore read from LDS as a matrix whose contraction index is
// contiguous ("k-contiguous"): A as [m][k], B as [n][k].  An accumulator tile
// stored back naturally gives [n][m] with 4 consecutive m per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int WAVE = 64;

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Four consecutive elements of type T <-> float4 (8-byte or 16-byte accesses).
template <typename T> struct Vec4;
template <> struct Vec4<bf16> {
    typedef bf16x4 type;
    static __device__ __forceinline__ f32x4 to_f32(type v) {
        f32x4 r;
        r[0] = (float)v[0]; r[1] = (float)v[1]; r[2] = (float)v[2]; r[3] = (float)v[3];
        return r;
    }
    static __device__ __forceinline__ type from_f32(f32x4 v) {
        type r;
        r[0] = (bf16)v[0]; r[1] = (bf16)v[1]; r[2] = (bf16)v[2]; r[3] = (bf16)v[3];
        return r;
    }
};
template <> struct Vec4<float> {
    typedef f32x4 type;
    static __device__ __forceinline__ f32x4 to_f32(type v) { return v; }
    static __device__ __forceinline__ type from_f32(f32x4 v) { return v; }
};

template <typename T>
__device__ __forceinline__ f32x4 load4(const T* p) {
    return Vec4<T>::to_f32(*reinterpret_cast<const typename Vec4<T>::type*>(p));
}
template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 v) {
    *reinterpret_cast<typename Vec4<T>::type*>(p) = Vec4<T>::from_f32(v);
}

// Matrix-core tile product abstraction over the operand type.
template <typename T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int K = 32;   // contraction per instruction
    static constexpr int KPL = 8;  // contraction elements per lane
    typedef bf16x8 frag;
    // p points at element [m or n = 0][k = 0] of a k-contiguous matrix with
    // leading dimension ld (elements); 16-byte aligned rows required.
    static __device__ __forceinline__ frag load(const bf16* p, int ld, int lane) {
        return *reinterpret_cast<const bf16x8*>(p + (lane & 15) * ld + (lane >> 4) * 8);
    }
    // fragment whose row (this lane's m or n) starts at `row`
    static __device__ __forceinline__ frag loadr(const bf16* row, int lane) {
        return *reinterpret_cast<const bf16x8*>(row + (lane >> 4) * 8);
    }
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // scale the 8 operand elements by per-k factors (fp32), re-rounded to bf16
    static __device__ __forceinline__ frag scale(frag a, const float* f) {
        frag r;
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = (bf16)((float)a[i] * f[i]);
        return r;
    }
};

template <> struct Mma<float> {
    static constexpr int K = 4;
    static constexpr int KPL = 1;
    typedef float frag;
    static __device__ __forceinline__ frag load(const float* p, int ld, int lane) {
        return p[(lane & 15) * ld + (lane >> 4)];
    }
    static __device__ __forceinline__ frag loadr(const float* row, int lane) { return row[lane >> 4]; }
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag scale(frag a, const float* f) { return a * f[0]; }
};

// acc += A[16 x Kdim] * B[Kdim x 16], with this lane's A row starting at `ra`
// and its B row (column of B) at `rb`, both k-contiguous in LDS.  All
// fragments are read before the first product so their latencies overlap.
template <typename T, int KDIM>
__device__ __forceinline__ f32x4 tile_mma_r(const T* ra, const T* rb, f32x4 acc, int lane) {
    constexpr int NK = KDIM / Mma<T>::K;
    typename Mma<T>::frag a[NK], b[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        a[k] = Mma<T>::loadr(ra + k * Mma<T>::K, lane);
        b[k] = Mma<T>::loadr(rb + k * Mma<T>::K, lane);
    }
#pragma unroll
    for (int k = 0; k < NK; ++k) acc = Mma<T>::mma(a[k], b[k], acc);
    return acc;
}

// Same, for A given as [m][k] at pa (ld lda) and B as [n][k] at pb (ld ldb).
template <typename T, int KDIM>
__device__ __forceinline__ f32x4 tile_mma(const T* pa, int lda, const T* pb, int ldb, f32x4 acc,
                                          int lane) {
    return tile_mma_r<T, KDIM>(pa + (lane & 15) * lda, pb + (lane & 15) * ldb, acc, lane);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace kda
