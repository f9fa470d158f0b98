// kda_decode.hip -- one-token decode step of the KDA state layer on gfx950.
//
// Per (sequence, head) the token applies the KDA row of the table on page "The
// argument, in one page" ("Everything, in one table"):
//     S' = Diag(a) (I - beta k^T k) S + beta k^T v,      o = q S'
// Decode cost is the bytes of state read per step (same table, softmax row:
// the cost column counts bytes read per decode step), so the kernel reads each
// fp32 state once and writes it once.  With y = k S and z = (q * a) S (two
// reductions over the dk rows, taken from the same registers):
//     S'[c][j] = a_c (S[c][j] - beta k_c y_j) + beta k_c v_j
//     o_j      = z_j - beta (q*a . k) y_j + beta (q . k) v_j
//
// The decay-first ordering (ORD1, per-channel decay only),
//     S' = (I - beta k^T k) Diag(a) S + beta k^T v,
// reads y = (k * a) S instead:
//     S'[c][j] = a_c S[c][j] - beta k_c y_j + beta k_c v_j
//     o_j      = z_j - beta (q . k) y_j + beta (q . k) v_j
//
// With an input prologue (kda_prologue_t) the raw token inputs are transformed
// on load: beta = 1 / (1 + e^{-x}), log a = max(-softplus(x), min) so that
// a = max(1 / (1 + e^{x}), e^{min}), and k is scaled by r = (|k|^2 + eps)^{-1/2},
// which enters y, the two dot products and the update linearly (y and the dots
// are scaled after their reductions).
//
// One workgroup per state.  Thread (row group rg, column group cg) owns four
// consecutive columns 4cg..4cg+3 of rows rg, rg + RG, ...; a wavefront covers
// whole consecutive rows, so every 16-byte load and store is coalesced.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename T, int DK, int DV, bool SCALAR>
struct DecodeShape {
    static constexpr int CG = DV / 4;                           // column groups
    static constexpr int RG = (DK < 256 / CG) ? DK : 256 / CG;  // row groups
    static constexpr int NT = CG * RG;                          // threads
    static constexpr int RPT = DK / RG;                         // rows per thread
    static constexpr int NW = NT / WAVE;                        // wavefronts
    static_assert(NT % WAVE == 0 && DK % RG == 0, "decode shape");
};

template <typename T, int DK, int DV, bool SCALAR, bool ORD1>
__global__ void __launch_bounds__(256)
kda_decode_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                  const float* __restrict__ log_a, const float* __restrict__ beta,
                  const float* S_in, float* S_out, T* __restrict__ o, Prologue pro) {
    typedef DecodeShape<T, DK, DV, SCALAR> Sh;
    constexpr int CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT, NW = Sh::NW;
    __shared__ float s_k[DK], s_q[DK], s_qa[DK], s_a[DK], s_v[DV], s_dot[3];
    __shared__ f32x4 s_red[2][NW][CG];

    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int lane = tid % WAVE, wv = tid / WAVE;
    const int64_t head = blockIdx.x;  // n * H + h
    const float* Sp = S_in + head * (int64_t)(DK * DV);
    float* So = S_out + head * (int64_t)(DK * DV);

    // 1. the token's vectors first (their loads then complete ahead of the state's,
    //    the counter of outstanding loads draining in order), then the state tile:
    //    RPT 16-byte loads in flight per thread
    static_assert(DK <= Sh::NT && DV <= Sh::NT, "one vector element per thread");
    const int cc = tid < DK ? tid : 0, jj = tid < DV ? tid : 0;
    float b = beta[head];
    float la = SCALAR ? log_a[head] : log_a[head * DK + cc];
    const T qv = q[head * DK + cc], kv = k[head * DK + cc], vv0 = v[head * DV + jj];
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sp + (rg + RG * i) * DV + 4 * cg));

    // 2. per-token vectors
    if (pro.beta_logits) b = 1.f / (1.f + __expf(-b));
    if (tid < DK) {
        if (pro.log_a_raw) la = fmaxf(-(fmaxf(la, 0.f) + log1pf(__expf(-fabsf(la)))), pro.log_a_min);
        const float a = __expf(la);
        const float qc = to_f32(qv);
        s_k[tid] = to_f32(kv);
        s_a[tid] = a;
        s_q[tid] = qc;
        s_qa[tid] = qc * a;
    }
    if (tid < DV) s_v[tid] = to_f32(vv0);
    __syncthreads();

    // q.a.k and q.k for the output, and the key's scale (wave 0)
    if (wv == 0) {
        float d1 = 0.f, d2 = 0.f, kk = 0.f;
        for (int c = lane; c < DK; c += WAVE) {
            d1 += s_qa[c] * s_k[c];
            d2 += s_q[c] * s_k[c];
            kk += s_k[c] * s_k[c];
        }
#pragma unroll
        for (int off = WAVE / 2; off > 0; off >>= 1) {
            d1 += __shfl_xor(d1, off);
            d2 += __shfl_xor(d2, off);
            kk += __shfl_xor(kk, off);
        }
        const float r = pro.normalize_k ? rsqrtf(kk + PROLOGUE_EPS) : 1.f;
        if (lane == 0) { s_dot[0] = d1 * r; s_dot[1] = d2 * r; s_dot[2] = r; }
    }

    // 3. partial y = k S and z = (q*a) S over this thread's rows
    f32x4 y = zero4(), z = zero4();
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const float kr = ORD1 ? s_k[r] * s_a[r] : s_k[r], qr = s_qa[r];
        y += kr * s[i];
        z += qr * s[i];
    }
    // reduce over the row groups inside the wavefront (lanes with equal cg)
#pragma unroll
    for (int off = CG; off < WAVE; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            y[e] += __shfl_xor(y[e], off);
            z[e] += __shfl_xor(z[e], off);
        }
    }
    if (lane < CG) {
        s_red[0][wv][cg] = y;
        s_red[1][wv][cg] = z;
    }
    __syncthreads();
    y = s_red[0][0][cg];
    z = s_red[1][0][cg];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        y += s_red[0][w][cg];
        z += s_red[1][w][cg];
    }
    const float kr_scale = s_dot[2];  // 1 without the prologue's key normalisation
    y *= kr_scale;

    // 4. update in registers and write the state once
    f32x4 vv;
    vv[0] = s_v[4 * cg]; vv[1] = s_v[4 * cg + 1]; vv[2] = s_v[4 * cg + 2]; vv[3] = s_v[4 * cg + 3];
    const f32x4 bv = b * vv;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const float kr = s_k[r] * kr_scale, ar = s_a[r];
        const float bk = b * kr;
        f32x4 ns = ORD1 ? ar * s[i] - bk * y + kr * bv : ar * (s[i] - bk * y) + kr * bv;
        __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(So + r * DV + 4 * cg));
    }
    // 5. output o = z - beta (q*a.k) y + beta (q.k) v   (ORD1: (q.k) in both terms)
    if (rg == 0) {
        const float d1 = ORD1 ? s_dot[1] : s_dot[0], d2 = s_dot[1];
        f32x4 out = z - (b * d1) * y + (b * d2) * vv;
        store4(o + head * DV + 4 * cg, out);
    }
}

#define KDA_DECODE_CASE(T, DK_, DV_, SC, O1)                                                     \
    if (dk == DK_ && dv == DV_) {                                                                \
        typedef DecodeShape<T, DK_, DV_, SC> Sh;                                                 \
        hipLaunchKernelGGL((kda_decode_kernel<T, DK_, DV_, SC, O1>), dim3(heads), dim3(Sh::NT), 0,\
                           stream, (const T*)q, (const T*)k, (const T*)v, log_a, beta, S_in,     \
                           S_out, (T*)o, pro);                                                   \
        return hipGetLastError();                                                                \
    }

#define KDA_DECODE_DIMS(T, SC, O1)                                                                      \
    KDA_DECODE_CASE(T, 16, 16, SC, O1) KDA_DECODE_CASE(T, 16, 32, SC, O1) KDA_DECODE_CASE(T, 16, 64, SC, O1)  \
    KDA_DECODE_CASE(T, 16, 128, SC, O1) KDA_DECODE_CASE(T, 32, 16, SC, O1) KDA_DECODE_CASE(T, 32, 32, SC, O1) \
    KDA_DECODE_CASE(T, 32, 64, SC, O1) KDA_DECODE_CASE(T, 32, 128, SC, O1) KDA_DECODE_CASE(T, 64, 16, SC, O1) \
    KDA_DECODE_CASE(T, 64, 32, SC, O1) KDA_DECODE_CASE(T, 64, 64, SC, O1) KDA_DECODE_CASE(T, 64, 128, SC, O1) \
    KDA_DECODE_CASE(T, 128, 16, SC, O1) KDA_DECODE_CASE(T, 128, 32, SC, O1)                                  \
    KDA_DECODE_CASE(T, 128, 64, SC, O1) KDA_DECODE_CASE(T, 128, 128, SC, O1)

bool decode_supported(int dtype, int dk, int dv) {
    auto ok = [](int d) { return d == 16 || d == 32 || d == 64 || d == 128; };
    return (dtype == 0 || dtype == 1) && ok(dk) && ok(dv);
}

// order 1 comes with per-channel decay only (the host maps scalar decay to order 0)
hipError_t launch_decode(int dtype, int dk, int dv, int scalar, int order, const Prologue& pro, int64_t heads,
                         const void* q,
                         const void* k, const void* v, const float* log_a, const float* beta,
                         const float* S_in, float* S_out, void* o, hipStream_t stream) {
    if (dtype == 1) {
        if (scalar) { KDA_DECODE_DIMS(bf16, true, false) }
        else if (order) { KDA_DECODE_DIMS(bf16, false, true) }
        else { KDA_DECODE_DIMS(bf16, false, false) }
    } else {
        if (scalar) { KDA_DECODE_DIMS(float, true, false) }
        else if (order) { KDA_DECODE_DIMS(float, false, true) }
        else { KDA_DECODE_DIMS(float, false, false) }
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
