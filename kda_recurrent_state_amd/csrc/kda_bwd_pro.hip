// kda_bwd_pro.hip -- the input prologue around the prefill's gradient.
//
// The prologue (kda_prologue_t) turns a layer's raw projections into the
// recurrence's inputs: unit keys k = x / sqrt(|x|^2 + eps), a logistic write
// strength beta = 1 / (1 + e^-z) and a log-decay log a = max(-softplus(y), lo).
// The pages fix no gate parameterisation; these are the usual learned gates.
// For the gradient of a call with a prologue, the transformed inputs are
// formed once (kda_pro_apply_kernel), the gradient runs on them, and the chain
// rule through the transforms is applied to its outputs in place
// (kda_pro_grad_kernel):
//   dx = (dk - k (k . dk)) / sqrt(|x|^2 + eps)   (k the unit key, per token and head)
//   dz = dbeta * beta (1 - beta)
//   dy = dlog_a * (-1 / (1 + e^-y)) where -softplus(y) >= lo, else 0
// Both are elementwise over (token, head) rows, HBM-bound: a row of dk
// channels is covered by dk / 4 consecutive lanes, four channels each, and
// the key's norm and dot product are summed over those lanes.
#include "kda_device.hpp"
#include "kda_chunk_common.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr float LN2 = 0.6931471805599453f;

struct ProArgs {
    const void* k;         // raw keys [rows, DK]
    const float* log_a;    // raw log-decay inputs [rows, DK] or [rows]
    const float* beta;     // raw beta inputs [rows]
    void* k_out;           // apply: unit keys; grad: dk in place
    float* la_out;         // apply: log a; grad: dlog_a in place
    float* b_out;          // apply: beta; grad: dbeta in place
    int64_t rows;
    int scalar;
    int nk, bl, la;
    float lo2;             // clip of log2 a (-inf: none)
};

// sum over the G consecutive lanes that hold one row, in a fixed order
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

__device__ __forceinline__ float sigmoid(float z) { return 1.f / (1.f + __expf(-z)); }

template <typename T, int DK>
__global__ __launch_bounds__(256) void kda_pro_apply_kernel(ProArgs a) {
    constexpr int G = DK / 4, RPB = 256 / G;
    const int tid = threadIdx.x, g = tid % G;
    int64_t row = (int64_t)blockIdx.x * RPB + tid / G;
    const bool live = row < a.rows;
    if (!live) row = a.rows - 1;  // every lane of a row group takes part in the sums
    const int64_t e = row * DK + 4 * g;
    if (a.nk) {
        f32x4 k = load4(static_cast<const T*>(a.k) + e);
        const float ss = group_sum<G>(k[0] * k[0] + k[1] * k[1] + k[2] * k[2] + k[3] * k[3]);
        const float r = rsqrtf(ss + PROLOGUE_EPS);
        if (live) store4(static_cast<T*>(a.k_out) + e, f32x4{k[0] * r, k[1] * r, k[2] * r, k[3] * r});
    }
    if (!live) return;
    if (a.la) {
        if (a.scalar) {
            if (g == 0) a.la_out[row] = prologue_log2_a(a.log_a[row], a.lo2) * LN2;
        } else {
            const f32x4 y = *reinterpret_cast<const f32x4*>(a.log_a + e);
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = prologue_log2_a(y[i], a.lo2) * LN2;
            *reinterpret_cast<f32x4*>(a.la_out + e) = o;
        }
    }
    if (a.bl && g == 0) a.b_out[row] = sigmoid(a.beta[row]);
}

template <typename T, int DK>
__global__ __launch_bounds__(256) void kda_pro_grad_kernel(ProArgs a) {
    constexpr int G = DK / 4, RPB = 256 / G;
    const int tid = threadIdx.x, g = tid % G;
    int64_t row = (int64_t)blockIdx.x * RPB + tid / G;
    const bool live = row < a.rows;
    if (!live) row = a.rows - 1;
    const int64_t e = row * DK + 4 * g;
    if (a.nk) {
        const f32x4 x = load4(static_cast<const T*>(a.k) + e);
        const f32x4 dkh = load4(static_cast<const T*>(a.k_out) + e);
        const float ss = group_sum<G>(x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]);
        const float r = rsqrtf(ss + PROLOGUE_EPS);
        const f32x4 kh = f32x4{x[0] * r, x[1] * r, x[2] * r, x[3] * r};
        const float dot = group_sum<G>(kh[0] * dkh[0] + kh[1] * dkh[1] + kh[2] * dkh[2] + kh[3] * dkh[3]);
        f32x4 dx;
#pragma unroll
        for (int i = 0; i < 4; ++i) dx[i] = (dkh[i] - kh[i] * dot) * r;
        if (live) store4(static_cast<T*>(a.k_out) + e, dx);
    }
    if (!live) return;
    if (a.la) {
        // d log a / dy = -sigmoid(y) while the clip is not active
        auto dy = [&](float y, float d) {
            return prologue_log2_a(y, -INFINITY) >= a.lo2 ? -d * sigmoid(y) : 0.f;
        };
        if (a.scalar) {
            if (g == 0) a.la_out[row] = dy(a.log_a[row], a.la_out[row]);
        } else {
            const f32x4 y = *reinterpret_cast<const f32x4*>(a.log_a + e);
            f32x4 d = *reinterpret_cast<const f32x4*>(a.la_out + e);
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] = dy(y[i], d[i]);
            *reinterpret_cast<f32x4*>(a.la_out + e) = d;
        }
    }
    if (a.bl && g == 0) {
        const float b = sigmoid(a.beta[row]);
        a.b_out[row] = a.b_out[row] * b * (1.f - b);
    }
}

template <typename T, int DK>
hipError_t pro_launch(bool grad, const ProArgs& a, hipStream_t st) {
    constexpr int RPB = 256 / (DK / 4);
    const int64_t blocks = (a.rows + RPB - 1) / RPB;
    if (grad)
        hipLaunchKernelGGL((kda_pro_grad_kernel<T, DK>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((kda_pro_apply_kernel<T, DK>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prologue(bool grad, int dtype, int dk, int scalar, const Prologue& pro, int64_t rows,
                               const void* k, const float* log_a, const float* beta, void* k_out, float* la_out,
                               float* b_out, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    ProArgs a;
    a.k = k; a.log_a = log_a; a.beta = beta; a.k_out = k_out; a.la_out = la_out; a.b_out = b_out;
    a.rows = rows; a.scalar = scalar;
    a.nk = pro.normalize_k; a.bl = pro.beta_logits; a.la = pro.log_a_raw;
    a.lo2 = pro.log_a_min * LOG2E;
    if (dtype == 1) {
        if (dk == 128) return pro_launch<bf16, 128>(grad, a, st);
        if (dk == 64) return pro_launch<bf16, 64>(grad, a, st);
        if (dk == 32) return pro_launch<bf16, 32>(grad, a, st);
        if (dk == 16) return pro_launch<bf16, 16>(grad, a, st);
    } else {
        if (dk == 128) return pro_launch<float, 128>(grad, a, st);
        if (dk == 64) return pro_launch<float, 64>(grad, a, st);
        if (dk == 32) return pro_launch<float, 32>(grad, a, st);
        if (dk == 16) return pro_launch<float, 16>(grad, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
