// kda_launch.hpp -- host-side launchers shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Input prologue switches (kda_prologue_t), passed to the kernels that run it.
struct Prologue {
    int32_t normalize_k = 0, beta_logits = 0, log_a_raw = 0;
    float log_a_min = 0.f;
    bool any() const { return normalize_k || beta_logits || log_a_raw; }
};
constexpr float PROLOGUE_EPS = 1e-6f;

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_a;
    const float* beta;
    const float* S0;
    const int32_t* cu_seqlens;  // device; may be null (equal lengths)
    void* o;
    float* S_T;                 // may be null
    int32_t num_seqs;
    int32_t num_heads;
    int64_t total_tokens;
    int32_t dk, dv;
    int32_t dtype;              // 0 fp32, 1 bf16
    int32_t scalar_decay;
    int32_t chunk;              // 32 or 64
    int32_t split;              // workgroups per (sequence, head) along dv
    int32_t order;              // 1: decay first (per-channel decay only), else 0
    float* snap;                // state snapshots [rows, H, dk, dv], or null
    int64_t snap_rows;
    int32_t snap_every;         // tokens between snapshots (a multiple of chunk), 0 = none
    Prologue pro;               // input prologue (none by default)
};

// The input prologue around the prefill's gradient, over rows (token, head):
// grad = false writes the transformed inputs (k_out, la_out, b_out) from the raw
// ones; grad = true applies the chain rule through the transforms in place to
// the gradient's dk (k_out), dlog_a (la_out) and dbeta (b_out).  Transforms that
// pro does not request are skipped (their outputs are not touched).
hipError_t launch_bwd_prologue(bool grad, int dtype, int dk, int scalar, const Prologue& pro, int64_t rows,
                               const void* k, const float* log_a, const float* beta, void* k_out, float* la_out,
                               float* b_out, hipStream_t st);

bool decode_supported(int dtype, int dk, int dv);
hipError_t launch_decode(int dtype, int dk, int dv, int scalar, int order, const Prologue& pro, int64_t heads,
                         const void* q,
                         const void* k, const void* v, const float* log_a, const float* beta,
                         const float* S_in, float* S_out, void* o, hipStream_t stream);

// true if a chunk kernel exists for (dtype, dk, dv / split, chunk)
bool chunk_supported(int dtype, int dk, int dvs, int chunk, int scalar);
hipError_t launch_chunk(const ChunkArgs& a, hipStream_t stream);

// Two-pass prefill: a chunk-parallel pass writes one operator block per
// (sequence, head, chunk) of a segment of m chunks; a sequential pass applies them.
struct PrepLaunch {
    const void* q;
    const void* k;
    const float* log_a;
    const float* beta;
    const int32_t* cu_seqlens;  // device; may be null (equal lengths eq_len)
    int64_t eq_len;
    void* ws;                   // blocks [units][m]
    int32_t num_heads;
    int64_t units;              // num_seqs * num_heads
    int32_t m;                  // chunks per unit in the segment
    int64_t chunk0;             // first chunk of the segment
    int32_t dk, chunk, scalar;
    int32_t order;              // as in ChunkArgs
    Prologue pro;
};
struct ScanLaunch {
    const void* v;
    void* o;
    const int32_t* cu_seqlens;
    int64_t eq_len;
    const void* ws;
    const float* S_in;          // may be null (zero state)
    float* S_out;
    int32_t num_heads;
    int64_t units;
    int32_t dk, dv, split, m, chunk;
    int64_t chunk0;
    int32_t order;              // as in ChunkArgs
    float* snap;                // as in ChunkArgs
    int64_t snap_rows;
    int32_t snap_every;
    const int32_t* ord;         // sequences longest first (launch_seq_rank), or null: index order
};
// Longest-first order of the sequences of cu_seqlens: ord[r] = sequence of rank r.
hipError_t launch_seq_rank(const int32_t* cu_seqlens, int num_seqs, int32_t* ord, hipStream_t stream);
int prep_block_bytes(int dk, int chunk, int order);  // 0 if no prep kernel for (dk, chunk)
hipError_t launch_prep(const PrepLaunch& a, hipStream_t stream);
hipError_t launch_prep2(const PrepLaunch& a, hipStream_t stream);  // dk = 128, chunk 32
bool two_pass_supported(int dtype, int dk, int dvs, int chunk);
hipError_t launch_scan(const ScanLaunch& a, hipStream_t stream);

// Backward of the prefill (erase-first order): three kernels after a forward
// prefill that kept the state at every 64th token of each sequence.
struct BwdLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* log_a;
    const float* beta;
    const float* S0;            // may be null (zero initial states)
    const int32_t* cu_seqlens;  // device; may be null (equal lengths eq_len)
    int64_t eq_len;
    const void* dO;
    const float* dST;           // may be null (zero)
    void* dq;
    void* dk;
    void* dv;
    float* dlog_a;
    float* dbeta;
    float* dS0;                 // may be null (not written)
    const float* snap;          // forward states, one row per 64 tokens of each sequence
    int64_t snap_rows;          // rows snap holds; a row at or past it reads as a zero state
    void* ops;                  // operator blocks, bwd_block_bytes each
    float* xbuf;                // derivatives at chunk ends, [chunks][dk][dv]
    void* scr;                  // bwd_scratch_bytes per chunk
    int32_t num_heads;
    int64_t units;
    int32_t nsub_max, nch_max;  // 16- and 64-token pieces of the longest sequence
    int32_t kdim, vdim, dtype, scalar;
    int32_t order;              // 1: decay-first (per-channel decay), else erase-first
};
int bwd_block_bytes(int dtype, int dk);
int64_t bwd_scratch_bytes(int dtype, int dk, int dv);  // per 64-token chunk
bool bwd_supported(int dtype, int dk, int dv);
hipError_t launch_bwd(const BwdLaunch& a, hipStream_t stream);

}  // namespace kda
