// kda_api.cpp -- the extern "C" entry points declared in include/kda.h.
//
// Host-side argument validation, choice of kernel configuration, launch on the
// caller's stream.  Nothing here allocates device memory.  State kept: the
// thread-local text of the last error, and per device the address of the fixed
// scratch array that kda_chunk_fwd_noalloc uses (looked up on its first call).
#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/kda.h"
#include "kda_launch.hpp"

// Scratch of kda_chunk_fwd_noalloc (the two-pass workspace of a caller that
// cannot allocate): a fixed array in device memory, of which every GPU the
// library runs on holds its own copy until the process ends.  Host code uses
// only the per-device address from hipGetSymbolAddress, never this name.
static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return KDA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool width_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Common checks of the dims structure.
int check_dims(const kda_dims_t* d) {
    if (!d) return fail(KDA_ERR_INVALID_ARGUMENT, "dims is NULL");
    if (d->num_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs = %d < 0", d->num_seqs);
    if (d->num_heads <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_heads = %d <= 0", d->num_heads);
    if (d->total_tokens < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "total_tokens = %lld < 0", (long long)d->total_tokens);
    if (d->qkv_dtype != KDA_F32 && d->qkv_dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "qkv_dtype = %d is not KDA_F32 or KDA_BF16", d->qkv_dtype);
    if (d->scalar_decay != 0 && d->scalar_decay != 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "scalar_decay = %d is not 0 or 1", d->scalar_decay);
    if (d->order != KDA_ORDER_ERASE_FIRST && d->order != KDA_ORDER_DECAY_FIRST)
        return fail(KDA_ERR_INVALID_ARGUMENT, "order = %d is not a kda_order_t", d->order);
    if (!width_ok(d->dk) || !width_ok(d->dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk = %d, dv = %d: each must be 16, 32, 64 or 128", d->dk, d->dv);
    return KDA_OK;
}

// Non-null pointers with the alignment the kernels' vector accesses need.
int check_ptrs(const void* const* ptrs, const char* const* names, const int* align, int count) {
    for (int i = 0; i < count; ++i) {
        if (!ptrs[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
        if ((uintptr_t)ptrs[i] % (uintptr_t)align[i])
            return fail(KDA_ERR_MISALIGNED, "%s is not %d-byte aligned", names[i], align[i]);
    }
    return KDA_OK;
}

// Smallest dv split that gives at least 256 workgroups (one per compute unit),
// among the splits compiled for this shape.
int choose_split(const kda_dims_t* d, int chunk) {
    const int64_t units = (int64_t)d->num_seqs * d->num_heads;
    int best = 0;
    for (int split = 1; split <= 8; split *= 2) {
        if (d->dv % split) break;
        if (!kda::chunk_supported(d->qkv_dtype, d->dk, d->dv / split, chunk, d->scalar_decay)) continue;
        best = split;
        if (units * split >= 256) break;
    }
    return best;
}

// Validates a prologue (NULL: none) and copies it for the launchers.
int check_prologue(const kda_prologue_t* pr, kda::Prologue* out) {
    *out = kda::Prologue();
    if (!pr) return KDA_OK;
    auto flag = [](int32_t f) { return f == 0 || f == 1; };
    if (!flag(pr->normalize_k) || !flag(pr->beta_logits) || !flag(pr->log_a_raw))
        return fail(KDA_ERR_INVALID_ARGUMENT, "prologue flags must be 0 or 1 (got %d, %d, %d)", pr->normalize_k,
                    pr->beta_logits, pr->log_a_raw);
    if (pr->log_a_raw && (isnan(pr->log_a_min) || pr->log_a_min > 0.f))
        return fail(KDA_ERR_INVALID_ARGUMENT, "prologue log_a_min = %g must be <= 0 (or -INFINITY)",
                    (double)pr->log_a_min);
    out->normalize_k = pr->normalize_k;
    out->beta_logits = pr->beta_logits;
    out->log_a_raw = pr->log_a_raw;
    out->log_a_min = pr->log_a_raw ? pr->log_a_min : 0.f;
    return KDA_OK;
}

// Order the kernels run: with one decay value per token and head the two
// orders are the same map, and the erase-first kernels serve both.
int kernel_order(const kda_dims_t* d) { return d->scalar_decay ? 0 : d->order; }
// The two-pass method runs a scalar decay (Gated DeltaNet) through its
// decay-first kernels: the same map, with two Gram products instead of four, no
// write term outside E and blocks without KT (29,184 instead of 37,376 bytes at
// dk = 128).
int two_pass_order(const kda_dims_t* d) { return d->scalar_decay ? 1 : d->order; }

// Plan of a prefill call: which method, chunk, split and, for the two-pass
// method, the workspace layout [sequence order][states of all units][operator
// blocks].
struct Plan {
    int method = KDA_METHOD_SINGLE;
    int chunk = 32, split = 0;
    int64_t units = 0, max_chunks = 0;
    size_t block = 0, state_bytes = 0, order_bytes = 0, min_bytes = 0, pref_bytes = 0;
    size_t bwd_pref_bytes = 0;  // the preferred workspace of the backward's prefill rerun
    bool two_pass_ok = false;
};

// Sequences the state pass can take longest first: the rank kernel compares
// every pair, so the order is formed up to this many sequences (a few
// microseconds), and index order is kept beyond.
constexpr int kMaxRankedSeqs = 4096;

// Operator bytes per segment of the preferred workspace.  Each segment costs a
// launch of both passes and a ramp of each; on the 288 GB parts a few GiB is
// cheap, and fewer, longer segments measured faster than cache-sized ones (the
// 64-sequence varlen batch: 14.5 ms in ten segments of 4 GiB, 13.9 ms in three
// of 16 GiB; the 2 x 32K batch needs 2.4 GB, one segment either way).  The
// backward's prefill rerun keeps 4 GiB segments: its workspace holds much
// more besides.
constexpr size_t kSegmentTarget = size_t(16) << 30;
constexpr size_t kBwdSegmentTarget = size_t(4) << 30;

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Smallest split with at least 256 workgroups among the two-pass shapes, and
// with slices of at most 64 columns: the 128-column state pass holds two
// column blocks of a 128-row state per wavefront and spills registers (on the
// 64-sequence varlen batch split 2 runs 15.5 ms against 16.4 ms at split 1).
int choose_split_two_pass(const kda_dims_t* d, int chunk) {
    const int64_t units = (int64_t)d->num_seqs * d->num_heads;
    int best = 0;
    for (int split = 1; split <= 8; split *= 2) {
        if (d->dv % split) break;
        if (!kda::two_pass_supported(d->qkv_dtype, d->dk, d->dv / split, chunk)) continue;
        best = split;
        if (units * split >= 256 && d->dv / split <= 64) break;
    }
    return best;
}

// Validates the dims-level prefill arguments and fills the plan's shape part.
int plan_prefill(const kda_dims_t* d, bool have_cu, Plan* pl) {
    int st = check_dims(d);
    if (st) return st;
    pl->chunk = d->chunk_size == 0 ? 32 : d->chunk_size;
    if (pl->chunk != 32 && pl->chunk != 64)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size = %d: must be 0, 32 or 64", d->chunk_size);
    if (d->method < KDA_METHOD_AUTO || d->method > KDA_METHOD_TWO_PASS)
        return fail(KDA_ERR_INVALID_ARGUMENT, "method = %d is not a kda_method_t", d->method);
    if (d->max_seqlen < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "max_seqlen = %lld < 0", (long long)d->max_seqlen);
    if (d->dv_split != 0 && d->dv_split != 1 && d->dv_split != 2 && d->dv_split != 4 && d->dv_split != 8)
        return fail(KDA_ERR_INVALID_ARGUMENT, "dv_split = %d: must be 0, 1, 2, 4 or 8", d->dv_split);
    pl->units = (int64_t)d->num_seqs * d->num_heads;
    if (d->num_seqs == 0) return KDA_OK;
    int64_t maxlen = d->total_tokens;
    if (!have_cu) maxlen = d->total_tokens / d->num_seqs;
    else if (d->max_seqlen > 0) maxlen = d->max_seqlen < d->total_tokens ? d->max_seqlen : d->total_tokens;
    pl->max_chunks = (maxlen + pl->chunk - 1) / pl->chunk;
    // two-pass shape
    int split2 = d->dv_split;
    if (split2 == 0) split2 = choose_split_two_pass(d, pl->chunk);
    else if (d->dv % split2 || !kda::two_pass_supported(d->qkv_dtype, d->dk, d->dv / split2, pl->chunk))
        split2 = 0;
    pl->block = (size_t)kda::prep_block_bytes(d->dk, pl->chunk, two_pass_order(d));
    pl->two_pass_ok = split2 > 0 && pl->block > 0 && d->method != KDA_METHOD_SINGLE;
    if (d->method == KDA_METHOD_TWO_PASS && !pl->two_pass_ok)
        return fail(KDA_ERR_UNSUPPORTED, "no two-pass prefill for dtype %d, dk %d, dv %d, chunk %d, dv_split %d",
                    d->qkv_dtype, d->dk, d->dv, pl->chunk, d->dv_split);
    if (pl->two_pass_ok) {
        pl->state_bytes = round256((size_t)pl->units * d->dk * d->dv * 4);
        const size_t per_chunk = (size_t)pl->units * pl->block;
        int64_t m = (int64_t)(kSegmentTarget / per_chunk);
        if (m > pl->max_chunks) m = pl->max_chunks;
        if (m < 1) m = 1;
        // With more state-pass workgroups than compute units, sequences of
        // different lengths finish unevenly in index order; the walk then takes
        // them longest first (simulated on the 64-sequence varlen batch: 19-30 %
        // above the even finish in index order, within 1 % longest first).
        const int64_t groups = pl->units * split2;
        if (have_cu && d->num_seqs >= 2 && d->num_seqs <= kMaxRankedSeqs && groups > 256)
            pl->order_bytes = round256((size_t)d->num_seqs * 4);
        pl->min_bytes = pl->order_bytes + pl->state_bytes + per_chunk;
        pl->pref_bytes = pl->order_bytes + pl->state_bytes + per_chunk * (size_t)m;
        int64_t mb = (int64_t)(kBwdSegmentTarget / per_chunk);
        if (mb > pl->max_chunks) mb = pl->max_chunks;
        if (mb < 1) mb = 1;
        pl->bwd_pref_bytes = pl->order_bytes + pl->state_bytes + per_chunk * (size_t)mb;
        pl->split = split2;
    }
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_version(void) { return 10000; }

const char* kda_status_string(int status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
        default: return "KDA_ERR_UNKNOWN";
    }
}

const char* kda_last_error(void) { return g_last_error; }

int kda_chunk_workspace_size(const kda_dims_t* d, size_t* bytes) {
    if (!bytes) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
    Plan pl;
    int st = plan_prefill(d, true, &pl);
    if (st) return st;
    *bytes = pl.two_pass_ok ? pl.pref_bytes : 0;
    return ok();
}

int kda_chunk_plan(const kda_dims_t* d, int packed, size_t workspace_bytes, int* method, int* chunk,
                   int* dv_split) {
    if (!method || !chunk || !dv_split) return fail(KDA_ERR_INVALID_ARGUMENT, "method, chunk or dv_split is NULL");
    Plan pl;
    int st = plan_prefill(d, packed != 0, &pl);
    if (st) return st;
    *chunk = pl.chunk;
    *method = KDA_METHOD_SINGLE;
    *dv_split = 0;
    if (d->num_seqs == 0) return ok();
    // as chunk_fwd_impl decides (the public entry points reserve the running states)
    if (pl.two_pass_ok) {
        const size_t need = pl.order_bytes + pl.state_bytes + (size_t)pl.units * pl.block;
        if (workspace_bytes >= need) {
            *method = KDA_METHOD_TWO_PASS;
            *dv_split = pl.split;
            return ok();
        }
        if (d->method == KDA_METHOD_TWO_PASS)
            return fail(KDA_ERR_INVALID_ARGUMENT, "two-pass prefill needs a workspace of at least %zu bytes (got %zu)",
                        need, workspace_bytes);
    }
    int split = d->dv_split;
    if (split == 0) {
        split = choose_split(d, pl.chunk);
        if (split == 0)
            return fail(KDA_ERR_UNSUPPORTED, "no prefill kernel for dtype %d, dk %d, dv %d, chunk %d", d->qkv_dtype,
                        d->dk, d->dv, pl.chunk);
    } else if (d->dv % split || !kda::chunk_supported(d->qkv_dtype, d->dk, d->dv / split, pl.chunk, d->scalar_decay)) {
        return fail(KDA_ERR_UNSUPPORTED, "no prefill kernel for dtype %d, dk %d, dv %d / split %d, chunk %d",
                    d->qkv_dtype, d->dk, d->dv, split, pl.chunk);
    }
    *dv_split = split;
    return ok();
}

int kda_chunk_workspace_min(const kda_dims_t* d, size_t* bytes) {
    if (!bytes) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
    Plan pl;
    int st = plan_prefill(d, true, &pl);
    if (st) return st;
    *bytes = pl.two_pass_ok ? pl.min_bytes : 0;
    return ok();
}

int kda_chunk_fwd(const kda_dims_t* d, const void* q, const void* k, const void* v,
                  const float* log_a, const float* beta, const float* S0,
                  const int32_t* cu_seqlens, void* o, float* S_T, void* workspace,
                  size_t workspace_bytes, void* stream) {
    return kda_chunk_fwd_snapshots(d, q, k, v, log_a, beta, S0, cu_seqlens, o, S_T, nullptr, 0, 0, workspace,
                                   workspace_bytes, stream);
}

int kda_chunk_fwd_snapshots(const kda_dims_t* d, const void* q, const void* k, const void* v,
                            const float* log_a, const float* beta, const float* S0,
                            const int32_t* cu_seqlens, void* o, float* S_T, float* snapshots,
                            int64_t snapshot_rows, int64_t snapshot_every, void* workspace,
                            size_t workspace_bytes, void* stream) {
    return kda_chunk_fwd_ex(d, nullptr, q, k, v, log_a, beta, S0, cu_seqlens, o, S_T, snapshots, snapshot_rows,
                            snapshot_every, workspace, workspace_bytes, stream);
}

// The prefill behind every kda_chunk_fwd* entry point.  Workspace layout: the
// longest-first sequence order (order_bytes, only for batches the state pass
// takes in that order), the running states of all units, then the operator
// blocks (at state_off).  The
// public entry points always reserve the states (their documented minimum);
// kda_chunk_fwd_noalloc reserves them only when S_T is NULL (otherwise S_T holds
// the running state), which leaves its fixed scratch to the blocks.
static int chunk_fwd_impl(const kda_dims_t* d, const kda_prologue_t* prologue, const void* q, const void* k,
                          const void* v, const float* log_a, const float* beta, const float* S0,
                          const int32_t* cu_seqlens, void* o, float* S_T, float* snapshots, int64_t snapshot_rows,
                          int64_t snapshot_every, void* workspace, size_t workspace_bytes, bool reserve_states,
                          void* stream) {
    Plan pl;
    int st = plan_prefill(d, cu_seqlens != nullptr, &pl);
    if (st) return st;
    kda::Prologue pro;
    if ((st = check_prologue(prologue, &pro))) return st;
    const int chunk = pl.chunk;
    if (snapshot_every < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "snapshot_every = %lld < 0", (long long)snapshot_every);
    if (snapshot_every == 0 && snapshots && snapshot_rows > 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "a snapshot buffer needs snapshot_every > 0");
    if (snapshot_every > 0) {
        if (snapshot_every % chunk)
            return fail(KDA_ERR_INVALID_ARGUMENT, "snapshot_every = %lld is not a multiple of the chunk size %d",
                        (long long)snapshot_every, chunk);
        if (snapshot_every > 0x7fffffff)
            return fail(KDA_ERR_INVALID_ARGUMENT, "snapshot_every = %lld is too large", (long long)snapshot_every);
        if (snapshot_rows < 0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "snapshot_rows = %lld < 0", (long long)snapshot_rows);
        if (snapshot_rows > 0 && !snapshots)
            return fail(KDA_ERR_INVALID_ARGUMENT, "snapshots is NULL but snapshot_rows = %lld",
                        (long long)snapshot_rows);
        if (snapshots && !aligned16(snapshots))
            return fail(KDA_ERR_MISALIGNED, "snapshots is not 16-byte aligned");
    }
    // no snapshot rows to write: the plain prefill
    if (snapshot_every == 0 || snapshot_rows == 0) { snapshots = nullptr; snapshot_every = 0; snapshot_rows = 0; }
    if (d->num_seqs == 0) {
        if (d->total_tokens != 0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs = 0 but total_tokens = %lld",
                        (long long)d->total_tokens);
        return ok();
    }
    if (!cu_seqlens && d->total_tokens % d->num_seqs != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "cu_seqlens is NULL but total_tokens = %lld is not a multiple of num_seqs = %d",
                    (long long)d->total_tokens, d->num_seqs);
    if (d->total_tokens > 0) {
        const void* ptrs[] = {q, k, v, log_a, beta, o};
        const char* names[] = {"q", "k", "v", "log_a", "beta", "o"};
        const int align[] = {16, 16, 16, d->scalar_decay ? 4 : 16, 4, 16};
        if ((st = check_ptrs(ptrs, names, align, 6))) return st;
    }
    if (S0 && !aligned16(S0)) return fail(KDA_ERR_MISALIGNED, "S0 is not 16-byte aligned");
    if (S_T && !aligned16(S_T)) return fail(KDA_ERR_MISALIGNED, "S_T is not 16-byte aligned");
    if (cu_seqlens && ((uintptr_t)cu_seqlens & 3u))
        return fail(KDA_ERR_MISALIGNED, "cu_seqlens is not 4-byte aligned");

    // method
    bool two_pass = false;
    const size_t state_off = pl.order_bytes + ((reserve_states || !S_T) ? pl.state_bytes : 0);
    if (pl.two_pass_ok) {
        const size_t need = state_off + (size_t)pl.units * pl.block;
        const bool have_ws = workspace && workspace_bytes >= need;
        if (d->method == KDA_METHOD_TWO_PASS && !have_ws)
            return fail(KDA_ERR_INVALID_ARGUMENT, "two-pass prefill needs a workspace of at least %zu bytes (got %zu)",
                        need, workspace ? workspace_bytes : (size_t)0);
        two_pass = have_ws;
    }
    if (two_pass) {
        if ((uintptr_t)workspace & 255u) return fail(KDA_ERR_MISALIGNED, "workspace is not 256-byte aligned");
        const size_t per_chunk = (size_t)pl.units * pl.block;
        int64_t m = (int64_t)((workspace_bytes - state_off) / per_chunk);
        if (m > pl.max_chunks) m = pl.max_chunks;
        if (m < 1) m = 1;
        if (pl.units * m > 0x7fffffff || pl.units * pl.split > 0x7fffffff)
            return fail(KDA_ERR_INVALID_ARGUMENT, "too many (sequence, head) units: %lld", (long long)pl.units);
        const int64_t nseg = pl.max_chunks > 0 ? (pl.max_chunks + m - 1) / m : 1;
        uint8_t* ws = static_cast<uint8_t*>(workspace);
        int32_t* ord = pl.order_bytes ? reinterpret_cast<int32_t*>(ws) : nullptr;
        float* run = S_T ? S_T : reinterpret_cast<float*>(ws + pl.order_bytes);
        uint8_t* blocks = ws + state_off;
        const int64_t eq_len = cu_seqlens ? 0 : d->total_tokens / d->num_seqs;
        if (ord) {
            hipError_t e = kda::launch_seq_rank(cu_seqlens, d->num_seqs, ord, (hipStream_t)stream);
            if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill sequence order launch: %s", hipGetErrorString(e));
        }
        for (int64_t sgi = 0; sgi < nseg; ++sgi) {
            const int64_t chunk0 = sgi * m;
            hipError_t e = hipSuccess;
            if (d->total_tokens > 0) {
                kda::PrepLaunch pa;
                pa.q = q; pa.k = k; pa.log_a = log_a; pa.beta = beta; pa.cu_seqlens = cu_seqlens;
                pa.eq_len = eq_len; pa.ws = blocks; pa.num_heads = d->num_heads; pa.units = pl.units;
                pa.m = (int32_t)m; pa.chunk0 = chunk0; pa.dk = d->dk; pa.chunk = chunk; pa.scalar = d->scalar_decay;
                pa.order = two_pass_order(d); pa.pro = pro;
                e = kda::launch_prep(pa, (hipStream_t)stream);
                if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill operator pass launch: %s", hipGetErrorString(e));
            }
            kda::ScanLaunch sa;
            sa.v = v; sa.o = o; sa.cu_seqlens = cu_seqlens; sa.eq_len = eq_len; sa.ws = blocks;
            sa.S_in = sgi == 0 ? S0 : run; sa.S_out = run; sa.num_heads = d->num_heads; sa.units = pl.units;
            sa.dk = d->dk; sa.dv = d->dv; sa.split = pl.split; sa.m = (int32_t)m; sa.chunk = chunk;
            sa.chunk0 = chunk0; sa.order = two_pass_order(d); sa.snap = snapshots; sa.snap_rows = snapshot_rows;
            sa.snap_every = (int32_t)snapshot_every;
            sa.ord = ord;
            e = kda::launch_scan(sa, (hipStream_t)stream);
            if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill state pass launch: %s", hipGetErrorString(e));
        }
        return ok();
    }

    int split = d->dv_split;
    if (split == 0) {
        split = choose_split(d, chunk);
        if (split == 0)
            return fail(KDA_ERR_UNSUPPORTED, "no prefill kernel for dtype %d, dk %d, dv %d, chunk %d",
                        d->qkv_dtype, d->dk, d->dv, chunk);
    } else if (d->dv % split || !kda::chunk_supported(d->qkv_dtype, d->dk, d->dv / split, chunk, d->scalar_decay)) {
        return fail(KDA_ERR_UNSUPPORTED, "no prefill kernel for dtype %d, dk %d, dv %d / split %d, chunk %d",
                    d->qkv_dtype, d->dk, d->dv, split, chunk);
    }
    const int64_t blocks = (int64_t)d->num_seqs * d->num_heads * split;
    if (blocks > 0x7fffffff)
        return fail(KDA_ERR_INVALID_ARGUMENT, "too many (sequence, head, slice) units: %lld", (long long)blocks);

    kda::ChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.log_a = log_a; a.beta = beta; a.S0 = S0;
    a.cu_seqlens = cu_seqlens; a.o = o; a.S_T = S_T;
    a.num_seqs = d->num_seqs; a.num_heads = d->num_heads; a.total_tokens = d->total_tokens;
    a.dk = d->dk; a.dv = d->dv; a.dtype = d->qkv_dtype; a.scalar_decay = d->scalar_decay;
    a.chunk = chunk; a.split = split; a.order = kernel_order(d);
    a.snap = snapshots; a.snap_rows = snapshot_rows; a.snap_every = (int32_t)snapshot_every;
    a.pro = pro;
    hipError_t e = kda::launch_chunk(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    return ok();
}


int kda_chunk_fwd_ex(const kda_dims_t* d, const kda_prologue_t* prologue, const void* q, const void* k,
                     const void* v, const float* log_a, const float* beta, const float* S0,
                     const int32_t* cu_seqlens, void* o, float* S_T, float* snapshots, int64_t snapshot_rows,
                     int64_t snapshot_every, void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_fwd_impl(d, prologue, q, k, v, log_a, beta, S0, cu_seqlens, o, S_T, snapshots, snapshot_rows,
                          snapshot_every, workspace, workspace_bytes, true, stream);
}

// Per-device address of `scratch`, looked up once per device with that device
// current (each GPU holds its own copy of the array at its own address).
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64] = {};

static int scratch_address(void* stream, void** out) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(KDA_ERR_HIP, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(KDA_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p)
            return fail(KDA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

int kda_chunk_fwd_noalloc(const kda_dims_t* d, const void* q, const void* k, const void* v, const float* log_a,
                          const float* beta, const float* S0, const int32_t* cu_seqlens, void* o, float* S_T,
                          void* stream) {
    Plan pl;
    int st = plan_prefill(d, cu_seqlens != nullptr, &pl);
    if (st) return st;
    if (!pl.two_pass_ok || d->num_seqs == 0)  // single-pass: no scratch at all
        return chunk_fwd_impl(d, nullptr, q, k, v, log_a, beta, S0, cu_seqlens, o, S_T, nullptr, 0, 0, nullptr, 0,
                              false, stream);
    const size_t need = pl.order_bytes + (S_T ? 0 : pl.state_bytes) + (size_t)pl.units * pl.block;
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "the two-pass prefill of %lld (sequence, head) units needs %zu bytes of scratch%s; the fixed "
                    "scratch holds %zu (use kda_chunk_fwd with a workspace, or the single-pass method)",
                    (long long)pl.units, need, S_T ? "" : " (S_T is NULL: the running states too)",
                    (size_t)KDA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((st = scratch_address(stream, &ws))) return st;
    return chunk_fwd_impl(d, nullptr, q, k, v, log_a, beta, S0, cu_seqlens, o, S_T, nullptr, 0, 0, ws,
                          (size_t)KDA_NOALLOC_SCRATCH_BYTES, false, stream);
}

}  // extern "C"

namespace {
// Backward workspace: [prefill's two-pass workspace][o scratch][states every 64
// tokens][operator blocks per 16 tokens][state derivatives per 64-token chunk]
// [per chunk: start state, E and Y of each 16-token piece, kept by the gradient pass].
struct BwdPlan {
    Plan fwd;
    size_t fwd_ws = 0, o_bytes = 0, snap_bytes = 0, ops_bytes = 0, x_bytes = 0, scr_bytes = 0, total = 0;
    int64_t snap_rows = 0, maxlen = 0;
};


// Transformed inputs of a backward with a prologue: keys, log a, beta.
size_t prologue_bytes(const kda_dims_t* d) {
    const size_t rows = (size_t)(d->total_tokens > 0 ? d->total_tokens : 0) * (size_t)d->num_heads;
    const size_t esize = d->qkv_dtype == KDA_BF16 ? 2 : 4;
    return round256(rows * d->dk * esize) + round256(rows * (d->scalar_decay ? 1 : d->dk) * 4) + round256(rows * 4);
}

// saved: the caller hands in the forward's states at every 64th token, so the
// workspace holds no rerun (no prefill workspace, outputs or states of its own).
int plan_bwd(const kda_dims_t* d, bool have_cu, bool saved, BwdPlan* bp) {
    int st = plan_prefill(d, have_cu, &bp->fwd);
    if (st) return st;
    if (!kda::bwd_supported(d->qkv_dtype, d->dk, d->dv))
        return fail(KDA_ERR_UNSUPPORTED, "no backward for dtype %d, dk %d, dv %d", d->qkv_dtype, d->dk, d->dv);
    const int64_t T = d->total_tokens, N = d->num_seqs, H = d->num_heads;
    const size_t state = (size_t)d->dk * d->dv * 4;
    bp->snap_rows = T / 64;
    if (!saved) {
        bp->fwd_ws = bp->fwd.two_pass_ok ? bp->fwd.bwd_pref_bytes : 0;
        bp->o_bytes = round256((size_t)T * H * d->dv * (d->qkv_dtype == KDA_BF16 ? 2 : 4));
        bp->snap_bytes = round256((size_t)bp->snap_rows * H * state);
    }
    bp->ops_bytes = round256((size_t)(T / 16 + N) * H * kda::bwd_block_bytes(d->qkv_dtype, d->dk));
    bp->x_bytes = round256((size_t)(T / 64 + N) * H * state);
    bp->scr_bytes = round256((size_t)(T / 64 + N) * H * (size_t)kda::bwd_scratch_bytes(d->qkv_dtype, d->dk, d->dv));
    bp->total = round256(bp->fwd_ws) + bp->o_bytes + bp->snap_bytes + bp->ops_bytes + bp->x_bytes + bp->scr_bytes;
    bp->maxlen = N > 0 ? bp->fwd.max_chunks * bp->fwd.chunk : 0;
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_decode_step(const kda_dims_t* d, const void* q, const void* k, const void* v,
                    const float* log_a, const float* beta, const float* S_in, float* S_out,
                    void* o, void* stream) {
    return kda_decode_step_ex(d, nullptr, q, k, v, log_a, beta, S_in, S_out, o, stream);
}

int kda_decode_step_ex(const kda_dims_t* d, const kda_prologue_t* prologue, const void* q, const void* k,
                       const void* v, const float* log_a, const float* beta, const float* S_in, float* S_out,
                       void* o, void* stream) {
    int st = check_dims(d);
    if (st) return st;
    kda::Prologue pro;
    if ((st = check_prologue(prologue, &pro))) return st;
    if (d->total_tokens != d->num_seqs)
        return fail(KDA_ERR_INVALID_ARGUMENT, "decode needs total_tokens (%lld) == num_seqs (%d)",
                    (long long)d->total_tokens, d->num_seqs);
    if (d->num_seqs == 0) return ok();
    const void* ptrs[] = {q, k, v, log_a, beta, S_in, S_out, o};
    const char* names[] = {"q", "k", "v", "log_a", "beta", "S_in", "S_out", "o"};
    const int align[] = {16, 16, 16, 4, 4, 16, 16, 16};
    if ((st = check_ptrs(ptrs, names, align, 8))) return st;
    if (!kda::decode_supported(d->qkv_dtype, d->dk, d->dv))
        return fail(KDA_ERR_UNSUPPORTED, "no decode kernel for dtype %d, dk %d, dv %d", d->qkv_dtype, d->dk, d->dv);
    const int64_t heads = (int64_t)d->num_seqs * d->num_heads;
    if (heads > 0x7fffffff) return fail(KDA_ERR_INVALID_ARGUMENT, "too many states: %lld", (long long)heads);
    hipError_t e = kda::launch_decode(d->qkv_dtype, d->dk, d->dv, d->scalar_decay, kernel_order(d), pro, heads, q, k,
                                      v, log_a, beta, S_in, S_out, o, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return ok();
}

int kda_chunk_bwd_workspace_size(const kda_dims_t* d, size_t* bytes) {
    if (!bytes) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
    BwdPlan bp;
    int st = plan_bwd(d, true, false, &bp);
    if (st) return st;
    *bytes = bp.total;
    return ok();
}

int kda_chunk_bwd_ex_workspace_size(const kda_dims_t* d, const kda_prologue_t* prologue, int saved, size_t* bytes) {
    if (!bytes) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
    kda::Prologue pro;
    int st = check_prologue(prologue, &pro);
    if (st) return st;
    BwdPlan bp;
    if ((st = plan_bwd(d, true, saved != 0, &bp))) return st;
    *bytes = bp.total + (pro.any() ? prologue_bytes(d) : 0);
    return ok();
}

int kda_chunk_bwd_saved_workspace_size(const kda_dims_t* d, size_t* bytes) {
    if (!bytes) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
    BwdPlan bp;
    int st = plan_bwd(d, true, true, &bp);
    if (st) return st;
    *bytes = bp.total;
    return ok();
}

}  // extern "C"

namespace {

// The backward's four stages.  states == nullptr (saved false): the prefill is run
// again for the states at every 64th token; otherwise they are the caller's rows.
int chunk_bwd_impl(const kda_dims_t* d, const void* q, const void* k, const void* v, const float* log_a,
                   const float* beta, const float* S0, const int32_t* cu_seqlens, bool saved, const float* states,
                   int64_t state_rows, const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                   float* dlog_a, float* dbeta, float* dS0, void* workspace, size_t workspace_bytes, void* stream,
                   bool check_only = false) {
    BwdPlan bp;
    int st = plan_bwd(d, cu_seqlens != nullptr, saved, &bp);
    if (st) return st;
    if (d->num_seqs == 0) {
        if (d->total_tokens != 0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs = 0 but total_tokens = %lld", (long long)d->total_tokens);
        return ok();
    }
    if (!cu_seqlens && d->total_tokens % d->num_seqs != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "cu_seqlens is NULL but total_tokens = %lld is not a multiple of num_seqs = %d",
                    (long long)d->total_tokens, d->num_seqs);
    if (d->total_tokens > 0) {
        const void* ptrs[] = {q, k, v, log_a, beta, dO, dq, dk, dv, dlog_a, dbeta};
        const char* names[] = {"q", "k", "v", "log_a", "beta", "dO", "dq", "dk", "dv", "dlog_a", "dbeta"};
        const int a4 = d->scalar_decay ? 4 : 16;
        const int align[] = {16, 16, 16, a4, 4, 16, 16, 16, 16, a4, 4};
        if ((st = check_ptrs(ptrs, names, align, 11))) return st;
    }
    if (S0 && !aligned16(S0)) return fail(KDA_ERR_MISALIGNED, "S0 is not 16-byte aligned");
    if (dS_T && !aligned16(dS_T)) return fail(KDA_ERR_MISALIGNED, "dS_T is not 16-byte aligned");
    if (dS0 && !aligned16(dS0)) return fail(KDA_ERR_MISALIGNED, "dS0 is not 16-byte aligned");
    if (cu_seqlens && ((uintptr_t)cu_seqlens & 3u))
        return fail(KDA_ERR_MISALIGNED, "cu_seqlens is not 4-byte aligned");
    if (!workspace || workspace_bytes < bp.total)
        return fail(KDA_ERR_INVALID_ARGUMENT, "the backward needs a workspace of at least %zu bytes (got %zu)",
                    bp.total, workspace ? workspace_bytes : (size_t)0);
    if ((uintptr_t)workspace & 255u) return fail(KDA_ERR_MISALIGNED, "workspace is not 256-byte aligned");
    if (saved) {
        // rows the kernels may read: one per whole 64 tokens of each sequence
        // (known on the host only for equal lengths)
        const int64_t need = cu_seqlens ? 0 : (int64_t)d->num_seqs * ((d->total_tokens / d->num_seqs) / 64);
        if (state_rows < need)
            return fail(KDA_ERR_INVALID_ARGUMENT, "states holds %lld rows, the sequences need %lld",
                        (long long)state_rows, (long long)need);
        if (!states && d->total_tokens >= 64)
            return fail(KDA_ERR_INVALID_ARGUMENT, "states is NULL (the states at every 64th token are needed)");
        if (states && !aligned16(states)) return fail(KDA_ERR_MISALIGNED, "states is not 16-byte aligned");
    }
    const int64_t units = (int64_t)d->num_seqs * d->num_heads;
    const int64_t nsub_max = (bp.maxlen + 15) / 16, nch_max = (bp.maxlen + 63) / 64;
    if (units > 65535 || nsub_max > 0x7fffffff)
        return fail(KDA_ERR_INVALID_ARGUMENT, "too many (sequence, head) units for the backward: %lld",
                    (long long)units);
    if (check_only) return ok();
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint8_t* fwd_ws = bp.fwd_ws ? ws : nullptr;
    size_t off = round256(bp.fwd_ws);
    void* o_scratch = ws + off;
    off += bp.o_bytes;
    float* snap = reinterpret_cast<float*>(ws + off);
    off += bp.snap_bytes;
    void* ops = ws + off;
    off += bp.ops_bytes;
    float* xbuf = reinterpret_cast<float*>(ws + off);
    off += bp.x_bytes;
    void* scr = ws + off;

    int64_t snap_rows = bp.snap_rows;
    if (saved) {
        snap = const_cast<float*>(states);
        snap_rows = states ? state_rows : 0;
    } else if (bp.snap_rows > 0) {
        // the prefill again, keeping the state at every 64th token (nothing to
        // keep when no sequence reaches 64 tokens)
        st = kda_chunk_fwd_snapshots(d, q, k, v, log_a, beta, S0, cu_seqlens, o_scratch, nullptr, snap,
                                     bp.snap_rows, 64, fwd_ws, bp.fwd_ws, stream);
        if (st) return st;
    }

    kda::BwdLaunch a;
    a.q = q; a.k = k; a.v = v; a.log_a = log_a; a.beta = beta; a.S0 = S0;
    a.cu_seqlens = cu_seqlens; a.eq_len = cu_seqlens ? 0 : d->total_tokens / d->num_seqs;
    a.dO = dO; a.dST = dS_T; a.dq = dq; a.dk = dk; a.dv = dv; a.dlog_a = dlog_a; a.dbeta = dbeta; a.dS0 = dS0;
    a.snap = snap; a.snap_rows = snap_rows; a.ops = ops; a.xbuf = xbuf; a.scr = scr;
    a.num_heads = d->num_heads; a.units = units; a.nsub_max = (int32_t)nsub_max; a.nch_max = (int32_t)nch_max;
    a.kdim = d->dk; a.vdim = d->dv; a.dtype = d->qkv_dtype; a.scalar = d->scalar_decay;
    a.order = kernel_order(d);
    hipError_t e = kda::launch_bwd(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    return ok();
}

// The backward with an input prologue: the transformed inputs are formed in
// the workspace past the gradient's own share, the gradient runs on them, and
// the chain rule through the transforms is applied to dk, dlog_a and dbeta.
int chunk_bwd_ex_impl(const kda_dims_t* d, const kda_prologue_t* prologue, const void* q, const void* k,
                      const void* v, const float* log_a, const float* beta, const float* S0,
                      const int32_t* cu_seqlens, const float* states, int64_t state_rows, const void* dO,
                      const float* dS_T, void* dq, void* dk, void* dv, float* dlog_a, float* dbeta, float* dS0,
                      void* workspace, size_t workspace_bytes, void* stream) {
    kda::Prologue pro;
    int st = check_prologue(prologue, &pro);
    if (st) return st;
    const bool saved = states != nullptr;
    if (!pro.any())
        return chunk_bwd_impl(d, q, k, v, log_a, beta, S0, cu_seqlens, saved, states, state_rows, dO, dS_T, dq, dk,
                              dv, dlog_a, dbeta, dS0, workspace, workspace_bytes, stream);
    BwdPlan bp;
    if ((st = plan_bwd(d, cu_seqlens != nullptr, saved, &bp))) return st;
    const size_t extra = prologue_bytes(d);
    if (!workspace || workspace_bytes < bp.total + extra)
        return fail(KDA_ERR_INVALID_ARGUMENT, "the backward with a prologue needs a workspace of at least %zu bytes "
                    "(got %zu)", bp.total + extra, workspace ? workspace_bytes : (size_t)0);
    if ((uintptr_t)workspace & 255u) return fail(KDA_ERR_MISALIGNED, "workspace is not 256-byte aligned");
    const int64_t rows = d->total_tokens * d->num_heads;
    const size_t esize = d->qkv_dtype == KDA_BF16 ? 2 : 4;
    uint8_t* px = static_cast<uint8_t*>(workspace) + bp.total;
    void* k_t = px;
    float* la_t = reinterpret_cast<float*>(px + round256((size_t)rows * d->dk * esize));
    float* b_t = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(la_t) +
                                          round256((size_t)rows * (d->scalar_decay ? 1 : d->dk) * 4));
    const void* k_in = pro.normalize_k ? k_t : k;
    const float* la_in = pro.log_a_raw ? la_t : log_a;
    const float* b_in = pro.beta_logits ? b_t : beta;
    // every argument is checked before anything is enqueued: the raw inputs
    // here, the rest by the gradient's own checks (on the transformed inputs)
    if (rows > 0) {
        const void* ptrs[] = {k, log_a, beta};
        const char* names[] = {"k", "log_a", "beta"};
        const int align[] = {16, d->scalar_decay ? 4 : 16, 4};
        if ((st = check_ptrs(ptrs, names, align, 3))) return st;
    }
    st = chunk_bwd_impl(d, q, k_in, v, la_in, b_in, S0, cu_seqlens, saved, states, state_rows, dO, dS_T, dq, dk, dv,
                        dlog_a, dbeta, dS0, workspace, bp.total, stream, true);
    if (st) return st;
    if (rows > 0) {
        hipError_t e = kda::launch_bwd_prologue(false, d->qkv_dtype, d->dk, d->scalar_decay, pro, rows, k, log_a,
                                                beta, k_t, la_t, b_t, (hipStream_t)stream);
        if (e != hipSuccess) return fail(KDA_ERR_HIP, "prologue launch: %s", hipGetErrorString(e));
    }
    st = chunk_bwd_impl(d, q, k_in, v, la_in, b_in, S0, cu_seqlens, saved, states, state_rows, dO, dS_T, dq, dk, dv,
                        dlog_a, dbeta, dS0, workspace, bp.total, stream);
    if (st) return st;
    if (rows > 0) {
        hipError_t e = kda::launch_bwd_prologue(true, d->qkv_dtype, d->dk, d->scalar_decay, pro, rows, k, log_a, beta,
                                                dk, dlog_a, dbeta, (hipStream_t)stream);
        if (e != hipSuccess) return fail(KDA_ERR_HIP, "prologue gradient launch: %s", hipGetErrorString(e));
    }
    return ok();
}

}  // namespace

extern "C" {

int kda_chunk_bwd_ex(const kda_dims_t* d, const kda_prologue_t* prologue, const void* q, const void* k,
                     const void* v, const float* log_a, const float* beta, const float* S0,
                     const int32_t* cu_seqlens, const float* states, int64_t state_rows, const void* dO,
                     const float* dS_T, void* dq, void* dk, void* dv, float* dlog_a, float* dbeta, float* dS0,
                     void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_bwd_ex_impl(d, prologue, q, k, v, log_a, beta, S0, cu_seqlens, states, state_rows, dO, dS_T, dq,
                             dk, dv, dlog_a, dbeta, dS0, workspace, workspace_bytes, stream);
}

int kda_chunk_bwd(const kda_dims_t* d, const void* q, const void* k, const void* v, const float* log_a,
                  const float* beta, const float* S0, const int32_t* cu_seqlens, const void* dO, const float* dS_T,
                  void* dq, void* dk, void* dv, float* dlog_a, float* dbeta, float* dS0, void* workspace,
                  size_t workspace_bytes, void* stream) {
    return chunk_bwd_impl(d, q, k, v, log_a, beta, S0, cu_seqlens, false, nullptr, 0, dO, dS_T, dq, dk, dv, dlog_a,
                          dbeta, dS0, workspace, workspace_bytes, stream);
}

int kda_chunk_bwd_saved(const kda_dims_t* d, const void* q, const void* k, const void* v, const float* log_a,
                        const float* beta, const float* S0, const int32_t* cu_seqlens, const float* states,
                        int64_t state_rows, const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                        float* dlog_a, float* dbeta, float* dS0, void* workspace, size_t workspace_bytes,
                        void* stream) {
    return chunk_bwd_impl(d, q, k, v, log_a, beta, S0, cu_seqlens, true, states, state_rows, dO, dS_T, dq, dk, dv,
                          dlog_a, dbeta, dS0, workspace, workspace_bytes, stream);
}

}  // extern "C"
