/*
 * kda.h -- C ABI of the MI355X (gfx950) gated delta-rule state layer.
 *
 * The layer keeps, per (sequence, head), a fixed-size state S of shape dk x dv
 * (page "The argument, in one page", section "Everything, in one table", row
 * "Linear attention": the state replaces the growing cache and never grows).
 * Every token updates it with the KDA rule of the same table (row "KDA"):
 *
 *     S <- Diag(a_t) (I - beta_t k_t^T k_t) S + beta_t k_t^T v_t,   a_t = exp(log_a_t)
 *
 * i.e. erase what S holds along the key k_t, decay every key row c of S by its
 * own a_t[c], then write beta_t k_t^T v_t; the output is the read after the
 * update, o_t = q_t S.  kda_dims_t.order selects the variant that decays
 * before it erases (kda_order_t below).  With one log_a value per (token, head) this is the
 * "Gated DeltaNet" row; with log_a = 0 it is the "Delta rule" row.
 *
 * Two entry points compute it:
 *   kda_chunk_fwd    -- prefill over packed variable-length sequences by the
 *                       chunkwise (WY) form (row "Chunkwise / WY" of the same
 *                       table: the same map, one C x C triangular solve per
 *                       chunk plus dense products on the matrix cores);
 *   kda_decode_step  -- one token per sequence, updating S in place.
 * Both take the initial state in and give the final state out, since the
 * state cannot be rebuilt from nearby tokens and reuse needs it exported
 * (glossary page "Linear attention", section "Why it matters").
 *
 * Conventions (both entry points)
 *   - Every pointer is DEVICE memory owned by the caller (e.g. allocated by
 *     PyTorch).  The library allocates nothing and keeps no global state.
 *   - Layouts are contiguous, row-major, with the last index fastest.
 *     Tokens of all sequences are packed along one axis of length T.
 *   - The call validates its arguments on the host, enqueues its kernels on
 *     `stream` (a hipStream_t; NULL = the null stream) and returns without
 *     waiting.  On a non-OK status nothing was enqueued and outputs are
 *     untouched; kda_last_error() then describes the reason (thread-local).
 *     Faults during execution surface at the caller's next synchronisation.
 *   - No scaling of q and no normalisation of k happen inside: callers fold
 *     any 1/sqrt(dk) into q and normalise k themselves.
 *   - log_a must be finite and <= 0 (0 < a <= 1); beta is unrestricted.  Every
 *     such decay is supported exactly (to rounding): the chunked prefill splits
 *     decay factors around 16-token references in chunks whose tokens all have
 *     log_a >= -8.3 (log2 a >= -12), and takes a chunk with a steeper token by
 *     one exponential of a run of consecutive decays per term (slower: an extra
 *     kernel pass over the marked chunks in the two-pass method).  Decode takes
 *     a = exp(log_a) per token.
 *   - Alignment: q, k, v, o and the fp32 states must be 16-byte aligned, as
 *     must a per-channel log_a in prefill; beta, a scalar log_a, any decode
 *     log_a, and cu_seqlens need 4-byte alignment.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef KDA_API
#define KDA_API __attribute__((visibility("default")))
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, inconsistent dims */
    KDA_ERR_UNSUPPORTED = 2,      /* a (dk, dv, dtype, chunk) combination not compiled */
    KDA_ERR_MISALIGNED = 3,       /* a pointer below its required alignment (see above) */
    KDA_ERR_HIP = 4               /* the HIP runtime rejected a launch */
} kda_status_t;

typedef enum {
    KDA_F32 = 0,  /* q, k, v, o in float32: products on fp32 matrix cores */
    KDA_BF16 = 1  /* q, k, v, o in bfloat16: products on bf16 matrix cores, fp32 state */
} kda_dtype_t;

/* Prefill algorithm.  Both compute the same chunkwise form. */
typedef enum {
    KDA_METHOD_AUTO = 0,      /* two-pass when compiled for the shape and a workspace is
                                 given, else single-pass */
    KDA_METHOD_SINGLE = 1,    /* one kernel; each workgroup walks its sequence and forms
                                 every chunk's operators itself; no workspace */
    KDA_METHOD_TWO_PASS = 2   /* a chunk-parallel pass writes each chunk's operators to
                                 the workspace, a sequential pass applies them; needs a
                                 workspace (kda_chunk_workspace_size); bf16 only */
} kda_method_t;

/*
 * Order of decay and erase in the update.  The KDA row of the table (page "The
 * argument, in one page", section "Everything, in one table") writes
 * Diag(a)(I - beta k^T k) S: erase along k, then decay.  Gated delta-rule
 * layers are also written with the decay applied to S first,
 * (I - beta k^T k) Diag(a) S, so that the erase reads the decayed state; the
 * two are the same map when a is one scalar per token and head
 * (scalar_decay = 1), and differ with a per-channel a.
 */
typedef enum {
    KDA_ORDER_ERASE_FIRST = 0,  /* S <- Diag(a)(I - beta k^T k) S + beta k^T v (the table's KDA row) */
    KDA_ORDER_DECAY_FIRST = 1   /* S <- (I - beta k^T k) Diag(a) S + beta k^T v */
} kda_order_t;

typedef struct {
    int32_t num_seqs;     /* N: sequences (prefill) or sequences of one token (decode) */
    int32_t num_heads;    /* H */
    int64_t total_tokens; /* T: packed tokens over all sequences (decode: T == N) */
    int32_t dk;           /* key width: 16, 32, 64 or 128 (bf16 prefill: 32, 64 or 128;
                             fp32 prefill: 16, 32 or 64, and 128 with 16-column dv
                             slices, i.e. dv_split = dv / 16) */
    int32_t dv;           /* value width: 16, 32, 64 or 128 */
    int32_t qkv_dtype;    /* kda_dtype_t of q, k, v and o */
    int32_t scalar_decay; /* 0: log_a is [T, H, dk] (KDA); 1: log_a is [T, H] (Gated DeltaNet) */
    int32_t chunk_size;   /* prefill chunk C: 0 = default (32), else 32 or 64; 64 is
                             compiled only where its LDS image fits (small dk, dv) */
    int32_t dv_split;     /* prefill: workgroups per (sequence, head) along dv;
                             0 = choose from the problem size, else 1, 2, 4 or 8
                             (each slice dv / split must be 16, 32 or 64) */
    int32_t method;       /* prefill: kda_method_t */
    int32_t order;        /* kda_order_t: where the decay sits in the update */
    int64_t max_seqlen;   /* prefill: an upper bound on the longest sequence, or 0 if
                             unknown (then total_tokens is assumed).  Used only to size
                             the two-pass workspace segments. */
} kda_dims_t;

/*
 * Chunked prefill.
 *   q, k      [T, H, dk]   qkv_dtype
 *   v         [T, H, dv]   qkv_dtype
 *   log_a     [T, H, dk] float32 (scalar_decay = 0) or [T, H] float32 (= 1)
 *   beta      [T, H]       float32
 *   S0        [N, H, dk, dv] float32 initial states, or NULL for zeros
 *   cu_seqlens[N + 1]      int32 token offsets (device): sequence n is tokens
 *                          [cu_seqlens[n], cu_seqlens[n+1]); cu_seqlens[0] = 0,
 *                          non-decreasing, cu_seqlens[N] = T.  Empty sequences
 *                          are allowed (their S_T equals S0).  NULL means N
 *                          sequences of equal length T / N (T % N must be 0).
 *   o         [T, H, dv]   qkv_dtype output, o_t = q_t S_t
 *   S_T       [N, H, dk, dv] float32 final states, or NULL to skip.  May alias
 *             S0 (every workgroup reads its part of S0 before it writes S_T).
 *   workspace device scratch for the two-pass method (256-byte aligned), or
 *             NULL; workspace_bytes its size.  The two-pass method processes the
 *             sequences in segments of as many chunks as the workspace holds
 *             (at least one); its contents are not needed after the call.
 *             Calls that share a workspace must be ordered on one stream.
 * Results do not depend on method, chunk_size or dv_split beyond rounding order.
 * Returns a kda_status_t.
 */
KDA_API int kda_chunk_fwd(const kda_dims_t* dims, const void* q, const void* k, const void* v,
                  const float* log_a, const float* beta, const float* S0,
                  const int32_t* cu_seqlens, void* o, float* S_T, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * Chunked prefill that also exports the state at regular positions of every
 * sequence, for prefix reuse and checkpointing: the state is the only record
 * of the tokens before it, so a continuation from a shared prefix needs a
 * stored copy (glossary page "Linear attention", section "Why it matters").
 *   snapshot_every  L: tokens between snapshots, > 0 and a multiple of the
 *                   chunk size (32, or 64 with chunk_size = 64).
 *   snapshots       [R, H, dk, dv] float32 (16-byte aligned), not aliasing any
 *                   other argument.  Sequence n of length len_n contributes
 *                   floor(len_n / L) rows, in sequence order: its row s is the
 *                   state after its first (s + 1) L tokens, at row
 *                   P_n + s with P_n = sum over m < n of floor(len_m / L).
 *                   The row for s = floor(len_n / L) - 1 equals S_T when L
 *                   divides len_n.  Each row is exactly what S_T of a call on
 *                   that prefix returns (same method, chunk and split).
 *   snapshot_rows   R, the rows the buffer holds.  Rows at or past R are not
 *                   written (the lengths are on the device, so the host
 *                   cannot check R against P_N).
 * All other arguments and the error behaviour are those of kda_chunk_fwd,
 * which is this call with snapshots = NULL and snapshot_every = 0.
 */
KDA_API int kda_chunk_fwd_snapshots(const kda_dims_t* dims, const void* q, const void* k, const void* v,
                            const float* log_a, const float* beta, const float* S0,
                            const int32_t* cu_seqlens, void* o, float* S_T, float* snapshots,
                            int64_t snapshot_rows, int64_t snapshot_every, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Optional input prologue, applied as the kernels load their inputs, so that a
 * layer's raw projections need no separate pass over memory.  The pages fix no
 * gate parameterisation; these are the transforms of the usual learned gates:
 */
typedef struct {
    int32_t normalize_k;  /* 1: k_t <- k_t / sqrt(sum_c k_tc^2 + 1e-6), per token and head (fp32) */
    int32_t beta_logits;  /* 1: beta holds logits: beta_t <- 1 / (1 + exp(-beta_t)) */
    int32_t log_a_raw;    /* 1: log_a holds pre-activations x (any finite value):
                             log a <- max(-softplus(x), log_a_min), softplus(x) = log(1 + e^x) */
    float log_a_min;      /* lower clip of log a with log_a_raw: <= 0, or -INFINITY for none */
} kda_prologue_t;

/*
 * kda_chunk_fwd_snapshots with an input prologue (NULL, or all fields 0: none).
 * The prologue runs where the kernels load their inputs: in the two-pass
 * method's operator pass, or in the single-pass kernel (fp32 inputs, the other
 * shapes, KDA_METHOD_SINGLE, no workspace).  Everything else is as
 * kda_chunk_fwd_snapshots.
 */
KDA_API int kda_chunk_fwd_ex(const kda_dims_t* dims, const kda_prologue_t* prologue, const void* q,
                     const void* k, const void* v, const float* log_a, const float* beta,
                     const float* S0, const int32_t* cu_seqlens, void* o, float* S_T,
                     float* snapshots, int64_t snapshot_rows, int64_t snapshot_every,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The call allocates nothing; it takes the two-pass
 * workspace from a fixed array of KDA_NOALLOC_SCRATCH_BYTES in device memory,
 * one per GPU, held from the library's first use on that GPU until the process
 * ends.  Arguments, layouts and results are those of kda_chunk_fwd (method,
 * chunk and dv split from dims; no prologue, no snapshots).  When S_T is given
 * it holds the running state, and the scratch holds only operator blocks: a
 * call needs units x 37,376 bytes for one chunk per (sequence, head) at dk = 128
 * (units x 20,736 at dk = 64), plus units x dk x dv x 4 when S_T is NULL
 * (and a 256-byte-rounded 4 bytes per sequence for packed batches of more than
 * 256 state-pass workgroups, which the state pass takes longest first), and
 * fails with KDA_ERR_INVALID_ARGUMENT (nothing enqueued) when that exceeds the
 * scratch; larger segments of chunks run when more fits.  Shapes without a
 * two-pass kernel run single-pass and use no scratch.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
KDA_API int kda_chunk_fwd_noalloc(const kda_dims_t* dims, const void* q, const void* k, const void* v,
                                  const float* log_a, const float* beta, const float* S0,
                                  const int32_t* cu_seqlens, void* o, float* S_T, void* stream);

/*
 * Workspace the two-pass prefill prefers for these dims (segments of up to
 * 16 GiB of operator blocks: about 1.2 KB per token and head at dk = 128, so a
 * whole 2 x 32-head x 32K-token batch runs as one segment), or 0 if the call
 * would run single-pass (method SINGLE, or no two-pass kernel for the shape).
 * The minimum that still runs two-pass is what one chunk per (sequence, head)
 * needs: see kda_chunk_workspace_min.  Both include, for packed batches
 * (cu_seqlens) of 2 to 4096 sequences with more state-pass workgroups than the
 * GPU's 256 compute units, 4 bytes per sequence (rounded to 256) for the
 * order in which the state pass takes them: longest first, so that the long
 * walks do not start last.
 */
KDA_API int kda_chunk_workspace_size(const kda_dims_t* dims, size_t* bytes);
KDA_API int kda_chunk_workspace_min(const kda_dims_t* dims, size_t* bytes);

/*
 * The kernel configuration a kda_chunk_fwd call with these dims would run,
 * without running it (host only; no device is touched):
 *   packed           1 if the call passes cu_seqlens, 0 if not
 *   workspace_bytes  the workspace the call passes (0 for none)
 *   method           out: KDA_METHOD_SINGLE or KDA_METHOD_TWO_PASS
 *   chunk            out: the chunk size C
 *   dv_split         out: workgroups per (sequence, head) along dv (0 when
 *                    num_seqs is 0: nothing runs)
 * Returns the status the call would return for these dims and workspace size
 * (before its pointer checks): KDA_ERR_UNSUPPORTED for a shape not compiled,
 * KDA_ERR_INVALID_ARGUMENT for a two-pass method asked for without enough
 * workspace or a NULL output pointer.
 */
KDA_API int kda_chunk_plan(const kda_dims_t* dims, int packed, size_t workspace_bytes, int* method, int* chunk,
                           int* dv_split);

/*
 * Gradient of the prefill, for training.  On the pages the delta rule's cost is
 * a sequential dependency that blocks parallel training, and the chunkwise (WY)
 * form is what makes it parallel (page "The argument, in one page", section
 * "Everything, in one table", rows "Delta rule" and "Chunkwise / WY"); this is
 * the derivative of that same map, S_t = Diag(a_t)(I - beta_t k_t^T k_t) S_{t-1}
 * + beta_t k_t^T v_t, o_t = q_t S_t (row "KDA"; with scalar_decay, row "Gated
 * DeltaNet").
 *
 * For a loss L with dL/do = dO and dL/dS_T = dS_T, the call writes the
 * derivatives of L with respect to every input of kda_chunk_fwd:
 *   q, k, v, log_a, beta, S0, cu_seqlens   as for kda_chunk_fwd (the forward inputs)
 *   dO        [T, H, dv]   qkv_dtype
 *   dS_T      [N, H, dk, dv] float32, or NULL for zero
 *   dq, dk    [T, H, dk]   qkv_dtype outputs
 *   dv        [T, H, dv]   qkv_dtype output
 *   dlog_a    float32 output with the shape of log_a ([T, H] with a scalar decay:
 *             the sum over channels)
 *   dbeta     [T, H]       float32 output
 *   dS0       [N, H, dk, dv] float32 output, or NULL to skip; written also when
 *             S0 is NULL (the derivative at the zero initial state)
 *   workspace device memory of at least kda_chunk_bwd_workspace_size bytes,
 *             256-byte aligned; its contents are not needed after the call.
 *             Calls that share a workspace must be ordered on one stream.
 * The call first reruns the prefill (method, chunk_size and dv_split as in dims)
 * keeping the state at every 64th token, then three kernels walk 16-token
 * pieces: operators per piece, the derivative with respect to the state
 * backwards through each sequence, and the gradients of each 64-token chunk.
 * Both orders (dims.order; the decay-first map's chunk form is the erase-first
 * one with each token's decay applied before its own read, and differs only in
 * the last step of dlog_a); bf16 with dk, dv in {32, 64, 128}, fp32
 * with dk, dv in {16, 32, 64}, in both cases dk and dv equal or a factor 2
 * apart.  No input prologue (kda_chunk_bwd_ex takes one).  Outputs must not alias
 * inputs or each other.  Returns a kda_status_t.
 */
KDA_API int kda_chunk_bwd(const kda_dims_t* dims, const void* q, const void* k, const void* v,
                  const float* log_a, const float* beta, const float* S0,
                  const int32_t* cu_seqlens, const void* dO, const float* dS_T, void* dq, void* dk,
                  void* dv, float* dlog_a, float* dbeta, float* dS0, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Workspace kda_chunk_bwd needs for these dims (about 5.9 KB per token and head
 * at dk = dv = 128, plus what the prefill's two-pass method prefers). */
KDA_API int kda_chunk_bwd_workspace_size(const kda_dims_t* dims, size_t* bytes);

/*
 * kda_chunk_bwd for a training step whose forward call kept its states: the
 * state at every 64th token of each sequence, as kda_chunk_fwd_snapshots
 * writes it with snapshot_every = 64 (same dims and inputs; any method, chunk
 * or dv split, which change the states only by rounding).  The backward then
 * runs no prefill of its own: it is the three gradient kernels alone, with a
 * smaller workspace (kda_chunk_bwd_saved_workspace_size).
 *   states      [R, H, dk, dv] float32, 16-byte aligned, read only: row P_n + s
 *               is the state of sequence n after its first 64 (s + 1) tokens,
 *               P_n = sum over m < n of floor(len_m / 64).  May be NULL only
 *               when total_tokens < 64 (no row is needed).
 *   state_rows  R.  Without cu_seqlens the call checks R >= N floor(T / (64 N))
 *               and returns KDA_ERR_INVALID_ARGUMENT otherwise; with cu_seqlens
 *               the lengths are on the device, so the caller passes at least
 *               P_N rows: a row at or past R is read as a zero state (wrong
 *               gradients for that chunk, but no access outside the buffer).
 * Every other argument, the supported shapes and the error behaviour are those
 * of kda_chunk_bwd, whose gradients this returns (bit for bit when the forward
 * ran with the same method, chunk and dv split as kda_chunk_bwd's rerun).
 */
KDA_API int kda_chunk_bwd_saved(const kda_dims_t* dims, const void* q, const void* k, const void* v,
                                const float* log_a, const float* beta, const float* S0,
                                const int32_t* cu_seqlens, const float* states, int64_t state_rows,
                                const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                                float* dlog_a, float* dbeta, float* dS0, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * kda_chunk_bwd for a forward call that ran an input prologue (kda_chunk_fwd_ex),
 * optionally from the forward's kept states.  k, log_a and beta are the raw
 * inputs the forward took, and dk, dlog_a, dbeta are the derivatives with
 * respect to them: through k = x / sqrt(|x|^2 + 1e-6), beta = 1 / (1 + e^-z)
 * and log a = max(-softplus(y), log_a_min), whose derivative is taken as 0
 * where the clip is active (-softplus(y) < log_a_min).  The transformed inputs
 * are formed in the workspace, the gradient runs on them, and the chain rule
 * through the transforms is applied to dk, dlog_a and dbeta in place.
 *   prologue    as for kda_chunk_fwd_ex (NULL or all fields 0: none)
 *   states      NULL: the prefill is run again, as kda_chunk_bwd does; else the
 *               forward's states at every 64th token, as for kda_chunk_bwd_saved
 *   workspace   at least kda_chunk_bwd_ex_workspace_size bytes (saved = states
 *               is not NULL), 256-byte aligned
 * The other arguments, the supported shapes and the error behaviour are those of
 * kda_chunk_bwd (with states: kda_chunk_bwd_saved); every argument is checked
 * before anything is enqueued.
 */
KDA_API int kda_chunk_bwd_ex(const kda_dims_t* dims, const kda_prologue_t* prologue, const void* q,
                             const void* k, const void* v, const float* log_a, const float* beta,
                             const float* S0, const int32_t* cu_seqlens, const float* states,
                             int64_t state_rows, const void* dO, const float* dS_T, void* dq, void* dk,
                             void* dv, float* dlog_a, float* dbeta, float* dS0, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Workspace kda_chunk_bwd_ex needs: kda_chunk_bwd's (saved = 0) or
 * kda_chunk_bwd_saved's (saved != 0), plus, with a prologue, the transformed
 * keys, log a and beta (T H dk elements of qkv_dtype, T H dk or T H floats, and
 * T H floats, each rounded up to 256 bytes). */
KDA_API int kda_chunk_bwd_ex_workspace_size(const kda_dims_t* dims, const kda_prologue_t* prologue,
                                            int saved, size_t* bytes);

/* Workspace kda_chunk_bwd_saved needs for these dims (about 4.6 KB per token and
 * head at dk = dv = 128: the gradient kernels' share of kda_chunk_bwd's). */
KDA_API int kda_chunk_bwd_saved_workspace_size(const kda_dims_t* dims, size_t* bytes);

/*
 * One decode step: one token per sequence (T == N).
 *   q, k      [N, H, dk]   qkv_dtype
 *   v         [N, H, dv]   qkv_dtype
 *   log_a     [N, H, dk] or [N, H] float32, beta [N, H] float32
 *   S_in      [N, H, dk, dv] float32 state before the token
 *   S_out     [N, H, dk, dv] float32 state after the token; may equal S_in
 *             (in-place update).  Each state is read once and written once.
 *   o         [N, H, dv]   qkv_dtype output, o = q S_out
 * Returns a kda_status_t.
 */
KDA_API int kda_decode_step(const kda_dims_t* dims, const void* q, const void* k, const void* v,
                    const float* log_a, const float* beta, const float* S_in, float* S_out,
                    void* o, void* stream);

/* kda_decode_step with an input prologue (NULL, or all fields 0: none); every
 * shape that kda_decode_step supports. */
KDA_API int kda_decode_step_ex(const kda_dims_t* dims, const kda_prologue_t* prologue, const void* q,
                       const void* k, const void* v, const float* log_a, const float* beta,
                       const float* S_in, float* S_out, void* o, void* stream);

/* Static text for a status code. */
KDA_API const char* kda_status_string(int status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
KDA_API const char* kda_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
KDA_API int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
