// Driver for the sanitizer build of the C-ABI's host side (kda_api.cpp built with
// AddressSanitizer and UndefinedBehaviorSanitizer on its host code): every case is
// refused by the host validation (or has nothing to do), so no kernel is launched
// and no fake address is dereferenced.  Sizes are pushed to their extremes so
// that overflow in the size arithmetic would show.  Exit status 0 when every
// status is the documented one.  Test infrastructure (CPU only, no GPU needed).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static const uintptr_t GOOD = 0x7F0000000000ull;  // 16-byte aligned, never dereferenced
static int failures = 0;

static kda_dims_t dims(int32_t N = 2, int32_t H = 4, int64_t T = 128, int32_t dk = 128, int32_t dv = 128) {
    kda_dims_t d;
    memset(&d, 0, sizeof(d));
    d.num_seqs = N; d.num_heads = H; d.total_tokens = T; d.dk = dk; d.dv = dv; d.qkv_dtype = KDA_BF16;
    return d;
}

static void expect(const char* what, int got, int want) {
    if (got != want) {
        printf("%s: status %d, expected %d (%s)\n", what, got, want, kda_last_error());
        ++failures;
    }
}

static const void* P(uintptr_t x) { return (const void*)x; }

static int prefill(const kda_dims_t* d, uintptr_t q = GOOD, uintptr_t o = GOOD, uintptr_t cu = GOOD,
                   uintptr_t ws = 0, size_t ws_bytes = 0, uintptr_t S0 = 0) {
    return kda_chunk_fwd(d, P(q), P(GOOD), P(GOOD), (const float*)GOOD, (const float*)GOOD, (const float*)S0,
                         (const int32_t*)cu, (void*)o, (float*)GOOD, (void*)ws, ws_bytes, nullptr);
}

int main() {
    kda_dims_t d = dims();
    expect("null dims", prefill(nullptr), KDA_ERR_INVALID_ARGUMENT);
    d = dims(); d.num_heads = 0; expect("heads 0", prefill(&d), KDA_ERR_INVALID_ARGUMENT);
    d = dims(); d.dk = 48; expect("dk 48", prefill(&d), KDA_ERR_UNSUPPORTED);
    d = dims(); d.dv_split = 3; expect("split 3", prefill(&d), KDA_ERR_INVALID_ARGUMENT);
    d = dims(); expect("q null", prefill(&d, 0), KDA_ERR_INVALID_ARGUMENT);
    d = dims(); expect("q misaligned", prefill(&d, GOOD + 2), KDA_ERR_MISALIGNED);
    d = dims(); expect("S0 misaligned", prefill(&d, GOOD, GOOD, GOOD, 0, 0, GOOD + 8), KDA_ERR_MISALIGNED);
    d = dims(); d.total_tokens = 127; expect("no cu, uneven", prefill(&d, GOOD, GOOD, 0), KDA_ERR_INVALID_ARGUMENT);
    d = dims(0, 4, 0); expect("nothing to do", prefill(&d, 0, 0, 0), KDA_OK);
    d = dims(); d.method = KDA_METHOD_TWO_PASS; expect("two-pass no workspace", prefill(&d), KDA_ERR_INVALID_ARGUMENT);
    d = dims(); d.method = KDA_METHOD_TWO_PASS;
    expect("two-pass small workspace", prefill(&d, GOOD, GOOD, GOOD, GOOD, 64), KDA_ERR_INVALID_ARGUMENT);
    expect("two-pass misaligned workspace", prefill(&d, GOOD, GOOD, GOOD, GOOD + 16, size_t(1) << 30),
           KDA_ERR_MISALIGNED);

    // workspace sizes at the extremes of the dims (no overflow, consistent answers)
    size_t pref = 0, least = 0;
    d = dims(2, 32, 2 * 32768);
    expect("ws size", kda_chunk_workspace_size(&d, &pref), KDA_OK);
    expect("ws min", kda_chunk_workspace_min(&d, &least), KDA_OK);
    if (!(least > 0 && pref >= least)) { printf("workspace sizes %zu %zu\n", pref, least); ++failures; }
    size_t huge = 0;
    d = dims(1 << 20, 64, int64_t(1) << 40); d.max_seqlen = int64_t(1) << 22;
    expect("ws size huge", kda_chunk_workspace_size(&d, &huge), KDA_OK);
    d = dims(2, 4, 128);
    expect("ws size null out", kda_chunk_workspace_size(&d, nullptr), KDA_ERR_INVALID_ARGUMENT);
    size_t bwd = 0;
    d = dims(2, 32, 2 * 32768);
    expect("bwd ws size", kda_chunk_bwd_workspace_size(&d, &bwd), KDA_OK);
    if (bwd <= pref) { printf("bwd workspace %zu\n", bwd); ++failures; }

    // snapshots
    d = dims();
    expect("snap every 48",
           kda_chunk_fwd_snapshots(&d, P(GOOD), P(GOOD), P(GOOD), (const float*)GOOD, (const float*)GOOD, nullptr,
                                   (const int32_t*)GOOD, (void*)GOOD, (float*)GOOD, (float*)GOOD, 4, 48, nullptr, 0,
                                   nullptr),
           KDA_ERR_INVALID_ARGUMENT);
    expect("snap huge interval",
           kda_chunk_fwd_snapshots(&d, P(GOOD), P(GOOD), P(GOOD), (const float*)GOOD, (const float*)GOOD, nullptr,
                                   (const int32_t*)GOOD, (void*)GOOD, (float*)GOOD, (float*)GOOD, 4,
                                   int64_t(1) << 40, nullptr, 0, nullptr),
           KDA_ERR_INVALID_ARGUMENT);

    // prologue
    kda_prologue_t pro;
    memset(&pro, 0, sizeof(pro));
    pro.normalize_k = 2;
    d = dims();
    expect("prologue flag 2",
           kda_chunk_fwd_ex(&d, &pro, P(GOOD), P(GOOD), P(GOOD), (const float*)GOOD, (const float*)GOOD, nullptr,
                            (const int32_t*)GOOD, (void*)GOOD, (float*)GOOD, nullptr, 0, 0, nullptr, 0, nullptr),
           KDA_ERR_INVALID_ARGUMENT);

    // decode
    d = dims(2, 4, 3);
    expect("decode T != N",
           kda_decode_step(&d, P(GOOD), P(GOOD), P(GOOD), (const float*)GOOD, (const float*)GOOD,
                           (const float*)GOOD, (float*)GOOD, (void*)GOOD, nullptr),
           KDA_ERR_INVALID_ARGUMENT);
    d = dims(2, 4, 2); d.dk = 24;
    expect("decode dk 24",
           kda_decode_step(&d, P(GOOD), P(GOOD), P(GOOD), (const float*)GOOD, (const float*)GOOD,
                           (const float*)GOOD, (float*)GOOD, (void*)GOOD, nullptr),
           KDA_ERR_UNSUPPORTED);

    // allocation-free prefill: beyond its fixed scratch, refused before any device call
    d = dims(1, 4096, 64); d.method = KDA_METHOD_TWO_PASS;
    expect("noalloc too big",
           kda_chunk_fwd_noalloc(&d, P(GOOD), P(GOOD), P(GOOD), (const float*)GOOD, (const float*)GOOD, nullptr,
                                 (const int32_t*)GOOD, (void*)GOOD, (float*)GOOD, nullptr),
           KDA_ERR_INVALID_ARGUMENT);

    // backward
    d = dims(); d.dk = 32; d.dv = 128;
    expect("bwd unsupported shape",
           kda_chunk_bwd(&d, P(GOOD), P(GOOD), P(GOOD), (const float*)GOOD, (const float*)GOOD, nullptr,
                         (const int32_t*)GOOD, P(GOOD), nullptr, (void*)GOOD, (void*)GOOD, (void*)GOOD, (float*)GOOD,
                         (float*)GOOD, nullptr, (void*)GOOD, size_t(1) << 40, nullptr),
           KDA_ERR_UNSUPPORTED);
    d = dims();
    expect("bwd saved without states",
           kda_chunk_bwd_saved(&d, P(GOOD), P(GOOD), P(GOOD), (const float*)GOOD, (const float*)GOOD, nullptr,
                               (const int32_t*)GOOD, nullptr, 0, P(GOOD), nullptr, (void*)GOOD, (void*)GOOD,
                               (void*)GOOD, (float*)GOOD, (float*)GOOD, nullptr, (void*)GOOD, size_t(1) << 40,
                               nullptr),
           KDA_ERR_INVALID_ARGUMENT);
    kda_prologue_t bad_pro = {2, 0, 0, 0.f};
    expect("bwd_ex bad prologue",
           kda_chunk_bwd_ex(&d, &bad_pro, P(GOOD), P(GOOD), P(GOOD), (const float*)GOOD, (const float*)GOOD, nullptr,
                            (const int32_t*)GOOD, nullptr, 0, P(GOOD), nullptr, (void*)GOOD, (void*)GOOD, (void*)GOOD,
                            (float*)GOOD, (float*)GOOD, nullptr, (void*)GOOD, size_t(1) << 40, nullptr),
           KDA_ERR_INVALID_ARGUMENT);
    kda_prologue_t all_pro = {1, 1, 1, -8.f};
    expect("bwd_ex workspace too small",
           kda_chunk_bwd_ex(&d, &all_pro, P(GOOD), P(GOOD), P(GOOD), (const float*)GOOD, (const float*)GOOD, nullptr,
                            (const int32_t*)GOOD, nullptr, 0, P(GOOD), nullptr, (void*)GOOD, (void*)GOOD, (void*)GOOD,
                            (float*)GOOD, (float*)GOOD, nullptr, (void*)GOOD, 4096, nullptr),
           KDA_ERR_INVALID_ARGUMENT);

    for (int s = -1; s < 6; ++s)
        if (!kda_status_string(s) || !*kda_status_string(s)) ++failures;
    printf(failures ? "api sanitizer check FAILED (%d)\n" : "api sanitizer check ok\n", failures);
    return failures ? 1 : 0;
}
