"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments with the documented status codes before touching a GPU (CPU only).

Fake device addresses are used: every case below is refused by host-side
validation, so nothing is dereferenced or launched.
"""
import ctypes
import os
import re

import pytest

import kda_recurrent_state_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, MISALIGNED = 0, 1, 2, 3
GOOD = 0x7F0000000000  # 16-byte aligned fake device address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    return kda.load_library()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"KDA_API\s+[\w\s\*]+?\b(kda_\w+)\s*\(", text)


def test_header_declares_entry_points():
    names = declared_functions()
    assert {"kda_chunk_fwd", "kda_chunk_fwd_snapshots", "kda_chunk_workspace_size", "kda_chunk_workspace_min", "kda_decode_step",
            "kda_status_string", "kda_last_error", "kda_version"} <= set(names)


def test_every_declared_symbol_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported by {kda.library_path()}"


def dims(**kw):
    base = dict(num_seqs=2, num_heads=4, total_tokens=128, dk=128, dv=128, qkv_dtype=1,
                scalar_decay=0, chunk_size=0, dv_split=0, method=0, order=0, max_seqlen=0)
    base.update(kw)
    return kda._Dims(**base)


def prefill(lib, d, q=GOOD, k=GOOD, v=GOOD, la=GOOD, beta=GOOD, S0=None, cu=GOOD, o=GOOD, ST=GOOD,
            ws=None, ws_bytes=0):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    dp = None if d is None else ctypes.byref(d)
    return lib.kda_chunk_fwd(dp, P(q), P(k), P(v), P(la), P(beta), P(S0), P(cu), P(o), P(ST), P(ws),
                             ctypes.c_size_t(ws_bytes), None)


def decode(lib, d, q=GOOD, k=GOOD, v=GOOD, la=GOOD, beta=GOOD, Si=GOOD, So=GOOD, o=GOOD):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.kda_decode_step(ctypes.byref(d), P(q), P(k), P(v), P(la), P(beta), P(Si), P(So), P(o), None)


@pytest.mark.parametrize("case,expect", [
    (dict(d=None), INVALID),
    (dict(d=dims(num_heads=0)), INVALID),
    (dict(d=dims(num_seqs=-1)), INVALID),
    (dict(d=dims(total_tokens=-5)), INVALID),
    (dict(d=dims(qkv_dtype=7)), INVALID),
    (dict(d=dims(scalar_decay=2)), INVALID),
    (dict(d=dims(dk=48)), UNSUPPORTED),
    (dict(d=dims(dv=256)), UNSUPPORTED),
    (dict(d=dims(chunk_size=48)), UNSUPPORTED),
    (dict(d=dims(dv_split=3)), INVALID),
    (dict(d=dims(qkv_dtype=1, dk=16, dv=16)), UNSUPPORTED),  # no bf16 kernel below dk=32
    (dict(d=dims(qkv_dtype=0, dk=128, dv=128, dv_split=4)), UNSUPPORTED),  # fp32 at dk=128: 16-column slices only
    (dict(d=dims(), q=None), INVALID),
    (dict(d=dims(), beta=None), INVALID),
    (dict(d=dims(), o=None), INVALID),
    (dict(d=dims(), q=GOOD + 2), MISALIGNED),
    (dict(d=dims(), la=GOOD + 4), MISALIGNED),
    (dict(d=dims(), S0=GOOD + 8), MISALIGNED),
    (dict(d=dims(), cu=GOOD + 2), MISALIGNED),
    (dict(d=dims(total_tokens=127), cu=None), INVALID),
    (dict(d=dims(num_seqs=0, total_tokens=5)), INVALID),
    (dict(d=dims(num_seqs=0, total_tokens=0), q=None, cu=None), OK),  # nothing to do
    (dict(d=dims(method=3)), INVALID),
    (dict(d=dims(order=2)), INVALID),
    (dict(d=dims(order=-1)), INVALID),
    (dict(d=dims(max_seqlen=-1)), INVALID),
    (dict(d=dims(method=2, qkv_dtype=0, dk=64, dv=64)), UNSUPPORTED),  # two-pass is bf16 only
    (dict(d=dims(method=2)), INVALID),                                   # no workspace
    (dict(d=dims(method=2), ws=GOOD, ws_bytes=64), INVALID),             # workspace too small
    (dict(d=dims(method=2), ws=GOOD + 16, ws_bytes=1 << 30), MISALIGNED),
])
def test_prefill_validation(lib, case, expect):
    st = prefill(lib, **case)
    assert st == expect, (st, lib.kda_last_error())
    if expect != OK:
        assert lib.kda_last_error().decode() != ""
    else:
        assert lib.kda_last_error().decode() == ""


def prefill_snap(lib, d, snaps=GOOD, rows=4, every=64, cu=GOOD):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.kda_chunk_fwd_snapshots(ctypes.byref(d), P(GOOD), P(GOOD), P(GOOD), P(GOOD), P(GOOD), None,
                                       P(cu), P(GOOD), P(GOOD), P(snaps), ctypes.c_int64(rows),
                                       ctypes.c_int64(every), None, ctypes.c_size_t(0), None)


@pytest.mark.parametrize("case,expect", [
    (dict(every=48), INVALID),                          # not a multiple of the chunk (32)
    (dict(every=32, d=dims(chunk_size=64)), INVALID),   # not a multiple of the chunk (64)
    (dict(every=-32), INVALID),
    (dict(every=0), INVALID),                           # a buffer but no interval
    (dict(snaps=None), INVALID),                        # rows but no buffer
    (dict(rows=-1), INVALID),
    (dict(snaps=GOOD + 2), MISALIGNED),
    (dict(snaps=GOOD + 4), MISALIGNED),
    (dict(every=1 << 40), INVALID),
    (dict(d=dims(num_seqs=0, total_tokens=0)), OK),     # nothing to do
    (dict(d=dims(num_seqs=0, total_tokens=0), every=0, snaps=None, rows=0), OK),
])
def test_snapshot_validation(lib, case, expect):
    case.setdefault("d", dims())
    st = prefill_snap(lib, **case)
    assert st == expect, (st, lib.kda_last_error())


@pytest.mark.parametrize("case,expect", [
    (dict(d=dims(total_tokens=3)), INVALID),
    (dict(d=dims(total_tokens=2), Si=None), INVALID),
    (dict(d=dims(total_tokens=2), So=GOOD + 4), MISALIGNED),
    (dict(d=dims(total_tokens=2, dk=24)), UNSUPPORTED),
    (dict(d=dims(total_tokens=2, order=3)), INVALID),
    (dict(d=dims(num_seqs=0, total_tokens=0), q=None), OK),
])
def test_decode_validation(lib, case, expect):
    assert decode(lib, **case) == expect


def test_scalar_arrays_need_only_4_byte_alignment(lib):
    """beta and a scalar log_a pass with 4-byte alignment; the call then stops
    at the misaligned output, so nothing is launched."""
    st = prefill(lib, dims(scalar_decay=1), la=GOOD + 4, beta=GOOD + 4, o=GOOD + 2)
    assert st == MISALIGNED and lib.kda_last_error().decode().startswith("o is not")
    st = decode(lib, dims(total_tokens=2), la=GOOD + 4, beta=GOOD + 4, o=GOOD + 2)
    assert st == MISALIGNED and lib.kda_last_error().decode().startswith("o is not")


def test_workspace_sizes(lib):
    size, least = ctypes.c_size_t(0), ctypes.c_size_t(0)
    d = dims(num_seqs=2, num_heads=32, total_tokens=2 * 32768)
    assert lib.kda_chunk_workspace_size(ctypes.byref(d), ctypes.byref(size)) == OK
    assert lib.kda_chunk_workspace_min(ctypes.byref(d), ctypes.byref(least)) == OK
    units, state = 64, 64 * 128 * 128 * 4
    assert least.value > state and (least.value - state) % units == 0
    block = (least.value - state) // units
    assert block % 256 == 0 and size.value >= least.value and (size.value - state) % (units * block) == 0
    assert (size.value - state) <= (16 << 30)  # segments of at most 16 GiB of blocks
    d.max_seqlen = 32768  # with the longest sequence known, this batch fits one segment
    assert lib.kda_chunk_workspace_size(ctypes.byref(d), ctypes.byref(size)) == OK
    assert size.value - state == units * block * (32768 // 32)
    d = dims(method=1)
    assert lib.kda_chunk_workspace_size(ctypes.byref(d), ctypes.byref(size)) == OK and size.value == 0
    d = dims(qkv_dtype=0, dk=64, dv=64)  # fp32 runs single-pass only
    assert lib.kda_chunk_workspace_size(ctypes.byref(d), ctypes.byref(size)) == OK and size.value == 0


def test_workspace_holds_the_sequence_order(lib):
    """Packed batches with more state-pass workgroups than the 256 compute
    units reserve 4 bytes per sequence (rounded to 256) for the longest-first
    order; smaller batches and batches beyond 4096 sequences do not."""
    def least(**kw):
        n = ctypes.c_size_t(0)
        assert lib.kda_chunk_workspace_min(ctypes.byref(dims(**kw)), ctypes.byref(n)) == OK
        return n.value
    block, state = 37376, 128 * 128 * 4
    # 300 units at split 2 (64-column slices): 600 workgroups, ordered
    assert least(num_seqs=300, num_heads=1, total_tokens=30000) == 1280 + 300 * (state + block)
    # 64 units at split 4: 256 workgroups, all resident at once, index order
    assert least(num_seqs=2, num_heads=32, total_tokens=64) == 64 * (state + block)
    # 5000 sequences: beyond the ranked maximum, index order
    assert least(num_seqs=5000, num_heads=1, total_tokens=5000) == 5000 * (state + block)


def test_status_strings(lib):
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(3) == b"KDA_ERR_MISALIGNED"
    assert lib.kda_status_string(99) == b"KDA_ERR_UNKNOWN"
    assert lib.kda_version() >= 10000


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 1, 32)
    with pytest.raises(RuntimeError, match="HIP device"):
        kda.chunk_fwd(x, x, x, torch.zeros(4, 1, 32), torch.zeros(4, 1))


def test_snapshot_rows_counts_whole_intervals():
    assert kda.snapshot_rows([0, 300, 307, 435, 435, 596], 64) == 4 + 0 + 2 + 0 + 2
    assert kda.snapshot_rows(None, 64, total_tokens=640, num_seqs=2) == 2 * 5
    assert kda.snapshot_rows(None, 64, total_tokens=0, num_seqs=0) == 0
    with pytest.raises(ValueError):
        kda.snapshot_rows([0, 10], 0)


def test_decay_first_blocks_hold_no_write_operator(lib):
    """Decay-first operator blocks drop the dk x C write operator: at dk = 128,
    C = 32 a block is 8192 bytes smaller.  With a scalar decay both orders run
    the same kernels and need the same workspace."""
    def least(**kw):
        n = ctypes.c_size_t(0)
        assert lib.kda_chunk_workspace_min(ctypes.byref(dims(**kw)), ctypes.byref(n)) == OK
        return n.value
    units = 2 * 4
    assert least(order=0) - least(order=1) == units * 8192
    assert least(order=0, dk=64, dv=64) - least(order=1, dk=64, dv=64) == units * 4096
    assert least(order=1, scalar_decay=1) == least(order=0, scalar_decay=1)


def prefill_ex(lib, d, pro, ws=None, ws_bytes=0):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    pp = None if pro is None else ctypes.byref(pro)
    return lib.kda_chunk_fwd_ex(ctypes.byref(d), pp, P(GOOD), P(GOOD), P(GOOD), P(GOOD), P(GOOD), None, P(GOOD),
                                P(GOOD), P(GOOD), None, ctypes.c_int64(0), ctypes.c_int64(0), P(ws),
                                ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("fields,d,expect", [
    ((2, 0, 0, 0.0), dims(), INVALID),                     # flags are 0 or 1
    ((0, 0, 1, 0.5), dims(), INVALID),                     # log_a_min above 0
    ((0, 0, 1, float("nan")), dims(), INVALID),
    # the single-pass kernel runs the prologue too: these pass every check and
    # fail here only at the launch (no GPU)
    ((1, 1, 1, -8.0), dims(qkv_dtype=0, dk=64, dv=64), "launch"),  # fp32 runs single-pass
    ((1, 1, 1, -8.0), dims(qkv_dtype=0, dk=128, dv=128), "launch"),  # fp32 at dk = 128: 16-column slices
    ((1, 0, 0, 0.0), dims(method=1), "launch"),             # single-pass asked for
    ((0, 1, 0, 0.0), dims(), "launch"),                     # no workspace: single-pass
    ((0, 0, 0, 0.0), dims(num_seqs=0, total_tokens=0), OK),
    ((1, 1, 1, float("-inf")), dims(num_seqs=0, total_tokens=0), OK),
])
def test_prologue_validation(lib, fields, d, expect):
    pro = kda._Prologue(*fields)
    st = prefill_ex(lib, d, pro)
    if expect == "launch":
        assert st not in (OK, INVALID, UNSUPPORTED, MISALIGNED), (st, lib.kda_last_error())
        assert "launch" in lib.kda_last_error().decode()
    else:
        assert st == expect, (st, lib.kda_last_error())


def test_decode_prologue_validation(lib):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    bad = kda._Prologue(0, 3, 0, 0.0)
    st = lib.kda_decode_step_ex(ctypes.byref(dims(total_tokens=2)), ctypes.byref(bad), P(GOOD), P(GOOD), P(GOOD),
                                P(GOOD), P(GOOD), P(GOOD), P(GOOD), P(GOOD), None)
    assert st == INVALID


def test_binding_prologue_fields():
    assert kda._prologue(None) is None
    p = kda._prologue(dict(normalize_k=True, log_a_raw=1))
    assert (p.normalize_k, p.beta_logits, p.log_a_raw, p.log_a_min) == (1, 0, 1, float("-inf"))
    with pytest.raises(ValueError):
        kda._prologue(dict(normalise_k=True))


# ---- kda_chunk_bwd: argument checks (nothing is launched) ----
def bwd_ws(lib, d):
    need = ctypes.c_size_t(0)
    st = lib.kda_chunk_bwd_workspace_size(ctypes.byref(d), ctypes.byref(need))
    return st, need.value


def backward(lib, d, ws_bytes=None, **ptrs):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    names = ["q", "k", "v", "la", "beta", "S0", "cu", "dO", "dST", "dq", "dk", "dv", "dla", "dbeta", "dS0", "ws"]
    vals = {n: GOOD for n in names}
    vals.update(S0=None, dST=None, dS0=None)
    vals.update(ptrs)
    if ws_bytes is None:
        st, ws_bytes = bwd_ws(lib, d)
        assert st == OK
    return lib.kda_chunk_bwd(ctypes.byref(d), *[P(vals[n]) for n in names[:-1]], P(vals["ws"]),
                             ctypes.c_size_t(ws_bytes), None)


def test_bwd_workspace_size(lib):
    st, b128 = bwd_ws(lib, dims(total_tokens=4096, num_seqs=2, max_seqlen=2048))
    assert st == OK and b128 > 0
    # grows with the tokens: kept states every 64 tokens, blocks every 16, derivatives every 64
    st, b256 = bwd_ws(lib, dims(total_tokens=8192, num_seqs=2, max_seqlen=4096))
    assert st == OK and b256 > 1.9 * b128 - (1 << 30)
    assert bwd_ws(lib, dims(order=1))[0] == OK                        # decay-first, per-channel
    assert bwd_ws(lib, dims(order=1, scalar_decay=1))[0] == OK       # one map with a scalar gate
    assert bwd_ws(lib, dims(dk=128, dv=64))[0] == OK                   # dk, dv a factor 2 apart
    assert bwd_ws(lib, dims(dk=32, dv=64))[0] == OK
    assert bwd_ws(lib, dims(dk=128, dv=32))[0] == UNSUPPORTED          # a factor 4
    assert bwd_ws(lib, dims(dk=16, dv=16))[0] == UNSUPPORTED          # bf16 needs dk >= 32
    assert bwd_ws(lib, dims(dk=16, dv=16, qkv_dtype=0))[0] == OK
    assert bwd_ws(lib, dims(dk=16, dv=32, qkv_dtype=0))[0] == OK
    assert bwd_ws(lib, dims(dk=16, dv=64, qkv_dtype=0))[0] == UNSUPPORTED
    assert bwd_ws(lib, dims(dk=128, dv=128, qkv_dtype=0))[0] == UNSUPPORTED


@pytest.mark.parametrize("case,expect", [
    (dict(ws_bytes=1024), INVALID),                 # workspace too small
    (dict(ws=None), INVALID),
    (dict(ws=GOOD + 16), MISALIGNED),               # 256-byte alignment
    (dict(dO=None), INVALID),
    (dict(dq=None), INVALID),
    (dict(dbeta=None), INVALID),
    (dict(dla=GOOD + 4), MISALIGNED),               # per-channel dlog_a is read in 16-byte pieces
    (dict(dST=GOOD + 8), MISALIGNED),
    (dict(dS0=GOOD + 8), MISALIGNED),
    (dict(q=GOOD + 2), MISALIGNED),
])
def test_bwd_validation(lib, case, expect):
    d = dims()
    assert backward(lib, d, **case) == expect


def test_bwd_refuses_unsupported_shapes(lib):
    assert backward(lib, dims(dk=32, dv=128), ws_bytes=1 << 20) == UNSUPPORTED
    assert backward(lib, dims(order=2), ws_bytes=1 << 20) in (INVALID, UNSUPPORTED)


def bwd_saved(lib, d, states=GOOD, rows=2, ws_bytes=None, **ptrs):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    vals = {n: GOOD for n in ["q", "k", "v", "la", "beta", "cu", "dO", "dq", "dk", "dv", "dla", "dbeta", "ws"]}
    vals.update(S0=None, dST=None, dS0=None)
    vals.update(ptrs)
    if ws_bytes is None:
        need = ctypes.c_size_t(0)
        assert lib.kda_chunk_bwd_saved_workspace_size(ctypes.byref(d), ctypes.byref(need)) == OK
        ws_bytes = need.value
    g = lambda *ns: [P(vals[n]) for n in ns]
    return lib.kda_chunk_bwd_saved(ctypes.byref(d), *g("q", "k", "v", "la", "beta", "S0", "cu"), P(states),
                                   ctypes.c_int64(rows), *g("dO", "dST", "dq", "dk", "dv", "dla", "dbeta", "dS0",
                                                            "ws"), ctypes.c_size_t(ws_bytes), None)


def test_bwd_saved_workspace_is_the_gradient_share():
    """With the forward's states passed in, the workspace drops the rerun's
    prefill workspace, outputs and kept states."""
    lib = kda.load_library(build_if_missing=False)
    d = dims(total_tokens=65536, num_seqs=2, num_heads=32, max_seqlen=32768)
    full, saved = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.kda_chunk_bwd_workspace_size(ctypes.byref(d), ctypes.byref(full)) == OK
    assert lib.kda_chunk_bwd_saved_workspace_size(ctypes.byref(d), ctypes.byref(saved)) == OK
    pref = ctypes.c_size_t(0)
    assert lib.kda_chunk_workspace_size(ctypes.byref(d), ctypes.byref(pref)) == OK
    rerun = pref.value + 65536 * 32 * 128 * 2 + (65536 // 64) * 32 * 128 * 128 * 4
    assert abs(full.value - saved.value - rerun) < 4096
    d1 = dims(dk=128, dv=32)
    assert lib.kda_chunk_bwd_saved_workspace_size(ctypes.byref(d1), ctypes.byref(saved)) == UNSUPPORTED


@pytest.mark.parametrize("case,expect", [
    (dict(states=None), INVALID),                   # 128 tokens: rows are needed
    (dict(cu=None, rows=1), INVALID),               # equal lengths 2 x 64: two rows
    (dict(states=GOOD + 8), MISALIGNED),
    (dict(ws_bytes=1024), INVALID),
    (dict(dq=None), INVALID),
])
def test_bwd_saved_validation(lib, case, expect):
    assert bwd_saved(lib, dims(), **case) == expect


def test_bwd_saved_states_optional_below_64_tokens(lib):
    """Fewer than 64 tokens: no state row can be read, so states may be NULL;
    the call gets past every argument check (it then needs the GPU, and fails
    here only at the launch)."""
    st = bwd_saved(lib, dims(total_tokens=40, num_seqs=2), states=None, rows=0)
    assert st not in (INVALID, MISALIGNED, UNSUPPORTED)


def _cpu_prefill_inputs(T=40, H=2, dk=32, dv=16, N=2):
    import torch
    q = torch.zeros(T, H, dk, dtype=torch.bfloat16)
    return dict(q=q, k=q.clone(), v=torch.zeros(T, H, dv, dtype=torch.bfloat16),
                log_a=torch.zeros(T, H, dk), beta=torch.zeros(T, H),
                cu_seqlens=torch.tensor([0, 25, T], dtype=torch.int32)), (T, H, dk, dv, N)


@pytest.mark.parametrize("which", ["out", "final_state"])
def test_prefill_rejects_wrong_output_shapes(which):
    """The library cannot see sizes: a too-small output tensor is refused by the
    binding (ValueError) before any device check or call."""
    import torch
    inp, (T, H, dk, dv, N) = _cpu_prefill_inputs()
    bad = {"out": torch.zeros(T - 1, H, dv, dtype=torch.bfloat16),
           "final_state": torch.zeros(N, H, dk, dv - 1)}[which]
    with pytest.raises(ValueError, match=which):
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], cu_seqlens=inp["cu_seqlens"],
                      **{which: bad})
    with pytest.raises(RuntimeError, match="no CPU path"):  # right shapes: refused for the device
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], cu_seqlens=inp["cu_seqlens"])


@pytest.mark.parametrize("which", ["out", "S_out"])
def test_decode_rejects_wrong_output_shapes(which):
    import torch
    N, H, dk, dv = 3, 2, 32, 16
    q = torch.zeros(N, H, dk, dtype=torch.bfloat16)
    args = (q, q.clone(), torch.zeros(N, H, dv, dtype=torch.bfloat16), torch.zeros(N, H, dk), torch.zeros(N, H),
            torch.zeros(N, H, dk, dv))
    bad = {"out": torch.zeros(N, H, dv + 1, dtype=torch.bfloat16), "S_out": torch.zeros(N - 1, H, dk, dv)}[which]
    with pytest.raises(ValueError, match=which):
        kda.decode_step(*args, **{which: bad})
    with pytest.raises(RuntimeError, match="no CPU path"):
        kda.decode_step(*args)


def test_noalloc_rejects_beyond_its_scratch(lib):
    """kda_chunk_fwd_noalloc refuses, before touching a device, a two-pass call
    whose one-chunk segment does not fit its fixed scratch (4096 units x 37,376
    bytes > 128 MiB), and says so."""
    P = lambda x: ctypes.c_void_p(x)
    d = dims(num_seqs=1, num_heads=4096, total_tokens=64, method=2)
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(d), P(GOOD), P(GOOD), P(GOOD), P(GOOD), P(GOOD), None, P(GOOD),
                                   P(GOOD), P(GOOD), None)
    assert st == INVALID
    assert b"scratch" in lib.kda_last_error()
    # without S_T the running states count too: 1400 units x (64 KiB + 37,376 bytes) > 128 MiB
    d = dims(num_seqs=1, num_heads=1400, total_tokens=64, method=2)
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(d), P(GOOD), P(GOOD), P(GOOD), P(GOOD), P(GOOD), None, P(GOOD),
                                   P(GOOD), None, None)
    assert st == INVALID and b"S_T is NULL" in lib.kda_last_error()


def test_chunk_plan(lib):
    """kda_chunk_plan reports the configuration a prefill call would run, and
    the status it would return, without touching a device."""
    def plan(d, packed=1, ws=0):
        m, c, s = ctypes.c_int(-1), ctypes.c_int(-1), ctypes.c_int(-1)
        st = lib.kda_chunk_plan(ctypes.byref(d), packed, ctypes.c_size_t(ws), ctypes.byref(m), ctypes.byref(c),
                                ctypes.byref(s))
        return st, m.value, c.value, s.value
    d = dims(num_seqs=2, num_heads=32, total_tokens=2 * 32768, max_seqlen=32768)
    need = ctypes.c_size_t(0)
    assert lib.kda_chunk_workspace_size(ctypes.byref(d), ctypes.byref(need)) == OK
    assert plan(d, 0, need.value) == (OK, 2, 32, 4)        # the benchmark's call: two-pass, C = 32, dv split 4
    assert plan(d, 0, 0) == (OK, 1, 32, 4)                 # no workspace: single-pass
    assert plan(dims(qkv_dtype=0, dk=128, dv=128, num_heads=1), 1, 0)[:2] == (OK, 1)
    assert plan(dims(qkv_dtype=0, dk=128, dv=128, num_heads=1), 1, 0)[3] == 8   # fp32 at dk = 128: 16 columns
    assert plan(dims(method=2), 1, 0)[0] == INVALID        # two-pass without a workspace
    assert plan(dims(dk=48))[0] == UNSUPPORTED
    assert plan(dims(qkv_dtype=0, dk=128, dv=128, dv_split=4))[0] == UNSUPPORTED
    assert plan(dims(num_seqs=0, total_tokens=0)) == (OK, 1, 32, 0)
    m = ctypes.c_int(0)
    assert lib.kda_chunk_plan(ctypes.byref(dims()), 1, ctypes.c_size_t(0), ctypes.byref(m), None, None) == INVALID
