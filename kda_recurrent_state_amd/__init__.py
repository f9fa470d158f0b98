"""MI355X-native gated delta-rule (KDA / Gated DeltaNet) state layer.

Thin Python binding over the C ABI in ``include/kda.h`` (``libkda.so``, built
for gfx950 from ``csrc/``).  This module only marshals arguments: PyTorch
provides device memory and the current HIP stream; every step of the layer
runs in the library's HIP kernels.  There is no CPU or PyTorch fallback: if
the library or a GPU is missing, calls raise.

    o, S_T = chunk_fwd(q, k, v, log_a, beta, S0=None, cu_seqlens=None)
    o, S_T, snaps = chunk_fwd_snapshots(q, k, v, log_a, beta, S0, cu_seqlens,
                                        snapshot_every=1024)   # prefix states
    o, S   = decode_step(q, k, v, log_a, beta, S)        # S updated in place

Shapes (tokens of all sequences packed along the first axis):
    q, k [T, H, dk]; v [T, H, dv]; log_a [T, H, dk] (KDA) or [T, H] (Gated
    DeltaNet); beta [T, H]; states [N, H, dk, dv] float32.  q/k/v are bf16 or
    fp32 (o has the same dtype); log_a, beta and states are fp32.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # loads the HIP runtime the library then shares

__all__ = ["chunk_fwd", "chunk_fwd_snapshots", "snapshot_rows", "chunk_workspace_size", "chunk_plan", "chunk_bwd",
           "chunk_bwd_workspace_size", "decode_step", "KdaError", "library_path", "load_library",
           "METHOD_AUTO", "METHOD_SINGLE", "METHOD_TWO_PASS", "ORDER_ERASE_FIRST", "ORDER_DECAY_FIRST"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")
_lock = threading.Lock()
_lib = None

KDA_F32, KDA_BF16 = 0, 1


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class _Dims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32), ("scalar_decay", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("dv_split", ctypes.c_int32),
                ("method", ctypes.c_int32), ("order", ctypes.c_int32), ("max_seqlen", ctypes.c_int64)]


class _Prologue(ctypes.Structure):
    _fields_ = [("normalize_k", ctypes.c_int32), ("beta_logits", ctypes.c_int32), ("log_a_raw", ctypes.c_int32),
                ("log_a_min", ctypes.c_float)]


def _prologue(pro):
    """kda_prologue_t from a dict with keys normalize_k, beta_logits, log_a_raw,
    log_a_min (None: no prologue)."""
    if pro is None:
        return None
    unknown = set(pro) - {"normalize_k", "beta_logits", "log_a_raw", "log_a_min"}
    if unknown:
        raise ValueError(f"unknown prologue fields {sorted(unknown)}")
    lo = pro.get("log_a_min")
    return _Prologue(int(bool(pro.get("normalize_k"))), int(bool(pro.get("beta_logits"))),
                     int(bool(pro.get("log_a_raw"))), float("-inf") if lo is None else float(lo))


METHOD_AUTO, METHOD_SINGLE, METHOD_TWO_PASS = 0, 1, 2
# where the decay sits in the update (kda_order_t): the table's KDA row erases
# first, S <- Diag(a)(I - b k^T k) S + b k^T v; DECAY_FIRST is
# S <- (I - b k^T k) Diag(a) S + b k^T v.  Equal for a scalar decay.
ORDER_ERASE_FIRST, ORDER_DECAY_FIRST = 0, 1


def library_path() -> str:
    return _LIB_PATH


def load_library(build_if_missing: bool = True):
    """Load libkda.so (building it with hipcc first if it is absent)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                if not build_if_missing:
                    raise RuntimeError(f"{_LIB_PATH} is not built")
                from . import _build
                _build.build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            lib.kda_chunk_fwd.restype = ctypes.c_int
            lib.kda_chunk_fwd.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P, P, P, P,
                                          ctypes.c_size_t, P]
            lib.kda_chunk_fwd_ex.restype = ctypes.c_int
            lib.kda_chunk_fwd_ex.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Prologue), P, P, P, P, P, P, P,
                                             P, P, P, ctypes.c_int64, ctypes.c_int64, P, ctypes.c_size_t, P]
            lib.kda_decode_step_ex.restype = ctypes.c_int
            lib.kda_decode_step_ex.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Prologue), P, P, P, P, P, P,
                                               P, P, P]
            lib.kda_chunk_fwd_snapshots.restype = ctypes.c_int
            lib.kda_chunk_fwd_snapshots.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P, P, P, P,
                                                    ctypes.c_int64, ctypes.c_int64, P, ctypes.c_size_t, P]
            lib.kda_chunk_bwd.restype = ctypes.c_int
            lib.kda_chunk_bwd.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                          ctypes.c_size_t, P]
            lib.kda_chunk_bwd_ex.restype = ctypes.c_int
            lib.kda_chunk_bwd_ex.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Prologue), P, P, P, P, P, P, P,
                                             P, ctypes.c_int64, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
            lib.kda_chunk_bwd_ex_workspace_size.restype = ctypes.c_int
            lib.kda_chunk_bwd_ex_workspace_size.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Prologue),
                                                            ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
            lib.kda_chunk_bwd_saved.restype = ctypes.c_int
            lib.kda_chunk_bwd_saved.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P, P, ctypes.c_int64, P,
                                                P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
            for name in ("kda_chunk_workspace_size", "kda_chunk_workspace_min", "kda_chunk_bwd_workspace_size",
                         "kda_chunk_bwd_saved_workspace_size"):
                fn = getattr(lib, name)
                fn.restype = ctypes.c_int
                fn.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(ctypes.c_size_t)]
            lib.kda_chunk_plan.restype = ctypes.c_int
            lib.kda_chunk_plan.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int, ctypes.c_size_t,
                                           ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                           ctypes.POINTER(ctypes.c_int)]
            lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
            lib.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P, P, P, P]
            lib.kda_decode_step.restype = ctypes.c_int
            lib.kda_decode_step.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P, P, P]
            lib.kda_status_string.restype = ctypes.c_char_p
            lib.kda_status_string.argtypes = [ctypes.c_int]
            lib.kda_last_error.restype = ctypes.c_char_p
            lib.kda_last_error.argtypes = []
            lib.kda_version.restype = ctypes.c_int
            _lib = lib
        return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, ndim=None, shape=None):
    """Type, dtype, rank, exact shape and layout of one argument.  The library
    cannot see tensor sizes, so every buffer it writes is checked here."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got {tuple(t.shape)})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(ref, **tensors):
    """Every tensor on ref's HIP device (checked after all shapes)."""
    if ref.device.type != "cuda":
        raise RuntimeError(f"tensors must be on a HIP device (got {ref.device}); there is no CPU path")
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise RuntimeError(f"{name} is on {t.device}, not on {ref.device}")


def _check(lib, status):
    if status != 0:
        msg = lib.kda_last_error().decode() or lib.kda_status_string(status).decode()
        raise KdaError(status, msg)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32 (got {t.dtype})")


def _stream_handle(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def chunk_fwd(q, k, v, log_a, beta, S0=None, cu_seqlens=None, *, chunk_size: int = 0,
              dv_split: int = 0, out=None, final_state=True, num_seqs: int | None = None,
              method: int = METHOD_AUTO, workspace=None, max_seqlen: int | None = None,
              order: int = ORDER_ERASE_FIRST, prologue: dict | None = None):
    """Chunked prefill over packed sequences; returns (o, S_T or None).

    cu_seqlens: int32 device tensor [N+1], or None for num_seqs (default 1)
    sequences of equal length.  final_state=False skips S_T; passing a tensor
    writes S_T into it (it may be S0 itself).

    method: METHOD_AUTO, METHOD_SINGLE or METHOD_TWO_PASS.  The two-pass method
    needs device scratch: pass a uint8 tensor as `workspace`, or leave it None
    to have one of the library's preferred size allocated (torch's caching
    allocator) for this call.  max_seqlen bounds the longest sequence (with
    cu_seqlens); when None it is read from cu_seqlens, which synchronises.
    order: ORDER_ERASE_FIRST or ORDER_DECAY_FIRST.
    prologue: None, or a dict of kda_prologue_t fields (normalize_k, beta_logits,
    log_a_raw, log_a_min) transforming raw k, beta logits and log-decay
    pre-activations on load (two-pass prefill only)."""
    o, ST, _ = _prefill(q, k, v, log_a, beta, S0, cu_seqlens, chunk_size, dv_split, out, final_state,
                        num_seqs, method, workspace, max_seqlen, 0, None, order, prologue)
    return o, ST


def snapshot_rows(cu_seqlens, snapshot_every: int, *, total_tokens: int | None = None,
                  num_seqs: int | None = None) -> int:
    """Rows of the snapshot buffer a call needs: the sum over sequences of
    floor(len / snapshot_every).  From cu_seqlens (read on the host, which
    synchronises when it is a device tensor) or from equal lengths
    total_tokens / num_seqs."""
    L = int(snapshot_every)
    if L <= 0:
        raise ValueError("snapshot_every must be > 0")
    if cu_seqlens is None:
        n = 1 if num_seqs is None else int(num_seqs)
        return 0 if n == 0 else n * ((int(total_tokens) // n) // L)
    cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    return sum((b - a) // L for a, b in zip(cu[:-1], cu[1:]))


def chunk_fwd_snapshots(q, k, v, log_a, beta, S0=None, cu_seqlens=None, *, snapshot_every: int,
                        snapshots=None, chunk_size: int = 0, dv_split: int = 0, out=None, final_state=True,
                        num_seqs: int | None = None, method: int = METHOD_AUTO, workspace=None,
                        max_seqlen: int | None = None, order: int = ORDER_ERASE_FIRST,
                        prologue: dict | None = None):
    """chunk_fwd that also returns the state after every `snapshot_every` tokens
    of each sequence: (o, S_T or None, snapshots [R, H, dk, dv] float32).

    Sequence n contributes floor(len_n / snapshot_every) rows, in sequence
    order; its row s is the state after its first (s + 1) * snapshot_every
    tokens.  snapshot_every must be a multiple of the chunk size.  Pass a
    float32 tensor as `snapshots` to choose R (rows past R are not written),
    or leave it None to allocate exactly the rows needed (snapshot_rows, which
    reads cu_seqlens on the host)."""
    _need(q, "q", ndim=3)
    T, H, dk = q.shape
    dv = v.shape[2]
    if snapshots is None:
        N = (cu_seqlens.shape[0] - 1) if cu_seqlens is not None else (1 if num_seqs is None else int(num_seqs))
        R = snapshot_rows(cu_seqlens, snapshot_every, total_tokens=T, num_seqs=N)
        snapshots = torch.empty((R, H, dk, dv), dtype=torch.float32, device=q.device)
    else:
        _need(snapshots, "snapshots", torch.float32, 4)
        if snapshots.shape[1:] != (H, dk, dv):
            raise ValueError(f"snapshots must be [R,{H},{dk},{dv}] (got {tuple(snapshots.shape)})")
    return _prefill(q, k, v, log_a, beta, S0, cu_seqlens, chunk_size, dv_split, out, final_state, num_seqs,
                    method, workspace, max_seqlen, int(snapshot_every), snapshots, order, prologue)


def chunk_fwd_noalloc(q, k, v, log_a, beta, S0=None, cu_seqlens=None, *, chunk_size: int = 0,
                      dv_split: int = 0, out=None, final_state=True, num_seqs: int | None = None,
                      method: int = METHOD_AUTO, max_seqlen: int | None = None, order: int = ORDER_ERASE_FIRST):
    """chunk_fwd through kda_chunk_fwd_noalloc: the library allocates nothing and
    takes its two-pass workspace from a fixed device array (KDA_NOALLOC_SCRATCH_BYTES,
    128 MiB per GPU).  Outputs are allocated here unless `out` / `final_state`
    tensors are passed.  Calls that overlap on one GPU share that array and race."""
    o, ST, _ = _prefill(q, k, v, log_a, beta, S0, cu_seqlens, chunk_size, dv_split, out, final_state, num_seqs,
                        method, None, max_seqlen, 0, None, order, None, noalloc=True)
    return o, ST


def _prefill(q, k, v, log_a, beta, S0, cu_seqlens, chunk_size, dv_split, out, final_state, num_seqs,
             method, workspace, max_seqlen, snapshot_every, snapshots, order, prologue, noalloc=False):
    lib = load_library()
    _need(q, "q", ndim=3)
    T, H, dk = q.shape
    _need(k, "k", q.dtype, 3)
    _need(v, "v", q.dtype, 3)
    dv = v.shape[2]
    if k.shape != q.shape or v.shape[:2] != (T, H):
        raise ValueError("q, k, v shapes disagree")
    _need(log_a, "log_a", torch.float32)
    if log_a.shape == (T, H, dk):
        scalar = 0
    elif log_a.shape == (T, H):
        scalar = 1
    else:
        raise ValueError(f"log_a must be [T,H,dk] or [T,H] (got {tuple(log_a.shape)})")
    _need(beta, "beta", torch.float32)
    if beta.shape != (T, H):
        raise ValueError("beta must be [T,H]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
        N = cu_seqlens.shape[0] - 1
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    if S0 is not None:
        _need(S0, "S0", torch.float32)
        if S0.shape != (N, H, dk, dv):
            raise ValueError(f"S0 must be [{N},{H},{dk},{dv}] (got {tuple(S0.shape)})")
    if out is not None:
        _need(out, "out", q.dtype, shape=(T, H, dv))
    if isinstance(final_state, torch.Tensor):
        _need(final_state, "final_state", torch.float32, shape=(N, H, dk, dv))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
    _same_device(q, k=k, v=v, log_a=log_a, beta=beta, S0=S0, cu_seqlens=cu_seqlens, out=out,
                 final_state=final_state if isinstance(final_state, torch.Tensor) else None,
                 snapshots=snapshots, workspace=workspace)
    o = out if out is not None else torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if isinstance(final_state, torch.Tensor):
        ST = final_state
    elif final_state:
        ST = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    else:
        ST = None
    if max_seqlen is None:
        if cu_seqlens is not None and N > 0 and method != METHOD_SINGLE:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item())
        else:
            max_seqlen = 0
    d = _Dims(N, H, T, dk, dv, _dtype_code(q), scalar, int(chunk_size), int(dv_split), int(method), int(order),
              int(max_seqlen))
    if noalloc:
        st = lib.kda_chunk_fwd_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(beta),
                                       _ptr(S0), _ptr(cu_seqlens), _ptr(o), _ptr(ST), _stream_handle(q.device))
        _check(lib, st)
        return o, ST, None
    if workspace is None and method != METHOD_SINGLE:
        need = ctypes.c_size_t(0)
        _check(lib, lib.kda_chunk_workspace_size(ctypes.byref(d), ctypes.byref(need)))
        if need.value > 0:
            workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    ws_bytes = ctypes.c_size_t(0 if workspace is None else workspace.numel())
    pro = _prologue(prologue)
    if pro is not None:
        rows = 0 if snapshots is None else snapshots.shape[0]
        st = lib.kda_chunk_fwd_ex(ctypes.byref(d), ctypes.byref(pro), _ptr(q), _ptr(k), _ptr(v), _ptr(log_a),
                                  _ptr(beta), _ptr(S0), _ptr(cu_seqlens), _ptr(o), _ptr(ST),
                                  _ptr(snapshots) if rows > 0 else None, ctypes.c_int64(rows),
                                  ctypes.c_int64(snapshot_every if rows > 0 else 0), _ptr(workspace), ws_bytes,
                                  _stream_handle(q.device))
    elif snapshots is None:
        st = lib.kda_chunk_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(beta),
                               _ptr(S0), _ptr(cu_seqlens), _ptr(o), _ptr(ST), _ptr(workspace), ws_bytes,
                               _stream_handle(q.device))
    else:
        rows = snapshots.shape[0]
        st = lib.kda_chunk_fwd_snapshots(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(beta),
                                         _ptr(S0), _ptr(cu_seqlens), _ptr(o), _ptr(ST),
                                         _ptr(snapshots) if rows > 0 else None, ctypes.c_int64(rows),
                                         ctypes.c_int64(snapshot_every), _ptr(workspace), ws_bytes,
                                         _stream_handle(q.device))
    _check(lib, st)
    return o, ST, snapshots


def chunk_workspace_size(q, v, *, num_seqs=1, scalar_decay=False, chunk_size=0, dv_split=0,
                         method=METHOD_AUTO, max_seqlen=0, minimum=False, order=ORDER_ERASE_FIRST):
    """Bytes of workspace the prefill prefers (or, minimum=True, needs) for these
    shapes; 0 when it would run single-pass."""
    lib = load_library()
    T, H, dk = q.shape
    d = _Dims(int(num_seqs), H, T, dk, v.shape[2], _dtype_code(q), int(bool(scalar_decay)), int(chunk_size),
              int(dv_split), int(method), int(order), int(max_seqlen))
    need = ctypes.c_size_t(0)
    fn = lib.kda_chunk_workspace_min if minimum else lib.kda_chunk_workspace_size
    _check(lib, fn(ctypes.byref(d), ctypes.byref(need)))
    return need.value


def chunk_plan(q, v, *, num_seqs=1, packed=True, workspace_bytes=0, scalar_decay=False, chunk_size=0, dv_split=0,
               method=METHOD_AUTO, max_seqlen=0, order=ORDER_ERASE_FIRST):
    """The configuration chunk_fwd would run for these shapes and workspace size:
    (method, chunk, dv_split), method METHOD_SINGLE or METHOD_TWO_PASS."""
    lib = load_library()
    T, H, dk = q.shape
    d = _Dims(int(num_seqs), H, T, dk, v.shape[2], _dtype_code(q), int(bool(scalar_decay)), int(chunk_size),
              int(dv_split), int(method), int(order), int(max_seqlen))
    m, c, s = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(lib, lib.kda_chunk_plan(ctypes.byref(d), int(bool(packed)), ctypes.c_size_t(int(workspace_bytes)),
                                   ctypes.byref(m), ctypes.byref(c), ctypes.byref(s)))
    return m.value, c.value, s.value


def chunk_bwd(q, k, v, log_a, beta, dO, S0=None, cu_seqlens=None, dS_T=None, *, chunk_size: int = 0,
              dv_split: int = 0, num_seqs: int | None = None, method: int = METHOD_AUTO, workspace=None,
              max_seqlen: int | None = None, initial_state_grad=True, states=None, prologue: dict | None = None,
              order: int = ORDER_ERASE_FIRST):
    """Gradient of chunk_fwd (in the order `order`) for upstream derivatives dO
    [T,H,dv] (and dS_T [N,H,dk,dv], None for zero).  Returns a dict with "dq",
    "dk" [T,H,dk] and "dv" [T,H,dv] in q's dtype, "dlog_a" (log_a's shape) and
    "dbeta" [T,H] in float32, and "dS0" [N,H,dk,dv] float32 (None when
    initial_state_grad is False).  The forward inputs are passed again.

    states: the forward's states at every 64th token, [R,H,dk,dv] float32 as
    chunk_fwd_snapshots(..., snapshot_every=64) returns them; the call then
    runs no prefill of its own (kda_chunk_bwd_saved).  None: the call reruns
    the prefill to recover them, and chunk_size, dv_split and method choose that
    rerun.  prologue: the input prologue the forward ran (chunk_fwd's
    prologue); k, log_a and beta are then the raw inputs and dk, dlog_a, dbeta
    the derivatives with respect to them (kda_chunk_bwd_ex).  workspace: a
    uint8 tensor of at least chunk_bwd_workspace_size(saved=states is not None,
    prologue=prologue) bytes, or None to have one allocated."""
    lib = load_library()
    _need(q, "q", ndim=3)
    T, H, dk = q.shape
    _need(k, "k", q.dtype, 3)
    _need(v, "v", q.dtype, 3)
    dv = v.shape[2]
    if k.shape != q.shape or v.shape[:2] != (T, H):
        raise ValueError("q, k, v shapes disagree")
    _need(log_a, "log_a", torch.float32)
    if log_a.shape == (T, H, dk):
        scalar = 0
    elif log_a.shape == (T, H):
        scalar = 1
    else:
        raise ValueError(f"log_a must be [T,H,dk] or [T,H] (got {tuple(log_a.shape)})")
    _need(beta, "beta", torch.float32)
    if beta.shape != (T, H):
        raise ValueError("beta must be [T,H]")
    _need(dO, "dO", q.dtype, 3)
    if dO.shape != v.shape:
        raise ValueError("dO must have v's shape")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
        N = cu_seqlens.shape[0] - 1
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    for name, x in (("S0", S0), ("dS_T", dS_T)):
        if x is not None:
            _need(x, name, torch.float32)
            if x.shape != (N, H, dk, dv):
                raise ValueError(f"{name} must be [{N},{H},{dk},{dv}] (got {tuple(x.shape)})")
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
    saved = states is not None
    if saved:
        _need(states, "states", torch.float32, 4)
        if states.shape[1:] != (H, dk, dv):
            raise ValueError(f"states must be [R,{H},{dk},{dv}] (got {tuple(states.shape)})")
        rows = snapshot_rows(cu_seqlens, 64, total_tokens=T, num_seqs=N)
        if states.shape[0] < rows:
            raise ValueError(f"states holds {states.shape[0]} rows, the sequences need {rows}")
    _same_device(q, k=k, v=v, log_a=log_a, beta=beta, dO=dO, S0=S0, dS_T=dS_T, cu_seqlens=cu_seqlens,
                 workspace=workspace, states=states)
    if max_seqlen is None:
        if cu_seqlens is not None and N > 0:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item())
        else:
            max_seqlen = 0
    d = _Dims(N, H, T, dk, dv, _dtype_code(q), scalar, int(chunk_size), int(dv_split), int(method),
              int(order), int(max_seqlen))
    pro = _prologue(prologue)
    if workspace is None:
        need = ctypes.c_size_t(0)
        if pro is not None:
            _check(lib, lib.kda_chunk_bwd_ex_workspace_size(ctypes.byref(d), ctypes.byref(pro), int(saved),
                                                            ctypes.byref(need)))
        else:
            size_fn = lib.kda_chunk_bwd_saved_workspace_size if saved else lib.kda_chunk_bwd_workspace_size
            _check(lib, size_fn(ctypes.byref(d), ctypes.byref(need)))
        workspace = torch.empty(max(need.value, 256), dtype=torch.uint8, device=q.device)
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dlog_a": torch.empty_like(log_a), "dbeta": torch.empty_like(beta),
           "dS0": torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device) if initial_state_grad else None}
    grads = (_ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_a"]), _ptr(out["dbeta"]),
             _ptr(out["dS0"]), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream_handle(q.device))
    if pro is not None:
        st = lib.kda_chunk_bwd_ex(ctypes.byref(d), ctypes.byref(pro), _ptr(q), _ptr(k), _ptr(v), _ptr(log_a),
                                  _ptr(beta), _ptr(S0), _ptr(cu_seqlens), _ptr(states),
                                  ctypes.c_int64(states.shape[0] if saved else 0), _ptr(dO), _ptr(dS_T), *grads)
    elif saved:
        st = lib.kda_chunk_bwd_saved(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(beta),
                                     _ptr(S0), _ptr(cu_seqlens), _ptr(states), ctypes.c_int64(states.shape[0]),
                                     _ptr(dO), _ptr(dS_T), *grads)
    else:
        st = lib.kda_chunk_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(beta), _ptr(S0),
                               _ptr(cu_seqlens), _ptr(dO), _ptr(dS_T), *grads)
    _check(lib, st)
    return out


def chunk_bwd_workspace_size(q, v, *, num_seqs=1, scalar_decay=False, chunk_size=0, dv_split=0,
                             method=METHOD_AUTO, max_seqlen=0, saved=False, prologue: dict | None = None,
                             order: int = ORDER_ERASE_FIRST):
    """Bytes of workspace chunk_bwd needs for these shapes (saved=True: with the
    forward's states passed in, so without the prefill rerun; prologue: the
    input prologue the forward ran)."""
    lib = load_library()
    T, H, dk = q.shape
    d = _Dims(int(num_seqs), H, T, dk, v.shape[2], _dtype_code(q), int(bool(scalar_decay)), int(chunk_size),
              int(dv_split), int(method), int(order), int(max_seqlen))
    need = ctypes.c_size_t(0)
    pro = _prologue(prologue)
    if pro is not None:
        _check(lib, lib.kda_chunk_bwd_ex_workspace_size(ctypes.byref(d), ctypes.byref(pro), int(bool(saved)),
                                                        ctypes.byref(need)))
    else:
        fn = lib.kda_chunk_bwd_saved_workspace_size if saved else lib.kda_chunk_bwd_workspace_size
        _check(lib, fn(ctypes.byref(d), ctypes.byref(need)))
    return need.value


def decode_step(q, k, v, log_a, beta, S, *, out=None, S_out=None, order: int = ORDER_ERASE_FIRST,
                prologue: dict | None = None):
    """One token per sequence: q, k [N,H,dk], v [N,H,dv], log_a [N,H,dk] or
    [N,H], beta [N,H], S [N,H,dk,dv].  Updates S in place unless S_out is
    given; returns (o, state_after)."""
    lib = load_library()
    _need(q, "q", ndim=3)
    N, H, dk = q.shape
    _need(k, "k", q.dtype, 3)
    _need(v, "v", q.dtype, 3)
    dv = v.shape[2]
    _need(log_a, "log_a", torch.float32)
    if log_a.shape == (N, H, dk):
        scalar = 0
    elif log_a.shape == (N, H):
        scalar = 1
    else:
        raise ValueError("log_a must be [N,H,dk] or [N,H]")
    _need(beta, "beta", torch.float32)
    _need(S, "S", torch.float32)
    if S.shape != (N, H, dk, dv) or k.shape != q.shape or v.shape[:2] != (N, H) or beta.shape != (N, H):
        raise ValueError("decode shapes disagree")
    if S_out is not None:
        _need(S_out, "S_out", torch.float32, shape=(N, H, dk, dv))
    if out is not None:
        _need(out, "out", q.dtype, shape=(N, H, dv))
    _same_device(q, k=k, v=v, log_a=log_a, beta=beta, S=S, S_out=S_out, out=out)
    So = S if S_out is None else S_out
    o = out if out is not None else torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    d = _Dims(N, H, N, dk, dv, _dtype_code(q), scalar, 0, 0, 0, int(order), 0)
    pro = _prologue(prologue)
    if pro is not None:
        st = lib.kda_decode_step_ex(ctypes.byref(d), ctypes.byref(pro), _ptr(q), _ptr(k), _ptr(v), _ptr(log_a),
                                    _ptr(beta), _ptr(S), _ptr(So), _ptr(o), _stream_handle(q.device))
    else:
        st = lib.kda_decode_step(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(beta),
                                 _ptr(S), _ptr(So), _ptr(o), _stream_handle(q.device))
    _check(lib, st)
    return o, So
