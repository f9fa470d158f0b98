"""fp64 CPU oracle for the gated delta-rule (KDA / Gated DeltaNet) state layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product (the HIP
library and its Python binding) never imports, links or calls anything here,
and this package shares no code with it.

The arithmetic lives in ``kda_oracle.c``: a token-by-token recurrence in double
precision that follows the KDA / Gated DeltaNet / delta-rule rows of the table
"Everything, in one table" on the page "The argument, in one page".  This module
only marshals arrays into it (upcasting every input exactly to float64) and
builds it with the system C compiler.

Pinned by ``tests/test_oracle.py`` (worked example, closed forms, brute-force
matrix products, exact rational arithmetic, orthonormal recall, reductions to
linear attention and to a scalar first-order recurrence, linearity, continuation)
and ``tests/test_oracle_mutants.py`` (planted mistakes must fail a pin).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, no fast-math: IEEE double semantics)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-pthread", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load_library(path: str | None = None):
    """Load (building first if absent) an oracle shared library."""
    global _lib
    if path is not None:
        lib = ctypes.CDLL(path)
        _declare(lib)
        return lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = ctypes.CDLL(_LIB)
            _declare(_lib)
        return _lib


def _declare(lib) -> None:
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.kda_oracle_fwd.restype = ctypes.c_int
    lib.kda_oracle_fwd.argtypes = [I64, P, I64, I64, I64, P, P, P, P, ctypes.c_int, P, P,
                                   ctypes.c_int, P, P, ctypes.c_int]
    if hasattr(lib, "kda_oracle_bwd"):
        lib.kda_oracle_bwd.restype = ctypes.c_int
        lib.kda_oracle_bwd.argtypes = [I64, P, I64, I64, I64, P, P, P, P, ctypes.c_int, P, P,
                                       ctypes.c_int, P, P, P, P, P, P, P, P, ctypes.c_int]


MAX_THREADS = 16  # the host CPU share that goes with one GPU


def default_threads() -> int:
    """Threads of the oracle's pool: the CPUs this process may run on, at most
    MAX_THREADS (a machine shared by several GPUs grants each that many)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_THREADS))


def _f64(x) -> np.ndarray:
    """Exact upcast to a contiguous float64 array (bf16/fp32 -> fp64 is exact)."""
    if hasattr(x, "detach"):  # torch tensor (possibly bf16, possibly on a device)
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


# Prologue of the layer's inputs.  The pages fix no gate parameterisation; these
# are the transforms that turn a layer's raw projections into the recurrence's
# inputs in the usual learned gates (and in this project's input recipe): unit
# keys, a logistic write strength, a negative-softplus log-decay.
PROLOGUE_EPS = 1e-6


def prologue(k, log_a, beta, normalize_k=False, beta_logits=False, log_a_raw=False, log_a_min=None):
    """Apply the input prologue in fp64 and return (k, log_a, beta) as float64:
      normalize_k:  k_t <- k_t / sqrt(sum_c k_tc^2 + PROLOGUE_EPS), per token and head
      beta_logits:  beta_t <- 1 / (1 + exp(-beta_t))
      log_a_raw:    log_a <- -softplus(log_a) = -(max(x, 0) + log(1 + exp(-|x|))),
                    then clipped from below at log_a_min when that is given."""
    k, log_a, beta = _f64(k), _f64(log_a), _f64(beta)
    if normalize_k:
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + PROLOGUE_EPS)
    if beta_logits:
        beta = 1.0 / (1.0 + np.exp(-beta))
    if log_a_raw:
        log_a = -(np.maximum(log_a, 0.0) + np.log1p(np.exp(-np.abs(log_a))))
        if log_a_min is not None:
            log_a = np.maximum(log_a, float(log_a_min))
    return k, log_a, beta


def kda_oracle(q, k, v, log_a, beta, S0=None, cu_seqlens=None, order: int = 0,
               threads: int | None = None, lib=None, pro: dict | None = None):
    """Run the fp64 recurrence.

    q, k: [T, H, dk]; v: [T, H, dv]; log_a: [T, H, dk] (per channel) or [T, H]
    (scalar decay); beta: [T, H]; S0: [N, H, dk, dv] or None (zeros);
    cu_seqlens: [N+1] int offsets, or None for a single sequence of length T.
    order 0 is the table's KDA row (erase, decay, write); 1 is decay-first.

    pro: keyword arguments of prologue(), applied to the inputs first.

    Returns (o [T, H, dv], S_T [N, H, dk, dv]) as float64 arrays.
    """
    q, k, v, log_a, beta = (_f64(x) for x in (q, k, v, log_a, beta))
    if pro:
        k, log_a, beta = prologue(k, log_a, beta, **pro)
    T, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("inconsistent shapes")
    if log_a.shape == (T, H, dk):
        scalar = 0
    elif log_a.shape == (T, H):
        scalar = 1
    else:
        raise ValueError("log_a must be [T,H,dk] or [T,H]")
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    if cu[-1] != T:
        raise ValueError("cu_seqlens[-1] must equal T")
    s0 = None
    if S0 is not None:
        s0 = _f64(S0)
        if s0.shape != (N, H, dk, dv):
            raise ValueError("S0 must be [N,H,dk,dv]")
    o = np.zeros((T, H, dv), dtype=np.float64)
    ST = np.zeros((N, H, dk, dv), dtype=np.float64)
    nt = threads if threads is not None else default_threads()
    L = lib if lib is not None else load_library()
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = L.kda_oracle_fwd(N, ptr(cu), H, dk, dv, ptr(q), ptr(k), ptr(v), ptr(log_a), scalar,
                          ptr(beta), ptr(s0), int(order), ptr(o), ptr(ST), int(nt))
    if rc != 0:
        raise RuntimeError("kda_oracle_fwd failed with code %d" % rc)
    return o, ST


def prologue_bwd(k, log_a, beta, grads, normalize_k=False, beta_logits=False, log_a_raw=False, log_a_min=None):
    """Chain rule through prologue(): given the raw inputs (k, log_a, beta) and
    the derivatives "dk", "dlog_a", "dbeta" with respect to the transformed
    ones, return a copy of grads with those three taken with respect to the raw
    inputs (fp64):
      normalize_k:  with n = sqrt(|x|^2 + eps) and u = x / n,  dx = (du - u (u . du)) / n
      beta_logits:  with b = 1 / (1 + e^-z),                   dz = db b (1 - b)
      log_a_raw:    with y the pre-activation,                 dy = dlog_a (-1 / (1 + e^-y)),
                    and 0 where the clip at log_a_min is active (-softplus(y) < log_a_min)."""
    k, log_a, beta = _f64(k), _f64(log_a), _f64(beta)
    out = dict(grads)
    if normalize_k:
        n = np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + PROLOGUE_EPS)
        u, du = k / n, np.asarray(grads["dk"], dtype=np.float64)
        out["dk"] = (du - u * np.sum(u * du, axis=-1, keepdims=True)) / n
    if beta_logits:
        b = 1.0 / (1.0 + np.exp(-beta))
        out["dbeta"] = np.asarray(grads["dbeta"], dtype=np.float64) * b * (1.0 - b)
    if log_a_raw:
        d = -np.asarray(grads["dlog_a"], dtype=np.float64) / (1.0 + np.exp(-log_a))
        if log_a_min is not None:
            y = -(np.maximum(log_a, 0.0) + np.log1p(np.exp(-np.abs(log_a))))
            d = np.where(y >= float(log_a_min), d, 0.0)
        out["dlog_a"] = d
    return out


def kda_oracle_bwd(q, k, v, log_a, beta, S0=None, cu_seqlens=None, dO=None, dST=None,
                   order: int = 0, threads: int | None = None, lib=None, pro: dict | None = None):
    """Gradient of kda_oracle in fp64.

    For a scalar loss whose derivatives with respect to kda_oracle's outputs are
    dO [T, H, dv] and dST [N, H, dk, dv] (None: zero), return a dict with the
    derivatives with respect to its inputs: "dq", "dk" [T, H, dk], "dv" [T, H, dv],
    "dlog_a" (the shape of log_a), "dbeta" [T, H] and "dS0" [N, H, dk, dv], as
    float64 arrays.  The walk is the chain rule applied to one token's update at a
    time, backwards from the last token (kda_oracle.c, kda_oracle_bwd).

    pro: keyword arguments of prologue(): k, log_a and beta are then raw inputs,
    transformed first, and their derivatives are taken through the transforms
    (prologue_bwd).
    """
    if pro:
        raw = (_f64(k), _f64(log_a), _f64(beta))
        k, log_a, beta = prologue(*raw, **pro)
        g = kda_oracle_bwd(q, k, v, log_a, beta, S0=S0, cu_seqlens=cu_seqlens, dO=dO, dST=dST, order=order,
                           threads=threads, lib=lib)
        return prologue_bwd(*raw, g, **pro)
    q, k, v, log_a, beta = (_f64(x) for x in (q, k, v, log_a, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("inconsistent shapes")
    if log_a.shape == (T, H, dk):
        scalar = 0
    elif log_a.shape == (T, H):
        scalar = 1
    else:
        raise ValueError("log_a must be [T,H,dk] or [T,H]")
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    if cu[-1] != T:
        raise ValueError("cu_seqlens[-1] must equal T")
    s0 = None if S0 is None else _f64(S0)
    if s0 is not None and s0.shape != (N, H, dk, dv):
        raise ValueError("S0 must be [N,H,dk,dv]")
    do = np.zeros((T, H, dv)) if dO is None else _f64(dO)
    if do.shape != (T, H, dv):
        raise ValueError("dO must be [T,H,dv]")
    dst = None if dST is None else _f64(dST)
    if dst is not None and dst.shape != (N, H, dk, dv):
        raise ValueError("dST must be [N,H,dk,dv]")
    out = {"dq": np.zeros((T, H, dk)), "dk": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
           "dlog_a": np.zeros(log_a.shape), "dbeta": np.zeros((T, H)),
           "dS0": np.zeros((N, H, dk, dv))}
    nt = threads if threads is not None else default_threads()
    L = lib if lib is not None else load_library()
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = L.kda_oracle_bwd(N, ptr(cu), H, dk, dv, ptr(q), ptr(k), ptr(v), ptr(log_a), scalar,
                          ptr(beta), ptr(s0), int(order), ptr(do), ptr(dst), ptr(out["dq"]),
                          ptr(out["dk"]), ptr(out["dv"]), ptr(out["dlog_a"]), ptr(out["dbeta"]),
                          ptr(out["dS0"]), int(nt))
    if rc != 0:
        raise RuntimeError("kda_oracle_bwd failed with code %d" % rc)
    return out
