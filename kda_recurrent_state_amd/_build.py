"""Compile the HIP library (gfx950) in place: kda_recurrent_state_amd/libkda.so.

Every source is compiled by hipcc for gfx950 only, in parallel, then linked
into one shared library with a plain C ABI (include/kda.h).  Packed-fp32
instruction selection is turned off for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_chunk.hip", "kda_prep.hip", "kda_prep2.hip", "kda_scan.hip",
           "kda_bwd.hip", "kda_bwd_pro.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=fast",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fvisibility=hidden", "-Wno-unused-result", "-I" + os.path.join(os.path.dirname(HERE), "include")]
# The state pass runs one workgroup per compute unit, so each wavefront may use
# accumulator registers on top of its 256 vector registers; left to itself the
# compiler then keeps matrix-core results there and copies the state back and
# forth every chunk.  This keeps them in vector registers (the walk fits).
EXTRA = {"kda_scan.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         # the gradient pass holds a state and its derivative per wavefront; in this
         # form it fits without spilling to scratch memory at dk = dv = 128
         "kda_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmd = [hipcc, *lang, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")
        return obj

    with ThreadPoolExecutor(max_workers=jobs or min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
