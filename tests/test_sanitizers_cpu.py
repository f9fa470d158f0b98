"""CPU-only sanitizer builds (AddressSanitizer and UndefinedBehaviorSanitizer):
the fp64 oracle (oracle/kda_oracle.c, built with gcc) and the host side of the
C-ABI library (kda_api.cpp, host code instrumented, device code as usual),
each driven by a small program under tests/sanitize/ that exercises its index
arithmetic and argument checks.  No GPU is used: the API driver only makes calls
that the host validation refuses or that have nothing to do."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(ROOT, "kda_recurrent_state_amd", "_build")
HIPCC = "/opt/rocm/bin/hipcc"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _check_clean(r):
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    return tmp_path_factory.mktemp("san")


def test_oracle_under_asan_ubsan(outdir):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = os.path.join(outdir, "oracle_check")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-pthread", os.path.join(ROOT, "oracle", "kda_oracle.c"), os.path.join(SAN, "oracle_check.c"), "-lm",
          "-o", exe])
    r = _run([exe], env=ENV)
    _check_clean(r)
    assert "oracle sanitizer check ok" in r.stdout


def test_api_host_validation_under_asan_ubsan(outdir):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from kda_recurrent_state_amd import _build as library_build
    kernels = [os.path.splitext(f)[0] for f in library_build.SOURCES if f.endswith(".hip")]
    objs = [os.path.join(BUILD, k + ".o") for k in kernels]
    if not all(os.path.exists(o) for o in objs):
        from kda_recurrent_state_amd import _build
        _build.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    api_o, chk_o, exe = (os.path.join(outdir, n) for n in ("api.o", "check.o", "api_check"))
    _run([HIPCC, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san, "-I" + os.path.join(ROOT, "include"),
          "-c", os.path.join(ROOT, "kda_recurrent_state_amd", "csrc", "kda_api.cpp"), "-o", api_o])
    _run([HIPCC, "-O1", "-g", "-std=c++17", *san, "-I" + os.path.join(ROOT, "include"),
          "-c", os.path.join(SAN, "api_check.cpp"), "-o", chk_o])
    _run([HIPCC, "--offload-arch=gfx950", *san, chk_o, api_o, *objs, "-o", exe])
    r = _run([exe], env=ENV)
    _check_clean(r)
    assert "api sanitizer check ok" in r.stdout
