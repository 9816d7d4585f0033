"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two drivers, built here with the sanitizers and run:
  * tests/sanitize/oracle_driver.c with oracle/oracle.c (gcc): every oracle
    entry point on small ragged shapes, heap buffers of exactly the documented
    sizes;
  * tests/sanitize/abi_driver.c with the library's sources (hipcc, sanitizers
    on the host side only; the device code is built as usual and never run):
    every validation path of the C ABI, which returns before any HIP call.
Any out-of-bounds access, leak in the oracle, or undefined behaviour fails the
run (-fno-sanitize-recover).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "invariant_selected_token_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer", *SANITIZE,
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="no ROCm compilers")
def test_abi_validation_under_sanitizers(tmp_path):
    host_san = []
    for f in SANITIZE:          # host code only: each flag behind -Xarch_host
        host_san += ["-Xarch_host", f]
    hip = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC, *host_san]
    objs = []
    for src in ("kernels.hip", "api.hip"):
        o = str(tmp_path / (src + ".o"))
        _run([*hip, "-c", os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    d = str(tmp_path / "abi_driver.o")
    _run([CLANG, "-O1", "-g", *SANITIZE, "-I", INCLUDE, "-c", os.path.join(SAN, "abi_driver.c"),
          "-o", d])
    exe = str(tmp_path / "abi_san")
    _run([CLANGXX, *SANITIZE, *objs, d, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # leaks of the HIP runtime at exit are not ours
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert "all statuses as documented" in r.stdout
