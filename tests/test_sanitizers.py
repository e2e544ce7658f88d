"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU): the C oracle, run on
small inputs and through its error returns, and the C-ABI library's host side (argument checks,
workspace queries, status strings), driven through every error path.  Device code is built
without instrumentation (-Xarch_host puts the sanitizers on the host pass only)."""
import os
import shutil
import subprocess

import pytest

from long_context_sparse_lightning_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "long_context_sparse_lightning_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-fopenmp", os.path.join(ROOT, "oracle", "lsa_oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"), timeout=300)
    assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("g++") is None, reason="needs hipcc and g++")
def test_c_abi_host_side_under_asan_and_ubsan(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"] + san
    objs = []
    for src in build.LSA_SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        _run([HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj], timeout=600)
        objs.append(obj)
    # the driver is plain host C++: compiled and linked (against the HIP runtime) by g++
    exe = str(tmp_path / "abi_driver")
    _run(["g++", "-O1", "-g", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}",
          "-fsanitize=address,undefined", "-fno-omit-frame-pointer", os.path.join(HERE, "abi_driver.cpp")]
         + objs + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], timeout=300)
    r = _run([exe], env=ENV, timeout=300)
    assert "abi driver: ok" in r.stdout
