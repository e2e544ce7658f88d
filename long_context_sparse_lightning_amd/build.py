"""Build the gfx950 shared libraries in-tree with hipcc.

* ``liblsa.so``     -- the LSA hot path (kernels + C ABI of ``include/lsa.h``);
* ``liblsa_gen.so`` -- the seeded synthetic-input fills used by the tests and the bench.

Run ``python -m long_context_sparse_lightning_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc")
                       else "hipcc")

# Every HIP translation unit is built with packed-fp32 code generation switched off: the
# v_pk_*_f32 forms are avoided on this hardware.  (hipcc's host pass warns that it does not
# know the feature; that warning is harmless.)
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

LSA_SOURCES = ["lsa_api.hip", "lsa_indexer.hip", "lsa_topk.hip", "lsa_mla.hip", "lsa_frontend.hip",
               "lsa_hier.hip"]
GEN_SOURCES = ["lsa_gen.hip"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int = 4) -> list[str]:
    obj_dir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(obj_dir, exist_ok=True)
    units = [(s, os.path.join(obj_dir, s.replace(".hip", ".o"))) for s in LSA_SOURCES + GEN_SOURCES]

    def compile_one(u):
        src, obj = u
        _run([HIPCC] + COMMON_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(compile_one, units))
    objs = dict(units)
    out_lsa = os.path.join(PKG, "liblsa.so")
    out_gen = os.path.join(PKG, "liblsa_gen.so")
    _link([objs[s] for s in LSA_SOURCES], out_lsa, verbose)
    _link([objs[s] for s in GEN_SOURCES], out_gen, verbose)
    return [out_lsa, out_gen]


def clean() -> None:
    shutil.rmtree(os.path.join(ROOT, "_build"), ignore_errors=True)


if __name__ == "__main__":
    for p in build(verbose="-v" in sys.argv):
        print(p)
