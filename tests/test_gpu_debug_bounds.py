"""LSA_DEBUG_BOUNDS mode on the GPU: with the variable set, a call whose seqlens break the device-side
precondition (Lq <= seqlens[b] <= S_max) is refused with LSA_ERR_BAD_SHAPE before anything is
launched, and a valid call runs as usual.  The variable is read once per process, so the check
runs in a child process."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SCRIPT = r"""
import torch
from long_context_sparse_lightning_amd import lsa
dev = "cuda"
B, S, H = 2, 300, 4
q = torch.zeros(B, H, 80, dtype=torch.bfloat16, device=dev)
kv = torch.zeros(B, S, 80, dtype=torch.bfloat16, device=dev)
idx = torch.zeros(B, 64, dtype=torch.int32, device=dev)
ns = torch.full((B,), 64, dtype=torch.int32, device=dev)
ok = torch.tensor([300, 200], dtype=torch.int32, device=dev)
bad = torch.tensor([300, 301], dtype=torch.int32, device=dev)
lsa.lsa_sparse_mla_decode(q, kv, idx, ns, ok, 64, 0.1)
torch.cuda.synchronize()
try:
    lsa.lsa_sparse_mla_decode(q, kv, idx, ns, bad, 64, 0.1)
    raise SystemExit("bad seqlens accepted")
except lsa.LsaError as e:
    assert e.status == 2 and "seqlens[1] = 301" in str(e), str(e)
qi = torch.zeros(B, 1, 4, 32, dtype=torch.bfloat16, device=dev)
w = torch.zeros(B, 1, 4, dtype=torch.float32, device=dev)
k = torch.zeros(B, S, 32, dtype=torch.bfloat16, device=dev)
try:
    lsa.lsa_index_topk(qi, w, k, torch.tensor([0, 10], dtype=torch.int32, device=dev), 64, 4, 8)
    raise SystemExit("empty sequence accepted")
except lsa.LsaError as e:
    assert e.status == 2, str(e)
print("debug bounds ok")
"""


def test_debug_bounds_refuses_bad_seqlens():
    print("case LSA_DEBUG_BOUNDS child process", flush=True)
    env = dict(os.environ, LSA_DEBUG_BOUNDS="1", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", SCRIPT], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=180)
    assert r.returncode == 0 and "debug bounds ok" in r.stdout, r.stdout + r.stderr
