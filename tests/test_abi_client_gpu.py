"""The C ABI from plain C: tests/c/abi_client (built by build(), no Python or
torch inside it) plans and runs a small decode through include/pa.h alone;
its output must match the fp64 oracle on the bf16 bits it wrote, within
2e-3, and its run without lse must give the same output bit for bit.  The
client runs as a child process.  Needs an AMD GPU."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, max_err, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_client")


def test_plain_c_client_decode(tmp_path):
    say("plain C client of the ABI")
    assert os.path.exists(CLIENT), "tests/c/abi_client is missing: run __graft_entry__.build()"
    path = tmp_path / "client.bin"
    r = subprocess.run([CLIENT, str(path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    raw = path.read_bytes()
    B, Hq, Hkv, D, N, E = np.frombuffer(raw[:24], np.int32)
    off = 24

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(raw, dtype, count=int(n), offset=off)
        off += a.nbytes
        return a

    q = take(np.uint16, B * Hq * D).reshape(B, Hq, D)
    k = take(np.uint16, N * Hkv * D).reshape(N, Hkv, D)
    v = take(np.uint16, N * Hkv * D).reshape(N, Hkv, D)
    indptr = take(np.int32, B + 1)
    indices = take(np.int32, E)
    out = take(np.float32, B * Hq * D).reshape(B, Hq, D)
    lse = take(np.float32, B * Hq).reshape(B, Hq)
    out2 = take(np.float32, B * Hq * D).reshape(B, Hq, D)
    assert off == len(raw)
    ref, ref_lse = oracle.load().decode(q, k, v, indptr, indices, float(np.float32(D ** -0.5)), int(Hkv))
    e = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  max|d| out {e[0]:.3g} lse {e[1]:.3g}")
    assert e[0] <= TOL and e[1] <= TOL
    assert np.array_equal(out, out2)
