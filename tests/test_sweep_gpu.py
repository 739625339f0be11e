"""A seeded sweep over the paths and their parameters together: decode,
chunked prefill and cascade decode, each over bf16 and E4M3 pools, with head
shapes, list-length mixes (empty lists, one-entry lists, ragged tails, long
lists), forced splits, plain or XCD placement, pool scales and the fused
[slots, 2, Hkv, D] layout drawn per case.  Every output row and lse against
the fp64 oracle within 2e-3.  Each case prints its parameters before it runs.
Needs an AMD GPU."""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_pa_amd as pa
import workloads as W
from gpu_util import TOL, device, max_err, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

PATHS = ("decode", "prefill", "cascade")
N_CASES = 36


def _lengths(rng, B, path):
    mix = rng.integers(0, 3)
    if mix == 0:
        lengths = rng.integers(1, 70, B)                 # short lists, ragged single tiles
    elif mix == 1:
        lengths = rng.integers(1, 1500, B)
    else:
        lengths = rng.integers(900, 5000, B)             # long lists (split by the plan)
    if path == "decode" and B > 1 and rng.random() < 0.5:
        lengths[rng.integers(0, B)] = 0                 # an empty list
    if rng.random() < 0.3:
        lengths[rng.integers(0, B)] = 1
    return lengths


def draw(seed: int) -> dict:
    """The parameters of case `seed` (host only, no GPU)."""
    rng = np.random.Generator(np.random.PCG64(5000 + seed))
    path = PATHS[seed % 3]
    c = {"seed": seed, "path": path, "fp8": bool((seed // 3) % 2)}
    c["D"] = int(rng.choice([128, 256]))
    G = int(rng.choice([1, 2, 4, 8]))
    c["Hkv"] = int(rng.integers(1, 9))
    c["Hq"] = G * c["Hkv"]
    B = int(rng.integers(1, 13))
    lengths = _lengths(rng, B, path)
    c["flags"] = pa.PA_PLAN_NO_XCD_ORDER if rng.random() < 0.3 else 0
    if path == "cascade":
        c["group"] = int(rng.integers(1, B + 1))
        c["prefix"] = int(rng.integers(1, max(2, int(lengths.min()) + 1)))
        lengths = np.maximum(lengths, c["prefix"])
        if rng.random() < 0.5:
            c["flags"] |= pa.PA_PLAN_CASCADE_ALL
    elif rng.random() < 0.4:
        c["flags"] |= pa.PA_PLAN_FORCE_SPLITS(int(rng.choice([2, 3, 7])))
    if path == "prefill":
        c["chunks"] = [int(rng.integers(0, min(L, 300) + 1)) for L in lengths]
    c["lengths"] = [int(x) for x in lengths]
    c["fused"] = bool(rng.random() < 0.4)
    c["k_scale"] = float(np.float32(np.exp(rng.uniform(np.log(0.05), np.log(4.0)))))
    c["v_scale"] = float(np.float32(np.exp(rng.uniform(np.log(0.05), np.log(4.0)))))
    return c


def _pools(c, N, dev):
    """(k, v) views [N, Hkv, D]: separate pools, or the two halves of one
    fused [N, 2, Hkv, D] buffer (slot stride 2 * Hkv * D)."""
    Hkv, D, seed = c["Hkv"], c["D"], 7000 + c["seed"]
    if c["fp8"]:
        k, v = W.make_pools_e4m3(N, Hkv, D, seed, dev, k_scale=c["k_scale"], v_scale=c["v_scale"])
        k, v = k.view(torch.uint8), v.view(torch.uint8)
    else:
        k, v = W.make_pools(N, Hkv, D, seed, dev)
    if c["fused"]:
        fused = torch.stack([k, v], dim=1).contiguous()
        return fused[:, 0], fused[:, 1]
    return k, v


def _case_ids(c):
    return (f"{c['seed']}-{c['path']}-{'fp8' if c['fp8'] else 'bf16'}-{c['Hq']}x{c['Hkv']}x{c['D']}"
            f"{'-fused' if c['fused'] else ''}")


CASES = [draw(s) for s in range(N_CASES)]


@pytest.mark.parametrize("c", CASES, ids=_case_ids)
def test_sweep(c):
    say(f"sweep case {c}")
    dev = device()
    Hq, Hkv, D, path = c["Hq"], c["Hkv"], c["D"], c["path"]
    lengths = np.asarray(c["lengths"])
    B = lengths.size
    N = int(lengths.sum()) + 777
    rng = np.random.Generator(np.random.PCG64(6000 + c["seed"]))
    if path == "cascade":
        ip, idx = W.slot_lists(lengths, N, rng, c["group"], c["prefix"])
    else:
        ip, idx = W.slot_lists(lengths, N, rng)
    k, v = _pools(c, N, dev)
    scale = W.softmax_scale(D)
    idx_dev = torch.as_tensor(idx, device=dev)
    forced = (c["flags"] >> pa.PA_PLAN_FORCE_SPLITS_SHIFT) & 0xFFFF
    ks, vs = c["k_scale"], c["v_scale"]
    ref_o = oracle.load()
    kc = W.codes(k) if c["fp8"] else W.bits(k)
    vc = W.codes(v) if c["fp8"] else W.bits(v)
    if path == "prefill":
        qo = np.concatenate([[0], np.cumsum(c["chunks"])]).astype(np.int32)
        T = int(qo[-1])
        q = W.normal_bf16((T, Hq, D), 8000 + c["seed"], dev)
        rows = T
    else:
        q = W.normal_bf16((B, Hq, D), 8000 + c["seed"], dev)
        rows = B
    out = torch.full((rows, Hq, D), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((rows, Hq), float("nan"), dtype=torch.float32, device=dev)
    capacity = max(int(ip[-1]), 1, B * forced * 256)
    # forced prefill parts: n per (request, KV head, row tile of at most 256
    # chunk tokens), counted against max_q_total's tiles
    q_cap = max(rows, 1) if path != "prefill" or not forced else forced * (rows + B * 256)
    with pa.Plan(B, capacity, Hq, Hkv, D, max_q_total=q_cap) as plan:
        fl = c["flags"] | (pa.PA_PLAN_KV_FP8 if c["fp8"] else 0)
        if path == "prefill":
            plan.plan(ip, qo, flags=fl)
            if c["fp8"]:
                plan.prefill_fp8(q, k, v, idx_dev, scale, ks, vs, out, lse)
            else:
                plan.prefill(q, k, v, idx_dev, scale, out, lse)
        else:
            if path == "cascade":
                gi = np.concatenate([np.arange(0, B, c["group"]), [B]]).astype(np.int32)
                plan.plan_cascade(ip, gi, np.full(gi.size - 1, c["prefix"], np.int32), flags=fl)
            else:
                plan.plan(ip, flags=fl)
            if c["fp8"]:
                plan.decode_fp8(q, k, v, idx_dev, scale, ks, vs, out, lse)
            else:
                plan.decode(q, k, v, idx_dev, scale, out, lse)
        torch.cuda.synchronize()
    qb = W.bits(q)
    sel = None
    if path == "prefill":
        # every row while the oracle's work stays small, else every head of
        # each request's first and last chunk token and of 48 random tokens
        work = sum(C * L for C, L in zip(c["chunks"], c["lengths"])) * Hq * D
        if work > 2e9:
            toks = set(rng.integers(0, T, 48).tolist())
            for b in range(B):
                if qo[b + 1] > qo[b]:
                    toks |= {int(qo[b]), int(qo[b + 1]) - 1}
            sel = np.array([t * Hq + h for t in sorted(toks) for h in range(Hq)], np.int32)
        if c["fp8"]:
            ref, ref_lse = ref_o.prefill_fp8(qb, kc, vc, qo, ip, idx, scale, ks, vs, Hkv, sel=sel)
        else:
            ref, ref_lse = ref_o.prefill(qb, kc, vc, qo, ip, idx, scale, Hkv, sel=sel)
    elif c["fp8"]:
        ref, ref_lse = ref_o.decode_fp8(qb, kc, vc, ip, idx, scale, ks, vs, Hkv)
    else:
        ref, ref_lse = ref_o.decode(qb, kc, vc, ip, idx, scale, Hkv)
    e = (max_err(out.cpu().numpy(), ref, rows=sel),
         max_err(lse.cpu().numpy().reshape(-1), ref_lse.reshape(-1), rows=sel))
    n = rows * Hq if sel is None else sel.size
    say(f"  {n} of {rows * Hq} rows: max|d| out {e[0]:.3g} lse {e[1]:.3g}")
    assert e[0] <= TOL and e[1] <= TOL


def test_sweep_covers_the_parameters():
    """The drawn cases reach every path and pool type, both head dims, every
    group size, fused pools, forced splits and empty lists."""
    seen = {(c["path"], c["fp8"]) for c in CASES}
    assert seen == {(p, f) for p in PATHS for f in (False, True)}
    assert {c["D"] for c in CASES} == {128, 256}
    assert {c["Hq"] // c["Hkv"] for c in CASES} == {1, 2, 4, 8}
    assert any(c["fused"] for c in CASES)
    assert any((c["flags"] >> pa.PA_PLAN_FORCE_SPLITS_SHIFT) & 0xFFFF for c in CASES)
    assert any(0 in c["lengths"] for c in CASES)
