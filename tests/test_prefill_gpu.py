"""Chunked-prefill parity: the HIP matrix-core path (through the C ABI) against
the fp64 oracle on the same seeded bf16 inputs, within 2e-3.  Needs an AMD GPU."""
import numpy as np
import pytest
import torch

import paged_gqa_decode_pa_amd as pa
import workloads as W
from gpu_util import (TOL, device, max_err, oracle_decode, oracle_prefill, run_decode, run_prefill,
                      say)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _case(reqs, Hq, Hkv, D, num_slots, seed):
    """reqs: [(list length L, chunk length C)] -> (qo_indptr, kv_indptr, kv_indices, q, k, v)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray([L for L, _ in reqs])
    kv_indptr, kv_indices = W.slot_lists(lengths, num_slots, rng)
    qo_indptr = np.concatenate([[0], np.cumsum([C for _, C in reqs])]).astype(np.int32)
    dev = device()
    q = W.normal_bf16((int(qo_indptr[-1]), Hq, D), seed * 5 + 1, dev)
    k, v = W.make_pools(num_slots, Hkv, D, seed * 5 + 2, dev)
    return qo_indptr, kv_indptr, kv_indices, q, k, v


def _check(reqs, Hq, Hkv, D, seed, flags=0, num_slots=8192):
    qo, ip, idx, q, k, v = _case(reqs, Hq, Hkv, D, num_slots, seed)
    scale = W.softmax_scale(D)
    out, lse = run_prefill(q, k, v, qo, ip, torch.as_tensor(idx, device=device()), scale, Hkv,
                           flags=flags)
    ref, ref_lse = oracle_prefill(q, k, v, qo, ip, idx, scale, Hkv)
    e_out, e_lse = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  max|d| out={e_out:.3g} lse={e_lse:.3g}")
    assert e_out <= TOL and e_lse <= TOL
    return out, lse


SMALL = [
    # ([(L, C)], Hq, Hkv, D): tiles of 128/G chunk tokens, KV tiles of 64 (D=128) / 32 (D=256)
    ([(1, 1), (5, 5), (40, 33), (300, 64), (700, 129), (100, 0)], 32, 8, 128),
    ([(200, 200), (513, 130)], 8, 8, 128),          # group 1: 128-token tiles
    ([(64, 17), (1000, 300)], 16, 8, 128),          # group 2
    ([(90, 40), (333, 16), (2, 1)], 64, 8, 128),    # group 8: 16-token tiles
    ([(50, 50), (400, 100)], 16, 4, 256),
    ([(120, 7), (260, 200)], 8, 8, 256),
    ([(77, 77), (31, 3)], 32, 4, 256),
    ([(60, 20), (300, 150)], 16, 8, 256),           # group 2
]


@pytest.mark.parametrize("reqs,Hq,Hkv,D", SMALL,
                         ids=[f"{c[1]}x{c[2]}x{c[3]}-{i}" for i, c in enumerate(SMALL)])
def test_prefill_small_parity(reqs, Hq, Hkv, D):
    say(f"prefill small parity reqs={reqs} Hq={Hq} Hkv={Hkv} D={D}")
    _check(reqs, Hq, Hkv, D, seed=11 + Hq + D + len(reqs))


@pytest.mark.parametrize("n", [2, 5, 16])
def test_prefill_forced_splits(n):
    say(f"prefill forced splits n={n}")
    reqs = [(300, 64), (700, 129), (9, 9)]
    base, base_lse = _check(reqs, 32, 8, 128, seed=7)
    out, lse = _check(reqs, 32, 8, 128, seed=7, flags=pa.PA_PLAN_FORCE_SPLITS(n))
    assert max_err(out, base.astype(np.float64)) <= TOL


@pytest.mark.parametrize("D,Hq,Hkv,splits", [(128, 32, 8, 0), (128, 32, 8, 5), (256, 16, 4, 0)])
def test_prefill_scores_rising_along_the_list(D, Hq, Hkv, splits):
    """K rows scaled by 1, 4, 16, 64 in bands of 97 list entries (exact in
    bf16): the scores jump by far more than 16 log2 units inside tiles and
    between them, so the running maximum must move mid-range (the path that
    weighs a tile again after an fp16 overflow of its weights)."""
    say(f"prefill rising scores D={D} Hq={Hq} Hkv={Hkv} splits={splits}")
    reqs = [(700, 129), (1500, 64), (300, 300)]
    qo, ip, idx, q, k, v = _case(reqs, Hq, Hkv, D, 8192, seed=43 + D)
    fac = np.ones(k.shape[0], np.float32)
    for r in range(len(reqs)):
        band = np.minimum(np.arange(ip[r + 1] - ip[r]) // 97, 3)
        fac[idx[ip[r]:ip[r + 1]]] = 4.0 ** band
    f = torch.as_tensor(fac, device=k.device)[:, None, None]
    k2 = (k.float() * f).to(torch.bfloat16)
    assert torch.equal(k2.float(), k.float() * f)   # the scaling is exact
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(D)
    flags = pa.PA_PLAN_FORCE_SPLITS(splits) if splits else 0
    out, lse = run_prefill(q, k2, v, qo, ip, idx_dev, scale, Hkv, flags=flags)
    ref, ref_lse = oracle_prefill(q, k2, v, qo, ip, idx, scale, Hkv)
    e_out, e_lse = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  max|d| out={e_out:.3g} lse={e_lse:.3g} (oracle lse up to {np.abs(ref_lse[np.isfinite(ref_lse)]).max():.1f})")
    assert e_out <= TOL and e_lse <= TOL


def test_prefill_xcd_order_neutral_and_deterministic():
    say("prefill xcd order / determinism")
    reqs = [(500, 200), (1200, 64)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 8192, 3)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    a, _ = run_prefill(q, k, v, qo, ip, idx_dev, scale, 8)
    b, _ = run_prefill(q, k, v, qo, ip, idx_dev, scale, 8)
    c, _ = run_prefill(q, k, v, qo, ip, idx_dev, scale, 8, flags=pa.PA_PLAN_NO_XCD_ORDER)
    assert np.array_equal(a, b)
    assert np.array_equal(a, c)  # one unit per workgroup: placement does not change the sums


def test_prefill_chunk_of_one_equals_decode():
    say("prefill C=1 vs decode")
    reqs = [(1, 1), (77, 1), (600, 1)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 4096, 5)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    out_p, lse_p = run_prefill(q, k, v, qo, ip, idx_dev, scale, 8)
    out_d, lse_d = run_decode(q, k, v, ip, idx_dev, scale, 8)
    ref, ref_lse = oracle_decode(q, k, v, ip, idx, scale, 8)
    assert max_err(out_p, ref) <= TOL and max_err(lse_p, ref_lse) <= TOL
    assert max_err(out_p, out_d.astype(np.float64)) <= TOL


def test_prefill_poisoned_pool():
    say("prefill poisoned pool")
    reqs = [(150, 40), (333, 100)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 8192, 9)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    clean, _ = run_prefill(q, k, v, qo, ip, idx_dev, scale, 8)
    W.poison_unreferenced(k, idx)
    W.poison_unreferenced(v, idx)
    dirty, _ = run_prefill(q, k, v, qo, ip, idx_dev, scale, 8)
    assert np.array_equal(clean, dirty)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 4, 256)], ids=["D128", "D256"])
def test_prefill_large_pool_offsets(Hq, Hkv, D):
    """Slots beyond 2^31 bytes of pool address (64-bit row offsets)."""
    say(f"prefill large pool: 2,300,000 slots x {Hkv} heads x {D}")
    num_slots = 2_300_000
    dev = device()
    rng = np.random.Generator(np.random.PCG64(21))
    lengths = np.asarray([700, 260])
    ip, idx = W.slot_lists(lengths, num_slots, rng)
    idx[:64] = num_slots - 1 - np.arange(64)   # touch the very end of the pool
    qo = np.asarray([0, 200, 330], np.int32)
    q = W.normal_bf16((330, Hq, D), 22, dev)
    k, v = W.make_pools(num_slots, Hkv, D, 23, dev)
    scale = W.softmax_scale(D)
    out, lse = run_prefill(q, k, v, qo, ip, torch.as_tensor(idx, device=dev), scale, Hkv)
    ref, ref_lse = oracle_prefill(q, k, v, qo, ip, idx, scale, Hkv)
    assert max_err(out, ref) <= TOL and max_err(lse, ref_lse) <= TOL
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.slow
@pytest.mark.parametrize("spec", W.PREFILL_SPECS, ids=lambda s: s.name)
def test_prefill_workload_full_rows(spec):
    """Both chunked-prefill workloads at full size, in the benchmark's launch
    configuration: every output row against the oracle."""
    say(f"prefill workload {spec.name}: all rows")
    dev = device()
    case = W.make_prefill_case(spec, dev)
    idx_dev = torch.as_tensor(case.kv_indices, device=dev)
    out, lse = run_prefill(case.q, case.k_pool, case.v_pool, case.qo_indptr, case.kv_indptr, idx_dev,
                           case.sm_scale, spec.num_kv_heads)
    ref, ref_lse = oracle_prefill(case.q, case.k_pool, case.v_pool, case.qo_indptr, case.kv_indptr,
                                  case.kv_indices, case.sm_scale, spec.num_kv_heads)
    e_out, e_lse = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  {out.shape[0] * out.shape[1]} rows: max|d| out={e_out:.3g} lse={e_lse:.3g}")
    assert e_out <= TOL and e_lse <= TOL


@pytest.mark.parametrize("log2_scale,splits", [(16, 0), (100, 0), (16, 5), (100, 7)])
def test_prefill_values_beyond_fp16_range(log2_scale, splits):
    """The weighted sum runs on fp16 matrix cores; a unit whose V values
    overflow fp16 is run again with V scaled by a power of two.  V = 2^s x
    N(0, 1) (exact in bf16) must give 2^s x the result for N(0, 1), and the
    oracle within 2e-3 x 2^s; with KV ranges cut into parts, whose fp16
    partial rows carry that power of two beside them."""
    say(f"prefill with V scaled by 2^{log2_scale}, splits={splits}")
    reqs = [(300, 64), (700, 129), (40, 33)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 8192, seed=41)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    flags = pa.PA_PLAN_FORCE_SPLITS(splits) if splits else 0
    base, base_lse = run_prefill(q, k, v, qo, ip, idx_dev, scale, 8, flags=flags)
    f = 2.0 ** log2_scale
    big = (v.float() * f).to(torch.bfloat16)
    assert torch.equal(big.float(), v.float() * f)   # the scaling is exact
    out, lse = run_prefill(q, k, big, qo, ip, idx_dev, scale, 8, flags=flags)
    ref, ref_lse = oracle_prefill(q, k, big, qo, ip, idx, scale, 8)
    e = max_err(out / f, ref / f), max_err(lse, ref_lse)
    say(f"  max|d|/2^s vs oracle {e[0]:.3g}, lse {e[1]:.3g}; vs unscaled {max_err(out / f, base):.3g}")
    assert e[0] <= TOL and e[1] <= TOL
    assert max_err(out / f, base) <= TOL and max_err(lse, base_lse) <= 1e-6


@pytest.mark.parametrize("splits", [0, 5])
def test_prefill_values_beyond_fp16_range_in_part_of_the_list(splits):
    """Only the V rows of the first 150 list entries of each request scaled by
    2^16: the parts of a cut range then run with different powers of two, each
    stored beside its partial rows and undone in the merge."""
    say(f"prefill with V scaled by 2^16 on the first 150 entries, splits={splits}")
    reqs = [(300, 64), (700, 129), (40, 33)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 8192, seed=42)
    fac = np.ones(v.shape[0], np.float32)
    for r in range(len(reqs)):
        fac[idx[ip[r]:ip[r] + 150]] = 65536.0
    f = torch.as_tensor(fac, device=v.device)[:, None, None]
    big = (v.float() * f).to(torch.bfloat16)
    assert torch.equal(big.float(), v.float() * f)   # the scaling is exact
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    flags = pa.PA_PLAN_FORCE_SPLITS(splits) if splits else 0
    out, lse = run_prefill(q, k, big, qo, ip, idx_dev, scale, 8, flags=flags)
    ref, ref_lse = oracle_prefill(q, k, big, qo, ip, idx, scale, 8)
    e = max_err(out / 65536.0, ref / 65536.0), max_err(lse, ref_lse)
    say(f"  max|d|/2^16 vs oracle {e[0]:.3g}, lse {e[1]:.3g}")
    assert e[0] <= TOL and e[1] <= TOL


def test_prefill_forced_splits_capacity():
    """The documented room for forced prefill parts: 2 requests of 640 chunk
    tokens (10 tiles of 64 tokens per KV head, 160 tiles) in a plan with
    max_q_total 1280 hold 1024 + 8 * (20 + 2) = 1200 units, so 7 parts per
    tile (1120 units) fit and give the oracle's result; 64 parts per tile
    (10240 units) are refused with PA_ERR_CAPACITY before anything runs."""
    say("prefill forced-split capacity")
    reqs = [(1000, 640), (1000, 640)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 4096, seed=51)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    out = torch.full((1280, 32, 128), float("nan"), dtype=torch.float32, device=device())
    with pa.Plan(2, int(ip[-1]), 32, 8, 128, max_q_total=1280) as plan:
        plan.plan(ip, qo, flags=pa.PA_PLAN_FORCE_SPLITS(7))
        plan.prefill(q, k, v, idx_dev, scale, out)
        torch.cuda.synchronize()
        with pytest.raises(pa.PAError) as e:
            plan.plan(ip, qo, flags=pa.PA_PLAN_FORCE_SPLITS(64))
        assert e.value.status == pa.PA_ERR_CAPACITY
    ref, _ = oracle_prefill(q, k, v, qo, ip, idx, scale, 8)
    assert max_err(out.cpu().numpy(), ref) <= TOL


def test_prefill_refuses_misaligned_out():
    """Output rows are written four floats at a time: an out buffer that is
    only 4-byte aligned is refused on the host, for bf16 and E4M3 pools."""
    say("prefill with a misaligned out buffer")
    reqs = [(100, 20)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 1024, seed=53)
    idx_dev = torch.as_tensor(idx, device=device())
    n = 20 * 32 * 128
    out = torch.empty(n + 4, dtype=torch.float32, device=device())[1:1 + n].view(20, 32, 128)
    assert out.data_ptr() % 16 == 4
    k8, v8 = W.make_pools_e4m3(1024, 8, 128, 54, device())
    with pa.Plan(1, int(ip[-1]), 32, 8, 128, max_q_total=20) as plan:
        plan.plan(ip, qo)
        for run in (lambda: plan.prefill(q, k, v, idx_dev, 0.088, out),
                    lambda: plan.prefill_fp8(q, k8, v8, idx_dev, 0.088, 1.0, 1.0, out)):
            with pytest.raises(pa.PAError) as e:
                run()
            assert e.value.status == pa.PA_ERR_INVALID_ARG
