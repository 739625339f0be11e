"""Chunked prefill over 8-bit (OCP FP8 E4M3) pools with per-pool scales,
through the C ABI (pa_prefill_chunk_run_fp8), against the fp64 oracle on the
same codes, within 2e-3.  Needs an AMD GPU."""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_pa_amd as pa
import workloads as W
from gpu_util import TOL, device, max_err, run_prefill, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

KS, VS = W.FP8_K_SCALE, W.FP8_V_SCALE


def _case(reqs, Hq, Hkv, D, num_slots, seed, k_scale=KS, v_scale=VS):
    """reqs: [(list length L, chunk length C)] -> (qo_indptr, kv_indptr, kv_indices, q, k, v)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray([L for L, _ in reqs])
    kv_indptr, kv_indices = W.slot_lists(lengths, num_slots, rng)
    qo_indptr = np.concatenate([[0], np.cumsum([C for _, C in reqs])]).astype(np.int32)
    dev = device()
    q = W.normal_bf16((int(qo_indptr[-1]), Hq, D), seed * 5 + 1, dev)
    k, v = W.make_pools_e4m3(num_slots, Hkv, D, seed * 5 + 2, dev, k_scale=k_scale, v_scale=v_scale)
    return qo_indptr, kv_indptr, kv_indices, q, k, v


def run_prefill_fp8(q, k, v, qo_indptr, kv_indptr, idx_dev, sm_scale, Hkv, k_scale=KS, v_scale=VS, flags=0):
    T, Hq, D = q.shape
    B = len(kv_indptr) - 1
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.float32, device=q.device)
    lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device=q.device)
    with pa.Plan(max(B, 1), max(int(kv_indptr[-1]), 1), Hq, Hkv, D, max_q_total=max(T, 1)) as plan:
        plan.plan(kv_indptr, qo_indptr, flags=flags)
        plan.prefill_fp8(q, k, v, idx_dev, sm_scale, k_scale, v_scale, out, lse)
        torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _oracle(q, k, v, qo, ip, idx, scale, Hkv, k_scale=KS, v_scale=VS, sel=None):
    return oracle.load().prefill_fp8(W.bits(q), W.codes(k), W.codes(v), qo, ip, np.asarray(idx, np.int32),
                                     scale, k_scale, v_scale, Hkv, sel=sel)


def _check(reqs, Hq, Hkv, D, seed, flags=0, num_slots=8192, k_scale=KS, v_scale=VS):
    qo, ip, idx, q, k, v = _case(reqs, Hq, Hkv, D, num_slots, seed, k_scale, v_scale)
    scale = W.softmax_scale(D)
    out, lse = run_prefill_fp8(q, k, v, qo, ip, torch.as_tensor(idx, device=device()), scale, Hkv,
                               k_scale, v_scale, flags)
    ref, ref_lse = _oracle(q, k, v, qo, ip, idx, scale, Hkv, k_scale, v_scale)
    e_out, e_lse = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  max|d| out={e_out:.3g} lse={e_lse:.3g}")
    assert e_out <= TOL and e_lse <= TOL
    return out, lse


SMALL = [
    # ([(L, C)], Hq, Hkv, D): tiles of 128/G chunk tokens, KV tiles of 64 (D=128) / 32 (D=256)
    ([(1, 1), (5, 5), (40, 33), (300, 64), (700, 129), (100, 0)], 32, 8, 128),
    ([(200, 200), (513, 130)], 8, 8, 128),          # group 1
    ([(64, 17), (1000, 300)], 16, 8, 128),          # group 2
    ([(90, 40), (333, 16), (2, 1)], 64, 8, 128),    # group 8
    ([(50, 50), (400, 100)], 16, 4, 256),
    ([(120, 7), (260, 200)], 8, 8, 256),
    ([(77, 77), (31, 3)], 32, 4, 256),
    ([(60, 20), (300, 150)], 16, 8, 256),           # group 2
    ([(500, 90), (45, 45)], 12, 3, 128),            # odd KV-head count
]


@pytest.mark.parametrize("reqs,Hq,Hkv,D", SMALL,
                         ids=[f"{c[1]}x{c[2]}x{c[3]}-{i}" for i, c in enumerate(SMALL)])
def test_prefill_fp8_small_parity(reqs, Hq, Hkv, D):
    say(f"prefill fp8 small parity reqs={reqs} Hq={Hq} Hkv={Hkv} D={D}")
    _check(reqs, Hq, Hkv, D, seed=61 + Hq + D + len(reqs))


@pytest.mark.parametrize("n", [2, 5, 16])
def test_prefill_fp8_forced_splits(n):
    """KV ranges cut into parts: the fp16 partial rows of code values merged
    in the kernel, v_scale applied after the merge."""
    say(f"prefill fp8 forced splits n={n}")
    reqs = [(300, 64), (700, 129), (9, 9)]
    base, _ = _check(reqs, 32, 8, 128, seed=8)
    out, _ = _check(reqs, 32, 8, 128, seed=8, flags=pa.PA_PLAN_FORCE_SPLITS(n))
    assert max_err(out, base.astype(np.float64)) <= TOL


@pytest.mark.parametrize("k_scale,v_scale,v_gen,splits", [(0.37, 1.3, 1.3, 0), (3.1, 0.07, 0.07, 5),
                                                          (0.02, 1000.0, 0.02, 0), (0.02, 1000.0, 0.02, 7)])
def test_prefill_fp8_scales(k_scale, v_scale, v_gen, splits):
    """Pool scales that are not powers of two; and V codes of ~50 x N(0, 1)
    (drawn as N(0, 1) / 0.02) read under v_scale 1000, so that rows times the
    scale reach ~10^5: fp16 partial rows would overflow if the scale were
    applied before the merge of a cut range.  Errors relative to the size of
    the values, v_scale / v_gen."""
    say(f"prefill fp8 scales k={k_scale} v={v_scale} (codes of N(0,1)/{v_gen}) splits={splits}")
    reqs = [(300, 64), (700, 129), (40, 33), (1, 1)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 8192, 71, k_scale, v_gen)
    scale = W.softmax_scale(128)
    flags = pa.PA_PLAN_FORCE_SPLITS(splits) if splits else 0
    out, lse = run_prefill_fp8(q, k, v, qo, ip, torch.as_tensor(idx, device=device()), scale, 8,
                               k_scale, v_scale, flags)
    ref, ref_lse = _oracle(q, k, v, qo, ip, idx, scale, 8, k_scale, v_scale)
    size = v_scale / v_gen
    e_out, e_lse = max_err(out / size, ref / size), max_err(lse, ref_lse)
    say(f"  max|out| {np.abs(out).max():.3g}; max|d|/{size:g}={e_out:.3g} lse={e_lse:.3g}")
    assert e_out <= TOL and e_lse <= TOL


def test_prefill_fp8_unit_scales_equal_bf16_prefill():
    """With unit scales, the fp8 prefill and the bf16 prefill over pools that
    hold the codes' values (exact in bf16) run the same operands through the
    same matrix cores: bit-identical outputs."""
    say("prefill fp8 vs bf16 prefill on the widened codes")
    reqs = [(300, 64), (700, 129), (40, 33), (5, 5)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 8192, 72, 1.0, 1.0)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    out8, lse8 = run_prefill_fp8(q, k, v, qo, ip, idx_dev, scale, 8, 1.0, 1.0)
    kb, vb = k.to(torch.bfloat16), v.to(torch.bfloat16)
    out, lse = run_prefill(q, kb, vb, qo, ip, idx_dev, scale, 8)
    assert np.array_equal(out8, out) and np.array_equal(lse8, lse)


def test_prefill_fp8_chunk_of_one_equals_decode():
    say("prefill fp8 C=1 vs fp8 decode")
    reqs = [(1, 1), (77, 1), (600, 1)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 4096, 73)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    out_p, lse_p = run_prefill_fp8(q, k, v, qo, ip, idx_dev, scale, 8)
    ref, ref_lse = oracle.load().decode_fp8(W.bits(q), W.codes(k), W.codes(v), ip, idx, scale, KS, VS, 8)
    assert max_err(out_p, ref) <= TOL and max_err(lse_p, ref_lse) <= TOL


def test_prefill_fp8_poisoned_pool():
    """NaN codes (0x7F) in every unreferenced slot change nothing."""
    say("prefill fp8 poisoned pool")
    reqs = [(150, 40), (333, 100)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 8192, 74)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    clean, _ = run_prefill_fp8(q, k, v, qo, ip, idx_dev, scale, 8)
    mask = torch.ones(k.shape[0], dtype=torch.bool, device=k.device)
    mask[torch.as_tensor(idx, device=k.device, dtype=torch.int64)] = False
    k.view(torch.uint8)[mask] = 0x7F
    v.view(torch.uint8)[mask] = 0x7F
    dirty, _ = run_prefill_fp8(q, k, v, qo, ip, idx_dev, scale, 8)
    assert np.array_equal(clean, dirty)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 4, 256)], ids=["D128", "D256"])
def test_prefill_fp8_large_pool_offsets(Hq, Hkv, D):
    """Slots beyond 2^31 bytes of an 8-bit pool (64-bit row offsets)."""
    say(f"prefill fp8 large pool: 2,300,000 slots x {Hkv} heads x {D}")
    num_slots = 2_300_000
    dev = device()
    rng = np.random.Generator(np.random.PCG64(75))
    lengths = np.asarray([700, 260])
    ip, idx = W.slot_lists(lengths, num_slots, rng)
    idx[:64] = num_slots - 1 - np.arange(64)   # touch the very end of the pool
    qo = np.asarray([0, 200, 330], np.int32)
    q = W.normal_bf16((330, Hq, D), 76, dev)
    k, v = W.make_pools_e4m3(num_slots, Hkv, D, 77, dev)
    scale = W.softmax_scale(D)
    out, lse = run_prefill_fp8(q, k, v, qo, ip, torch.as_tensor(idx, device=dev), scale, Hkv)
    ref, ref_lse = _oracle(q, k, v, qo, ip, idx, scale, Hkv)
    assert max_err(out, ref) <= TOL and max_err(lse, ref_lse) <= TOL
    del k, v
    torch.cuda.empty_cache()


def test_prefill_fp8_bad_scales():
    say("prefill fp8: non-finite scales are rejected")
    qo, ip, idx, q, k, v = _case([(40, 10)], 32, 8, 128, 1024, 78)
    out = torch.empty((10, 32, 128), dtype=torch.float32, device=device())
    idx_dev = torch.as_tensor(idx, device=device())
    with pa.Plan(1, 40, 32, 8, 128, max_q_total=10) as plan:
        plan.plan(ip, qo)
        for ks, vs in [(float("nan"), 1.0), (1.0, float("inf"))]:
            with pytest.raises(pa.PAError) as err:
                plan.prefill_fp8(q, k, v, idx_dev, 0.088, ks, vs, out)
            assert err.value.status == pa.PA_ERR_INVALID_ARG


@pytest.mark.slow
@pytest.mark.parametrize("spec", W.PREFILL_SPECS, ids=lambda s: s.name)
def test_prefill_fp8_workload_full_rows(spec):
    """Both chunked-prefill workloads at full size over E4M3 pools, in the
    benchmark's launch configuration: every output row against the oracle."""
    say(f"prefill fp8 workload {spec.name}: all rows")
    dev = device()
    qo, ip, idx = W.prefill_lists(spec)
    T = int(qo[-1])
    q = W.normal_bf16((T, spec.num_qo_heads, spec.head_dim), spec.seed, dev)
    k, v = W.make_pools_e4m3(spec.num_slots, spec.num_kv_heads, spec.head_dim, W.layer_seed(spec.seed, 0), dev)
    scale = W.softmax_scale(spec.head_dim)
    out, lse = run_prefill_fp8(q, k, v, qo, ip, torch.as_tensor(idx, device=dev), scale, spec.num_kv_heads)
    ref, ref_lse = _oracle(q, k, v, qo, ip, idx, scale, spec.num_kv_heads)
    e_out, e_lse = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  {out.shape[0] * out.shape[1]} rows: max|d| out={e_out:.3g} lse={e_lse:.3g}")
    assert e_out <= TOL and e_lse <= TOL


@pytest.mark.parametrize("k_scale,v_scale", [(-0.37, -1.3), (0.0, 0.7), (0.37, 0.0)])
def test_prefill_fp8_nonpositive_scales(k_scale, v_scale):
    """Scales of any sign: a negative k_scale runs as |scale| on the negated
    query, a zero k_scale gives every score 0 (the mean of the visible V
    rows), a zero v_scale a zero output; against the oracle, with KV cuts."""
    say(f"prefill fp8 scales k={k_scale} v={v_scale}")
    reqs = [(300, 64), (700, 129), (40, 33)]
    qo, ip, idx, q, k, v = _case(reqs, 32, 8, 128, 8192, 96, 0.37, 1.3)
    scale = W.softmax_scale(128)
    for flags in (0, pa.PA_PLAN_FORCE_SPLITS(5)):
        out, lse = run_prefill_fp8(q, k, v, qo, ip, torch.as_tensor(idx, device=device()), scale, 8,
                                   k_scale, v_scale, flags)
        ref, ref_lse = _oracle(q, k, v, qo, ip, idx, scale, 8, k_scale, v_scale)
        e = max_err(out, ref), max_err(lse, ref_lse)
        say(f"  flags {flags:#x}: max|d| out {e[0]:.3g} lse {e[1]:.3g}")
        assert e[0] <= TOL and e[1] <= TOL
