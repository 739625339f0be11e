"""pa_decode_run_noalloc: decode without a plan object and without any
allocation (its workspace is a device array inside the library).  Called
through the C ABI and checked against pa_decode_run (the plan path) and the
fp64 oracle within 2e-3, on two calls in a row, the second smaller than the
first, so that the second call runs on a workspace the first left behind.
Needs an AMD GPU."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import TOL, all_rows_written, device, max_err, oracle_decode, run_decode, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _case(lengths, Hq, Hkv, D, num_slots, seed):
    dev = device()
    rng = np.random.Generator(np.random.PCG64(seed))
    ip, idx = W.slot_lists(np.asarray(lengths), num_slots, rng)
    q = W.normal_bf16((len(lengths), Hq, D), seed * 3 + 1, dev)
    k, v = W.make_pools(num_slots, Hkv, D, seed * 3 + 2, dev)
    return ip, idx, q, k, v


def _noalloc(q, k, v, ip, idx, Hkv):
    import paged_gqa_decode_pa_amd as pa
    B, Hq, D = q.shape
    dev = q.device
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    pa.pa_decode_run_noalloc(q, k, v, torch.as_tensor(ip, device=dev), torch.as_tensor(idx, device=dev),
                             W.softmax_scale(D), out, lse, num_kv_heads=Hkv)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check(lengths, Hq, Hkv, D, num_slots, seed):
    say(f"no-alloc decode lengths={lengths[:8]}{'...' if len(lengths) > 8 else ''} "
        f"B={len(lengths)} Hq={Hq} Hkv={Hkv} D={D}")
    ip, idx, q, k, v = _case(lengths, Hq, Hkv, D, num_slots, seed)
    out, lse = _noalloc(q, k, v, ip, idx, Hkv)
    ref_run, ref_run_lse = run_decode(q, k, v, ip, torch.as_tensor(idx, device=device()),
                                      W.softmax_scale(D), Hkv)
    ref, ref_lse = oracle_decode(q, k, v, ip, idx, W.softmax_scale(D), Hkv)
    e_run = max(max_err(out, ref_run), max_err(lse, ref_run_lse))
    e = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  vs pa_decode_run {e_run:.3g}; vs oracle out {e[0]:.3g} lse {e[1]:.3g}")
    assert all_rows_written(out) and all_rows_written(lse)
    assert e_run <= TOL and e[0] <= TOL and e[1] <= TOL


# (lengths, Hq, Hkv, D, pool slots): each pair is run in this order, the
# second call smaller than the first
PAIRS = [
    (([3000, 17, 0, 4096, 1, 255, 700, 2000], 32, 8, 128, 20000),
     ([5, 0, 300], 32, 8, 128, 20000)),
    (([1500, 1, 9000, 64], 16, 4, 256, 12000),
     ([1], 16, 4, 256, 100)),                       # fewer list entries than workgroups
    (([800, 1200, 77, 3], 64, 8, 128, 4000),        # 8 query heads per KV head
     ([40, 2], 8, 8, 128, 500)),                    # group 1
]


@pytest.mark.parametrize("first,second", PAIRS, ids=["g4_d128", "g4_d256", "g8_then_g1"])
def test_noalloc_two_calls_match_plan_path(first, second):
    _check(*first, seed=sum(first[0]) % 997 + 1)
    _check(*second, seed=sum(second[0]) % 991 + 2)


def test_noalloc_batch64_workload_all_rows():
    """The batch-64 shared-prefix workload (layer 0) through the no-allocation
    path, every row against the oracle, then a smaller call after it."""
    spec = W.BATCH64_SHARED_PREFIX
    say(f"no-alloc decode {spec.name} layer 0, all rows")
    case = W.make_decode_case(spec, device(), layers=1)
    out, lse = _noalloc(case.q, case.k_pools[0], case.v_pools[0], case.kv_indptr, case.kv_indices,
                        spec.num_kv_heads)
    ref, ref_lse = oracle_decode(case.q, case.k_pools[0], case.v_pools[0], case.kv_indptr,
                                 case.kv_indices, case.sm_scale, spec.num_kv_heads)
    e = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  vs oracle out {e[0]:.3g} lse {e[1]:.3g}")
    assert e[0] <= TOL and e[1] <= TOL
    del case
    torch.cuda.empty_cache()
    _check([100, 200, 300], 32, 8, 128, 1000, seed=5)


def test_noalloc_invalid_offsets_give_nan():
    """Offsets that are not a CSR array (found on the device) give NaN, not a
    result that looks valid; the next valid call is unaffected."""
    import paged_gqa_decode_pa_amd as pa
    say("no-alloc decode with decreasing kv_indptr")
    dev = device()
    ip, idx, q, k, v = _case([10, 20, 30], 32, 8, 128, 100, seed=9)
    bad = torch.as_tensor(np.array([0, 10, 5, 60], np.int32), device=dev)
    out = torch.zeros((3, 32, 128), dtype=torch.float32, device=dev)
    lse = torch.zeros((3, 32), dtype=torch.float32, device=dev)
    pa.pa_decode_run_noalloc(q, k, v, bad, torch.as_tensor(idx, device=dev), 0.1, out, lse, num_kv_heads=8)
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(lse).all()
    _check([10, 20, 30], 32, 8, 128, 100, seed=9)


def test_noalloc_host_errors():
    import paged_gqa_decode_pa_amd as pa
    say("no-alloc decode argument errors")
    dev = device()
    q = torch.zeros((2, 32, 128), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((10, 8, 128), dtype=torch.bfloat16, device=dev)
    ip = torch.zeros(3, dtype=torch.int32, device=dev)
    idx = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.zeros((2, 32, 128), dtype=torch.float32, device=dev)
    vp = ctypes_void_p = __import__("ctypes").c_void_p
    st = pa._lib.pa_decode_run_noalloc(vp(q.data_ptr()), vp(k.data_ptr()), vp(k.data_ptr()), 10, 0,
                                       vp(ip.data_ptr()), vp(idx.data_ptr()), 5000, 32, 8, 128, 0.1,
                                       vp(out.data_ptr()), None, None)
    assert st == pa.PA_ERR_CAPACITY
    st = pa._lib.pa_decode_run_noalloc(vp(q.data_ptr()), vp(k.data_ptr()), vp(k.data_ptr()), 10, 0,
                                       vp(ip.data_ptr()), vp(idx.data_ptr()), 2, 32, 8, 96, 0.1,
                                       vp(out.data_ptr()), None, None)
    assert st == pa.PA_ERR_UNSUPPORTED
    st = pa._lib.pa_decode_run_noalloc(vp(q.data_ptr()), vp(k.data_ptr()), vp(k.data_ptr()), 10, 0,
                                       vp(ip.data_ptr()), vp(idx.data_ptr()), 2, 32, 8, 128, float("inf"),
                                       vp(out.data_ptr()), None, None)
    assert st == pa.PA_ERR_INVALID_ARG
