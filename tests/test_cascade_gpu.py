"""Cascade decode (pa_plan_cascade): each group's shared prefix is attended
once by the matrix-core prefix units and merged into the decode kernel's
results.  The output must match the fp64 oracle on the full lists within
2e-3 and the plain decode plan within 5e-4.  Needs an AMD GPU."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import TOL, device, max_err, oracle_decode, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# Cascade and plain decode of the same lists agree to this (the bar against
# the oracle stays 2e-3): the prefix units weight V on fp16 matrix cores,
# each weight rounded once to fp16 (relative error <= 2^-11), where the decode
# kernel keeps fp32 weights.
CASCADE_VS_PLAIN = 5e-4


def _groups(B, size):
    gi = list(range(0, B, size)) + [B]
    return np.array(gi, np.int32)


def _case(lengths, group_size, prefix_len, Hq, Hkv, D, num_slots, seed):
    dev = device()
    rng = np.random.Generator(np.random.PCG64(seed))
    ip, idx = W.slot_lists(np.asarray(lengths), num_slots, rng, group_size, prefix_len)
    q = W.normal_bf16((len(lengths), Hq, D), seed * 5 + 1, dev)
    k, v = W.make_pools(num_slots, Hkv, D, seed * 5 + 2, dev)
    return ip, idx, q, k, v


def _run(plan_fn, ip, idx, q, k, v, Hkv, flags=0):
    import paged_gqa_decode_pa_amd as pa
    B, Hq, D = q.shape
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=q.device)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device)
    with pa.Plan(B, int(ip[-1]), Hq, Hkv, D) as plan:
        plan_fn(plan)
        plan.decode(q, k, v, torch.as_tensor(idx, device=q.device), W.softmax_scale(D), out, lse)
        torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check(ip, idx, q, k, v, Hkv, gi, pl):
    import paged_gqa_decode_pa_amd as pa
    # prefix units for every group, however small (the default leaves small
    # groups to the plain split)
    cas, cas_lse = _run(lambda p: p.plan_cascade(ip, gi, pl, flags=pa.PA_PLAN_CASCADE_ALL),
                        ip, idx, q, k, v, Hkv)
    ref_plain, ref_plain_lse = _run(lambda p: p.plan(ip), ip, idx, q, k, v, Hkv)
    d_plain = max(max_err(cas, ref_plain), max_err(cas_lse, ref_plain_lse))
    ref, ref_lse = oracle_decode(q, k, v, ip, idx, W.softmax_scale(q.shape[-1]), Hkv)
    e = max_err(cas, ref), max_err(cas_lse, ref_lse)
    say(f"  vs plain {d_plain:.3g}; vs oracle out {e[0]:.3g} lse {e[1]:.3g} (all rows)")
    assert d_plain <= CASCADE_VS_PLAIN
    assert e[0] <= TOL and e[1] <= TOL


CASES = [
    # (lengths, group size, prefix, Hq, Hkv, D)
    ([1200, 1500, 3000, 900, 2000, 2600, 1100, 1300, 700, 701, 2222, 4000], 4, 700, 32, 8, 128),
    ([1024] * 4 + [1500] * 4, 4, 1024, 32, 8, 128),      # some lists are all prefix
    ([300 + 17 * i for i in range(40)], 40, 290, 32, 8, 128),   # 40 members: subgroups of 32 + 8
    ([5, 70, 64, 65, 1, 1], 2, 1, 32, 8, 128),            # one-entry prefixes, ragged tiles
    ([800, 950, 1000, 1200, 333, 444], 3, 300, 64, 8, 128),     # 8 query heads per KV head
    ([700, 1900, 1000, 1200], 2, 650, 16, 4, 256),        # head_dim 256
    ([400, 800, 1600, 3200], 1, 0, 32, 8, 128),           # no sharing: plain decode
    ([500, 600, 700, 800, 900], 5, 400, 8, 8, 128),       # 1 query head per KV head
    ([900, 1000, 1100, 1300], 4, 500, 16, 8, 128),        # 2 query heads per KV head
    ([600, 700, 800], 3, 333, 32, 4, 256),                # head_dim 256, 8 query heads per KV head
]


@pytest.mark.parametrize("lengths,gsize,plen,Hq,Hkv,D", CASES,
                         ids=[f"{c[3]}x{c[4]}x{c[5]}-g{c[1]}-p{c[2]}-{i}" for i, c in enumerate(CASES)])
def test_cascade_parity(lengths, gsize, plen, Hq, Hkv, D):
    say(f"cascade lengths={lengths[:6]}... groups of {gsize} prefix {plen} Hq={Hq} Hkv={Hkv} D={D}")
    ip, idx, q, k, v = _case(lengths, gsize, plen, Hq, Hkv, D, 40000, seed=len(lengths) + plen + D)
    gi = _groups(len(lengths), gsize)
    pl = np.full(gi.size - 1, plen, np.int32)
    _check(ip, idx, q, k, v, Hkv, gi, pl)


def test_mixed_groups():
    """Groups with and without prefixes, a singleton with a prefix, in one plan."""
    say("cascade mixed groups")
    lengths = [900, 1100, 1000, 600, 2000, 2100, 50, 3000]
    ip, idx, q, k, v = _case(lengths, 2, 40, 32, 8, 128, 20000, seed=77)
    gi = np.array([0, 2, 4, 6, 7, 8], np.int32)
    pl = np.array([40, 0, 40, 50, 3000], np.int32)
    _check(ip, idx, q, k, v, 8, gi, pl)


def test_batch64_workload_full_rows():
    """The batch-64 workload's 16 groups of 4 sharing 1024 slots, in the
    benchmark's launch configuration; every row against the oracle."""
    spec = W.BATCH64_SHARED_PREFIX
    say("cascade batch64 workload (all rows)")
    case = W.make_decode_case(spec, device(), layers=1)
    gi = _groups(spec.batch, spec.prefix_group_size)
    pl = np.full(gi.size - 1, spec.prefix_len, np.int32)
    _check(case.kv_indptr, case.kv_indices, case.q, case.k_pools[0], case.v_pools[0],
           spec.num_kv_heads, gi, pl)
    del case
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_system_prompt_workload_full_rows():
    """64 requests sharing a 4096-slot system prompt (subgroups of 32 under
    the default policy); every row against the oracle."""
    spec = W.SYSTEM_PROMPT_B64
    say("cascade system-prompt workload (all rows)")
    case = W.make_decode_case(spec, device(), layers=1)
    gi = np.array([0, spec.batch], np.int32)
    pl = np.array([spec.prefix_len], np.int32)
    q, k, v = case.q, case.k_pools[0], case.v_pools[0]
    cas, cas_lse = _run(lambda p: p.plan_cascade(case.kv_indptr, gi, pl), case.kv_indptr,
                        case.kv_indices, q, k, v, spec.num_kv_heads)
    plain, plain_lse = _run(lambda p: p.plan(case.kv_indptr), case.kv_indptr, case.kv_indices,
                            q, k, v, spec.num_kv_heads)
    assert max_err(cas, plain) <= CASCADE_VS_PLAIN and max_err(cas_lse, plain_lse) <= CASCADE_VS_PLAIN
    ref, ref_lse = oracle_decode(q, k, v, case.kv_indptr, case.kv_indices, case.sm_scale,
                                 spec.num_kv_heads)
    e = max_err(cas, ref), max_err(cas_lse, ref_lse)
    say(f"  vs oracle out {e[0]:.3g} lse {e[1]:.3g}")
    assert e[0] <= TOL and e[1] <= TOL
    del case
    torch.cuda.empty_cache()


def test_small_groups_default_is_plain_decode():
    """Without PA_PLAN_CASCADE_ALL, groups of 4 requests get no prefix units:
    the result is the plain decode's, bit for bit."""
    say("cascade default policy on small groups")
    lengths = [1000, 1200, 1400, 1600, 900, 950, 990, 1300]
    ip, idx, q, k, v = _case(lengths, 4, 500, 32, 8, 128, 10000, seed=15)
    gi, pl = _groups(8, 4), np.array([500, 500], np.int32)
    a, la = _run(lambda p: p.plan_cascade(ip, gi, pl), ip, idx, q, k, v, 8)
    b, lb = _run(lambda p: p.plan(ip), ip, idx, q, k, v, 8)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_plan_modes_alternate():
    """One plan object: cascade, plain, cascade again; each run matches."""
    import paged_gqa_decode_pa_amd as pa
    say("cascade / plain alternation on one plan")
    lengths = [1000, 1200, 1400, 1600]
    ip, idx, q, k, v = _case(lengths, 4, 500, 32, 8, 128, 10000, seed=5)
    gi, pl = _groups(4, 4), np.array([500], np.int32)
    idx_dev = torch.as_tensor(idx, device=device())
    outs = []
    with pa.Plan(4, int(ip[-1]), 32, 8, 128) as plan:
        for mode in ("cascade", "plain", "cascade"):
            if mode == "cascade":
                plan.plan_cascade(ip, gi, pl, flags=pa.PA_PLAN_CASCADE_ALL)
            else:
                plan.plan(ip)
            o = torch.full((4, 32, 128), float("nan"), dtype=torch.float32, device=device())
            plan.decode(q, k, v, idx_dev, W.softmax_scale(128), o)
            outs.append(o)
        # the same cascade plan over E4M3 pools of zero codes: every V is 0
        plan.plan_cascade(ip, gi, pl, flags=pa.PA_PLAN_CASCADE_ALL | pa.PA_PLAN_KV_FP8)
        k8 = torch.zeros((k.shape[0], 8, 128), dtype=torch.uint8, device=device())
        o8 = torch.full((4, 32, 128), float("nan"), dtype=torch.float32, device=device())
        plan.decode_fp8(q, k8, k8, idx_dev, W.softmax_scale(128), 1.0, 1.0, o8)
        torch.cuda.synchronize()
        assert torch.equal(o8, torch.zeros_like(o8))
    a, b, c = (o.cpu().numpy() for o in outs)
    assert np.array_equal(a, c) and max_err(a, b) <= CASCADE_VS_PLAIN


def _run_fp8(plan_fn, ip, idx, q, k, v, Hkv, k_scale, v_scale):
    import paged_gqa_decode_pa_amd as pa
    B, Hq, D = q.shape
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=q.device)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device)
    with pa.Plan(B, int(ip[-1]), Hq, Hkv, D) as plan:
        plan_fn(plan)
        plan.decode_fp8(q, k, v, torch.as_tensor(idx, device=q.device), W.softmax_scale(D), k_scale, v_scale,
                        out, lse)
        torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


FP8_CASES = [CASES[0], CASES[2], CASES[3], CASES[4], CASES[5], CASES[9]]


@pytest.mark.parametrize("lengths,gsize,plen,Hq,Hkv,D", FP8_CASES,
                         ids=[f"{c[3]}x{c[4]}x{c[5]}-g{c[1]}-p{c[2]}-{i}" for i, c in enumerate(FP8_CASES)])
def test_cascade_fp8_parity(lengths, gsize, plen, Hq, Hkv, D):
    """Cascade plans over E4M3 pools (pa_decode_run_fp8): prefix units read
    the codes on the matrix cores; scales that are not powers of two."""
    import oracle
    import paged_gqa_decode_pa_amd as pa
    say(f"cascade fp8 parity {Hq}x{Hkv}x{D} groups of {gsize}, prefix {plen}")
    dev = device()
    ks, vs = 0.37, 1.3
    rng = np.random.Generator(np.random.PCG64(80 + len(lengths)))
    ip, idx = W.slot_lists(np.asarray(lengths), 20000, rng, gsize, plen)
    q = W.normal_bf16((len(lengths), Hq, D), 81, dev)
    k, v = W.make_pools_e4m3(20000, Hkv, D, 82, dev, k_scale=ks, v_scale=vs)
    B = len(lengths)
    gi = _groups(B, gsize)
    pl = np.full(gi.size - 1, plen, np.int32)
    fl = pa.PA_PLAN_KV_FP8
    cas, cas_lse = _run_fp8(lambda p: p.plan_cascade(ip, gi, pl, flags=pa.PA_PLAN_CASCADE_ALL | fl),
                            ip, idx, q, k, v, Hkv, ks, vs)
    plain, plain_lse = _run_fp8(lambda p: p.plan(ip, flags=fl), ip, idx, q, k, v, Hkv, ks, vs)
    ref, ref_lse = oracle.load().decode_fp8(W.bits(q), W.codes(k), W.codes(v), ip, idx, W.softmax_scale(D),
                                            ks, vs, Hkv)
    d_plain = max(max_err(cas, plain), max_err(cas_lse, plain_lse))
    e = max_err(cas, ref), max_err(cas_lse, ref_lse)
    say(f"  vs plain {d_plain:.3g}; vs oracle out {e[0]:.3g} lse {e[1]:.3g} (all rows)")
    assert d_plain <= CASCADE_VS_PLAIN
    assert e[0] <= TOL and e[1] <= TOL


@pytest.mark.slow
def test_system_prompt_workload_fp8_full_rows():
    """The system-prompt workload over E4M3 pools under its cascade plan (as
    bench.py --workload system_prompt --cascade --kv fp8 runs it): every row
    against the oracle, and within 5e-4 of the plain E4M3 plan."""
    import oracle
    import paged_gqa_decode_pa_amd as pa
    spec = W.SYSTEM_PROMPT_B64
    say("cascade system-prompt workload over E4M3 pools (all rows)")
    dev = device()
    case = W.make_decode_case(spec, dev, layers=0)
    k, v = W.make_pools_e4m3(spec.num_slots, spec.num_kv_heads, spec.head_dim, W.layer_seed(spec.seed, 0), dev)
    ks, vs = W.FP8_K_SCALE, W.FP8_V_SCALE
    gi = np.array([0, spec.batch], np.int32)
    pl = np.array([spec.prefix_len], np.int32)
    fl = pa.PA_PLAN_KV_FP8
    cas, cas_lse = _run_fp8(lambda p: p.plan_cascade(case.kv_indptr, gi, pl, flags=fl), case.kv_indptr,
                            case.kv_indices, case.q, k, v, spec.num_kv_heads, ks, vs)
    plain, plain_lse = _run_fp8(lambda p: p.plan(case.kv_indptr, flags=fl), case.kv_indptr, case.kv_indices,
                                case.q, k, v, spec.num_kv_heads, ks, vs)
    assert max_err(cas, plain) <= CASCADE_VS_PLAIN and max_err(cas_lse, plain_lse) <= CASCADE_VS_PLAIN
    ref, ref_lse = oracle.load().decode_fp8(W.bits(case.q), W.codes(k), W.codes(v), case.kv_indptr,
                                            case.kv_indices, case.sm_scale, ks, vs, spec.num_kv_heads)
    e = max_err(cas, ref), max_err(cas_lse, ref_lse)
    say(f"  vs oracle out {e[0]:.3g} lse {e[1]:.3g}")
    assert e[0] <= TOL and e[1] <= TOL
    del case, k, v
    torch.cuda.empty_cache()


def test_graph_replay():
    """A captured cascade run (prefix kernel + decode kernel) replays bit-exactly."""
    import paged_gqa_decode_pa_amd as pa
    say("cascade graph replay")
    lengths = [1500, 1700, 900, 2500, 1000, 1100]
    ip, idx, q, k, v = _case(lengths, 3, 800, 32, 8, 128, 20000, seed=9)
    gi, pl = _groups(6, 3), np.array([800, 800], np.int32)
    dev = device()
    idx_dev = torch.as_tensor(idx, device=dev)
    out = torch.empty((6, 32, 128), dtype=torch.float32, device=dev)
    with pa.Plan(6, int(ip[-1]), 32, 8, 128) as plan:
        plan.plan_cascade(ip, gi, pl, flags=pa.PA_PLAN_CASCADE_ALL)
        plan.decode(q, k, v, idx_dev, W.softmax_scale(128), out)
        torch.cuda.synchronize()
        eager = out.clone()
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            plan.decode(q, k, v, idx_dev, W.softmax_scale(128), out, stream=side)
        torch.cuda.synchronize()
        for _ in range(3):
            out.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager)


@pytest.mark.parametrize("layout", ["singletons", "one_big_group"])
def test_capacity_extremes(layout):
    """The most prefix units or slots a plan has to hold: 64 one-request groups
    (pairs < workgroups, two parts each) and one group of 128 requests (four
    subgroups, 16 parts each: exactly the reserved slots)."""
    import paged_gqa_decode_pa_amd as pa
    say(f"cascade capacity {layout}")
    if layout == "singletons":
        lengths, gsize, plen = [700 + 13 * i for i in range(64)], 1, 600
    else:
        lengths, gsize, plen = [1200 + 7 * i for i in range(128)], 128, 1100
    ip, idx, q, k, v = _case(lengths, gsize, plen, 32, 8, 128, 200000, seed=len(lengths))
    gi = _groups(len(lengths), gsize)
    pl = np.full(gi.size - 1, plen, np.int32)
    _check(ip, idx, q, k, v, 8, gi, pl)
