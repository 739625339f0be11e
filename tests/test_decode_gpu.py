"""Decode parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded bf16 inputs, element by element, within 2e-3; index handling
bit-exact.  Needs an AMD GPU."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import TOL, all_rows_written, device, max_err, oracle_decode, run_decode, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _lists(lengths, num_slots, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return W.slot_lists(np.asarray(lengths), num_slots, rng)


def _case(lengths, Hq, Hkv, D, num_slots, seed):
    dev = device()
    ip, idx = _lists(lengths, num_slots, seed)
    q = W.normal_bf16((len(lengths), Hq, D), seed * 3 + 1, dev)
    k, v = W.make_pools(num_slots, Hkv, D, seed * 3 + 2, dev)
    return ip, idx, q, k, v


SMALL = [
    # (lengths, Hq, Hkv, D) -- tiles of 16 (D=128) / 8 (D=256) tokens per wave, ragged tails
    ([1, 15, 16, 17, 63, 64, 65, 200, 1023], 32, 8, 128),
    ([0, 1, 2, 300, 0, 77], 32, 8, 128),
    ([5, 129, 700], 8, 8, 128),      # group 1
    ([33, 250], 16, 8, 128),         # group 2
    ([47, 512], 64, 8, 128),         # group 8
    ([1, 7, 8, 9, 300, 1500], 16, 4, 256),
    ([3, 999], 4, 4, 256),
    ([40, 2], 16, 8, 256),
    ([100, 31], 32, 4, 256),
]


@pytest.mark.parametrize("lengths,Hq,Hkv,D", SMALL, ids=[f"{c[1]}x{c[2]}x{c[3]}-{i}" for i, c in enumerate(SMALL)])
def test_small_parity(lengths, Hq, Hkv, D):
    say(f"small parity lengths={lengths} Hq={Hq} Hkv={Hkv} D={D}")
    ip, idx, q, k, v = _case(lengths, Hq, Hkv, D, 4096, seed=sum(lengths) + Hq + D)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(D)
    out, lse = run_decode(q, k, v, ip, idx_dev, scale, Hkv)
    ref, ref_lse = oracle_decode(q, k, v, ip, idx, scale, Hkv)
    e_out, e_lse = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  max|d| out={e_out:.3g} lse={e_lse:.3g}")
    assert e_out <= TOL and e_lse <= TOL


@pytest.mark.parametrize("spec", [W.SINGLE_REQUEST_256, W.QWEN3_4B_BATCH8], ids=lambda s: s.name)
def test_workload_full_parity(spec):
    say(f"full parity {spec.name}")
    case = W.make_decode_case(spec, device(), layers=1)
    idx_dev = torch.as_tensor(case.kv_indices, device=device())
    out, lse = run_decode(case.q, case.k_pools[0], case.v_pools[0], case.kv_indptr, idx_dev,
                          case.sm_scale, spec.num_kv_heads)
    ref, ref_lse = oracle_decode(case.q, case.k_pools[0], case.v_pools[0], case.kv_indptr,
                                 case.kv_indices, case.sm_scale, spec.num_kv_heads)
    e_out, e_lse = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  max|d| out={e_out:.3g} lse={e_lse:.3g}")
    assert e_out <= TOL and e_lse <= TOL


def _bench_config_layers(spec, layers, warm_steps=6):
    """Decode the given layers of a full-size workload as the benchmark does:
    one plan object with the speed feedback on (its weights moved by a few
    warm steps first), one pa_plan, then every layer's run reusing it.
    Returns {layer: (out, lse, k, v)} with the outputs on the host."""
    import paged_gqa_decode_pa_amd as pa
    dev = device()
    ip, idx = W.decode_lists(spec)
    q = W.normal_bf16((spec.batch, spec.num_qo_heads, spec.head_dim), spec.seed, dev)
    idx_dev = torch.as_tensor(idx, device=dev)
    scale = W.softmax_scale(spec.head_dim)
    pools = {l: W.make_pools(spec.num_slots, spec.num_kv_heads, spec.head_dim,
                             W.layer_seed(spec.seed, l), dev) for l in layers}
    shape = (spec.batch, spec.num_qo_heads, spec.head_dim)
    res = {}
    with pa.Plan(spec.batch, int(ip[-1]), spec.num_qo_heads, spec.num_kv_heads, spec.head_dim) as plan:
        warm = torch.empty(shape, dtype=torch.float32, device=dev)
        for _ in range(warm_steps):
            plan.plan(ip, flags=pa.PA_PLAN_SPEED_FEEDBACK)
            for l in layers:
                plan.decode(q, pools[l][0], pools[l][1], idx_dev, scale, warm)
            torch.cuda.synchronize()
        plan.plan(ip, flags=pa.PA_PLAN_SPEED_FEEDBACK)
        outs = {l: (torch.full(shape, float("nan"), dtype=torch.float32, device=dev),
                    torch.full(shape[:2], float("nan"), dtype=torch.float32, device=dev)) for l in layers}
        for l in layers:
            plan.decode(q, pools[l][0], pools[l][1], idx_dev, scale, outs[l][0], outs[l][1])
        torch.cuda.synchronize()
        say(f"  workgroup weights in use: {plan.workgroup_weights().min():.3f} .. "
            f"{plan.workgroup_weights().max():.3f}")
    for l in layers:
        res[l] = (outs[l][0].cpu().numpy(), outs[l][1].cpu().numpy(), pools[l][0], pools[l][1])
    return ip, idx, q, scale, res


@pytest.mark.slow
@pytest.mark.parametrize("spec,layers", [(W.BATCH64_SHARED_PREFIX, (0, 17, 35)),
                                         (W.HEADDIM256_BATCH32, (0,))],
                         ids=["batch64_prefix_layers_0_17_35", "headdim256"])
def test_workload_full_rows(spec, layers):
    """Full-size workloads in the benchmark's launch configuration (one plan
    with the speed feedback, reused by every layer): every row of every
    listed layer against the oracle."""
    say(f"full-row parity {spec.name} layers {layers}")
    ip, idx, q, scale, res = _bench_config_layers(spec, layers)
    for l in layers:
        out, lse, k, v = res[l]
        ref, ref_lse = oracle_decode(q, k, v, ip, idx, scale, spec.num_kv_heads)
        e_out, e_lse = max_err(out, ref), max_err(lse, ref_lse)
        say(f"  layer {l}: max|d| out={e_out:.3g} lse={e_lse:.3g} over all {out.shape[0] * out.shape[1]} rows")
        assert e_out <= TOL and e_lse <= TOL
    del res
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [1, 2, 7, 64, 256])
def test_split_invariance(n):
    """Forcing any partition count gives the automatic result within 1e-5 and
    the oracle within 2e-3; parts may be empty."""
    say(f"forced splits {n}")
    lengths = [1, 100, 3000, 64, 255]
    ip, idx, q, k, v = _case(lengths, 32, 8, 128, 8192, seed=7)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    import paged_gqa_decode_pa_amd as pa
    auto, auto_lse = run_decode(q, k, v, ip, idx_dev, scale, 8)
    out, lse = run_decode(q, k, v, ip, idx_dev, scale, 8, flags=pa.PA_PLAN_FORCE_SPLITS(n))
    assert max_err(out, auto) <= 1e-5 and max_err(lse, auto_lse) <= 1e-5
    ref, ref_lse = oracle_decode(q, k, v, ip, idx, scale, 8)
    assert max_err(out, ref) <= TOL and max_err(lse, ref_lse) <= TOL


def test_xcd_order_is_result_neutral():
    import paged_gqa_decode_pa_amd as pa
    say("xcd order vs natural order")
    ip, idx, q, k, v = _case([700, 2000, 5, 1300] * 5, 32, 8, 128, 40000, seed=8)
    idx_dev = torch.as_tensor(idx, device=device())
    a, la = run_decode(q, k, v, ip, idx_dev, W.softmax_scale(128), 8)
    b, lb = run_decode(q, k, v, ip, idx_dev, W.softmax_scale(128), 8, flags=pa.PA_PLAN_NO_XCD_ORDER)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_single_token_is_exact():
    """L = 1: the output is the value row, bit for bit."""
    say("L=1 exactness")
    dev = device()
    B, Hq, Hkv, D, N = 40, 32, 8, 128, 5000
    ip, idx = _lists([1] * B, N, 11)
    q = W.normal_bf16((B, Hq, D), 12, dev)
    k, v = W.make_pools(N, Hkv, D, 13, dev)
    out, _ = run_decode(q, k, v, ip, torch.as_tensor(idx, device=dev), W.softmax_scale(D), Hkv)
    vrows = v[torch.as_tensor(idx, device=dev).long()].float().cpu().numpy()   # [B, Hkv, D]
    want = np.repeat(vrows, Hq // Hkv, axis=1)
    assert all_rows_written(out) and np.array_equal(out, want)


def _slot_tag_pool(num_slots, Hkv, D, dev):
    """V rows whose first four values spell the slot id in base 256 (exact in bf16)."""
    v = torch.zeros((num_slots, Hkv, D), dtype=torch.bfloat16, device=dev)
    ids = torch.arange(num_slots, device=dev, dtype=torch.int64)
    for digit in range(4):
        v[:, :, digit] = ((ids >> (8 * digit)) & 255).to(torch.bfloat16)[:, None]
    return v


@pytest.mark.parametrize("num_slots,Hq,Hkv,D", [(70000, 32, 8, 128), ((1 << 24) + 1000, 8, 1, 128),
                                                (2_300_000, 16, 8, 128), (1_048_575, 32, 8, 128),
                                                (1_600_000, 32, 8, 128), (1_100_000, 16, 4, 256)],
                         ids=["small_pool", "over_2^24_slots", "over_4GiB", "just_below_2GiB",
                              "between_2_and_4GiB", "head_dim_256_past_2GiB"])
def test_slot_tags_bit_exact(num_slots, Hq, Hkv, D):
    """Each single-slot request returns its slot id exactly, including the last
    slot of pools on both sides of 2 GiB (where row offsets stop fitting a
    signed 32-bit offset), past 4 GiB and past 2^24 slots."""
    dev = device()
    say(f"slot tags num_slots={num_slots} Hkv={Hkv} ({num_slots * Hkv * D * 2 / 2**30:.2f} GiB per pool)")
    rng = np.random.Generator(np.random.PCG64(num_slots))
    chosen = np.concatenate([[num_slots - 1, 0, num_slots - 2], rng.integers(0, num_slots, 61)]).astype(np.int32)
    B = chosen.size
    ip = np.arange(B + 1, dtype=np.int32)
    v = _slot_tag_pool(num_slots, Hkv, D, dev)
    k = torch.zeros_like(v)
    q = W.normal_bf16((B, Hq, D), 5, dev)
    out, _ = run_decode(q, k, v, ip, torch.as_tensor(chosen, device=dev), W.softmax_scale(D), Hkv)
    digits = np.rint(out[:, :, :4]).astype(np.int64)
    decoded = digits[..., 0] + 256 * digits[..., 1] + 65536 * digits[..., 2] + 16777216 * digits[..., 3]
    assert np.array_equal(decoded, np.repeat(chosen[:, None], Hq, axis=1))
    assert np.array_equal(out[:, :, :4], digits.astype(np.float32))
    del v, k
    torch.cuda.empty_cache()


def test_poisoned_pool_matches_clean():
    """NaN in every slot no list references changes nothing (no stray reads)."""
    say("poisoned pool")
    lengths = [1, 17, 250, 1000, 3]
    ip, idx, q, k, v = _case(lengths, 32, 8, 128, 6000, seed=21)
    idx_dev = torch.as_tensor(idx, device=device())
    clean, clean_lse = run_decode(q, k, v, ip, idx_dev, W.softmax_scale(128), 8)
    W.poison_unreferenced(k, idx)
    W.poison_unreferenced(v, idx)
    out, lse = run_decode(q, k, v, ip, idx_dev, W.softmax_scale(128), 8)
    assert np.array_equal(out, clean) and np.array_equal(lse, clean_lse)


def test_deterministic():
    say("run-to-run determinism")
    ip, idx, q, k, v = _case([3000, 4000, 10], 32, 8, 128, 9000, seed=22)
    idx_dev = torch.as_tensor(idx, device=device())
    a = run_decode(q, k, v, ip, idx_dev, W.softmax_scale(128), 8)
    b = run_decode(q, k, v, ip, idx_dev, W.softmax_scale(128), 8)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_empty_lists():
    say("empty lists")
    ip, idx, q, k, v = _case([0, 5, 0, 0], 32, 8, 128, 100, seed=23)
    out, lse = run_decode(q, k, v, ip, torch.as_tensor(idx, device=device()), W.softmax_scale(128), 8)
    for b in (0, 2, 3):
        assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
    ref, _ = oracle_decode(q, k, v, ip, idx, W.softmax_scale(128), 8)
    assert max_err(out[1], ref[1]) <= TOL


def test_fused_pool_layout():
    """A [slots, 2, Hkv, D] buffer with slot_stride = 2*Hkv*D gives the same bits."""
    say("fused KV buffer")
    dev = device()
    ip, idx, q, k, v = _case([123, 456], 32, 8, 128, 2000, seed=24)
    fused = torch.stack([k, v], dim=1).contiguous()          # [N, 2, Hkv, D]
    idx_dev = torch.as_tensor(idx, device=dev)
    a = run_decode(q, k, v, ip, idx_dev, W.softmax_scale(128), 8)
    b = run_decode(q, fused[:, 0], fused[:, 1], ip, idx_dev, W.softmax_scale(128), 8)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_shared_and_duplicate_slots():
    """Lists overlapping across requests and repeating a slot inside one list."""
    say("shared and duplicate slots")
    dev = device()
    idx = np.array([5, 6, 7, 5, 5, 6, 7, 7, 9, 5, 6], np.int32)
    ip = np.array([0, 3, 8, 11], np.int32)
    q = W.normal_bf16((3, 32, 128), 31, dev)
    k, v = W.make_pools(16, 8, 128, 32, dev)
    out, lse = run_decode(q, k, v, ip, torch.as_tensor(idx, device=dev), W.softmax_scale(128), 8)
    ref, ref_lse = oracle_decode(q, k, v, ip, idx, W.softmax_scale(128), 8)
    assert max_err(out, ref) <= TOL and max_err(lse, ref_lse) <= TOL


def test_plan_reused_across_layers():
    """One pa_plan, several layers with their own pools (one decode step)."""
    import paged_gqa_decode_pa_amd as pa
    say("plan reuse over 3 layers")
    dev = device()
    spec = W.QWEN3_4B_BATCH8
    case = W.make_decode_case(spec, dev, layers=3)
    idx_dev = torch.as_tensor(case.kv_indices, device=dev)
    outs = []
    with pa.Plan(spec.batch, int(case.kv_indptr[-1]), 32, 8, 128) as plan:
        plan.plan(case.kv_indptr)
        for layer in range(3):
            o = torch.full((spec.batch, 32, 128), float("nan"), dtype=torch.float32, device=dev)
            plan.decode(case.q, case.k_pools[layer], case.v_pools[layer], idx_dev, case.sm_scale, o)
            outs.append(o)
        torch.cuda.synchronize()
    for layer in range(3):
        ref, _ = oracle_decode(case.q, case.k_pools[layer], case.v_pools[layer], case.kv_indptr,
                               case.kv_indices, case.sm_scale, 8)
        assert max_err(outs[layer].cpu().numpy(), ref) <= TOL


def test_run_errors_are_reported():
    import paged_gqa_decode_pa_amd as pa
    say("error paths")
    dev = device()
    ip, idx, q, k, v = _case([10, 20], 32, 8, 128, 100, seed=25)
    idx_dev = torch.as_tensor(idx, device=dev)
    out = torch.empty((2, 32, 128), dtype=torch.float32, device=dev)
    with pa.Plan(2, 30, 32, 8, 128) as plan:
        with pytest.raises(pa.PAError) as e:                  # no pa_plan yet
            plan.decode(q, k, v, idx_dev, 0.1, out)
        assert e.value.status == pa.PA_ERR_PLAN_MISMATCH
        with pytest.raises(pa.PAError) as e:                  # batch above capacity
            plan.plan(np.array([0, 1, 2, 3], np.int32))
        assert e.value.status == pa.PA_ERR_CAPACITY
        with pytest.raises(pa.PAError) as e:                  # tokens above capacity
            plan.plan(np.array([0, 20, 31], np.int32))
        assert e.value.status == pa.PA_ERR_CAPACITY
        plan.plan(ip)
        with pytest.raises(pa.PAError) as e:                  # decode plan, prefill run
            plan.prefill(q, k, v, idx_dev, 0.1, out)
        assert e.value.status == pa.PA_ERR_PLAN_MISMATCH
        qflat = torch.empty(q.numel() + 8, dtype=torch.bfloat16, device=dev)
        q_mis = qflat[1:1 + q.numel()].view(q.shape)          # 2-byte misaligned
        with pytest.raises(pa.PAError) as e:
            plan.decode(q_mis, k, v, idx_dev, 0.1, out)
        assert e.value.status == pa.PA_ERR_INVALID_ARG
        with pytest.raises(pa.PAError) as e:
            plan.decode(q, k, v, idx_dev, float("nan"), out)
        assert e.value.status == pa.PA_ERR_INVALID_ARG
        with pytest.raises(pa.PAError) as e:
            plan.decode(q, k, v, idx_dev, 0.1, out, slot_stride=100)
        assert e.value.status == pa.PA_ERR_INVALID_ARG
        plan.decode(q, k, v, idx_dev, 0.1, out)                # still usable
        torch.cuda.synchronize()


def test_profile_events():
    import paged_gqa_decode_pa_amd as pa
    say("kernel timing events")
    dev = device()
    ip, idx, q, k, v = _case([2000] * 8, 32, 8, 128, 20000, seed=26)
    idx_dev = torch.as_tensor(idx, device=dev)
    out = torch.empty((8, 32, 128), dtype=torch.float32, device=dev)
    with pa.Plan(8, int(ip[-1]), 32, 8, 128) as plan:
        plan.plan(ip)
        pa.pa_profile_begin(plan.handle, 4)
        for _ in range(6):
            plan.decode(q, k, v, idx_dev, 0.1, out)
        ms, n = pa.pa_profile_end(plan.handle)
    assert n == 4 and ms > 0


@pytest.mark.parametrize("flags_n", [0, 7, 64])
def test_merge_protocol_repeatable(flags_n):
    """Split lists are merged in-kernel by the part that arrives last.  Many
    back-to-back launches (arrival counts reset by the kernels themselves)
    must give bit-identical results, equal to the oracle within 2e-3."""
    import paged_gqa_decode_pa_amd as pa
    say(f"in-kernel merge repeatability, forced splits {flags_n}")
    dev = device()
    spec = W.QWEN3_4B_BATCH8
    case = W.make_decode_case(spec, dev, layers=1)
    idx = torch.as_tensor(case.kv_indices, device=dev)
    flags = pa.PA_PLAN_FORCE_SPLITS(flags_n) if flags_n else 0
    capacity = max(int(case.kv_indptr[-1]), spec.batch * flags_n * 256)
    outs = [torch.full((spec.batch, 32, 128), float("nan"), dtype=torch.float32, device=dev)
            for _ in range(40)]
    with pa.Plan(spec.batch, capacity, 32, 8, 128) as plan:
        plan.plan(case.kv_indptr, flags=flags)
        for o in outs:
            plan.decode(case.q, case.k_pools[0], case.v_pools[0], idx, case.sm_scale, o)
        torch.cuda.synchronize()
    first = outs[0].cpu().numpy()
    for o in outs[1:]:
        assert np.array_equal(o.cpu().numpy(), first)
    ref, _ = oracle_decode(case.q, case.k_pools[0], case.v_pools[0], case.kv_indptr,
                           case.kv_indices, case.sm_scale, 8)
    assert max_err(first, ref) <= TOL


def test_plan_info_and_binding_shape_checks():
    """pa_plan_info reports the last plan; the binding rejects tensors that do
    not match it before anything reaches the C ABI."""
    import paged_gqa_decode_pa_amd as pa
    say("plan info and binding shape checks")
    dev = device()
    ip, idx, q, k, v = _case([10, 20, 30], 32, 8, 128, 100, seed=27)
    idx_dev = torch.as_tensor(idx, device=dev)
    out = torch.full((3, 32, 128), float("nan"), dtype=torch.float32, device=dev)
    with pa.Plan(4, 100, 32, 8, 128) as plan:
        assert plan.info()["mode"] == 0
        plan.plan(ip)
        assert plan.info() == dict(mode=1, rows=3, num_qo_heads=32, num_kv_heads=8, head_dim=128)
        with pytest.raises(ValueError):                      # q of another batch
            plan.decode(q[:2].contiguous(), k, v, idx_dev, 0.1, out[:2])
        with pytest.raises(ValueError):                      # out too small
            plan.decode(q, k, v, idx_dev, 0.1, out[:2])
        with pytest.raises(ValueError):                      # strided slot ids
            plan.decode(q, k, v, torch.as_tensor(np.repeat(idx, 2), device=dev)[::2], 0.1, out)
        with pytest.raises(ValueError):                      # V pool shorter than num_slots
            plan.decode(q, k, v[:50], idx_dev, 0.1, out, num_slots=100)
        plan.decode(q, k, v, idx_dev, W.softmax_scale(128), out)
        torch.cuda.synchronize()
    ref, ref_lse = oracle_decode(q, k, v, ip, idx, W.softmax_scale(128), 8)
    assert max_err(out.cpu().numpy(), ref) <= TOL


def test_index_check_debug_mode(monkeypatch):
    """With the PA_CHECK debug option, a run whose slot list holds an id
    outside the pool is refused on the host (the kernel never sees it)."""
    import paged_gqa_decode_pa_amd as pa
    say("PA_CHECK debug mode")
    monkeypatch.setattr(pa, "CHECK_INDICES", True)
    dev = device()
    ip, idx, q, k, v = _case([10, 20], 32, 8, 128, 100, seed=28)
    bad = idx.copy()
    bad[13] = 100
    out = torch.full((2, 32, 128), float("nan"), dtype=torch.float32, device=dev)
    with pa.Plan(2, 30, 32, 8, 128) as plan:
        plan.plan(ip)
        with pytest.raises(pa.PAError) as e:
            plan.decode(q, k, v, torch.as_tensor(bad, device=dev), 0.1, out)
        assert e.value.status == pa.PA_ERR_INVALID_ARG and "kv_indices[13]" in e.value.detail
        plan.decode(q, k, v, torch.as_tensor(idx, device=dev), W.softmax_scale(128), out)
        torch.cuda.synchronize()
    assert all_rows_written(out.cpu().numpy())
