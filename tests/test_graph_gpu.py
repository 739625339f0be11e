"""Capture of a multi-layer step in a HIP graph.

A plan is computed once per step and every layer's run reads the plan's
device tables, so the runs of one step can be captured once and replayed
(the plan/run split of the Agent-Infer page, section "分页 KV 缓存"; graph
capture of the decode step is stage 6 of the table in its section "优化历程").
Runs allocate nothing and reset their own arrival counters, so a replay must
give the eager result bit for bit.  Each replay follows eager work (the
outputs are poisoned) and a synchronisation, and every replay is checked."""
import numpy as np
import pytest
import torch

import paged_gqa_decode_pa_amd as pa
import workloads as W
from gpu_util import TOL, device, max_err, oracle_decode, oracle_prefill, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LAYERS = 4


def _replay_and_check(step, outs, eager, replays=3):
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        step(s)
    torch.cuda.synchronize()
    for rep in range(replays):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert np.array_equal(o.cpu().numpy(), e, equal_nan=True), f"replay {rep} differs"
    del g


@pytest.mark.parametrize("splits", [0, 3], ids=["auto", "forced3"])
def test_decode_layers_graph_replay(splits):
    say(f"graph capture: {LAYERS}-layer decode step, B=8, splits={splits}")
    dev = device()
    rng = np.random.Generator(np.random.PCG64(31))
    B, Hq, Hkv, D, N = 8, 32, 8, 128, 65536
    ip, idx = W.slot_lists(rng.integers(512, 4097, B), N, rng)
    q = W.normal_bf16((B, Hq, D), 32, dev)
    pools = [W.make_pools(N, Hkv, D, 40 + l, dev) for l in range(LAYERS)]
    idx_dev = torch.as_tensor(idx, device=dev)
    scale = W.softmax_scale(D)
    outs = [torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
    lses = [torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
    with pa.Plan(B, int(ip[-1]), Hq, Hkv, D) as plan:
        plan.plan(ip, flags=pa.PA_PLAN_FORCE_SPLITS(splits) if splits else 0)

        def step(stream):
            for l in range(LAYERS):
                plan.decode(q, pools[l][0], pools[l][1], idx_dev, scale, outs[l], lses[l], stream=stream)

        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        eager = [o.cpu().numpy() for o in outs] + [x.cpu().numpy() for x in lses]
        for l in range(LAYERS):
            ref, ref_lse = oracle_decode(q, pools[l][0], pools[l][1], ip, idx, scale, Hkv)
            assert max_err(eager[l], ref) <= TOL and max_err(eager[LAYERS + l], ref_lse) <= TOL
        _replay_and_check(step, outs + lses, eager)


def test_decode_graph_replay_after_replan_with_other_cuts():
    """A replay reads the device tables of the plan current at replay time.
    The same lists re-planned with other budgets (XCD weights here; the speed
    feedback does the same from step to step) keep the workgroup count but
    cut the lists into other units and merges: the captured launches must
    find them at the same table addresses, and the replay must equal an eager
    run of the new plan bit for bit (regression: the merge table used to
    follow the units, so its address moved with their count)."""
    say("graph replay after a re-plan of the same lists with other cuts")
    dev = device()
    rng = np.random.Generator(np.random.PCG64(43))
    B, Hq, Hkv, D, N = 24, 32, 8, 128, 65536
    ip, idx = W.slot_lists(rng.integers(300, 4097, B), N, rng)
    q = W.normal_bf16((B, Hq, D), 44, dev)
    pools = [W.make_pools(N, Hkv, D, 45 + l, dev) for l in range(2)]
    idx_dev = torch.as_tensor(idx, device=dev)
    scale = W.softmax_scale(D)
    outs = [torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev) for _ in range(2)]
    w_a, w_b = [1.0] * 8, [3.0, 0.3, 1.0, 1.0, 0.5, 2.0, 1.0, 0.7]
    for mw in (256, 512, 768):
        a = pa.pa_partition(ip, None, Hq, Hkv, D, max_workgroups=mw, xcd_weights=w_a)
        b = pa.pa_partition(ip, None, Hq, Hkv, D, max_workgroups=mw, xcd_weights=w_b)
        say(f"  {mw} workgroups: units {a[0][-1]} -> {b[0][-1]}, merges {len(a[2])} -> {len(b[2])}")
        assert len(a[0]) == len(b[0]) and (a[0][-1] != b[0][-1] or len(a[2]) != len(b[2]))
    with pa.Plan(B, int(ip[-1]), Hq, Hkv, D) as plan:
        pa.pa_plan_set_xcd_weights(plan.handle, w_a)
        plan.plan(ip)

        def step(stream):
            for l in range(2):
                plan.decode(q, pools[l][0], pools[l][1], idx_dev, scale, outs[l], stream=stream)

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step(s)
        torch.cuda.synchronize()
        pa.pa_plan_set_xcd_weights(plan.handle, w_b)
        plan.plan(ip)
        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        eager = [o.cpu().numpy() for o in outs]
        for l in range(2):
            ref, _ = oracle_decode(q, pools[l][0], pools[l][1], ip, idx, scale, Hkv)
            assert max_err(eager[l], ref) <= TOL
        for rep in range(3):
            for o in outs:
                o.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for o, e in zip(outs, eager):
                assert np.array_equal(o.cpu().numpy(), e), f"replay {rep} differs"
        del g


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_layers_graph_replay(kv):
    say(f"graph capture: {LAYERS}-layer prefill step with split KV ranges, {kv} pools")
    import oracle
    fp8 = kv == "fp8"
    ks, vs = W.FP8_K_SCALE, W.FP8_V_SCALE
    dev = device()
    rng = np.random.Generator(np.random.PCG64(37))
    Hq, Hkv, D, N = 32, 8, 128, 16384
    reqs = [(700, 64), (1500, 16)]     # few tiles: KV ranges are cut and merged
    ip, idx = W.slot_lists(np.asarray([L for L, _ in reqs]), N, rng)
    qo = np.concatenate([[0], np.cumsum([C for _, C in reqs])]).astype(np.int32)
    T = int(qo[-1])
    q = W.normal_bf16((T, Hq, D), 38, dev)
    make = W.make_pools_e4m3 if fp8 else W.make_pools
    pools = [make(N, Hkv, D, 50 + l, dev) for l in range(LAYERS)]
    idx_dev = torch.as_tensor(idx, device=dev)
    scale = W.softmax_scale(D)
    outs = [torch.full((T, Hq, D), float("nan"), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
    lses = [torch.full((T, Hq), float("nan"), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
    with pa.Plan(len(reqs), int(ip[-1]), Hq, Hkv, D, max_q_total=T) as plan:
        plan.plan(ip, qo)

        def step(stream):
            for l in range(LAYERS):
                if fp8:
                    plan.prefill_fp8(q, pools[l][0], pools[l][1], idx_dev, scale, ks, vs, outs[l], lses[l],
                                     stream=stream)
                else:
                    plan.prefill(q, pools[l][0], pools[l][1], idx_dev, scale, outs[l], lses[l], stream=stream)

        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        eager = [o.cpu().numpy() for o in outs] + [x.cpu().numpy() for x in lses]
        for l in range(LAYERS):
            if fp8:
                ref, ref_lse = oracle.load().prefill_fp8(W.bits(q), W.codes(pools[l][0]), W.codes(pools[l][1]),
                                                         qo, ip, idx, scale, ks, vs, Hkv)
            else:
                ref, ref_lse = oracle_prefill(q, pools[l][0], pools[l][1], qo, ip, idx, scale, Hkv)
            assert max_err(eager[l], ref) <= TOL and max_err(eager[LAYERS + l], ref_lse) <= TOL
        _replay_and_check(step, outs + lses, eager)


def test_fp8_decode_step_with_append_graph_replay():
    """A whole decode step over 8-bit pools captured once: per layer, the
    step's new token of every request appended (K rotated, both encoded) at
    the end of its list, then the fp8 decode over the lists.  The appended
    slots are wiped before every replay, so the captured appends must write
    them again; outputs bit for bit as the eager step's, which match the
    oracle over the pools the appends produced."""
    import oracle
    say(f"graph capture: {LAYERS}-layer fp8 decode step with appends")
    dev = device()
    rng = np.random.Generator(np.random.PCG64(39))
    B, Hq, Hkv, D, N = 8, 32, 8, 128, 65536
    ks, vs = W.FP8_K_SCALE, W.FP8_V_SCALE
    lengths = rng.integers(300, 3000, B)
    ip, idx = W.slot_lists(lengths, N, rng)
    new_slots = torch.as_tensor(idx[ip[1:] - 1].astype(np.int32), device=dev)
    positions = torch.as_tensor((lengths - 1).astype(np.int32), device=dev)
    q = W.normal_bf16((B, Hq, D), 40, dev)
    k_new = [W.normal_bf16((B, Hkv, D), 41 + 2 * l, dev) for l in range(LAYERS)]
    v_new = [W.normal_bf16((B, Hkv, D), 42 + 2 * l, dev) for l in range(LAYERS)]
    pools = [W.make_pools_e4m3(N, Hkv, D, 60 + l, dev) for l in range(LAYERS)]
    idx_dev = torch.as_tensor(idx, device=dev)
    scale = W.softmax_scale(D)
    outs = [torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
    sel = new_slots.to(torch.int64)
    with pa.Plan(B, int(ip[-1]), Hq, Hkv, D) as plan:
        plan.plan(ip, flags=pa.PA_PLAN_KV_FP8)

        def step(stream):
            for l in range(LAYERS):
                pa.pa_kv_append_fp8(k_new[l], v_new[l], new_slots, pools[l][0], pools[l][1], ks, vs,
                                    positions=positions, rope_theta=1e6, stream=stream)
                plan.decode_fp8(q, pools[l][0], pools[l][1], idx_dev, scale, ks, vs, outs[l], stream=stream)

        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        eager = [o.cpu().numpy() for o in outs]
        for l in range(LAYERS):
            ref, _ = oracle.load().decode_fp8(W.bits(q), W.codes(pools[l][0]), W.codes(pools[l][1]), ip, idx,
                                              scale, ks, vs, Hkv)
            assert max_err(eager[l], ref) <= TOL
        appended = [(W.codes(pools[l][0].view(torch.uint8)[sel]), W.codes(pools[l][1].view(torch.uint8)[sel]))
                    for l in range(LAYERS)]
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=s):
            step(s)
        torch.cuda.synchronize()
        for rep in range(3):
            for l in range(LAYERS):
                outs[l].fill_(float("nan"))
                pools[l][0].view(torch.uint8)[sel] = 0
                pools[l][1].view(torch.uint8)[sel] = 0
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for l in range(LAYERS):
                assert np.array_equal(outs[l].cpu().numpy(), eager[l]), f"replay {rep} layer {l} differs"
                assert np.array_equal(W.codes(pools[l][0].view(torch.uint8)[sel]), appended[l][0])
                assert np.array_equal(W.codes(pools[l][1].view(torch.uint8)[sel]), appended[l][1])
        del g


def test_one_graph_per_batch_size():
    """The serving pattern of a captured decode step: one plan, one set of
    static buffers and one captured step per batch size.  Each step writes
    its new lists and queries into that batch size's buffers, re-plans, and
    replays the captured step while pa_plan_launch_shape is unchanged (a step
    whose work fills the GPU keeps it whatever its lengths), capturing again
    otherwise.  Every replay equals an eager run of the same plan bit for bit
    and matches the oracle; batch 32 is captured once for all its steps."""
    say("one captured decode step per batch size, lists changing every step")
    dev = device()
    Hq, Hkv, D, N = 32, 8, 128, 400000
    rng = np.random.Generator(np.random.PCG64(47))
    pools = [W.make_pools(N, Hkv, D, 48 + l, dev) for l in range(2)]
    scale = W.softmax_scale(D)
    cap_entries = 32 * 4096
    slots = {}      # batch -> plan, buffers, graph and its launch shape
    captures = {32: 0, 8: 0}
    try:
        for step, B in enumerate([32, 8, 32, 32, 8]):
            lo, hi = (2048, 4096) if B == 32 else (512, 4096)
            ip, idx = W.slot_lists(rng.integers(lo, hi + 1, B), N, rng)
            if B not in slots:
                slots[B] = {"plan": pa.Plan(B, cap_entries, Hq, Hkv, D),
                            "q": torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev),
                            "idx": torch.zeros(cap_entries, dtype=torch.int32, device=dev),
                            "outs": [torch.empty((B, Hq, D), dtype=torch.float32, device=dev) for _ in range(2)],
                            "graph": None, "shape": None}
            sl = slots[B]
            plan, qb, ib, outs = sl["plan"], sl["q"], sl["idx"], sl["outs"]
            qb.copy_(W.normal_bf16((B, Hq, D), 49 + step, dev))
            ib[:idx.size].copy_(torch.as_tensor(idx, device=dev))
            plan.plan(ip)
            shape = plan.launch_shape()

            def layers(stream, dst=outs):
                for l in range(2):
                    plan.decode(qb, pools[l][0], pools[l][1], ib, scale, dst[l], stream=stream)

            if sl["graph"] is None or sl["shape"] != shape:
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    layers(s)
                torch.cuda.synchronize()
                sl["graph"], sl["shape"] = g, shape
                captures[B] += 1
            eager = [torch.full_like(o, float("nan")) for o in outs]
            layers(torch.cuda.current_stream(), eager)
            for o in outs:
                o.fill_(float("nan"))
            torch.cuda.synchronize()
            sl["graph"].replay()
            torch.cuda.synchronize()
            say(f"  step {step}: batch {B}, launch shape {shape}, captures so far {captures}")
            for l in range(2):
                got = outs[l].cpu().numpy()
                assert np.array_equal(got, eager[l].cpu().numpy()), f"step {step} layer {l}: replay differs"
                ref, _ = oracle_decode(qb, pools[l][0], pools[l][1], ip, idx, scale, Hkv)
                assert max_err(got, ref) <= TOL
        assert captures[32] == 1, captures
    finally:
        for sl in slots.values():
            sl["graph"] = None
            sl["plan"].close()
