"""Plans are independent: each owns its work table, partial results and
arrival counters, so runs of different plans may overlap on different
streams (two runs of one plan may not).  Two plans over different lists,
one decode and one chunked prefill, split so that both merge partial
results, are issued alternately on two streams (default priority) many
times; every output must equal that plan's result run alone, bit for bit,
and the results match the fp64 oracle.  Needs an AMD GPU."""
import numpy as np
import pytest
import torch

import paged_gqa_decode_pa_amd as pa
import workloads as W
from gpu_util import TOL, device, max_err, oracle_decode, oracle_prefill, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ROUNDS = 20


def test_two_plans_on_two_streams():
    say("two plans, two streams, interleaved")
    dev = device()
    Hq, Hkv, D, N = 32, 8, 128, 65536
    rng = np.random.Generator(np.random.PCG64(91))
    k, v = W.make_pools(N, Hkv, D, 92, dev)
    # plan A: decode over 16 lists, split into 5 parts each
    ip_a, idx_a = W.slot_lists(rng.integers(600, 3000, 16), N // 2, rng)
    q_a = W.normal_bf16((16, Hq, D), 93, dev)
    # plan B: chunked prefill of 4 requests (slots in the other half of the pool)
    reqs = [(1500, 64), (900, 16), (2500, 40), (300, 300)]
    ip_b, idx_b = W.slot_lists(np.asarray([L for L, _ in reqs]), N // 2, rng)
    idx_b = idx_b + N // 2
    qo_b = np.concatenate([[0], np.cumsum([C for _, C in reqs])]).astype(np.int32)
    T = int(qo_b[-1])
    q_b = W.normal_bf16((T, Hq, D), 94, dev)
    ia, ib = torch.as_tensor(idx_a, device=dev), torch.as_tensor(idx_b, device=dev)
    scale = W.softmax_scale(D)
    s1, s2 = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    with pa.Plan(16, int(ip_a[-1]) + 16 * 5 * 256, Hq, Hkv, D) as pa_, \
            pa.Plan(4, int(ip_b[-1]), Hq, Hkv, D, max_q_total=T) as pb:
        pa_.plan(ip_a, flags=pa.PA_PLAN_FORCE_SPLITS(5))
        pb.plan(ip_b, qo_b)
        base_a = torch.empty((16, Hq, D), dtype=torch.float32, device=dev)
        base_b = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
        pa_.decode(q_a, k, v, ia, scale, base_a)
        torch.cuda.synchronize()
        pb.prefill(q_b, k, v, ib, scale, base_b)
        torch.cuda.synchronize()
        ref_a, _ = oracle_decode(q_a, k, v, ip_a, idx_a, scale, Hkv)
        ref_b, _ = oracle_prefill(q_b, k, v, qo_b, ip_b, idx_b, scale, Hkv)
        assert max_err(base_a.cpu().numpy(), ref_a) <= TOL
        assert max_err(base_b.cpu().numpy(), ref_b) <= TOL
        outs_a = [torch.full_like(base_a, float("nan")) for _ in range(ROUNDS)]
        outs_b = [torch.full_like(base_b, float("nan")) for _ in range(ROUNDS)]
        s1.wait_stream(torch.cuda.current_stream(dev))
        s2.wait_stream(torch.cuda.current_stream(dev))
        for r in range(ROUNDS):
            pa_.decode(q_a, k, v, ia, scale, outs_a[r], stream=s1)
            pb.prefill(q_b, k, v, ib, scale, outs_b[r], stream=s2)
        torch.cuda.synchronize()
        for r in range(ROUNDS):
            assert torch.equal(outs_a[r], base_a), f"decode round {r} differs"
            assert torch.equal(outs_b[r], base_b), f"prefill round {r} differs"
