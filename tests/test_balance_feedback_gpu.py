"""Work weights of the automatic decode split (per XCD, set by the caller;
per workgroup, measured by PA_PLAN_SPEED_FEEDBACK): a weighted partition
gives the unweighted result up to summation order and the oracle within
2e-3, the feedback keeps every step's result within the same bounds while it
moves the weights, and the weights stay in their documented range.  Needs an
AMD GPU."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import TOL, device, max_err, oracle_decode, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

HQ, HKV, D = 32, 8, 128


def _fill_case(seed):
    """Enough list entries that the automatic split fills every workgroup
    slot of the GPU (the only launches whose timing feeds the weights)."""
    dev = device()
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = rng.integers(2000, 6000, size=16)
    ip, idx = W.slot_lists(lengths, 120000, rng)
    q = W.normal_bf16((16, HQ, D), seed + 1, dev)
    k, v = W.make_pools(120000, HKV, D, seed + 2, dev)
    return ip, idx, q, k, v


def _run(plan, q, k, v, idx_dev, scale):
    out = torch.full((q.shape[0], HQ, D), float("nan"), dtype=torch.float32, device=q.device)
    lse = torch.full((q.shape[0], HQ), float("nan"), dtype=torch.float32, device=q.device)
    plan.decode(q, k, v, idx_dev, scale, out, lse)
    return out, lse


def test_weights_roundtrip_and_validation():
    import paged_gqa_decode_pa_amd as pa
    say("xcd weights set/get")
    with pa.Plan(4, 1000, HQ, HKV, D) as plan:
        w = plan.xcd_weights()
        assert w.size == pa.PA_NUM_XCD and np.all(w == 1.0)
        ww = plan.workgroup_weights()
        assert ww.size >= 256 and np.all(ww == 1.0)
        plan.set_xcd_weights([2.0, 2.0, 2.0, 2.0, 1.0, 1.0, 1.0, 1.0])
        got = plan.xcd_weights()
        np.testing.assert_allclose(got, [4 / 3] * 4 + [2 / 3] * 4, rtol=1e-6)
        for bad in ([1.0] * 7, [1.0] * 7 + [0.1], [1.0] * 7 + [5.0], [1.0] * 7 + [float("nan")]):
            with pytest.raises(pa.PAError) as e:
                plan.set_xcd_weights(bad)
            assert e.value.status == pa.PA_ERR_INVALID_ARG
        np.testing.assert_allclose(plan.xcd_weights(), got)   # unchanged by the failures


def test_weighted_partition_parity():
    import paged_gqa_decode_pa_amd as pa
    say("weighted partition vs equal split vs oracle")
    ip, idx, q, k, v = _fill_case(21)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(D)
    with pa.Plan(16, int(ip[-1]), HQ, HKV, D) as plan:
        plan.plan(ip)
        a, la = _run(plan, q, k, v, idx_dev, scale)
        plan.set_xcd_weights([0.6, 1.4, 1.0, 1.2, 0.8, 1.0, 1.3, 0.7])
        plan.plan(ip)
        b, lb = _run(plan, q, k, v, idx_dev, scale)
        torch.cuda.synchronize()
    a, la, b, lb = (t.cpu().numpy() for t in (a, la, b, lb))
    assert max_err(b, a) <= 1e-5 and max_err(lb, la) <= 1e-5
    ref, ref_lse = oracle_decode(q, k, v, ip, idx, scale, HKV)
    e = max_err(b, ref), max_err(lb, ref_lse)
    say(f"  max|d| out={e[0]:.3g} lse={e[1]:.3g}")
    assert e[0] <= TOL and e[1] <= TOL


def test_feedback_over_steps():
    """Eight decode steps of two layers with the feedback on: every step's
    output matches the first within 1e-5 (only the cut points move), the
    first and last match the oracle, the workgroup weights leave 1 once the
    clock copies arrive and stay within bounds with mean 1."""
    import paged_gqa_decode_pa_amd as pa
    say("speed feedback over 8 steps")
    ip, idx, q, k, v = _fill_case(33)
    k2, v2 = W.make_pools(120000, HKV, D, 99, device())
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(D)
    outs, weights = [], []
    with pa.Plan(16, int(ip[-1]), HQ, HKV, D) as plan:
        for step in range(8):
            plan.plan(ip, flags=pa.PA_PLAN_SPEED_FEEDBACK)
            weights.append(plan.workgroup_weights())
            o0, l0 = _run(plan, q, k, v, idx_dev, scale)
            o1, _ = _run(plan, q, k2, v2, idx_dev, scale)
            torch.cuda.synchronize()
            outs.append((o0.cpu().numpy(), l0.cpu().numpy(), o1.cpu().numpy()))
        final = plan.workgroup_weights()
        assert np.all(plan.xcd_weights() == 1.0)   # the feedback leaves the XCD weights alone
    say(f"  weight spread per step: {[(round(float(w.min()), 3), round(float(w.max()), 3)) for w in weights]}")
    for o0, l0, o1 in outs[1:]:
        assert max_err(o0, outs[0][0]) <= 1e-5 and max_err(l0, outs[0][1]) <= 1e-5
        assert max_err(o1, outs[0][2]) <= 1e-5
    ref, ref_lse = oracle_decode(q, k, v, ip, idx, scale, HKV)
    for o0, l0, _ in (outs[0], outs[-1]):
        assert max_err(o0, ref) <= TOL and max_err(l0, ref_lse) <= TOL
    assert np.all(weights[0] == 1.0)
    assert np.any(final != 1.0), "no clock record reached the plan"
    for w in weights + [final]:
        assert np.all(w >= 0.5 / 1.5 - 1e-6) and np.all(w <= 1.5 * 1.5 + 1e-6)
        assert abs(float(w.mean()) - 1.0) < 1e-3
