"""The append step (pa_kv_append): new tokens' K/V rows written to their
slots, K (and optionally Q) rotated by RoPE, against the fp64 oracle's
rotation on the same bf16 bits.  Slot placement and V are bit-exact; a
rotated value must equal the oracle's double-precision rotation rounded once
to bf16 (nearest-even, no float32 step), bit for bit: the kernel also rounds
its double-precision rotation once.  Needs a GPU."""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_pa_amd as pa
import workloads as W
from gpu_util import TOL, device, max_err, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

THETA = 1e6   # Qwen3's RoPE base


def _bf16_round(x64: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, rounded once to nearest-even straight from the
    double (no float32 step, so no double rounding).  Values must be zero or
    normal in bf16 (|x| >= 2^-126), as every rotated N(0, 1) value here is."""
    x = np.ascontiguousarray(x64, dtype=np.float64)
    mag = np.abs(x)
    assert np.all((mag == 0) | ((mag >= 2.0 ** -126) & (mag < 3.0e38))), "outside bf16's normal range"
    u = x.view(np.uint64)
    # keep 7 of the double's 52 fraction bits: add half an ulp of the kept
    # part (minus one when the kept part is even: ties go to even), truncate
    drop = np.uint64(45)
    lsb = (u >> drop) & np.uint64(1)
    r = ((u + (np.uint64(1) << np.uint64(44)) - np.uint64(1) + lsb) >> drop) << drop
    f32 = r.view(np.float64).astype(np.float32)   # exact: r holds a bf16 value
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    def key(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(key(a_bits) - key(b_bits))


def _pools(N, Hkv, D, seed, dev):
    k, v = W.make_pools(N, Hkv, D, seed, dev)
    return k, v, W.bits(k).copy(), W.bits(v).copy()


def _check_append(T, Hq, Hkv, D, N, seed, theta=THETA, with_q=True, positions_hi=40000):
    dev = device()
    rng = np.random.Generator(np.random.PCG64(seed))
    k_pool, v_pool, k_before, v_before = _pools(N, Hkv, D, seed + 1, dev)
    k_new = W.normal_bf16((T, Hkv, D), seed + 2, dev)
    v_new = W.normal_bf16((T, Hkv, D), seed + 3, dev)
    q = W.normal_bf16((T, Hq, D), seed + 4, dev) if with_q else None
    q_before = W.bits(q).copy() if with_q else None
    out_loc = rng.permutation(N)[:T].astype(np.int32)
    positions = rng.integers(0, positions_hi, T).astype(np.int32)
    pa.pa_kv_append(k_new, v_new, torch.as_tensor(out_loc, device=dev), k_pool, v_pool,
                    positions=torch.as_tensor(positions, device=dev), rope_theta=theta, q=q)
    torch.cuda.synchronize()
    k_after, v_after = W.bits(k_pool), W.bits(v_pool)
    ref = oracle.load()
    kb, vb = W.bits(k_new), W.bits(v_new)
    # untouched slots
    others = np.setdiff1d(np.arange(N), out_loc)
    assert np.array_equal(k_after[others], k_before[others]), "K rows outside out_loc changed"
    assert np.array_equal(v_after[others], v_before[others]), "V rows outside out_loc changed"
    # V copied bit for bit
    assert np.array_equal(v_after[out_loc], vb), "V rows differ"
    # K rotated
    k_ref = ref.rope(kb, positions, theta) if theta > 0 else None
    exp_k = _bf16_round(k_ref) if theta > 0 else kb
    dk = _ulp_distance(k_after[out_loc], exp_k)
    say(f"  K: max ulp {dk.max()}, exact {np.mean(dk == 0) * 100:.4f}%")
    assert dk.max() == 0
    if with_q:
        q_after = W.bits(q)
        if theta > 0:
            dq = _ulp_distance(q_after, _bf16_round(ref.rope(q_before, positions, theta)))
            say(f"  Q: max ulp {dq.max()}, exact {np.mean(dq == 0) * 100:.4f}%")
            assert dq.max() == 0
        else:
            assert np.array_equal(q_after, q_before)
    return k_pool, v_pool, k_ref, out_loc, positions


@pytest.mark.parametrize("T,Hq,Hkv,D", [(64, 32, 8, 128), (7, 32, 8, 128), (33, 16, 4, 256), (1, 8, 8, 128)])
def test_append_rope_parity(T, Hq, Hkv, D):
    say(f"append + rope T={T} Hq={Hq} Hkv={Hkv} D={D}")
    _check_append(T, Hq, Hkv, D, N=4096, seed=100 + T + D)


def test_append_without_rotation_copies():
    say("append without rotation")
    _check_append(40, 32, 8, 128, N=1024, seed=7, theta=0.0)


def test_append_position_zero_is_a_copy():
    say("append at position 0")
    dev = device()
    k_pool, v_pool, _, _ = _pools(256, 8, 128, 3, dev)
    k_new = W.normal_bf16((16, 8, 128), 4, dev)
    v_new = W.normal_bf16((16, 8, 128), 5, dev)
    loc = torch.arange(16, dtype=torch.int32, device=dev) * 3
    pa.pa_kv_append(k_new, v_new, loc, k_pool, v_pool,
                    positions=torch.zeros(16, dtype=torch.int32, device=dev), rope_theta=THETA)
    torch.cuda.synchronize()
    assert np.array_equal(W.bits(k_pool)[loc.cpu().numpy()], W.bits(k_new))


def test_append_out_of_range_slots_write_nothing():
    say("append with out-of-range slots")
    dev = device()
    N = 512
    k_pool, v_pool, k_before, v_before = _pools(N, 8, 128, 9, dev)
    k_new = W.normal_bf16((4, 8, 128), 10, dev)
    v_new = W.normal_bf16((4, 8, 128), 11, dev)
    loc = np.array([-1, 17, N, 40], np.int32)
    pa.pa_kv_append(k_new, v_new, torch.as_tensor(loc, device=dev), k_pool, v_pool,
                    positions=torch.as_tensor([5, 6, 7, 8], dtype=torch.int32, device=dev),
                    rope_theta=THETA)
    torch.cuda.synchronize()
    k_after, v_after = W.bits(k_pool), W.bits(v_pool)
    keep = np.setdiff1d(np.arange(N), [17, 40])
    assert np.array_equal(k_after[keep], k_before[keep]) and np.array_equal(v_after[keep], v_before[keep])
    assert np.array_equal(v_after[[17, 40]], W.bits(v_new)[[1, 3]])


def test_append_empty_and_bad_arguments():
    say("append: empty call and argument checks")
    dev = device()
    k_pool, v_pool, k_before, _ = _pools(64, 8, 128, 12, dev)
    e = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=dev)
    pa.pa_kv_append(e, e, torch.empty(0, dtype=torch.int32, device=dev), k_pool, v_pool)
    torch.cuda.synchronize()
    assert np.array_equal(W.bits(k_pool), k_before)
    k3 = W.normal_bf16((3, 8, 96), 13, dev)
    with pytest.raises(pa.PAError) as err:
        pa.pa_kv_append(k3, k3, torch.zeros(3, dtype=torch.int32, device=dev),
                        torch.zeros((64, 8, 96), dtype=torch.bfloat16, device=dev),
                        torch.zeros((64, 8, 96), dtype=torch.bfloat16, device=dev))
    assert err.value.status == pa.PA_ERR_UNSUPPORTED


def test_append_then_decode_attends_rotated_keys():
    """End to end: rows appended (K rotated) then attended by decode give the
    oracle's attention over the rotated keys (rounded to bf16, as stored)."""
    say("append then decode")
    dev = device()
    Hq, Hkv, D, N = 32, 8, 128, 8192
    rng = np.random.Generator(np.random.PCG64(21))
    B = 4
    lengths = np.array([300, 1, 77, 1024])
    ip, idx = W.slot_lists(lengths, N, rng)
    k_pool, v_pool = W.make_pools(N, Hkv, D, 22, dev)
    # the last entry of every list is the token appended this step
    new_slots = idx[ip[1:] - 1].astype(np.int32)
    positions = (lengths - 1).astype(np.int32)
    k_new = W.normal_bf16((B, Hkv, D), 23, dev)
    v_new = W.normal_bf16((B, Hkv, D), 24, dev)
    q = W.normal_bf16((B, Hq, D), 25, dev)
    q_raw = W.bits(q).copy()
    pa.pa_kv_append(k_new, v_new, torch.as_tensor(new_slots, device=dev), k_pool, v_pool,
                    positions=torch.as_tensor(positions, device=dev), rope_theta=THETA, q=q)
    scale = W.softmax_scale(D)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
    with pa.Plan(B, int(ip[-1]), Hq, Hkv, D) as plan:
        plan.plan(ip)
        plan.decode(q, k_pool, v_pool, torch.as_tensor(idx, device=dev), scale, out)
        torch.cuda.synchronize()
    ref_o = oracle.load()
    # expected pool: the oracle's rotation of the appended rows, stored as bf16
    k_exp = W.bits(k_pool).copy()
    k_exp[new_slots] = _bf16_round(ref_o.rope(W.bits(k_new), positions, THETA))
    q_exp = _bf16_round(ref_o.rope(q_raw, positions, THETA))
    d = _ulp_distance(W.bits(k_pool), k_exp).max()
    assert d == 0
    ref, _ = ref_o.decode(q_exp, k_exp, W.bits(v_pool), ip, idx, scale, Hkv)
    assert max_err(out.cpu().numpy(), ref) <= TOL


def test_append_large_pool_offsets():
    """Slots past 2^31 bytes of pool address."""
    say("append into a 2,300,000-slot pool")
    dev = device()
    N = 2_300_000
    k_pool = torch.zeros((N, 8, 128), dtype=torch.bfloat16, device=dev)
    v_pool = torch.zeros((N, 8, 128), dtype=torch.bfloat16, device=dev)
    loc = np.array([N - 1, N - 2, 5, 2_100_000], np.int32)
    k_new = W.normal_bf16((4, 8, 128), 31, dev)
    v_new = W.normal_bf16((4, 8, 128), 32, dev)
    pos = np.array([0, 9, 99, 999], np.int32)
    pa.pa_kv_append(k_new, v_new, torch.as_tensor(loc, device=dev), k_pool, v_pool,
                    positions=torch.as_tensor(pos, device=dev), rope_theta=THETA)
    torch.cuda.synchronize()
    got_k = W.bits(k_pool[torch.as_tensor(loc, device=dev, dtype=torch.int64)])
    got_v = W.bits(v_pool[torch.as_tensor(loc, device=dev, dtype=torch.int64)])
    assert np.array_equal(got_v, W.bits(v_new))
    exp_k = _bf16_round(oracle.load().rope(W.bits(k_new), pos, THETA))
    assert _ulp_distance(got_k, exp_k).max() == 0
    del k_pool, v_pool
    torch.cuda.empty_cache()
