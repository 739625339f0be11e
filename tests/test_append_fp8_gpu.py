"""The append step into 8-bit pools (pa_kv_append_fp8): the new tokens' K/V
rows stored as OCP FP8 E4M3 codes under per-pool scales, K (and optionally Q)
rotated by RoPE, against the fp64 oracle's rotation and encoding of the same
bf16 bits.

Slot placement is bit-exact, and so are the V codes: x / v_scale is one
correctly rounded double division on both sides.  The K codes are bit-exact
too, except where the oracle's double quotient lies within 1e-12 (relative)
of a midpoint between two codes: there the rotation's last-bit differences
(sin, cos and the power of theta come from different libraries) may take
either neighbour, and either is accepted.  Q stays bf16 and is checked as in
the bf16 append.  Needs a GPU."""
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


def _f32(x: float) -> float:
    return float(np.float32(x))


def _code_pools(N, Hkv, D, seed, dev):
    """Pools of random finite codes (both signs), so that untouched slots are
    recognisable."""
    g = torch.Generator(device=dev).manual_seed(seed)
    k = torch.randint(0, 0x7F, (N, Hkv, D), generator=g, device=dev, dtype=torch.uint8)
    v = torch.randint(0, 0x7F, (N, Hkv, D), generator=g, device=dev, dtype=torch.uint8)
    k |= (torch.randint(0, 2, (N, Hkv, D), generator=g, device=dev, dtype=torch.uint8) << 7)
    v |= (torch.randint(0, 2, (N, Hkv, D), generator=g, device=dev, dtype=torch.uint8) << 7)
    return k, v


def _near_tie(x: np.ndarray, ref: oracle.Oracle, abs_window: float = 0.0) -> np.ndarray:
    """Where |x| lies within 1e-12 (relative), or abs_window, of a midpoint
    between two neighbouring finite codes."""
    fin = ref.e4m3_values(np.arange(0x7F, dtype=np.uint8))
    mids = (fin[:-1] + fin[1:]) / 2
    a = np.abs(x).ravel()
    j = np.clip(np.searchsorted(mids, a), 1, mids.size - 1)
    d = np.minimum(np.abs(a - mids[j - 1]), np.abs(a - mids[j]))
    return (d <= np.maximum(1e-12 * np.maximum(a, 2.0 ** -10), abs_window)).reshape(x.shape)


def _check_k_codes(got, want, quotient, ref, what="K", abs_window=0.0):
    """Codes equal, or neighbours where the quotient is a near tie (within
    abs_window too: the two sides' rotations differ by about the angle's
    rounding, pos * 2^-52 radians, times the pair's size)."""
    diff = got != want
    if diff.any():
        tie = _near_tie(quotient, ref, abs_window)
        step = np.abs(got.astype(np.int32) - want.astype(np.int32))
        ok = tie & (step == 1) & ((got & 0x80) == (want & 0x80))
        assert np.all(ok[diff]), (f"{what} codes differ away from ties: {np.count_nonzero(diff & ~ok)} "
                                  f"e.g. got {got[diff & ~ok][:4]} want {want[diff & ~ok][:4]}")
    say(f"  {what}: {got.size} codes, {np.count_nonzero(diff)} near-tie neighbours")


def _bf16_round(x64: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, rounded once to nearest-even straight from the
    double (no float32 step).  Values must be zero or normal in bf16."""
    x = np.ascontiguousarray(x64, dtype=np.float64)
    mag = np.abs(x)
    assert np.all((mag == 0) | ((mag >= 2.0 ** -126) & (mag < 3.0e38))), "outside bf16's normal range"
    u = x.view(np.uint64)
    drop = np.uint64(45)
    lsb = (u >> drop) & np.uint64(1)
    r = ((u + (np.uint64(1) << np.uint64(44)) - np.uint64(1) + lsb) >> drop) << drop
    f32 = r.view(np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _append(k_new, v_new, out_loc, k_pool, v_pool, k_scale, v_scale, positions=None, theta=0.0, q=None):
    dev = k_new.device
    pa.pa_kv_append_fp8(k_new, v_new, torch.as_tensor(out_loc, device=dev), k_pool, v_pool,
                        k_scale, v_scale,
                        positions=None if positions is None else torch.as_tensor(positions, device=dev),
                        rope_theta=theta, q=q)
    torch.cuda.synchronize()


def _check_append(T, Hq, Hkv, D, N, seed, k_scale, v_scale, theta=THETA, with_q=True, positions_hi=40000):
    dev = device()
    rng = np.random.Generator(np.random.PCG64(seed))
    k_pool, v_pool = _code_pools(N, Hkv, D, seed + 1, dev)
    k_before, v_before = W.codes(k_pool).copy(), W.codes(v_pool).copy()
    k_new = W.normal_bf16((T, Hkv, D), seed + 2, dev)
    v_new = W.normal_bf16((T, Hkv, D), seed + 3, dev)
    q = W.normal_bf16((T, Hq, D), seed + 4, dev) if with_q else None
    q_before = W.bits(q).copy() if with_q else None
    out_loc = rng.permutation(N)[:T].astype(np.int32)
    positions = rng.integers(0, positions_hi, T).astype(np.int32)
    _append(k_new, v_new, out_loc, k_pool, v_pool, k_scale, v_scale, positions, theta, q)
    k_after, v_after = W.codes(k_pool), W.codes(v_pool)
    ref = oracle.load()
    k_want, v_want, k_values = ref.append_e4m3(W.bits(k_new), W.bits(v_new), positions, theta,
                                               k_scale, v_scale)
    others = np.setdiff1d(np.arange(N), out_loc)
    assert np.array_equal(k_after[others], k_before[others]), "K rows outside out_loc changed"
    assert np.array_equal(v_after[others], v_before[others]), "V rows outside out_loc changed"
    assert np.array_equal(v_after[out_loc], v_want), "V codes differ"
    _check_k_codes(k_after[out_loc], k_want, k_values / _f32(k_scale), ref)
    sat = np.count_nonzero((v_want & 0x7F) == 0x7E) + np.count_nonzero((k_want & 0x7F) == 0x7E)
    say(f"  {sat} saturated codes")
    if with_q:
        q_after = W.bits(q)
        if theta > 0:
            assert np.array_equal(q_after, _bf16_round(ref.rope(q_before, positions, theta))), "Q rotation"
        else:
            assert np.array_equal(q_after, q_before)
    return k_pool, v_pool


APPEND_CASES = [
    (64, 32, 8, 128, 0.37, 0.05),      # scales that are not powers of two
    (7, 32, 8, 128, 1.0, 1.0),
    (33, 16, 4, 256, 0.02, 2.5),
    (1, 8, 8, 128, 0.125, 0.125),
    (40, 12, 3, 128, 0.004, 0.003),    # |x| / scale past 448 for |x| > ~1.5: saturation
]


@pytest.mark.parametrize("T,Hq,Hkv,D,ks,vs", APPEND_CASES,
                         ids=[f"T{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}-{c[5]}" for c in APPEND_CASES])
def test_append_fp8_parity(T, Hq, Hkv, D, ks, vs):
    say(f"append fp8 T={T} Hq={Hq} Hkv={Hkv} D={D} k_scale={ks} v_scale={vs}")
    _check_append(T, Hq, Hkv, D, N=4096, seed=300 + T + D, k_scale=ks, v_scale=vs)


def test_append_fp8_without_rotation():
    say("append fp8 without rotation")
    _check_append(40, 32, 8, 128, N=1024, seed=17, k_scale=0.3, v_scale=0.7, theta=0.0)


def test_append_fp8_special_values():
    """NaN, infinities, signed zeros, huge and tiny values, and exact ties of
    the code grid, at position 0 (K unrotated): every code as the oracle's."""
    say("append fp8 special values")
    dev = device()
    ref = oracle.load()
    fin = ref.e4m3_values(np.arange(0x7F, dtype=np.uint8))
    mids = (fin[:-1] + fin[1:]) / 2                 # exact in bf16: at most 5 significant bits
    vals = np.concatenate([[np.nan, np.inf, -np.inf, 0.0, -0.0, 1e30, -1e30, 448.0, 464.0, 470.0,
                            2.0 ** -10, -2.0 ** -10, 2.0 ** -12, 3 * 2.0 ** -10], mids, -mids, fin])
    D, Hkv = 128, 2
    T = -(-vals.size // (Hkv * D))
    x = np.zeros(T * Hkv * D)
    x[:vals.size] = vals
    xb = torch.as_tensor(x.reshape(T, Hkv, D), dtype=torch.float32).to(torch.bfloat16).to(dev)
    k_pool, v_pool = _code_pools(64, Hkv, D, 5, dev)
    loc = np.arange(T, dtype=np.int32) * 2 + 1
    _append(xb, xb, loc, k_pool, v_pool, 1.0, 1.0, np.zeros(T, np.int32), THETA)
    k_want, v_want, _ = ref.append_e4m3(W.bits(xb), W.bits(xb), np.zeros(T, np.int32), THETA, 1.0, 1.0)
    assert np.array_equal(W.codes(v_pool)[loc], v_want), "V special codes"
    assert np.array_equal(W.codes(k_pool)[loc], k_want), "K special codes at position 0"
    flat = v_want.ravel()[:vals.size]
    assert flat[0] == 0x7F and flat[1] == 0x7E and flat[2] == 0xFE and flat[3] == 0x00 and flat[4] == 0x80


def test_append_fp8_out_of_range_slots_and_arguments():
    say("append fp8: out-of-range slots, empty call, argument checks")
    dev = device()
    N = 512
    k_pool, v_pool = _code_pools(N, 8, 128, 9, dev)
    k_before, v_before = W.codes(k_pool).copy(), W.codes(v_pool).copy()
    k_new = W.normal_bf16((4, 8, 128), 10, dev)
    v_new = W.normal_bf16((4, 8, 128), 11, dev)
    loc = np.array([-1, 17, N, 40], np.int32)
    _append(k_new, v_new, loc, k_pool, v_pool, 0.5, 0.5, np.array([5, 6, 7, 8], np.int32), THETA)
    k_after, v_after = W.codes(k_pool), W.codes(v_pool)
    keep = np.setdiff1d(np.arange(N), [17, 40])
    assert np.array_equal(k_after[keep], k_before[keep]) and np.array_equal(v_after[keep], v_before[keep])
    _, v_want, _ = oracle.load().append_e4m3(W.bits(k_new), W.bits(v_new), np.array([5, 6, 7, 8], np.int32),
                                             THETA, 0.5, 0.5)
    assert np.array_equal(v_after[[17, 40]], v_want[[1, 3]])
    # empty call writes nothing
    e = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=dev)
    pa.pa_kv_append_fp8(e, e, torch.empty(0, dtype=torch.int32, device=dev), k_pool, v_pool, 1.0, 1.0)
    torch.cuda.synchronize()
    assert np.array_equal(W.codes(k_pool), k_after)
    loc1 = torch.zeros(4, dtype=torch.int32, device=dev)
    for ks, vs in [(0.0, 1.0), (1.0, -1.0), (float("nan"), 1.0), (1.0, float("inf"))]:
        with pytest.raises(pa.PAError) as err:
            pa.pa_kv_append_fp8(k_new, v_new, loc1, k_pool, v_pool, ks, vs)
        assert err.value.status == pa.PA_ERR_INVALID_ARG
    k3 = W.normal_bf16((3, 8, 96), 13, dev)
    with pytest.raises(pa.PAError) as err:
        pa.pa_kv_append_fp8(k3, k3, torch.zeros(3, dtype=torch.int32, device=dev),
                            torch.zeros((64, 8, 96), dtype=torch.uint8, device=dev),
                            torch.zeros((64, 8, 96), dtype=torch.uint8, device=dev), 1.0, 1.0)
    assert err.value.status == pa.PA_ERR_UNSUPPORTED
    with pytest.raises(TypeError):
        pa.pa_kv_append_fp8(k_new, v_new, loc1, torch.zeros((N, 8, 128), dtype=torch.bfloat16, device=dev),
                            torch.zeros((N, 8, 128), dtype=torch.bfloat16, device=dev), 1.0, 1.0)
    assert np.array_equal(W.codes(k_pool), k_after) and np.array_equal(W.codes(v_pool), v_after)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 4, 256)])
def test_append_fp8_then_decode_fp8(Hq, Hkv, D):
    """End to end: the step's token appended into 8-bit pools (float8_e4m3fn
    tensors), then attended by the fp8 decode: the oracle's attention over
    the pools holding the oracle's codes, to the usual tolerance."""
    say(f"append fp8 then decode fp8 {Hq}x{Hkv}x{D}")
    dev = device()
    N = 8192
    ks, vs = W.FP8_K_SCALE, W.FP8_V_SCALE
    rng = np.random.Generator(np.random.PCG64(41 + D))
    lengths = np.array([300, 1, 77, 1024, 2])
    B = lengths.size
    ip, idx = W.slot_lists(lengths, N, rng)
    k_pool, v_pool = W.make_pools_e4m3(N, Hkv, D, 42, dev, k_scale=ks, v_scale=vs)
    new_slots = idx[ip[1:] - 1].astype(np.int32)
    positions = (lengths - 1).astype(np.int32)
    k_new = W.normal_bf16((B, Hkv, D), 43, dev)
    v_new = W.normal_bf16((B, Hkv, D), 44, dev)
    q = W.normal_bf16((B, Hq, D), 45, dev)
    q_raw = W.bits(q).copy()
    k_exp, v_exp = W.codes(k_pool).copy(), W.codes(v_pool).copy()
    _append(k_new, v_new, new_slots, k_pool, v_pool, ks, vs, positions, THETA, q)
    ref = oracle.load()
    k_codes, v_codes, k_values = ref.append_e4m3(W.bits(k_new), W.bits(v_new), positions, THETA, ks, vs)
    _check_k_codes(W.codes(k_pool)[new_slots], k_codes, k_values / _f32(ks), ref)
    k_exp[new_slots] = W.codes(k_pool)[new_slots]     # equal to the oracle's, or a tie's neighbour
    v_exp[new_slots] = v_codes
    assert np.array_equal(W.codes(v_pool), v_exp)
    scale = W.softmax_scale(D)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
    with pa.Plan(B, int(ip[-1]), Hq, Hkv, D) as plan:
        plan.plan(ip, flags=pa.PA_PLAN_KV_FP8)
        plan.decode_fp8(q, k_pool, v_pool, torch.as_tensor(idx, device=dev), scale, ks, vs, out)
        torch.cuda.synchronize()
    q_exp = _bf16_round(ref.rope(q_raw, positions, THETA))
    want, _ = ref.decode_fp8(q_exp, k_exp, v_exp, ip, idx, scale, ks, vs, Hkv)
    assert max_err(out.cpu().numpy(), want) <= TOL


def test_append_fp8_large_pool_offsets():
    """Slots past 2^31 bytes of an 8-bit pool (2.36 GB per pool)."""
    say("append fp8 into a 2,300,000-slot pool")
    dev = device()
    N = 2_300_000
    k_pool = torch.zeros((N, 8, 128), dtype=torch.uint8, device=dev)
    v_pool = torch.zeros((N, 8, 128), dtype=torch.uint8, device=dev)
    loc = np.array([N - 1, N - 2, 5, 2_100_000], np.int32)
    k_new = W.normal_bf16((4, 8, 128), 51, dev)
    v_new = W.normal_bf16((4, 8, 128), 52, dev)
    pos = np.array([0, 9, 99, 999], np.int32)
    _append(k_new, v_new, loc, k_pool, v_pool, 0.25, 0.5, pos, THETA)
    sel = torch.as_tensor(loc, device=dev, dtype=torch.int64)
    got_k, got_v = W.codes(k_pool[sel]), W.codes(v_pool[sel])
    ref = oracle.load()
    k_want, v_want, k_values = ref.append_e4m3(W.bits(k_new), W.bits(v_new), pos, THETA, 0.25, 0.5)
    assert np.array_equal(got_v, v_want)
    _check_k_codes(got_k, k_want, k_values / _f32(0.25), ref)
    assert int(k_pool[:N - 2].count_nonzero()) == int((k_want[2:] != 0).sum()), "codes written elsewhere"
    del k_pool, v_pool
    torch.cuda.empty_cache()
