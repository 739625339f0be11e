"""A seeded sweep of the append step (pa_kv_append and pa_kv_append_fp8):
element type, head shape, token count, positions up to 2^20, RoPE base
(none, 1e4, 1e6), pool scales, and the pool layout -- separate pools, the
two halves of one fused [slots, 2, Hkv, D] buffer, or slots padded past
Hkv*D -- drawn per case.  The written slots must hold the oracle's rows (bf16
bit for bit; E4M3 codes as in the E4M3 append test), and every other byte of
the buffers, padding included, must be unchanged.  Needs an AMD GPU."""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_pa_amd as pa
import workloads as W
from gpu_util import device, say
from test_append_fp8_gpu import _bf16_round, _check_k_codes, _f32


def _rotation_error(pos_hi: int) -> float:
    """Bound on |difference| between the two sides' rotated values: the angle
    pos * inv_freq carries a relative rounding of a few 2^-53 on either side
    (double products, sin/cos and the power of theta from different
    libraries), times a pair's size (|x| < 8 for these N(0, 1) rows)."""
    return max(pos_hi, 1) * 8 * 8 * 2.0 ** -53


def _check_bf16_rotated(got_bits, want_bits, y, window):
    """bf16 bits equal, or one bf16 step apart where the oracle's double y
    lies within `window` of the midpoint between the two."""
    diff = got_bits != want_bits
    if not diff.any():
        return 0
    wid = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g, w = wid(got_bits[diff]), wid(want_bits[diff])
    mid = (g + w) / 2
    ok = np.abs(y[diff] - mid) <= window + 1e-12 * np.abs(y[diff])
    key = lambda b: np.where(b & 0x8000, -(b.astype(np.int64) & 0x7FFF), b.astype(np.int64))
    step = np.abs(key(got_bits[diff]) - key(want_bits[diff]))
    assert np.all(ok & (step == 1)), f"{np.count_nonzero(~(ok & (step == 1)))} rotated values differ away from ties"
    return int(diff.sum())

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def draw(seed):
    rng = np.random.Generator(np.random.PCG64(9000 + seed))
    c = {"seed": seed, "fp8": bool(seed % 2), "D": int(rng.choice([128, 256])), "Hkv": int(rng.integers(1, 9)),
         "T": int(rng.integers(1, 200)), "theta": float(rng.choice([0.0, 1e4, 1e6])),
         "layout": str(rng.choice(["separate", "fused", "padded"])),
         "pos_hi": int(rng.choice([16, 40000, 1 << 20])),
         "k_scale": float(np.float32(np.exp(rng.uniform(np.log(0.02), np.log(2.0))))),
         "v_scale": float(np.float32(np.exp(rng.uniform(np.log(0.02), np.log(2.0)))))}
    c["Hq"] = c["Hkv"] * int(rng.choice([1, 2, 4, 8]))
    return c


CASES = [draw(s) for s in range(16)]


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"{c['seed']}-{'fp8' if c['fp8'] else 'bf16'}-{c['layout']}-"
                                                   f"T{c['T']}-{c['Hkv']}x{c['D']}")
def test_append_sweep(c):
    say(f"append sweep case {c}")
    dev = device()
    rng = np.random.Generator(np.random.PCG64(9100 + c["seed"]))
    T, Hq, Hkv, D = c["T"], c["Hq"], c["Hkv"], c["D"]
    N = T + 300
    row = Hkv * D
    eb = 1 if c["fp8"] else 2
    stride = {"separate": row, "fused": 2 * row, "padded": row + (16 if c["fp8"] else 8)}[c["layout"]]
    # raw buffers of random bytes, K and V views into them
    nbytes = N * stride * eb
    raw_k = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev)
    raw_v = raw_k if c["layout"] == "fused" else torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev)
    if not c["fp8"]:
        raw_k[1::2] &= 0x3F   # bf16 patterns of moderate magnitude (no NaN) in untouched rows
        raw_v[1::2] &= 0x3F
    dt = torch.uint8 if c["fp8"] else torch.bfloat16
    k_all, v_all = raw_k.view(dt), raw_v.view(dt)
    k_pool = torch.as_strided(k_all, (N, Hkv, D), (stride, D, 1))
    v_pool = torch.as_strided(v_all, (N, Hkv, D), (stride, D, 1), row if c["layout"] == "fused" else 0)
    before_k, before_v = raw_k.cpu().numpy().copy(), raw_v.cpu().numpy().copy()
    k_new = W.normal_bf16((T, Hkv, D), 9200 + c["seed"], dev)
    v_new = W.normal_bf16((T, Hkv, D), 9300 + c["seed"], dev)
    q = W.normal_bf16((T, Hq, D), 9400 + c["seed"], dev)
    q_before = W.bits(q).copy()
    loc = rng.permutation(N)[:T].astype(np.int32)
    pos = rng.integers(0, c["pos_hi"], T).astype(np.int32)
    loc_d, pos_d = torch.as_tensor(loc, device=dev), torch.as_tensor(pos, device=dev)
    if c["fp8"]:
        pa.pa_kv_append_fp8(k_new, v_new, loc_d, k_pool, v_pool, c["k_scale"], c["v_scale"], positions=pos_d,
                            rope_theta=c["theta"], q=q)
    else:
        pa.pa_kv_append(k_new, v_new, loc_d, k_pool, v_pool, positions=pos_d, rope_theta=c["theta"], q=q)
    torch.cuda.synchronize()
    ref = oracle.load()
    kb, vb = W.bits(k_new), W.bits(v_new)
    # expected bytes: the buffers as they were, with the slots' rows replaced
    want_k, want_v = before_k.copy(), before_v.copy()
    after_k, after_v = raw_k.cpu().numpy(), raw_v.cpu().numpy()
    window = _rotation_error(c["pos_hi"]) if c["theta"] > 0 else 0.0
    if c["fp8"]:
        k_codes, v_codes, k_values = ref.append_e4m3(kb, vb, pos, c["theta"], c["k_scale"], c["v_scale"])
        got_k = np.stack([after_k[s * stride: s * stride + row] for s in loc]).reshape(T, Hkv, D)
        _check_k_codes(got_k, k_codes, k_values / _f32(c["k_scale"]), ref,
                       abs_window=window / _f32(c["k_scale"]))
        k_rows = got_k.reshape(T, row)        # accepted codes (equal, or a near tie's neighbour)
        v_rows = v_codes.reshape(T, row)
    else:
        if c["theta"] > 0:
            y = ref.rope(kb, pos, c["theta"])
            got_k = np.stack([after_k[s * stride * 2: s * stride * 2 + row * 2] for s in loc]).view(np.uint16)
            ties = _check_bf16_rotated(got_k.reshape(T, Hkv, D), _bf16_round(y), y, window)
            say(f"  K: {ties} near-tie neighbours")
            k_rows = got_k.reshape(T, row).view(np.uint8).reshape(T, row * 2)
        else:
            k_rows = kb.reshape(T, row).view(np.uint8).reshape(T, row * 2)
        v_rows = vb.reshape(T, row).view(np.uint8).reshape(T, row * 2)
    rb = row * eb
    voff = row * eb if c["layout"] == "fused" else 0
    for i, s in enumerate(loc):
        want_k[s * stride * eb: s * stride * eb + rb] = k_rows[i]
        want_v[s * stride * eb + voff: s * stride * eb + voff + rb] = v_rows[i]
    if c["layout"] == "fused":
        # one buffer: both the K and V replacements apply to it
        merged = before_k.copy()
        for i, s in enumerate(loc):
            merged[s * stride * eb: s * stride * eb + rb] = k_rows[i]
            merged[s * stride * eb + voff: s * stride * eb + voff + rb] = v_rows[i]
        assert np.array_equal(after_k, merged), "fused buffer differs"
    else:
        assert np.array_equal(after_k, want_k), "K buffer differs outside or inside the written rows"
        assert np.array_equal(after_v, want_v), "V buffer differs outside or inside the written rows"
    q_after = W.bits(q)
    if c["theta"] > 0:
        yq = ref.rope(q_before, pos, c["theta"])
        _check_bf16_rotated(q_after, _bf16_round(yq), yq, window)
    else:
        assert np.array_equal(q_after, q_before)
