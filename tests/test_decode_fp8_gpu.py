"""Decode over 8-bit (OCP FP8 E4M3) pools with per-pool scales, through the
C ABI (pa_decode_run_fp8), against the fp64 oracle on the same codes.  Needs
an AMD GPU."""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_pa_amd as pa
import workloads as W
from gpu_util import TOL, device, max_err, run_decode, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

KS, VS = W.FP8_K_SCALE, W.FP8_V_SCALE


def run_fp8(q, k, v, ip, idx_dev, scale, Hkv, flags=0, k_scale=KS, v_scale=VS, fp8_plan=True):
    B, Hq, D = q.shape
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=q.device)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device)
    forced = (flags >> pa.PA_PLAN_FORCE_SPLITS_SHIFT) & 0xFFFF
    with pa.Plan(max(B, 1), max(int(ip[-1]), 1, B * forced * 256), Hq, Hkv, D) as plan:
        plan.plan(ip, flags=flags | (pa.PA_PLAN_KV_FP8 if fp8_plan else 0))
        plan.decode_fp8(q, k, v, idx_dev, scale, k_scale, v_scale, out, lse)
        torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _case(lengths, Hq, Hkv, D, N, seed, k_scale=KS, v_scale=VS):
    dev = device()
    rng = np.random.Generator(np.random.PCG64(seed))
    ip, idx = W.slot_lists(np.asarray(lengths), N, rng)
    q = W.normal_bf16((len(lengths), Hq, D), seed + 1, dev)
    k, v = W.make_pools_e4m3(N, Hkv, D, seed + 2, dev, k_scale=k_scale, v_scale=v_scale)
    return ip, idx, q, k, v


def _oracle(q, k, v, ip, idx, scale, Hkv, sel=None, k_scale=KS, v_scale=VS):
    return oracle.load().decode_fp8(W.bits(q), W.codes(k), W.codes(v), ip, idx, scale, k_scale, v_scale,
                                    Hkv, sel=sel)


CASES = [
    ([1, 7, 64, 300, 1025], 32, 8, 128),
    ([0, 2, 513], 32, 8, 128),
    ([100, 2000], 8, 8, 128),
    ([33, 700], 16, 8, 128),
    ([50, 900, 3], 64, 8, 128),
    ([17, 1500], 16, 4, 256),
    ([400, 5], 8, 8, 256),
    ([5, 800, 77], 12, 3, 128),     # odd KV-head count
    ([300, 40, 1], 8, 2, 128),
    ([90, 700], 16, 8, 256),        # group 2
    ([40, 333, 6], 32, 4, 256),     # group 8: 8 codes a lane, 32 lanes a row
]


@pytest.mark.parametrize("lengths,Hq,Hkv,D", CASES, ids=[f"{c[1]}x{c[2]}x{c[3]}-{i}" for i, c in enumerate(CASES)])
def test_fp8_small_parity(lengths, Hq, Hkv, D):
    say(f"fp8 decode parity lengths={lengths} Hq={Hq} Hkv={Hkv} D={D}")
    ip, idx, q, k, v = _case(lengths, Hq, Hkv, D, 8192, 300 + Hq + D + len(lengths))
    scale = W.softmax_scale(D)
    out, lse = run_fp8(q, k, v, ip, torch.as_tensor(idx, device=device()), scale, Hkv)
    ref, ref_lse = _oracle(q, k, v, ip, idx, scale, Hkv)
    e, el = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  max|d| out={e:.3g} lse={el:.3g}")
    assert e <= TOL and el <= TOL


@pytest.mark.parametrize("k_scale,v_scale", [(0.37, 1.3), (3.1, 0.07), (1.0, 1.0)])
@pytest.mark.parametrize("lengths,Hq,Hkv,D", [CASES[0], CASES[5]], ids=["32x8x128", "16x4x256"])
def test_fp8_general_scales(lengths, Hq, Hkv, D, k_scale, v_scale):
    """Per-pool scales that are not powers of two: the kernel's products of
    the scales are rounded to float32, the oracle's are exact; the results
    still agree within 2e-3."""
    say(f"fp8 decode, scales k={k_scale} v={v_scale}, lengths={lengths} Hq={Hq} Hkv={Hkv} D={D}")
    ip, idx, q, k, v = _case(lengths, Hq, Hkv, D, 8192, 500 + Hq + D, k_scale=k_scale, v_scale=v_scale)
    scale = W.softmax_scale(D)
    out, lse = run_fp8(q, k, v, ip, torch.as_tensor(idx, device=device()), scale, Hkv,
                       k_scale=k_scale, v_scale=v_scale)
    ref, ref_lse = _oracle(q, k, v, ip, idx, scale, Hkv, k_scale=k_scale, v_scale=v_scale)
    e, el = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  max|d| out={e:.3g} lse={el:.3g}")
    assert e <= TOL and el <= TOL


@pytest.mark.parametrize("Hq", [32, 64], ids=["G4", "G8"])
@pytest.mark.parametrize("n", [2, 7])
def test_fp8_forced_splits_agree(n, Hq):
    """Split counts change each part's running maximum and so the fp16
    rounding of the weights: each splitting is within 2^-11 x max|v - o| <=
    2^-10 x max|V| of the exact weighted mean, so two differ by at most 2^-9 x
    max|V|."""
    say(f"fp8 forced splits n={n} Hq={Hq}")
    ip, idx, q, k, v = _case([300, 1025, 9], Hq, 8, 128, 8192, 71)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    base, _ = run_fp8(q, k, v, ip, idx_dev, scale, 8)
    out, lse = run_fp8(q, k, v, ip, idx_dev, scale, 8, flags=pa.PA_PLAN_FORCE_SPLITS(n))
    vals = v.float()[torch.as_tensor(idx.astype(np.int64), device=idx_dev.device)] * VS
    bound = 2.0 ** -9 * float(vals.abs().max())
    d = max_err(out, base.astype(np.float64))
    ref, ref_lse = _oracle(q, k, v, ip, idx, scale, 8)
    say(f"  split vs unsplit {d:.3g} (bound {bound:.3g}); vs oracle {max_err(out, ref):.3g}")
    assert d <= bound
    assert max_err(out, ref) <= TOL and max_err(lse, ref_lse) <= TOL


@pytest.mark.parametrize("Hq", [64, 32], ids=["G8", "G4"])
def test_fp8_against_bf16_path_on_the_same_values(Hq):
    """With unit scales, decode over E4M3 codes against the bf16 decode over
    pools holding the codes' values (the codes widen exactly).  The E4M3 path
    runs the weighted sum on fp16 products over two tokens, the weights
    rounded once to fp16 (relative error <= 2^-11 each, and the row sums add
    the rounded weights): each output moves by at most 2^-11 x max|v - o| <=
    2^-10 x max|V| from the bf16 path's, and both stay within 2e-3 of the
    oracle."""
    say(f"fp8 vs bf16 path on identical values, Hq={Hq}")
    ip, idx, q, k, v = _case([1, 90, 600, 2049], Hq, 8, 128, 8192, 81)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    out8, lse8 = run_fp8(q, k, v, ip, idx_dev, scale, 8, k_scale=1.0, v_scale=1.0)
    kb, vb = k.to(torch.bfloat16), v.to(torch.bfloat16)
    out16, lse16 = run_decode(q, kb, vb, ip, idx_dev, scale, 8)
    vmax = float(vb.float()[torch.as_tensor(idx.astype(np.int64), device=idx_dev.device)].abs().max())
    bound = 2.0 ** -10 * vmax
    d = max_err(out8, out16.astype(np.float64))
    ref, ref_lse = _oracle(q, k, v, ip, idx, scale, 8, k_scale=1.0, v_scale=1.0)
    say(f"  max|fp8 - bf16| = {d:.3g} (bound {bound:.3g}); vs oracle {max_err(out8, ref):.3g}")
    assert d <= bound
    assert max_err(out8, ref) <= TOL and max_err(lse8, ref_lse) <= TOL


def test_fp8_with_a_bf16_sized_plan():
    """A plan made without PA_PLAN_KV_FP8 splits for the bf16 kernel's
    workgroup count, more than the E4M3 kernel keeps resident: the extra
    workgroups run later and the result is the same up to the split's
    rounding."""
    say("fp8 decode with a plan sized for bf16 pools")
    ip, idx, q, k, v = _case([4000, 3000, 5000, 100], 32, 8, 128, 32768, 61)
    idx_dev = torch.as_tensor(idx, device=device())
    scale = W.softmax_scale(128)
    out, lse = run_fp8(q, k, v, ip, idx_dev, scale, 8, fp8_plan=False)
    ref, ref_lse = _oracle(q, k, v, ip, idx, scale, 8)
    assert max_err(out, ref) <= TOL and max_err(lse, ref_lse) <= TOL


def test_fp8_poisoned_pool():
    """NaN codes in every unreferenced slot change nothing."""
    say("fp8 poisoned pool")
    dev = device()
    ip, idx, q, k, v = _case([150, 333, 2], 32, 8, 128, 4096, 91)
    idx_dev = torch.as_tensor(idx, device=dev)
    scale = W.softmax_scale(128)
    clean, _ = run_fp8(q, k, v, ip, idx_dev, scale, 8)
    keep = torch.zeros(k.shape[0], dtype=torch.bool, device=dev)
    keep[torch.as_tensor(idx.astype(np.int64), device=dev)] = True
    for pool in (k, v):
        pool.view(torch.uint8)[~keep] = 0x7F
    dirty, _ = run_fp8(q, k, v, ip, idx_dev, scale, 8)
    assert np.array_equal(clean, dirty)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 4, 256)], ids=["D128", "D256"])
def test_fp8_large_pool_offsets(Hq, Hkv, D):
    """Rows past 2^31 bytes of an 8-bit pool (64-bit row offsets)."""
    say(f"fp8 large pool: 2,300,000 slots x {Hkv} heads x {D}")
    dev = device()
    N = 2_300_000
    rng = np.random.Generator(np.random.PCG64(101))
    ip, idx = W.slot_lists(np.asarray([700, 260]), N, rng)
    idx[:64] = N - 1 - np.arange(64)
    q = W.normal_bf16((2, Hq, D), 102, dev)
    k, v = W.make_pools_e4m3(N, Hkv, D, 103, dev)
    scale = W.softmax_scale(D)
    out, lse = run_fp8(q, k, v, ip, torch.as_tensor(idx, device=dev), scale, Hkv)
    ref, ref_lse = _oracle(q, k, v, ip, idx, scale, Hkv)
    assert max_err(out, ref) <= TOL and max_err(lse, ref_lse) <= TOL
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k_scale,v_scale", [(KS, VS), (0.37, 1.3)], ids=["pow2_scales", "general_scales"])
def test_fp8_batch64_workload_full_rows(k_scale, v_scale):
    """The batch-64 shared-prefix workload over 8-bit pools, every row."""
    _full_rows(W.BATCH64_SHARED_PREFIX, k_scale, v_scale)


@pytest.mark.slow
@pytest.mark.parametrize("spec", [W.HEADDIM256_BATCH32, W.QWEN3_4B_BATCH8, W.SINGLE_REQUEST_256],
                         ids=lambda s: s.name)
def test_fp8_other_workloads_full_rows(spec):
    """The head_dim-256, batch-8 and single-request workloads over 8-bit
    pools (as bench.py --kv fp8 runs them), every row."""
    _full_rows(spec, KS, VS)


def _full_rows(spec, k_scale, v_scale):
    say(f"fp8 workload {spec.name}, scales {k_scale}/{v_scale}: all rows")
    dev = device()
    ip, idx = W.decode_lists(spec)
    q = W.normal_bf16((spec.batch, spec.num_qo_heads, spec.head_dim), spec.seed, dev)
    k, v = W.make_pools_e4m3(spec.num_slots, spec.num_kv_heads, spec.head_dim, W.layer_seed(spec.seed, 0),
                             dev, k_scale=k_scale, v_scale=v_scale)
    scale = W.softmax_scale(spec.head_dim)
    out, lse = run_fp8(q, k, v, ip, torch.as_tensor(idx, device=dev), scale, spec.num_kv_heads,
                       k_scale=k_scale, v_scale=v_scale)
    ref, ref_lse = _oracle(q, k, v, ip, idx, scale, spec.num_kv_heads, k_scale=k_scale, v_scale=v_scale)
    e, el = max_err(out, ref), max_err(lse, ref_lse)
    say(f"  all {out.shape[0] * out.shape[1]} rows: max|d| out={e:.3g} lse={el:.3g}")
    assert e <= TOL and el <= TOL
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pad,ok", [(16, True), (48, True), (8, False), (24, False)])
def test_decode_fp8_padded_slot_stride(pad, ok):
    """E4M3 pools whose slots are padded (slot stride Hkv*D + pad bytes): a
    stride that keeps every row 16-byte aligned decodes as the compact pool
    does; any other is refused on the host (rows are read 16 codes a lane)."""
    say(f"fp8 decode, slot stride Hkv*D + {pad}")
    Hq, Hkv, D, N = 32, 8, 128, 4096
    ip, idx, q, k, v = _case([5, 300, 77], Hq, Hkv, D, N, seed=95)
    stride = Hkv * D + pad
    dev = q.device
    kb = torch.zeros((N, stride), dtype=torch.uint8, device=dev)
    vb = torch.zeros((N, stride), dtype=torch.uint8, device=dev)
    kb[:, :Hkv * D] = k.view(torch.uint8).reshape(N, Hkv * D)
    vb[:, :Hkv * D] = v.view(torch.uint8).reshape(N, Hkv * D)
    kp = torch.as_strided(kb, (N, Hkv, D), (stride, D, 1))
    vp = torch.as_strided(vb, (N, Hkv, D), (stride, D, 1))
    idx_dev = torch.as_tensor(idx, device=dev)
    scale = W.softmax_scale(D)
    if not ok:
        out = torch.empty((3, Hq, D), dtype=torch.float32, device=dev)
        with pa.Plan(3, int(ip[-1]), Hq, Hkv, D) as plan:
            plan.plan(ip, flags=pa.PA_PLAN_KV_FP8)
            with pytest.raises(pa.PAError) as e:
                plan.decode_fp8(q, kp, vp, idx_dev, scale, KS, VS, out)
            assert e.value.status == pa.PA_ERR_INVALID_ARG
        return
    out, lse = run_fp8(q, kp, vp, ip, idx_dev, scale, Hkv)
    base, base_lse = run_fp8(q, k, v, ip, idx_dev, scale, Hkv)
    assert np.array_equal(out, base) and np.array_equal(lse, base_lse)
    ref, ref_lse = _oracle(q, k, v, ip, idx, scale, Hkv)
    assert max_err(out, ref) <= TOL and max_err(lse, ref_lse) <= TOL


@pytest.mark.parametrize("k_scale,v_scale", [(-0.37, -1.3), (0.0, 0.7), (0.37, 0.0)])
def test_decode_fp8_nonpositive_scales(k_scale, v_scale):
    """Scales of any sign through the fp8 decode (the scores carry
    sm_scale * k_scale, the output v_scale), with the automatic split and
    with forced parts: against the oracle."""
    say(f"fp8 decode scales k={k_scale} v={v_scale}")
    Hq, Hkv, D = 32, 8, 128
    ip, idx, q, k, v = _case([1, 7, 64, 300, 1025, 0], Hq, Hkv, D, 8192, seed=97)
    idx_dev = torch.as_tensor(idx, device=q.device)
    scale = W.softmax_scale(D)
    ref, ref_lse = _oracle(q, k, v, ip, idx, scale, Hkv, k_scale=k_scale, v_scale=v_scale)
    for flags in (0, pa.PA_PLAN_FORCE_SPLITS(7)):
        out, lse = run_fp8(q, k, v, ip, idx_dev, scale, Hkv, flags=flags, k_scale=k_scale, v_scale=v_scale)
        e = max_err(out, ref), max_err(lse, ref_lse)
        say(f"  flags {flags:#x}: max|d| out {e[0]:.3g} lse {e[1]:.3g}")
        assert e[0] <= TOL and e[1] <= TOL
