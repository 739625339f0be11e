"""Pins that tie the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes an oracle handle (``oracle.Oracle``) and raises
``AssertionError`` when the oracle disagrees with:
  * a library routine on a special case (torch's scaled_dot_product_attention
    in float64 with grouped-query heads, numpy/scipy reductions),
  * brute force at 50 significant digits (mpmath) on tiny inputs,
  * closed forms (one token, two tokens, zero query, constant values,
    saturated softmax, empty list; RoPE of unit vectors; E4M3 saturation and
    special values),
  * torch's float8_e4m3fn rounding inside the finite range, and exact
    rational brute force for the nearest E4M3 code,
  * invariances (slot order, slot relocation, split-and-merge; RoPE's
    relative-position property and pair norms), and for RoPE numpy complex
    multiplication.
The same pins run against deliberately broken oracle builds to show that each
plausible mistake is caught (``test_oracle_mutants.py``).
"""
from __future__ import annotations

from fractions import Fraction

import mpmath
import numpy as np
import torch
import torch.nn.functional as F

import workloads

TOL = 1e-12


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to bf16 (nearest-even, via torch) and return the bits."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return workloads.bits(t)


def _widen(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _random_bits(rng, shape, scale=1.0):
    return _bf16_bits(rng.standard_normal(shape) * scale)


def _exact_dot(a_bits, b_bits) -> Fraction:
    return sum((Fraction(float(x)) * Fraction(float(y))
                for x, y in zip(_widen(a_bits), _widen(b_bits))), Fraction(0))


def _contiguous_case(rng, lengths, Hq, Hkv, D, spare=3):
    lengths = list(lengths)
    N = sum(lengths) + spare
    q = _random_bits(rng, (len(lengths), Hq, D))
    k = _random_bits(rng, (N, Hkv, D))
    v = _random_bits(rng, (N, Hkv, D))
    indptr = np.zeros(len(lengths) + 1, np.int32)
    indptr[1:] = np.cumsum(lengths)
    indices = np.arange(sum(lengths), dtype=np.int32) + spare  # slots spare.. (skip the first)
    return q, k, v, indptr, indices


def _scattered_case(rng, lengths, Hq, Hkv, D, N):
    lengths = list(lengths)
    q = _random_bits(rng, (len(lengths), Hq, D))
    k = _random_bits(rng, (N, Hkv, D))
    v = _random_bits(rng, (N, Hkv, D))
    indptr = np.zeros(len(lengths) + 1, np.int32)
    indptr[1:] = np.cumsum(lengths)
    indices = rng.permutation(N)[: sum(lengths)].astype(np.int32)
    return q, k, v, indptr, indices


# ----------------------------------------------------------------------------
# decode pins
# ----------------------------------------------------------------------------
def pin_sdpa_decode(o):
    """Contiguous slots: equals torch SDPA (float64, enable_gqa) to 1e-12."""
    rng = np.random.default_rng(11)
    for (Hq, Hkv, D, lengths) in [(8, 2, 16, [5, 1, 9]), (4, 4, 8, [3, 7]),
                                  (8, 1, 32, [6]), (16, 2, 128, [33, 2])]:
        q, k, v, indptr, indices = _contiguous_case(rng, lengths, Hq, Hkv, D)
        scale = workloads.softmax_scale(D)
        out, _ = o.decode(q, k, v, indptr, indices, scale, Hkv)
        for b in range(len(lengths)):
            ids = indices[indptr[b]:indptr[b + 1]]
            qt = torch.from_numpy(_widen(q[b]))[None, :, None, :]            # [1,Hq,1,D]
            kt = torch.from_numpy(_widen(k[ids])).permute(1, 0, 2)[None]     # [1,Hkv,L,D]
            vt = torch.from_numpy(_widen(v[ids])).permute(1, 0, 2)[None]
            ref = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
            err = np.abs(out[b] - ref[0, :, 0, :].numpy()).max()
            assert err < TOL, f"sdpa mismatch {err} (Hq={Hq} Hkv={Hkv} D={D} b={b})"


def pin_bruteforce_tiny(o):
    """Scattered slots, tiny shapes: equals 50-digit brute force (no max shift)."""
    mpmath.mp.dps = 50
    rng = np.random.default_rng(12)
    for (Hq, Hkv, D, lengths, N) in [(4, 2, 4, [1, 3, 5], 16), (2, 1, 6, [4, 2], 9),
                                     (4, 4, 3, [5], 8)]:
        q, k, v, indptr, indices = _scattered_case(rng, lengths, Hq, Hkv, D, N)
        scale = workloads.softmax_scale(D)
        out, lse = o.decode(q, k, v, indptr, indices, scale, Hkv)
        g = Hq // Hkv
        qw, kw, vw = _widen(q), _widen(k), _widen(v)
        for b in range(len(lengths)):
            ids = indices[indptr[b]:indptr[b + 1]]
            for h in range(Hq):
                kh = h // g
                e = []
                for s in ids:
                    dot = mpmath.fsum(mpmath.mpf(float(qw[b, h, d])) * mpmath.mpf(float(kw[s, kh, d]))
                                      for d in range(D))
                    e.append(mpmath.exp(mpmath.mpf(float(np.float32(scale))) * dot))
                z = mpmath.fsum(e)
                for d in range(D):
                    ref = mpmath.fsum(e[j] * mpmath.mpf(float(vw[s, kh, d]))
                                      for j, s in enumerate(ids)) / z
                    assert abs(out[b, h, d] - float(ref)) < 1e-14, "brute-force out mismatch"
                assert abs(lse[b, h] - float(mpmath.log(z))) < 1e-13, "brute-force lse mismatch"


def pin_slot_order(o):
    """Shuffling each list, or moving rows to other slots, changes nothing (1e-12)."""
    rng = np.random.default_rng(13)
    N = 200
    q, k, v, indptr, indices = _scattered_case(rng, [17, 40, 3], 8, 2, 16, N)
    scale = workloads.softmax_scale(16)
    base, base_lse = o.decode(q, k, v, indptr, indices, scale, 2)
    shuffled = indices.copy()
    for b in range(3):
        seg = shuffled[indptr[b]:indptr[b + 1]]
        shuffled[indptr[b]:indptr[b + 1]] = rng.permutation(seg)
    out, lse = o.decode(q, k, v, indptr, shuffled, scale, 2)
    assert np.abs(out - base).max() < TOL and np.abs(lse - base_lse).max() < TOL, "slot order"
    move = rng.permutation(N)                    # row at slot s moves to slot move[s]
    k2, v2 = np.empty_like(k), np.empty_like(v)
    k2[move], v2[move] = k, v
    out, lse = o.decode(q, k2, v2, indptr, move[indices].astype(np.int32), scale, 2)
    assert np.abs(out - base).max() < TOL and np.abs(lse - base_lse).max() < TOL, "relocation"


def pin_single_token(o):
    """L = 1: out is the value row exactly; lse is the scaled dot product."""
    rng = np.random.default_rng(14)
    q, k, v, indptr, indices = _scattered_case(rng, [1, 1, 1], 8, 2, 32, 50)
    scale = workloads.softmax_scale(32)
    out, lse = o.decode(q, k, v, indptr, indices, scale, 2)
    for b in range(3):
        s = indices[b]
        for h in range(8):
            assert np.array_equal(out[b, h], _widen(v[s, h // 4])), "L=1 must return V exactly"
            ref = float(Fraction(float(np.float32(scale))) * _exact_dot(q[b, h], k[s, h // 4]))
            assert abs(lse[b, h] - ref) < TOL, "L=1 lse"


def pin_two_tokens(o):
    """L = 2: out = sigmoid(s1-s0) v1 + (1 - sigmoid(s1-s0)) v0, lse = logaddexp(s0, s1)."""
    rng = np.random.default_rng(15)
    q, k, v, indptr, indices = _scattered_case(rng, [2, 2], 4, 2, 16, 30)
    scale = workloads.softmax_scale(16)
    out, lse = o.decode(q, k, v, indptr, indices, scale, 2)
    sc = Fraction(float(np.float32(scale)))
    for b in range(2):
        s0_slot, s1_slot = indices[indptr[b]], indices[indptr[b] + 1]
        for h in range(4):
            kh = h // 2
            s0 = float(sc * _exact_dot(q[b, h], k[s0_slot, kh]))
            s1 = float(sc * _exact_dot(q[b, h], k[s1_slot, kh]))
            w1 = 1.0 / (1.0 + np.exp(-(s1 - s0)))
            ref = w1 * _widen(v[s1_slot, kh]) + (1.0 - w1) * _widen(v[s0_slot, kh])
            assert np.abs(out[b, h] - ref).max() < TOL, "two-token closed form"
            assert abs(lse[b, h] - np.logaddexp(s0, s1)) < TOL, "two-token lse"


def pin_zero_query(o):
    """q = 0 (or scale 0): out is the arithmetic mean of the value rows, lse = ln L."""
    rng = np.random.default_rng(16)
    q, k, v, indptr, indices = _scattered_case(rng, [7, 1, 30], 4, 1, 8, 64)
    zq = np.zeros_like(q)
    for qq, scale in [(zq, 0.125), (q, 0.0)]:
        out, lse = o.decode(qq, k, v, indptr, indices, scale, 1)
        for b in range(3):
            ids = indices[indptr[b]:indptr[b + 1]]
            ref = _widen(v[ids, 0]).mean(axis=0)
            assert np.abs(out[b] - ref[None]).max() < TOL, "zero query: mean of V"
            assert np.abs(lse[b] - np.log(len(ids))).max() < TOL, "zero query: lse = ln L"


def pin_constant_values(o):
    """All listed value rows equal: out equals that row whatever the weights."""
    rng = np.random.default_rng(17)
    q, k, v, indptr, indices = _scattered_case(rng, [9, 4], 8, 2, 16, 40)
    row = _random_bits(rng, (2, 16))
    v = v.copy()
    v[indices] = row
    out, _ = o.decode(q, k, v, indptr, indices, workloads.softmax_scale(16), 2)
    for h in range(8):
        assert np.abs(out[:, h] - _widen(row[h // 4])[None]).max() < TOL, "constant V"


def pin_saturated_softmax(o):
    """One key far above the rest: out is that key's value row; lse its score.

    The top score (2048) exceeds every other by more than the double exponent
    range, so an exponent taken without the right shift overflows."""
    rng = np.random.default_rng(18)
    D = 8
    q, k, v, indptr, indices = _scattered_case(rng, [6], 2, 1, D, 20)
    q = _bf16_bits(np.full((1, 2, D), 16.0))
    k = k.copy()
    star = indices[3]
    k[star] = _bf16_bits(np.full((1, D), 16.0))
    others = indices[indices != star]
    k[others] = _bf16_bits(np.clip(_widen(k[others]), -4, 4) * 0.5)
    out, lse = o.decode(q, k, v, indptr, indices, 1.0, 1)
    for h in range(2):
        assert np.isfinite(out[0, h]).all(), "saturated softmax must stay finite"
        assert np.abs(out[0, h] - _widen(v[star, 0])).max() < TOL, "saturated softmax"
        assert abs(lse[0, h] - 16.0 * 16.0 * D) < 1e-9, "saturated lse"


def pin_empty_list(o):
    """An empty list gives out = 0 and lse = -inf, and leaves its neighbours alone."""
    rng = np.random.default_rng(19)
    q, k, v, indptr, indices = _scattered_case(rng, [0, 5, 0], 4, 2, 8, 20)
    scale = workloads.softmax_scale(8)
    out, lse = o.decode(q, k, v, indptr, indices, scale, 2)
    for b in (0, 2):
        assert np.all(out[b] == 0.0) and np.all(np.isneginf(lse[b])), "empty list"
    ref, ref_lse = o.decode(q[1:2], k, v, np.array([0, 5], np.int32), indices, scale, 2)
    assert np.abs(out[1] - ref[0]).max() < TOL and np.abs(lse[1] - ref_lse[0]).max() < TOL


def pin_duplicate_slots(o):
    """A slot listed twice counts twice: equals SDPA over the duplicated rows."""
    rng = np.random.default_rng(20)
    D, Hq, Hkv = 16, 4, 2
    q = _random_bits(rng, (1, Hq, D))
    k = _random_bits(rng, (10, Hkv, D))
    v = _random_bits(rng, (10, Hkv, D))
    ids = np.array([4, 4, 7, 1, 4], np.int32)
    scale = workloads.softmax_scale(D)
    out, _ = o.decode(q, k, v, np.array([0, 5], np.int32), ids, scale, Hkv)
    qt = torch.from_numpy(_widen(q[0]))[None, :, None, :]
    kt = torch.from_numpy(_widen(k[ids])).permute(1, 0, 2)[None]
    vt = torch.from_numpy(_widen(v[ids])).permute(1, 0, 2)[None]
    ref = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
    assert np.abs(out[0] - ref[0, :, 0, :].numpy()).max() < TOL, "duplicate slots"


def pin_row_selection(o):
    """Computing a subset of rows gives the same values as computing all rows."""
    rng = np.random.default_rng(21)
    q, k, v, indptr, indices = _scattered_case(rng, [5, 9, 2], 8, 2, 16, 40)
    scale = workloads.softmax_scale(16)
    full, full_lse = o.decode(q, k, v, indptr, indices, scale, 2)
    sel = [0, 9, 23, 17]
    part, part_lse = o.decode(q, k, v, indptr, indices, scale, 2, sel=sel)
    fo, po = full.reshape(-1, 16), part.reshape(-1, 16)
    assert np.array_equal(fo[sel], po[sel]), "row selection"
    assert np.array_equal(full_lse.reshape(-1)[sel], part_lse.reshape(-1)[sel])
    others = [r for r in range(24) if r not in sel]
    assert np.isnan(po[others]).all(), "unselected rows untouched"


# ----------------------------------------------------------------------------
# merge pins
# ----------------------------------------------------------------------------
def pin_merge_of_splits(o):
    """Decode over parts of a list, merged, equals decode over the whole list."""
    rng = np.random.default_rng(22)
    D, Hq, Hkv = 16, 4, 2
    q, k, v, indptr, indices = _scattered_case(rng, [23], Hq, Hkv, D, 60)
    scale = workloads.softmax_scale(D)
    whole, whole_lse = o.decode(q, k, v, indptr, indices, scale, Hkv)
    for cuts in ([0, 23], [0, 11, 23], [0, 1, 2, 9, 9, 22, 23], list(range(24))):
        n = len(cuts) - 1
        parts = [o.decode(q, k, v, np.array([0, cuts[i + 1] - cuts[i]], np.int32),
                          indices[cuts[i]:cuts[i + 1]], scale, Hkv) for i in range(n)]
        for h in range(Hq):
            op = np.stack([p[0][0, h] for p in parts])
            lp = np.array([p[1][0, h] for p in parts])
            mo, ml = o.merge(op, lp)
            assert np.abs(mo - whole[0, h]).max() < TOL, f"merge out ({n} parts)"
            assert abs(ml - whole_lse[0, h]) < TOL, f"merge lse ({n} parts)"


def pin_merge_special_cases(o):
    """One part returns itself; equal lse averages; all-empty gives 0 / -inf."""
    rng = np.random.default_rng(23)
    a = rng.standard_normal((1, 8))
    mo, ml = o.merge(a, np.array([0.7]))
    assert np.abs(mo - a[0]).max() < TOL and abs(ml - 0.7) < TOL, "single part"
    b = rng.standard_normal((2, 8))
    mo, ml = o.merge(b, np.array([1.5, 1.5]))
    assert np.abs(mo - b.mean(axis=0)).max() < TOL and abs(ml - (1.5 + np.log(2))) < TOL
    mo, ml = o.merge(b, np.array([-np.inf, 2.0]))
    assert np.abs(mo - b[1]).max() < TOL and abs(ml - 2.0) < TOL, "empty part ignored"
    mo, ml = o.merge(b, np.array([-np.inf, -np.inf]))
    assert np.all(mo == 0) and np.isneginf(ml), "all parts empty"


# ----------------------------------------------------------------------------
# prefill pins
# ----------------------------------------------------------------------------
def _prefill_case(rng, cached, chunks, Hq, Hkv, D, N):
    lengths = [p + c for p, c in zip(cached, chunks)]
    _, k, v, indptr, indices = _scattered_case(rng, lengths, Hq, Hkv, D, N)
    qo = np.zeros(len(chunks) + 1, np.int32)
    qo[1:] = np.cumsum(chunks)
    q = _random_bits(rng, (int(qo[-1]), Hq, D))
    return q, k, v, qo, indptr, indices


def pin_prefill_sdpa(o):
    """Contiguous slots: equals SDPA with an explicit bottom-right causal mask."""
    rng = np.random.default_rng(24)
    for (Hq, Hkv, D, cached, chunks) in [(8, 2, 16, [5, 0, 3], [4, 3, 1]), (4, 1, 32, [9], [6])]:
        lengths = [p + c for p, c in zip(cached, chunks)]
        _, k, v, indptr, indices = _contiguous_case(rng, lengths, Hq, Hkv, D)
        qo = np.zeros(len(chunks) + 1, np.int32)
        qo[1:] = np.cumsum(chunks)
        q = _random_bits(rng, (int(qo[-1]), Hq, D))
        scale = workloads.softmax_scale(D)
        out, _ = o.prefill(q, k, v, qo, indptr, indices, scale, Hkv)
        for b, (P, C) in enumerate(zip(cached, chunks)):
            ids = indices[indptr[b]:indptr[b + 1]]
            L = P + C
            qt = torch.from_numpy(_widen(q[qo[b]:qo[b + 1]])).permute(1, 0, 2)[None]  # [1,Hq,C,D]
            kt = torch.from_numpy(_widen(k[ids])).permute(1, 0, 2)[None]
            vt = torch.from_numpy(_widen(v[ids])).permute(1, 0, 2)[None]
            mask = torch.ones(C, L, dtype=torch.bool).tril(diagonal=P)
            ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                                 enable_gqa=True)
            err = np.abs(out[qo[b]:qo[b + 1]] - ref[0].permute(1, 0, 2).numpy()).max()
            assert err < TOL, f"prefill sdpa mismatch {err}"


def pin_prefill_rows_are_decodes(o):
    """Chunk row i equals decode over the list's first P+i+1 entries; C = 1 is decode."""
    rng = np.random.default_rng(25)
    Hq, Hkv, D = 8, 2, 16
    q, k, v, qo, indptr, indices = _prefill_case(rng, [6, 0, 11], [5, 2, 1], Hq, Hkv, D, 64)
    scale = workloads.softmax_scale(D)
    out, lse = o.prefill(q, k, v, qo, indptr, indices, scale, Hkv)
    for b in range(3):
        L = indptr[b + 1] - indptr[b]
        C = qo[b + 1] - qo[b]
        for i in range(C):
            n = L - C + i + 1
            ref, ref_lse = o.decode(q[qo[b] + i][None], k, v, np.array([0, n], np.int32),
                                    indices[indptr[b]:indptr[b] + n], scale, Hkv)
            assert np.abs(out[qo[b] + i] - ref[0]).max() < TOL, "prefill row vs decode"
            assert np.abs(lse[qo[b] + i] - ref_lse[0]).max() < TOL


# ----------------------------------------------------------------------------
# rotary position embedding pins (the append step)
# ----------------------------------------------------------------------------
def pin_rope_complex_rotation(o):
    """Rotate-half RoPE is the complex product (x_i + j x_{i+D/2}) e^{j p theta^(-2i/D)}:
    numpy complex arithmetic agrees to 1e-12."""
    rng = np.random.default_rng(41)
    for (T, H, D, theta) in [(5, 3, 8, 10000.0), (4, 2, 128, 1e6), (3, 1, 256, 5e5)]:
        x = _random_bits(rng, (T, H, D))
        pos = rng.integers(0, 40000, T).astype(np.int32)
        y = o.rope(x, pos, theta)
        xw = _widen(x)
        half = D // 2
        z = xw[..., :half] + 1j * xw[..., half:]
        ang = pos[:, None, None].astype(np.float64) * theta ** (-2.0 * np.arange(half) / D)[None, None, :]
        r = z * np.exp(1j * ang)
        ref = np.concatenate([r.real, r.imag], axis=-1)
        assert np.abs(y - ref).max() < 1e-12 * max(1.0, np.abs(ref).max()), "rope != complex rotation"


def pin_rope_closed_form(o):
    """D = 4, x = e_0 (pair 0) or e_1 (pair 1): y = (cos a, 0, sin a, 0) with
    a = p, and (0, cos b, 0, sin b) with b = p / sqrt(theta)."""
    theta = 10000.0
    for p in (0, 1, 7, 1234):
        e0 = _bf16_bits(np.array([[[1.0, 0.0, 0.0, 0.0]]]))
        e1 = _bf16_bits(np.array([[[0.0, 1.0, 0.0, 0.0]]]))
        y0 = o.rope(e0, np.array([p], np.int32), theta)[0, 0]
        y1 = o.rope(e1, np.array([p], np.int32), theta)[0, 0]
        a, b = float(p), float(p) / np.sqrt(theta)
        assert np.allclose(y0, [np.cos(a), 0, np.sin(a), 0], atol=1e-13), "pair 0 closed form"
        assert np.allclose(y1, [0, np.cos(b), 0, np.sin(b)], atol=1e-13), "pair 1 closed form"


def pin_rope_position_zero(o):
    """Position 0 leaves every row unchanged, exactly."""
    rng = np.random.default_rng(42)
    x = _random_bits(rng, (6, 4, 128))
    y = o.rope(x, np.zeros(6, np.int32), 1e6)
    assert np.array_equal(y, _widen(x)), "position 0 must be the identity"


def pin_rope_relative_position(o):
    """<R(m) q, R(n) k> depends on m - n only: equal to <R(m - n) q, k> (1e-9 relative)."""
    rng = np.random.default_rng(43)
    D, theta = 64, 1e4
    q = _random_bits(rng, (1, 1, D))
    k = _random_bits(rng, (1, 1, D))
    for (m, n) in [(5, 2), (1000, 37), (30000, 29999), (17, 17)]:
        lhs = float(np.dot(o.rope(q, np.array([m], np.int32), theta)[0, 0],
                           o.rope(k, np.array([n], np.int32), theta)[0, 0]))
        rhs = float(np.dot(o.rope(q, np.array([m - n], np.int32), theta)[0, 0], _widen(k)[0, 0]))
        assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(rhs)), f"relative position ({m}, {n})"


def pin_rope_norm(o):
    """Each pair (i, i + D/2) keeps its length."""
    rng = np.random.default_rng(44)
    D = 128
    x = _random_bits(rng, (8, 2, D))
    y = o.rope(x, rng.integers(0, 1 << 20, 8).astype(np.int32), 1e6)
    xw = _widen(x)
    nx = np.hypot(xw[..., :D // 2], xw[..., D // 2:])
    ny = np.hypot(y[..., :D // 2], y[..., D // 2:])
    assert np.abs(nx - ny).max() < 1e-12, "rotation changed a pair's length"


# ----------------------------------------------------------------------------
# 8-bit (OCP FP8 E4M3) pool pins
# ----------------------------------------------------------------------------
_ALL_CODES = np.arange(256, dtype=np.uint8)


def pin_e4m3_matches_torch(o):
    """All 256 E4M3 codes decode to torch's float8_e4m3fn values (NaN codes included)."""
    ours = o.e4m3_values(_ALL_CODES)
    ref = torch.from_numpy(_ALL_CODES.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref)), "NaN codes differ"
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok]), "E4M3 values differ from torch"


def pin_e4m3_closed_forms(o):
    """1.0, the largest finite value 448, the smallest normal 2^-6 and
    subnormal 2^-9, signed zero, and the NaN codes."""
    v = o.e4m3_values(np.array([0x38, 0x7E, 0x08, 0x01, 0x00, 0x80, 0xB8, 0x7F, 0xFF], np.uint8))
    assert list(v[:4]) == [1.0, 448.0, 2.0 ** -6, 2.0 ** -9], "E4M3 closed forms"
    assert v[4] == 0.0 and v[5] == 0.0 and np.signbit(v[5]) and v[6] == -1.0, "E4M3 signs"
    assert np.isnan(v[7]) and np.isnan(v[8]), "E4M3 NaN codes"


def pin_e4m3_widening_exact(o):
    """The bf16 patterns the fp8 decode attends over hold the codes' values exactly."""
    vals = o.e4m3_values(_ALL_CODES)
    wid = _widen(o.e4m3_to_bf16(_ALL_CODES))
    ok = ~np.isnan(vals)
    assert np.array_equal(wid[ok], vals[ok]) and np.all(np.isnan(wid[~ok])), "widening not exact"


def _fp8_case(rng, lengths, Hq, Hkv, D, spare=2):
    N = sum(lengths) + spare
    q = _random_bits(rng, (len(lengths), Hq, D))
    kc = torch.from_numpy(rng.standard_normal((N, Hkv, D)) * 2).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    vc = torch.from_numpy(rng.standard_normal((N, Hkv, D)) * 4).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    indptr = np.zeros(len(lengths) + 1, np.int32)
    indptr[1:] = np.cumsum(lengths)
    indices = np.arange(sum(lengths), dtype=np.int32) + spare
    return q, kc, vc, indptr, indices


def _f32(x: float) -> float:
    return float(np.float32(x))


def pin_decode_fp8_sdpa(o):
    """fp8 pools with per-pool scales that are not powers of two (0.37, 1.3)
    and a softmax scale 1/sqrt(32) that is not one either: torch SDPA
    (float64) on the values scale * torch's float8_e4m3fn value, contiguous
    slots, to 1e-12.  Every product is formed in double; a float32 product
    of two scales moves the scores by ~1e-8 and fails this pin."""
    rng = np.random.default_rng(51)
    for Hq, Hkv, D, lengths, k_scale, v_scale in [(8, 2, 32, [5, 1, 12], 0.37, 1.3),
                                                  (4, 4, 16, [3, 9], 0.5, 0.25)]:
        q, kc, vc, indptr, indices = _fp8_case(rng, lengths, Hq, Hkv, D)
        scale = workloads.softmax_scale(D)
        out, lse = o.decode_fp8(q, kc, vc, indptr, indices, scale, k_scale, v_scale, Hkv)
        kf = torch.from_numpy(kc.copy()).view(torch.float8_e4m3fn).to(torch.float64) * _f32(k_scale)
        vf = torch.from_numpy(vc.copy()).view(torch.float8_e4m3fn).to(torch.float64) * _f32(v_scale)
        sm = _f32(scale)
        for b in range(len(lengths)):
            ids = torch.from_numpy(indices[indptr[b]:indptr[b + 1]].astype(np.int64))
            qt = torch.from_numpy(_widen(q[b]))[None, :, None, :]
            kt = kf[ids].permute(1, 0, 2)[None].contiguous()
            vt = vf[ids].permute(1, 0, 2)[None].contiguous()
            ref = F.scaled_dot_product_attention(qt, kt, vt, scale=sm, enable_gqa=True)
            err = np.abs(out[b] - ref[0, :, 0, :].numpy()).max()
            assert err < TOL, f"fp8 decode vs sdpa {err} (scales {k_scale}, {v_scale})"
            g = Hq // Hkv
            s = sm * torch.einsum("hd,khd->hk", qt[0, :, 0, :],
                                  kt[0].permute(1, 0, 2).repeat_interleave(g, dim=1))
            ref_lse = torch.logsumexp(s, dim=1).numpy()
            err = np.abs(lse[b] - ref_lse).max()
            assert err < TOL, f"fp8 decode lse vs logsumexp {err}"


def pin_decode_fp8_single_token(o):
    """One listed slot: the output is v_scale times the code's value, exactly
    (the rounding of that one double product), and lse is the scaled dot
    product of q with k_scale times the K codes' values, summed exactly; an
    empty list gives out = 0 and lse = -inf."""
    rng = np.random.default_rng(52)
    Hq, Hkv, D = 4, 2, 8
    q, kc, vc, indptr, indices = _fp8_case(rng, [1, 1, 0], Hq, Hkv, D, spare=5)
    indices = np.array([3, 6], np.int32)
    k_scale, v_scale, scale = 0.37, 1.3, 0.3
    out, lse = o.decode_fp8(q, kc, vc, indptr, indices, scale, k_scale, v_scale, Hkv)
    assert np.all(out[2] == 0.0) and np.all(np.isneginf(lse[2])), "fp8 empty list"
    kval = o.e4m3_values(kc)
    vval = o.e4m3_values(vc)
    for b in range(2):
        for h in range(Hq):
            kh = h // (Hq // Hkv)
            want = _f32(v_scale) * vval[indices[b], kh]
            assert np.array_equal(out[b, h], want), "fp8 L=1 output is not v_scale * value"
            dot = sum((Fraction(float(x)) * Fraction(_f32(k_scale) * float(y))
                       for x, y in zip(_widen(q[b, h]), kval[indices[b], kh])), Fraction(0))
            assert abs(lse[b, h] - _f32(scale) * float(dot)) < 1e-14, "fp8 L=1 lse"


def pin_decode_fp8_unit_scales_equal_bf16(o):
    """With unit scales the fp8 decode equals the bf16 decode over pools that
    hold the codes' values (every E4M3 value is a bf16 value)."""
    rng = np.random.default_rng(53)
    q, kc, vc, indptr, indices = _fp8_case(rng, [7, 30, 2], 8, 2, 16)
    scale = workloads.softmax_scale(16)
    out8, lse8 = o.decode_fp8(q, kc, vc, indptr, indices, scale, 1.0, 1.0, 2)
    kb = _bf16_bits(torch.from_numpy(kc.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy())
    vb = _bf16_bits(torch.from_numpy(vc.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy())
    out, lse = o.decode(q, kb, vb, indptr, indices, scale, 2)
    assert np.abs(out8 - out).max() < TOL and np.abs(lse8 - lse).max() < TOL, "fp8 vs bf16 decode"


def _fp8_prefill_case(rng, cached, chunks, Hq, Hkv, D, spare=2):
    lengths = [p + c for p, c in zip(cached, chunks)]
    q_dec, kc, vc, indptr, indices = _fp8_case(rng, lengths, Hq, Hkv, D, spare)
    qo = np.zeros(len(chunks) + 1, np.int32)
    qo[1:] = np.cumsum(chunks)
    q = _random_bits(rng, (int(qo[-1]), Hq, D))
    return q, kc, vc, qo, indptr, indices


def pin_prefill_fp8_sdpa(o):
    """Chunked prefill over E4M3 pools at scales that are not powers of two:
    torch SDPA (float64) with an explicit bottom-right causal mask on the
    values scale * torch's float8_e4m3fn value, contiguous slots, to 1e-12."""
    rng = np.random.default_rng(54)
    for (Hq, Hkv, D, cached, chunks, k_scale, v_scale) in [(8, 2, 16, [5, 0, 3], [4, 3, 1], 0.37, 1.3),
                                                           (4, 1, 32, [9], [6], 2.5, 0.07)]:
        q, kc, vc, qo, indptr, indices = _fp8_prefill_case(rng, cached, chunks, Hq, Hkv, D)
        scale = workloads.softmax_scale(D)
        out, lse = o.prefill_fp8(q, kc, vc, qo, indptr, indices, scale, k_scale, v_scale, Hkv)
        kf = torch.from_numpy(kc.copy()).view(torch.float8_e4m3fn).to(torch.float64) * _f32(k_scale)
        vf = torch.from_numpy(vc.copy()).view(torch.float8_e4m3fn).to(torch.float64) * _f32(v_scale)
        for b, (P, C) in enumerate(zip(cached, chunks)):
            ids = torch.from_numpy(indices[indptr[b]:indptr[b + 1]].astype(np.int64))
            qt = torch.from_numpy(_widen(q[qo[b]:qo[b + 1]])).permute(1, 0, 2)[None]
            kt = kf[ids].permute(1, 0, 2)[None].contiguous()
            vt = vf[ids].permute(1, 0, 2)[None].contiguous()
            mask = torch.ones(C, P + C, dtype=torch.bool).tril(diagonal=P)
            ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=_f32(scale),
                                                 enable_gqa=True)
            err = np.abs(out[qo[b]:qo[b + 1]] - ref[0].permute(1, 0, 2).numpy()).max()
            assert err < TOL, f"fp8 prefill vs sdpa {err}"


def pin_prefill_fp8_rows_are_decodes(o):
    """Chunk row i over E4M3 pools equals the fp8 decode over the list's first
    P+i+1 entries (scattered slots, empty cached prefixes included)."""
    rng = np.random.default_rng(55)
    Hq, Hkv, D = 8, 2, 16
    q, kc, vc, qo, indptr, indices = _fp8_prefill_case(rng, [6, 0, 11], [5, 2, 1], Hq, Hkv, D, spare=9)
    indices = rng.permutation(kc.shape[0])[:indices.size].astype(np.int32)
    scale, k_scale, v_scale = workloads.softmax_scale(D), 0.37, 1.3
    out, lse = o.prefill_fp8(q, kc, vc, qo, indptr, indices, scale, k_scale, v_scale, Hkv)
    for b in range(3):
        L = indptr[b + 1] - indptr[b]
        C = qo[b + 1] - qo[b]
        for i in range(C):
            n = L - C + i + 1
            ref, ref_lse = o.decode_fp8(q[qo[b] + i][None], kc, vc, np.array([0, n], np.int32),
                                        indices[indptr[b]:indptr[b] + n], scale, k_scale, v_scale, Hkv)
            assert np.abs(out[qo[b] + i] - ref[0]).max() < TOL, "fp8 prefill row vs fp8 decode"
            assert np.abs(lse[qo[b] + i] - ref_lse[0]).max() < TOL


def pin_prefill_fp8_unit_scales_equal_bf16(o):
    """With unit scales the fp8 prefill equals the bf16 prefill over pools
    that hold the codes' values."""
    rng = np.random.default_rng(56)
    q, kc, vc, qo, indptr, indices = _fp8_prefill_case(rng, [7, 30, 2], [3, 5, 2], 8, 2, 16)
    scale = workloads.softmax_scale(16)
    out8, lse8 = o.prefill_fp8(q, kc, vc, qo, indptr, indices, scale, 1.0, 1.0, 2)
    out, lse = o.prefill(q, o.e4m3_to_bf16(kc), o.e4m3_to_bf16(vc), qo, indptr, indices, scale, 2)
    assert np.abs(out8 - out).max() < TOL and np.abs(lse8 - lse).max() < TOL, "fp8 vs bf16 prefill"


# ----------------------------------------------------------------------------
# Writing 8-bit pools: the E4M3 encoder and the append's rows
# ----------------------------------------------------------------------------
def _torch_codes(x) -> np.ndarray:
    """torch's float8_e4m3fn codes of float32 values (nearest even; NaN past 464)."""
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


_FINITE = torch.from_numpy(np.arange(0x7F, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _nearest_code(x: float) -> int:
    """Brute force in exact rationals over torch's table of the 127 finite
    magnitudes: the nearest one, a tie to the even code, sign kept; past 448
    the nearest finite value is 448 itself."""
    if np.isnan(x):
        return 0x7F
    sign = 0x80 if np.signbit(x) else 0
    a = Fraction(448) if np.isinf(x) else abs(Fraction(float(x)))
    best = min(range(0x7F), key=lambda c: (abs(Fraction(float(_FINITE[c])) - a), c & 1))
    return sign | best


def pin_e4m3_encode_round_trip(o):
    """Every finite code's own value encodes back to that code (both zeros too)."""
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    assert np.array_equal(o.e4m3_encode(o.e4m3_values(codes)), codes), "E4M3 round trip"


def pin_e4m3_encode_matches_torch(o):
    """Inside the finite range (|x| <= 464, the last tie) the codes equal
    torch's float8_e4m3fn rounding of float32 inputs: every midpoint between
    neighbouring codes (ties to even), and log-uniform magnitudes from 2^-12
    (below the smallest subnormal) to 464 of both signs."""
    rng = np.random.default_rng(61)
    mids = ((_FINITE[:-1] + _FINITE[1:]) / 2).tolist() + [464.0]
    mag = np.exp2(rng.uniform(-12, np.log2(464.0), 20000))
    x = np.concatenate([mids, -np.array(mids), mag * rng.choice([-1.0, 1.0], mag.size)])
    x = x.astype(np.float32).astype(np.float64)
    ours, ref = o.e4m3_encode(x), _torch_codes(x)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, f"E4M3 encode differs from torch at {x[bad[:4]]}: {ours[bad[:4]]} vs {ref[bad[:4]]}"


def pin_e4m3_encode_exact_nearest(o):
    """Doubles off the float32 grid against exact rational brute force: one
    double-precision step either side of every midpoint (2^-40 relative, far
    below a float's resolution, so a float-rounded quotient lands on the tie
    and fails), random doubles, and the subnormal edges."""
    rng = np.random.default_rng(62)
    mids = (_FINITE[:-1] + _FINITE[1:]) / 2
    near = np.concatenate([mids * (1 + 2.0 ** -40), mids * (1 - 2.0 ** -40), mids[:1] * 0.999999])
    rand = np.exp2(rng.uniform(-11, 8.8, 400)) * rng.choice([-1.0, 1.0], 400) * (1 + rng.uniform(0, 1e-9, 400))
    x = np.concatenate([near, -near, rand, [2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11, -2.0 ** -12]])
    ours = o.e4m3_encode(x)
    want = np.array([_nearest_code(v) for v in x], np.uint8)
    bad = np.nonzero(ours != want)[0]
    assert bad.size == 0, f"E4M3 encode not nearest at {x[bad[:4]]}: {ours[bad[:4]]} vs {want[bad[:4]]}"


def pin_e4m3_encode_saturation_and_specials(o):
    """448 and beyond (infinity included) saturate to +-448 (0x7E / 0xFE),
    NaN gives 0x7F, zeros keep their sign, tiny values round to a signed zero."""
    x = np.array([448.0, 449.0, 463.9, 464.0, 470.0, 480.0, 1e300, np.inf,
                  -448.0, -470.0, -np.inf, np.nan, 0.0, -0.0, 2.0 ** -11, -2.0 ** -11])
    want = [0x7E] * 8 + [0xFE] * 3 + [0x7F, 0x00, 0x80, 0x00, 0x80]
    assert list(o.e4m3_encode(x)) == want, "E4M3 saturation or special values"


def pin_e4m3_encode_scale(o):
    """A power-of-two scale s moves the input exactly, so encode(x, s) equals
    encode(x / s, 1) (computed here by exact scaling); a value that is
    s * value(code) for a scale s that is not a power of two encodes back to
    that code when the product is exact."""
    rng = np.random.default_rng(63)
    x = np.exp2(rng.uniform(-8, 6, 2000)) * rng.choice([-1.0, 1.0], 2000)
    for s in (4.0, 0.25):
        assert np.array_equal(o.e4m3_encode(x, s), o.e4m3_encode(x / s, 1.0)), f"scale {s}"
    s = 0.375                                  # 3/8: exact in float, not a power of two
    codes = np.arange(0x7F, dtype=np.uint8)    # value * 3/8 is exact in double for every code
    assert np.array_equal(o.e4m3_encode(_FINITE[codes] * s, s), codes), "scale 0.375 round trip"


def pin_append_e4m3_rows(o):
    """The rows the 8-bit append writes: values that are exact multiples of
    the pool scales (K at scale 2, V at scale 0.5) come back as their codes at
    position 0 (no rotation), a swap of the scales or of K and V shows; at
    position p a unit vector e_0 rotates into (cos p, sin p) on the pair
    (0, D/2), whose codes are the nearest to math.cos / math.sin."""
    import math
    rng = np.random.default_rng(64)
    T, H, D = 3, 2, 8
    kc = rng.integers(0, 0x7F, (T, H, D)).astype(np.uint8)
    vc = rng.integers(0x80, 0xFF, (T, H, D)).astype(np.uint8)
    kb = _bf16_bits(o.e4m3_values(kc) * 2.0)
    vb = _bf16_bits(o.e4m3_values(vc) * 0.5)
    k_out, v_out, _ = o.append_e4m3(kb, vb, np.zeros(T, np.int32), 1e4, 2.0, 0.5)
    assert np.array_equal(k_out, kc) and np.array_equal(v_out, vc), "append codes at position 0"
    e0 = np.zeros((1, 1, D))
    e0[0, 0, 0] = 1.0
    for p in (1, 2, 1000):
        k_out, _, _ = o.append_e4m3(_bf16_bits(e0), _bf16_bits(e0), np.array([p], np.int32), 1e4, 1.0, 1.0)
        assert k_out[0, 0, 0] == _nearest_code(math.cos(p)), f"cos({p})"
        assert k_out[0, 0, D // 2] == _nearest_code(math.sin(p)), f"sin({p})"


ALL_PINS = [
    pin_sdpa_decode, pin_bruteforce_tiny, pin_slot_order, pin_single_token, pin_two_tokens,
    pin_zero_query, pin_constant_values, pin_saturated_softmax, pin_empty_list,
    pin_duplicate_slots, pin_row_selection, pin_merge_of_splits, pin_merge_special_cases,
    pin_prefill_sdpa, pin_prefill_rows_are_decodes,
    pin_rope_complex_rotation, pin_rope_closed_form, pin_rope_position_zero,
    pin_rope_relative_position, pin_rope_norm,
    pin_e4m3_matches_torch, pin_e4m3_closed_forms, pin_e4m3_widening_exact, pin_decode_fp8_sdpa,
    pin_decode_fp8_single_token, pin_decode_fp8_unit_scales_equal_bf16,
    pin_e4m3_encode_round_trip, pin_e4m3_encode_matches_torch, pin_e4m3_encode_exact_nearest,
    pin_e4m3_encode_saturation_and_specials, pin_e4m3_encode_scale, pin_append_e4m3_rows,
    pin_prefill_fp8_sdpa, pin_prefill_fp8_rows_are_decodes, pin_prefill_fp8_unit_scales_equal_bf16,
]
