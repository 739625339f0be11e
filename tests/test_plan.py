"""Host partitioner (pa_partition): coverage, partial/merge bookkeeping, XCD
placement and determinism.  The partition is one of many valid ones, so the
tests check what every valid partition must satisfy."""
from collections import defaultdict

import numpy as np
import pytest

import paged_gqa_decode_pa_amd as pa
import workloads as W

XCD = 8


def _indptr(lengths):
    ip = np.zeros(len(lengths) + 1, np.int32)
    ip[1:] = np.cumsum(lengths)
    return ip


def check_offsets(offs, units):
    assert offs[0] == 0 and offs[-1] == units.size and np.all(np.diff(offs) >= 0)


def check_decode(units, merges, n_partials, indptr, Hkv, forced=None):
    B = indptr.size - 1
    real = units[units["request"] >= 0]
    assert real.size == units.size, "no padding units"
    by_stream = defaultdict(list)
    for u in real:
        b, h = int(u["request"]), int(u["kv_head"])
        assert 0 <= b < B and 0 <= h < Hkv
        assert indptr[b] <= u["kv_begin"] <= u["kv_end"] <= indptr[b + 1]
        assert (u["q_begin"], u["q_end"]) == (b, b + 1)
        assert u["diag"] == u["kv_end"] - 1
        by_stream[(b, h)].append(u)
    assert set(by_stream) == {(b, h) for b in range(B) for h in range(Hkv)}
    seen_partials = []
    merge_of = {(int(m["request"]), int(m["kv_head"])): m for m in merges}
    assert len(merge_of) == len(merges)
    for (b, h), us in by_stream.items():
        us = sorted(us, key=lambda u: (u["kv_begin"], u["kv_end"]))
        # the parts tile the request's list exactly, in order, without overlap
        pos = indptr[b]
        for u in us:
            assert u["kv_begin"] == pos
            pos = u["kv_end"]
        assert pos == indptr[b + 1]
        if forced:
            assert len(us) == forced
            sizes = [u["kv_end"] - u["kv_begin"] for u in us]
            assert max(sizes) - min(sizes) <= 1
        if len(us) == 1:
            assert us[0]["partial"] == -1 and (b, h) not in merge_of
        else:
            parts = [int(u["partial"]) for u in us]
            assert min(parts) >= 0
            m = merge_of[(b, h)]
            assert m["n_parts"] == len(us)
            assert sorted(parts) == list(range(m["first_partial"], m["first_partial"] + len(us)))
            assert (m["q_begin"], m["q_end"]) == (b, b + 1)
            seen_partials += parts
    assert sorted(seen_partials) == list(range(n_partials))


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 4, 256), (8, 8, 128), (64, 8, 256)])
def test_decode_partition_random(seed, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lengths = rng.integers(0, 3000, size=B)
    lengths[rng.random(B) < 0.2] = 0
    ip = _indptr(lengths)
    for flags in (0, pa.PA_PLAN_NO_XCD_ORDER):
        for max_wg in (0, 1, 37, 2048):
            offs, units, merges, n_p = pa.pa_partition(ip, None, Hq, Hkv, D, flags, max_wg)
            check_offsets(offs, units)
            check_decode(units, merges, n_p, ip, Hkv)
            n_wg = offs.size - 1
            limit = max_wg if max_wg > 0 else 768
            if flags & pa.PA_PLAN_NO_XCD_ORDER:
                assert n_wg <= limit
            else:
                assert n_wg % XCD == 0 and n_wg <= limit + XCD


@pytest.mark.parametrize("n", [1, 2, 3, 7, 64, 256])
def test_forced_splits(n):
    ip = _indptr([0, 1, 5, 100, 333])
    offs, units, merges, n_p = pa.pa_partition(ip, None, 32, 8, 128, pa.PA_PLAN_FORCE_SPLITS(n))
    check_offsets(offs, units)
    assert np.all(np.diff(offs) <= 1), "forced parts run one per workgroup"
    check_decode(units, merges, n_p, ip, 8, forced=n)


def test_forced_split_limit():
    ip = _indptr([10])
    with pytest.raises(pa.PAError) as e:
        pa.pa_partition(ip, None, 32, 8, 128, pa.PA_PLAN_FORCE_SPLITS(257))
    assert e.value.status == pa.PA_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [[1, 5], [0, 5, 3], [0, -1]])
def test_bad_indptr(bad):
    with pytest.raises(pa.PAError) as e:
        pa.pa_partition(np.array(bad, np.int32), None, 32, 8, 128)
    assert e.value.status == pa.PA_ERR_INVALID_ARG


def test_unknown_flag():
    with pytest.raises(pa.PAError):
        pa.pa_partition(_indptr([5]), None, 32, 8, 128, 0x80)


def test_deterministic():
    ip, _ = W.decode_lists(W.BATCH64_SHARED_PREFIX)
    a = pa.pa_partition(ip, None, 32, 8, 128)
    b = pa.pa_partition(ip, None, 32, 8, 128)
    assert all(np.array_equal(x, y) for x, y in zip(a[:3], b[:3])) and a[3] == b[3]


def test_batch64_partition_shape():
    """The batch-64 shared-prefix workload: one workgroup per resident slot,
    equal budgets, each (head, request) list opening its own workgroup, and
    requests of one prefix group opened side by side on one XCD."""
    ip, _ = W.decode_lists(W.BATCH64_SHARED_PREFIX)
    max_wg = 768
    offs, units, merges, n_p = pa.pa_partition(ip, None, 32, 8, 128, 0, max_wg)
    check_offsets(offs, units)
    check_decode(units, merges, n_p, ip, 8)
    n_wg = offs.size - 1
    assert n_wg == max_wg
    cost = np.array([(units["kv_end"][offs[w]:offs[w + 1]] - units["kv_begin"][offs[w]:offs[w + 1]]).sum()
                     + 128 * (offs[w + 1] - offs[w]) for w in range(n_wg)])
    assert cost.max() <= cost.mean() * 1.05
    # the first unit of workgroup id wg(i) opens segment i = head * B + request
    per_xcd = n_wg // XCD
    B = ip.size - 1
    for i in range(8 * B):
        wg = (i % per_xcd) * XCD + i // per_xcd
        first = units[offs[wg]]
        h, b = divmod(i, B)
        assert (first["request"], first["kv_head"], first["kv_begin"]) == (b, h, ip[b])
        if b % 4 == 3:   # the group b-3..b sits on one XCD
            xcds = {((i - k) // per_xcd) for k in range(4)}
            assert len(xcds) == 1


def _wg_costs(offs, units):
    return np.array([(units["kv_end"][offs[w]:offs[w + 1]] - units["kv_begin"][offs[w]:offs[w + 1]]).sum()
                     + 128 * (offs[w + 1] - offs[w]) for w in range(offs.size - 1)])


def test_unit_weights_give_the_unweighted_partition():
    ip, _ = W.decode_lists(W.BATCH64_SHARED_PREFIX)
    a = pa.pa_partition(ip, None, 32, 8, 128)
    b = pa.pa_partition(ip, None, 32, 8, 128, xcd_weights=np.ones(XCD))
    assert all(np.array_equal(x, y) for x, y in zip(a[:3], b[:3])) and a[3] == b[3]
    # the feedback flag is a pa_plan matter: the partition ignores it
    c = pa.pa_partition(ip, None, 32, 8, 128, pa.PA_PLAN_SPEED_FEEDBACK)
    assert all(np.array_equal(x, y) for x, y in zip(a[:3], c[:3]))


def test_weighted_partition_budgets():
    """Workgroups on XCD x get weight_x times an equal share; every
    partition invariant still holds."""
    ip, _ = W.decode_lists(W.BATCH64_SHARED_PREFIX)
    w = np.array([0.7, 1.3, 1.0, 1.1, 0.9, 1.25, 0.8, 0.95])
    offs, units, merges, n_p = pa.pa_partition(ip, None, 32, 8, 128, 0, 768, xcd_weights=w)
    check_offsets(offs, units)
    check_decode(units, merges, n_p, ip, 8)
    cost = _wg_costs(offs, units)
    assert cost.size == 768
    xcd_of = np.arange(cost.size) % XCD
    per_xcd = np.array([cost[xcd_of == x].mean() for x in range(XCD)])
    share = per_xcd / per_xcd.mean()
    np.testing.assert_allclose(share, w / w.mean(), rtol=0.03)
    base = cost.sum() / (w[xcd_of]).sum()
    assert np.all(cost <= base * w[xcd_of] * 1.05 + 128)


@pytest.mark.parametrize("seed", range(6))
def test_weighted_partition_random(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 70))
    lengths = rng.integers(0, 6000, size=B)
    lengths[rng.random(B) < 0.2] = 0
    ip = _indptr(lengths)
    w = rng.uniform(0.25, 4.0, size=XCD)
    for flags in (0, pa.PA_PLAN_NO_XCD_ORDER, pa.PA_PLAN_FORCE_SPLITS(3)):
        for max_wg in (0, 37, 768):
            offs, units, merges, n_p = pa.pa_partition(ip, None, 32, 8, 128, flags, max_wg,
                                                       xcd_weights=w)
            check_offsets(offs, units)
            check_decode(units, merges, n_p, ip, 8, forced=3 if flags & 0xFF00 else None)
    # weights are ignored where the split is not the automatic XCD-ordered one
    for flags in (pa.PA_PLAN_NO_XCD_ORDER, pa.PA_PLAN_FORCE_SPLITS(3)):
        a = pa.pa_partition(ip, None, 32, 8, 128, flags, 768)
        b = pa.pa_partition(ip, None, 32, 8, 128, flags, 768, xcd_weights=w)
        assert all(np.array_equal(x, y) for x, y in zip(a[:3], b[:3]))


def test_workgroup_weighted_budgets():
    """Workgroup id w gets wg_weights[w] (times its XCD's weight) of an equal
    share, whichever bin lands on it."""
    ip, _ = W.decode_lists(W.BATCH64_SHARED_PREFIX)
    rng = np.random.default_rng(5)
    ww = rng.uniform(0.6, 1.4, size=768)
    xw = np.array([1.1, 0.9, 1.0, 1.0, 1.2, 0.8, 1.0, 1.0])
    offs, units, merges, n_p = pa.pa_partition(ip, None, 32, 8, 128, 0, 768, xcd_weights=xw,
                                               wg_weights=ww)
    check_offsets(offs, units)
    check_decode(units, merges, n_p, ip, 8)
    cost = _wg_costs(offs, units)
    want = ww * xw[np.arange(768) % XCD]
    ratio = (cost / cost.sum()) / (want / want.sum())
    assert np.percentile(np.abs(ratio - 1), 95) < 0.05 and ratio.max() < 1.1
    # short weight arrays: ids beyond them weigh 1; plain order ignores XCD weights
    for flags, x in ((0, None), (pa.PA_PLAN_NO_XCD_ORDER, xw)):
        for nw in (1, 100, 768, 1000):
            o2, u2, m2, p2 = pa.pa_partition(ip, None, 32, 8, 128, flags, 768, xcd_weights=x,
                                             wg_weights=np.full(nw, 0.7))
            check_offsets(o2, u2)
            check_decode(u2, m2, p2, ip, 8)


@pytest.mark.parametrize("w", [[1.0] * 7, [1.0] * 9, [1.0] * 7 + [0.2], [1.0] * 7 + [4.5],
                               [1.0] * 7 + [float("nan")], [1.0] * 7 + [float("inf")]])
def test_bad_weights(w):
    with pytest.raises(pa.PAError) as e:
        pa.pa_partition(_indptr([100, 200]), None, 32, 8, 128, xcd_weights=w)
    assert e.value.status == pa.PA_ERR_INVALID_ARG
    if len(w) == 8:
        with pytest.raises(pa.PAError) as e:
            pa.pa_partition(_indptr([100, 200]), None, 32, 8, 128, wg_weights=w)
        assert e.value.status == pa.PA_ERR_INVALID_ARG


def test_decode_small_batch_uses_fewer_workgroups():
    """A small step does not spread below the minimum useful piece."""
    ip = _indptr([256])
    offs, units, merges, n_p = pa.pa_partition(ip, None, 32, 8, 128, pa.PA_PLAN_NO_XCD_ORDER, 768)
    assert offs.size - 1 == 8          # 8 heads x 256 tokens, 256-token minimum
    check_decode(units, merges, n_p, ip, 8)


def check_prefill(units, merges, n_p, qo, ip, Hkv, group):
    B = ip.size - 1
    real = units[units["request"] >= 0]
    assert real.size == units.size
    tiles = defaultdict(list)
    for u in real:
        tiles[(int(u["request"]), int(u["kv_head"]), int(u["q_begin"]), int(u["q_end"]))].append(u)
    qt = pa.pa_prefill_tile_rows(128) // group
    want = set()
    for b in range(B):
        C = qo[b + 1] - qo[b]
        for h in range(Hkv):
            for t0 in range(0, C, qt):
                want.add((b, h, qo[b] + t0, qo[b] + min(C, t0 + qt)))
    assert set(tiles) == want
    merge_of = {(int(m["request"]), int(m["kv_head"]), int(m["q_begin"])): m for m in merges}
    all_parts = []
    for (b, h, q0, q1), us in tiles.items():
        L = ip[b + 1] - ip[b]
        C = qo[b + 1] - qo[b]
        P = L - C
        t0, t1 = q0 - qo[b], q1 - qo[b]
        us = sorted(us, key=lambda u: u["kv_begin"])
        pos = ip[b]
        for u in us:
            assert u["kv_begin"] == pos and u["diag"] == ip[b] + P + t0
            pos = u["kv_end"]
        assert pos == ip[b] + P + t1  # ends at the last row's causal window
        if len(us) > 1:
            m = merge_of[(b, h, q0)]
            parts = sorted(int(u["partial"]) for u in us)
            assert parts == list(range(m["first_partial"], m["first_partial"] + len(us)))
            all_parts += parts
        else:
            assert us[0]["partial"] == -1
    assert sorted(all_parts) == list(range(n_p))


@pytest.mark.parametrize("spec", W.PREFILL_SPECS, ids=lambda s: s.name)
def test_prefill_partition_workloads(spec):
    qo, ip, _ = W.prefill_lists(spec)
    offs, units, merges, n_p = pa.pa_partition(ip, qo, spec.num_qo_heads, spec.num_kv_heads, spec.head_dim)
    check_offsets(offs, units)
    assert np.all(np.diff(offs) <= 1)
    check_prefill(units, merges, n_p, qo, ip, spec.num_kv_heads, spec.num_qo_heads // spec.num_kv_heads)
    real = units[units["request"] >= 0]
    assert real.size >= 256


@pytest.mark.parametrize("seed", range(6))
def test_prefill_partition_random(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 6))
    chunks = rng.integers(0, 300, size=B)
    cached = rng.integers(0, 2000, size=B)
    ip = _indptr(chunks + cached)
    qo = _indptr(chunks)
    for Hq, Hkv in ((32, 8), (8, 8), (16, 2)):
        for flags in (0, pa.PA_PLAN_FORCE_SPLITS(3)):
            offs, units, merges, n_p = pa.pa_partition(ip, qo, Hq, Hkv, 128, flags)
            check_offsets(offs, units)
            check_prefill(units, merges, n_p, qo, ip, Hkv, Hq // Hkv)


def test_prefill_chunk_longer_than_list():
    with pytest.raises(pa.PAError) as e:
        pa.pa_partition(_indptr([5]), _indptr([6]), 32, 8, 128)
    assert e.value.status == pa.PA_ERR_INVALID_ARG


def test_forced_splits_capacity_guarantee():
    """The documented capacity: Hkv * (max_batch + max_kv_total / 256) units."""
    from paged_gqa_decode_pa_amd import pa_partition
    ip = _indptr([10, 20, 30])
    n = 50
    offs, units, merges, n_p = pa_partition(ip, None, 32, 8, 128, pa.PA_PLAN_FORCE_SPLITS(n))
    assert n_p == 3 * 8 * n
    assert n_p <= 8 * (3 + (3 * n * 256) // 256)


def test_prefill_kv_cut_one_round():
    """Chunk tiles that cannot fill the GPU get their KV ranges cut into about
    one part per compute unit (one round of the resident prefill
    workgroups); tiles that fill it alone are not cut.  Every part of a tile
    covers a disjoint, contiguous piece of its causal window."""
    rows = pa.pa_prefill_tile_rows(128)
    tiles512 = 8 * 8 * 512 // (rows // 4)        # requests x KV heads x tiles of rows/4 tokens
    tiles64 = 8 * 8 * max(1, 64 // (rows // 4))
    parts64 = -(-256 // tiles64)                # about one part per compute unit
    for spec, n_units, n_merges in ((W.PREFILL_CHUNK512, tiles512, 0),
                                    (W.PREFILL_CHUNK64, tiles64 * parts64, tiles64)):
        qo, ip, idx = W.prefill_lists(spec)
        offs, units, merges, n_p = pa.pa_partition(ip, qo, spec.num_qo_heads, spec.num_kv_heads,
                                                   spec.head_dim)
        assert len(units) == n_units and len(merges) == n_merges
        for m in merges:
            parts = units[(units["request"] == m["request"]) & (units["kv_head"] == m["kv_head"])
                          & (units["q_begin"] == m["q_begin"])]
            parts = np.sort(parts, order="kv_begin")
            assert len(parts) == m["n_parts"]
            assert parts["kv_begin"][0] == ip[m["request"]]
            assert np.all(parts["kv_begin"][1:] == parts["kv_end"][:-1])
            # the last part ends at the window of the tile's last row
            t1 = m["q_end"] - qo[m["request"]]
            P = (ip[m["request"] + 1] - ip[m["request"]]) - (qo[m["request"] + 1] - qo[m["request"]])
            assert parts["kv_end"][-1] == ip[m["request"]] + P + t1
