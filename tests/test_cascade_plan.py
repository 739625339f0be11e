"""Host partitioner of cascade decode plans (pa_partition_cascade): the
prefix units and the decode units together cover every (request, KV head)
list exactly once, every merge names exactly the slots its parts write, and
no two parts share a slot.  The GPU results are checked against the oracle
in test_cascade_gpu.py."""
from collections import defaultdict

import numpy as np
import pytest

import paged_gqa_decode_pa_amd as pa
import workloads as W

MAX_PARTS = 16


def _indptr(lengths):
    ip = np.zeros(len(lengths) + 1, np.int32)
    ip[1:] = np.cumsum(lengths)
    return ip


def check_cascade(ip, gi, pl, Hq, Hkv, flags=0, max_wg=0):
    offs, units, merges, n_p, pre = pa.pa_partition_cascade(ip, gi, pl, Hq, Hkv, 128, flags, max_wg)
    B, g = ip.size - 1, Hq // Hkv
    assert offs[0] == 0 and offs[-1] == units.size
    skip = np.zeros(B, np.int64)
    cached = np.zeros(B, np.int64)
    for k in range(gi.size - 1):
        # groups with fewer than 64 member query rows get no prefix units
        # unless every group is asked for; their shared prefix is read with
        # cached loads instead (when there is someone to share it with)
        members = gi[k + 1] - gi[k]
        if members * g >= 64 or flags & pa.PA_PLAN_CASCADE_ALL:
            skip[gi[k]:gi[k + 1]] = pl[k]
        elif members > 1:
            cached[gi[k]:gi[k + 1]] = pl[k]
    written = defaultdict(int)          # partial slot -> times written
    # decode units: the list after the prefix, in order, once
    by_seg = defaultdict(list)
    for u in units:
        b, h = int(u["request"]), int(u["kv_head"])
        assert u["part_stride"] == 0 and (u["q_begin"], u["q_end"]) == (b, b + 1)
        assert u["cached_end"] == (ip[b] + cached[b] if cached[b] > 0 else 0)
        by_seg[(b, h)].append(u)
    merge_of = {(int(m["request"]), int(m["kv_head"])): m for m in merges}
    assert len(merge_of) == merges.size
    for b in range(B):
        for h in range(Hkv):
            us = sorted(by_seg[(b, h)], key=lambda u: (u["kv_begin"], u["kv_end"]))
            assert us, "every segment has a decode unit (possibly empty)"
            pos = ip[b] + skip[b]
            for u in us:
                assert u["kv_begin"] == pos
                pos = u["kv_end"]
            assert pos == ip[b + 1]
            if skip[b] > 0 or len(us) > 1:
                m = merge_of[(b, h)]
                assert m["n_parts"] == len(us)
                parts = sorted(int(u["partial"]) for u in us)
                assert parts == list(range(m["first_partial"], m["first_partial"] + len(us)))
                for s in parts:
                    written[s] += 1
                if skip[b] > 0:
                    assert m["prefix_parts"] >= 1
                else:
                    assert m["prefix_parts"] == 0
            else:
                assert us[0]["partial"] == -1 and (b, h) not in merge_of
    # prefix units: per group, subgroups of <= tile rows / g members, each prefix cut
    # into K parts per head; member t of part k writes slot partial + t*K
    covered = defaultdict(list)
    for u in pre:
        s0, m_, h = int(u["q_begin"]), int(u["q_end"] - u["q_begin"]), int(u["kv_head"])
        K = int(u["part_stride"])
        assert 1 <= m_ <= pa.pa_prefill_tile_rows(128) // g and 1 <= K <= MAX_PARTS
        assert u["request"] == s0 and u["merge"] == -1 and u["diag"] == u["kv_end"] - 1
        for t in range(m_):
            b = s0 + t
            assert skip[b] > 0
            covered[(b, h)].append((int(u["kv_begin"]) - ip[s0], int(u["kv_end"]) - ip[s0]))
            written[int(u["partial"]) + t * K] += 1
            m = merge_of[(b, h)]
            assert m["prefix_parts"] == K
            assert m["prefix_first"] <= u["partial"] + t * K < m["prefix_first"] + K
    for b in range(B):
        for h in range(Hkv):
            if skip[b] == 0:
                assert (b, h) not in covered
                continue
            parts = sorted(covered[(b, h)])
            pos = 0
            for lo, hi in parts:
                assert lo == pos and hi > lo
                pos = hi
            assert pos == skip[b]
    assert all(v == 1 for v in written.values()), "a partial slot written twice"
    assert sorted(written) == list(range(n_p)), "partial slots dense"
    return offs, units, merges, n_p, pre


def test_batch64_groups():
    ip, _ = W.decode_lists(W.BATCH64_SHARED_PREFIX)
    gi = np.arange(0, 65, 4, dtype=np.int32)
    pl = np.full(16, 1024, np.int32)
    # groups of 4 requests (16 query rows per KV head) stay plain decode ...
    offs, units, merges, n_p, pre = check_cascade(ip, gi, pl, 32, 8, max_wg=768)
    assert pre.size == 0
    plain = pa.pa_partition(ip, None, 32, 8, 128, 0, 768)
    # the same split; only the prefix entries are marked for cached loads
    assert np.array_equal(plain[0], offs) and np.array_equal(plain[2], merges)
    fields = [f for f in units.dtype.names if f != "cached_end"]
    assert all(np.array_equal(plain[1][f], units[f]) for f in fields)
    assert np.all(plain[1]["cached_end"] == 0)
    assert np.all(units["cached_end"] == ip[units["request"]] + 1024)
    # ... unless every group is asked for
    offs, units, merges, n_p, pre = check_cascade(ip, gi, pl, 32, 8, pa.PA_PLAN_CASCADE_ALL, 768)
    assert pre.size == 16 * 8 * 6       # 1024 entries in 6 parts: ~768 prefix units
    assert offs.size - 1 == 768


def test_system_prompt_groups():
    ip, _ = W.decode_lists(W.SYSTEM_PROMPT_B64)
    gi = np.array([0, 64], np.int32)
    pl = np.array([4096], np.int32)
    offs, units, merges, n_p, pre = check_cascade(ip, gi, pl, 32, 8, max_wg=768)
    members = pa.pa_prefill_tile_rows(128) // 4          # requests per prefix unit
    assert pre.size == -(-64 // members) * 8 * 16        # subgroups x KV heads x 16 parts of 256 entries


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (16, 4), (64, 8), (8, 8)])
def test_random_groups(seed, Hq, Hkv):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 80))
    lengths = rng.integers(0, 4000, size=B)
    # random consecutive groups, some large (subgroups), some singletons
    cuts = sorted(set(rng.integers(1, B, size=int(rng.integers(0, B))).tolist()) | {0, B})
    gi = np.array(cuts, np.int32)
    pl = np.zeros(gi.size - 1, np.int32)
    for k in range(gi.size - 1):
        shortest = int(lengths[gi[k]:gi[k + 1]].min())
        pl[k] = int(rng.choice([0, shortest, rng.integers(0, shortest + 1)]))
    ip = _indptr(lengths)
    for flags in (0, pa.PA_PLAN_NO_XCD_ORDER, pa.PA_PLAN_CASCADE_ALL,
                  pa.PA_PLAN_CASCADE_ALL | pa.PA_PLAN_NO_XCD_ORDER):
        for max_wg in (0, 37):
            check_cascade(ip, gi, pl, Hq, Hkv, flags, max_wg)


def test_large_group_is_split():
    ip = _indptr([3000] * 70)
    gi = np.array([0, 70], np.int32)
    offs, units, merges, n_p, pre = check_cascade(ip, gi, np.array([2500], np.int32), 32, 8,
                                                  pa.PA_PLAN_CASCADE_ALL)
    members = sorted(set((int(u["q_begin"]), int(u["q_end"])) for u in pre))
    m = pa.pa_prefill_tile_rows(128) // 4
    assert members == [(s0, min(70, s0 + m)) for s0 in range(0, 70, m)]


def test_no_prefix_is_plain_decode():
    ip, _ = W.decode_lists(W.QWEN3_4B_BATCH8)
    gi = np.array([0, 4, 8], np.int32)
    a = pa.pa_partition(ip, None, 32, 8, 128)
    b = pa.pa_partition_cascade(ip, gi, np.zeros(2, np.int32), 32, 8, 128)
    assert all(np.array_equal(x, y) for x, y in zip(a[:3], b[:3])) and a[3] == b[3]
    assert np.all(b[1]["cached_end"] == 0)
    assert b[4].size == 0


@pytest.mark.parametrize("gi,pl", [
    ([0, 2], [5]),            # does not reach batch
    ([1, 3], [5]),            # does not start at 0
    ([0, 2, 1, 3], [1, 1, 1]),  # decreasing
    ([0, 3], [101]),          # longer than the shortest member list
    ([0, 3], [-1]),
    ([0, 0, 3], [4, 0]),      # prefix for an empty group
])
def test_bad_groups(gi, pl):
    ip = _indptr([100, 200, 300])
    with pytest.raises(pa.PAError) as e:
        pa.pa_partition_cascade(ip, np.array(gi, np.int32), np.array(pl, np.int32), 32, 8, 128)
    assert e.value.status == pa.PA_ERR_INVALID_ARG


def test_forced_splits_rejected():
    ip = _indptr([100, 200])
    with pytest.raises(pa.PAError):
        pa.pa_partition_cascade(ip, np.array([0, 2], np.int32), np.array([50], np.int32), 32, 8,
                                128, pa.PA_PLAN_FORCE_SPLITS(2))


@pytest.mark.parametrize("seed", range(8))
def test_prefix_counts_within_plan_capacity(seed):
    """The prefix units and slots of any cascade partition stay within what a
    plan reserves: units <= max(segments, min(16*segments, 2*W)) and slots <=
    max(segments, min(16*segments, 2*(rows/g)*W)), W = decode workgroups, rows = prefill tile rows."""
    rng = np.random.default_rng(500 + seed)
    Hq, Hkv = [(32, 8), (64, 8), (16, 4), (8, 8)][seed % 4]
    g = Hq // Hkv
    B = int(rng.integers(1, 200))
    lengths = rng.integers(64, 3000, size=B)
    cuts = sorted(set(rng.integers(1, B, size=int(rng.integers(0, max(1, B // 3)))).tolist()) | {0, B})
    gi = np.array(cuts, np.int32)
    pl = np.array([int(lengths[gi[k]:gi[k + 1]].min()) for k in range(gi.size - 1)], np.int32)
    W = 768
    offs, units, merges, n_p, pre = pa.pa_partition_cascade(ip := _indptr(lengths), gi, pl, Hq, Hkv,
                                                            128, pa.PA_PLAN_CASCADE_ALL, W)
    segs = B * Hkv
    decode_slots = sum(int(m["n_parts"]) for m in merges)
    prefix_slots = n_p - decode_slots
    assert pre.size <= max(segs, min(16 * segs, 2 * W))
    assert prefix_slots <= max(segs, min(16 * segs, 2 * (pa.pa_prefill_tile_rows(128) // g) * W))
