"""Seeded input generators: deterministic, shaped as the pages say, and
structurally as described (scattered distinct slots, shared prefixes)."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_shapes.json")


def test_shapes_match_pages():
    facts = {k: v["value"] for k, v in json.load(open(GOLDEN)).items() if not k.startswith("_")}
    for spec in (W.SINGLE_REQUEST_256, W.QWEN3_4B_BATCH8, W.BATCH64_SHARED_PREFIX,
                 W.PREFILL_CHUNK512, W.PREFILL_CHUNK64):
        assert (spec.num_qo_heads, spec.num_kv_heads, spec.head_dim) == (
            facts["qwen3_num_qo_heads"], facts["qwen3_num_kv_heads"], facts["qwen3_head_dim"])
    assert W.HEADDIM256_BATCH32.head_dim == facts["qwen35_full_attention_head_dim"]
    assert W.BATCH64_SHARED_PREFIX.num_layers == facts["qwen3_4b_num_layers"]
    assert W.QWEN3_4B_BATCH8.batch == facts["throughput_concurrency"]
    assert W.PREFILL_CHUNK512.chunk_len == facts["prefill_chunk_default"]
    assert W.PREFILL_CHUNK64.chunk_len == facts["prefill_chunk_with_decode"]


@pytest.mark.parametrize("spec", W.DECODE_SPECS, ids=lambda s: s.name)
def test_decode_lists(spec):
    indptr, indices = W.decode_lists(spec)
    indptr2, indices2 = W.decode_lists(spec)
    assert np.array_equal(indptr, indptr2) and np.array_equal(indices, indices2)
    assert indptr.dtype == np.int32 and indices.dtype == np.int32
    assert indptr[0] == 0 and indptr.size == spec.batch + 1
    lengths = np.diff(indptr)
    assert lengths.min() >= spec.len_lo and lengths.max() <= spec.len_hi
    assert indices.min() >= 0 and indices.max() < spec.num_slots
    lists = [indices[indptr[b]:indptr[b + 1]] for b in range(spec.batch)]
    for ids in lists:
        assert np.unique(ids).size == ids.size, "no slot repeats inside one request"
    if spec.prefix_group_size:
        g, P = spec.prefix_group_size, spec.prefix_len
        for b in range(spec.batch):
            lead = lists[b - b % g][:P]
            assert np.array_equal(lists[b][:P], lead), "group shares its prefix"
        owned = np.concatenate([ids[P:] for ids in lists] + [lists[b][:P] for b in range(0, spec.batch, g)])
        assert np.unique(owned).size == owned.size, "suffixes and prefixes distinct"
    else:
        assert np.unique(indices).size == indices.size, "slots distinct across requests"


def test_batch64_workload_size():
    indptr, indices = W.decode_lists(W.BATCH64_SHARED_PREFIX)
    assert 64 * 2048 <= indptr[-1] <= 64 * 8192
    assert np.unique(indices).size < indices.size  # prefixes shared


@pytest.mark.parametrize("spec", W.PREFILL_SPECS, ids=lambda s: s.name)
def test_prefill_lists(spec):
    qo, indptr, indices = W.prefill_lists(spec)
    assert np.array_equal(np.diff(qo), np.full(spec.batch, spec.chunk_len))
    assert np.array_equal(np.diff(indptr), np.full(spec.batch, spec.cached_len + spec.chunk_len))
    assert np.unique(indices).size == indices.size


def test_tensors_seeded_and_rounded():
    a = W.normal_bf16((3, 5, 7), 42)
    b = W.normal_bf16((3, 5, 7), 42)
    assert a.dtype == torch.bfloat16 and torch.equal(a, b)
    c = W.normal_bf16((3, 5, 7), 43)
    assert not torch.equal(a, c)
    d = W.normal_bf16((3, 5, 7), 42, chunk_elems=8)
    assert torch.equal(d, W.normal_bf16((3, 5, 7), 42, chunk_elems=8))
    assert W.softmax_scale(128) == float(np.float32(1 / np.sqrt(128)))


def test_poison_unreferenced():
    pool = torch.zeros(10, 2, 4, dtype=torch.bfloat16)
    W.poison_unreferenced(pool, [1, 5, 5, 9])
    ref = torch.isnan(pool).all(dim=(1, 2))
    assert ref.tolist() == [True, False, True, True, True, False, True, True, True, False]
