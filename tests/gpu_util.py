"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
the fp64 oracle on the same bf16 bits."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads as W

# Tolerance on the fp32 output (and the natural-log lse) against the fp64 oracle.
TOL = 2e-3


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda", 0)


def run_decode(q, k_pool, v_pool, kv_indptr, kv_indices_dev, sm_scale, num_kv_heads,
               flags=0, with_lse=True, slot_stride=None, num_slots=None):
    """HIP decode through the C ABI -> (out float32 [B,Hq,D], lse float32 [B,Hq]) on the host."""
    import paged_gqa_decode_pa_amd as pa
    B, Hq, D = q.shape
    kv_total = int(kv_indptr[-1])
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=q.device)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device) if with_lse else None
    forced = (flags >> pa.PA_PLAN_FORCE_SPLITS_SHIFT) & 0xFFFF
    capacity = max(kv_total, 1, B * forced * 256)   # room for the forced parts
    with pa.Plan(max(B, 1), capacity, Hq, num_kv_heads, D) as plan:
        plan.plan(kv_indptr, flags=flags)
        plan.decode(q, k_pool, v_pool, kv_indices_dev, sm_scale, out, lse,
                    slot_stride=slot_stride, num_slots=num_slots)
        torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if with_lse else None)


def oracle_decode(q, k_pool, v_pool, kv_indptr, kv_indices, sm_scale, num_kv_heads, sel=None):
    ref = oracle.load()
    return ref.decode(W.bits(q), W.bits(k_pool), W.bits(v_pool), kv_indptr,
                      np.asarray(kv_indices, np.int32), sm_scale, num_kv_heads, sel=sel)


def max_err(gpu: np.ndarray, ref: np.ndarray, rows=None) -> float:
    g = gpu.reshape(-1, gpu.shape[-1]) if gpu.ndim > 1 else gpu.reshape(-1, 1)
    r = ref.reshape(g.shape)
    if rows is not None:
        g, r = g[rows], r[rows]
    both_inf = np.isneginf(g) & np.isneginf(r)
    d = np.where(both_inf, 0.0, np.abs(g.astype(np.float64) - r))
    return float(np.nanmax(d)) if d.size else 0.0


def run_prefill(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices_dev, sm_scale, num_kv_heads,
                flags=0, with_lse=True):
    """HIP chunked prefill through the C ABI -> (out [T,Hq,D], lse [T,Hq]) on the host."""
    import paged_gqa_decode_pa_amd as pa
    T, Hq, D = q.shape
    B = len(kv_indptr) - 1
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.float32, device=q.device)
    lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device=q.device) if with_lse else None
    with pa.Plan(max(B, 1), max(int(kv_indptr[-1]), 1), Hq, num_kv_heads, D,
                 max_q_total=max(T, 1)) as plan:
        plan.plan(kv_indptr, qo_indptr, flags=flags)
        plan.prefill(q, k_pool, v_pool, kv_indices_dev, sm_scale, out, lse)
        torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if with_lse else None)


def oracle_prefill(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, sm_scale, num_kv_heads,
                   sel=None):
    ref = oracle.load()
    return ref.prefill(W.bits(q), W.bits(k_pool), W.bits(v_pool), qo_indptr, kv_indptr,
                       np.asarray(kv_indices, np.int32), sm_scale, num_kv_heads, sel=sel)
