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
    """Largest |gpu - ref| over the compared rows (float64).

    The arrays are viewed as rows of their last axis (a 1-D array as rows of
    one value); ``rows`` selects flat row indices to compare (None: all).
    Rows are picked by index, never skipped because a value is NaN: a GPU
    value that is NaN or infinite where the oracle's is finite (an output row
    the kernel never wrote keeps the NaN it was filled with) and a finite GPU
    value where the oracle's is not (a row the oracle did not compute, or a
    result that should be infinite) both count as an infinite error.  The one
    non-finite agreement accepted is -inf on both sides (the lse of an empty
    list)."""
    g = np.asarray(gpu)
    r = np.asarray(ref)
    if g.size != r.size:
        raise ValueError(f"gpu and oracle sizes differ: {g.shape} vs {r.shape}")
    g = g.reshape(-1, g.shape[-1]) if g.ndim > 1 else g.reshape(-1, 1)
    r = r.reshape(g.shape)
    if rows is not None:
        idx = np.asarray(rows, dtype=np.int64).reshape(-1)
        g, r = g[idx], r[idx]
    if g.size == 0:
        return 0.0
    g = g.astype(np.float64)
    finite = np.isfinite(g) & np.isfinite(r)
    agree = np.isneginf(g) & np.isneginf(r)
    if not np.all(finite | agree):
        return float("inf")
    d = np.abs(g[finite] - r[finite])
    return float(d.max()) if d.size else 0.0


def all_rows_written(gpu: np.ndarray) -> bool:
    """True when no output value is NaN (outputs are filled with NaN before a
    run, so a NaN left over is a row the kernel did not write)."""
    return not np.isnan(np.asarray(gpu)).any()


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
