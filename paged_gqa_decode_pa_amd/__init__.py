"""Python binding of libpa: paged grouped-query decode attention on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libpa.so`` behind the C ABI declared in ``include/pa.h``; the
functions here carry the same names as the C entry points and pass tensors as
device pointers.  PyTorch provides device memory and streams.

Importing this package loads ``libpa.so`` (built in-tree by
``paged_gqa_decode_pa_amd.build.build()``) and fails loudly if it is missing.
torch is imported first so that the library binds to the HIP runtime torch
already loaded.

Debug option: with the environment variable ``PA_CHECK=1`` set when the
package is imported, every run made through a ``Plan`` object first copies
``kv_indices`` to the host and checks it against the plan's slot lists and
the pool size with ``pa_check_kv_indices`` (a host synchronisation per run;
off by default, since the kernels do not check slot ids).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARG = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_CAPACITY = 3
PA_ERR_PLAN_MISMATCH = 4
PA_ERR_HIP = 5

PA_PLAN_FORCE_SPLITS_SHIFT = 8
PA_MAX_FORCED_SPLITS = 256
PA_MAX_KV_TOTAL = 1 << 29
PA_PLAN_NO_XCD_ORDER = 0x1
PA_PLAN_SPEED_FEEDBACK = 0x2
PA_PLAN_CASCADE_ALL = 0x4
PA_PLAN_KV_FP8 = 0x8
PA_NUM_XCD = 8


def PA_PLAN_FORCE_SPLITS(n: int) -> int:
    return (int(n) & 0xFFFF) << PA_PLAN_FORCE_SPLITS_SHIFT


class pa_work_unit(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("request", "kv_head", "kv_begin", "kv_end", "q_begin", "q_end", "partial", "diag",
                 "merge", "part_stride", "cached_end", "reserved2")]


class pa_merge_unit(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("request", "kv_head", "q_begin", "q_end", "first_partial", "n_parts",
                 "prefix_first", "prefix_parts")]


WORK_UNIT_DTYPE = np.dtype([(n, np.int32) for n, _ in pa_work_unit._fields_])
MERGE_UNIT_DTYPE = np.dtype([(n, np.int32) for n, _ in pa_merge_unit._fields_])


class PAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{where}: {pa_strerror(status)} ({detail})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIBRARY):
        raise ImportError(f"{LIBRARY} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIBRARY)
    i32, i64, u32, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_float
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.pa_plan_create.argtypes = [ctypes.POINTER(vp), i32, i64, i32, i32, i32, i32]
    lib.pa_plan_create.restype = ctypes.c_int
    lib.pa_plan.argtypes = [vp, i32p, i32p, i32, u32, vp]
    lib.pa_plan.restype = ctypes.c_int
    run = [vp, vp, vp, vp, i64, i64, vp, f32, vp, vp, vp]
    lib.pa_decode_run.argtypes = run
    lib.pa_decode_run.restype = ctypes.c_int
    lib.pa_prefill_chunk_run.argtypes = run
    lib.pa_prefill_chunk_run.restype = ctypes.c_int
    lib.pa_plan_destroy.argtypes = [vp]
    lib.pa_plan_destroy.restype = None
    lib.pa_strerror.argtypes = [ctypes.c_int]
    lib.pa_strerror.restype = ctypes.c_char_p
    lib.pa_last_error_detail.argtypes = []
    lib.pa_last_error_detail.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = i32
    lib.pa_prefill_tile_rows.argtypes = [i32]
    lib.pa_prefill_tile_rows.restype = i32
    lib.pa_partition.argtypes = [i32p, i32p, i32, i32, i32, i32, u32, i32, i32p, i32,
                                 ctypes.POINTER(pa_work_unit), i32,
                                 ctypes.POINTER(pa_merge_unit), i32, i32p, i32p, i32p, i32p]
    lib.pa_partition.restype = ctypes.c_int
    f32p = ctypes.POINTER(ctypes.c_float)
    lib.pa_partition_weighted.argtypes = [i32p, i32p, i32, i32, i32, i32, u32, i32, f32p, i32,
                                          f32p, i32, i32p, i32, ctypes.POINTER(pa_work_unit), i32,
                                          ctypes.POINTER(pa_merge_unit), i32, i32p, i32p, i32p,
                                          i32p]
    lib.pa_partition_weighted.restype = ctypes.c_int
    lib.pa_plan_xcd_weights.argtypes = [vp, f32p, i32, i32p]
    lib.pa_plan_xcd_weights.restype = ctypes.c_int
    lib.pa_plan_set_xcd_weights.argtypes = [vp, f32p, i32]
    lib.pa_plan_set_xcd_weights.restype = ctypes.c_int
    lib.pa_plan_cascade.argtypes = [vp, i32p, i32, i32p, i32, i32p, u32, vp]
    lib.pa_plan_cascade.restype = ctypes.c_int
    wup, mup = ctypes.POINTER(pa_work_unit), ctypes.POINTER(pa_merge_unit)
    lib.pa_partition_cascade.argtypes = [i32p, i32, i32p, i32, i32p, i32, i32, i32, u32, i32,
                                         i32p, i32, wup, i32, mup, i32, wup, i32,
                                         i32p, i32p, i32p, i32p, i32p]
    lib.pa_partition_cascade.restype = ctypes.c_int
    lib.pa_plan_workgroup_weights.argtypes = [vp, f32p, i32, i32p]
    lib.pa_plan_workgroup_weights.restype = ctypes.c_int
    lib.pa_profile_begin.argtypes = [vp, i32]
    lib.pa_profile_begin.restype = ctypes.c_int
    lib.pa_profile_end.argtypes = [vp, ctypes.POINTER(ctypes.c_double), i32p]
    lib.pa_profile_end.restype = ctypes.c_int
    lib.pa_plan_host_timing.argtypes = [vp, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double)]
    lib.pa_plan_host_timing.restype = ctypes.c_int
    lib.pa_decode_run_fp8.argtypes = [vp, vp, vp, vp, i64, i64, vp, f32, f32, f32, vp, vp, vp]
    lib.pa_decode_run_fp8.restype = ctypes.c_int
    lib.pa_prefill_chunk_run_fp8.argtypes = [vp, vp, vp, vp, i64, i64, vp, f32, f32, f32, vp, vp, vp]
    lib.pa_prefill_chunk_run_fp8.restype = ctypes.c_int
    lib.pa_kv_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, vp, i64, i64, vp]
    lib.pa_kv_append.restype = ctypes.c_int
    lib.pa_kv_append_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, f32, f32, vp, vp, i64, i64, vp]
    lib.pa_kv_append_fp8.restype = ctypes.c_int
    lib.pa_plan_launch_shape.argtypes = [vp, i32p, i32p]
    lib.pa_plan_launch_shape.restype = ctypes.c_int
    lib.pa_plan_info.argtypes = [vp, i32p, i32p, i32p, i32p, i32p]
    lib.pa_plan_info.restype = ctypes.c_int
    lib.pa_check_kv_indices.argtypes = [i32p, i32, i32p, i64, ctypes.POINTER(ctypes.c_int64)]
    lib.pa_check_kv_indices.restype = ctypes.c_int
    lib.pa_decode_run_noalloc.argtypes = [vp, vp, vp, i64, i64, vp, vp, i32, i32, i32, i32, f32, vp, vp, vp]
    lib.pa_decode_run_noalloc.restype = ctypes.c_int
    return lib


_lib = _load()

CHECK_INDICES = os.environ.get("PA_CHECK", "0") not in ("", "0")


def pa_strerror(status: int) -> str:
    return _lib.pa_strerror(int(status)).decode()


def pa_last_error_detail() -> str:
    return _lib.pa_last_error_detail().decode()


def pa_version() -> int:
    return int(_lib.pa_version())


def pa_prefill_tile_rows(head_dim: int) -> int:
    """Query rows of one prefill work unit (chunk tokens x Hq/Hkv) at head_dim."""
    return int(_lib.pa_prefill_tile_rows(int(head_dim)))


def _check(status: int, where: str):
    if status != PA_OK:
        raise PAError(status, where, pa_last_error_detail())


def _host_i32(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _i32p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def _dev_ptr(t: Optional[torch.Tensor], name: str, dtype=None) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _pool_stride(k_pool: torch.Tensor, v_pool: torch.Tensor, head_dim: int) -> int:
    """Slot stride (elements) of a pool whose rows are [.., Hkv, D] with contiguous heads."""
    for name, p in (("k_pool", k_pool), ("v_pool", v_pool)):
        if p.dim() < 2 or p.stride(-1) != 1 or (p.dim() >= 3 and p.stride(-2) != head_dim):
            raise ValueError(f"{name}: each slot must hold its Hkv rows of D contiguous values")
    if k_pool.stride(0) != v_pool.stride(0):
        raise ValueError("k_pool and v_pool must have the same slot stride")
    return int(k_pool.stride(0))


# ----------------------------------------------------------------------------
# C entry points
# ----------------------------------------------------------------------------
def pa_plan_create(max_batch: int, max_kv_total: int, max_q_total: int,
                   num_qo_heads: int, num_kv_heads: int, head_dim: int) -> ctypes.c_void_p:
    handle = ctypes.c_void_p()
    _check(_lib.pa_plan_create(ctypes.byref(handle), max_batch, max_kv_total, max_q_total,
                               num_qo_heads, num_kv_heads, head_dim), "pa_plan_create")
    return handle


def pa_plan(plan, kv_indptr, qo_indptr=None, flags: int = 0, stream=None) -> None:
    kv = _host_i32(kv_indptr)
    qo = _host_i32(qo_indptr)
    batch = kv.size - 1
    _check(_lib.pa_plan(plan, _i32p(kv), _i32p(qo), batch, flags, _stream(stream)), "pa_plan")


def pa_plan_cascade(plan, kv_indptr, group_indptr, prefix_len, flags: int = 0,
                    stream=None) -> None:
    kv = _host_i32(kv_indptr)
    gi = _host_i32(group_indptr)
    pl = _host_i32(prefix_len)
    ng = 0 if gi is None else gi.size - 1
    _check(_lib.pa_plan_cascade(plan, _i32p(kv), kv.size - 1, _i32p(gi), ng, _i32p(pl), flags,
                                _stream(stream)), "pa_plan_cascade")


def pa_plan_launch_shape(plan):
    """-> (n_workgroups, n_prefix_units) of the last pa_plan on this plan: the
    launch sizes a captured run keeps (replays stay valid while they match)."""
    wg, pre = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.pa_plan_launch_shape(plan, ctypes.byref(wg), ctypes.byref(pre)), "pa_plan_launch_shape")
    return wg.value, pre.value


def pa_plan_info(plan):
    """-> dict(mode, rows, num_qo_heads, num_kv_heads, head_dim) of the last
    pa_plan on this plan (mode 0: none, 1: decode, 2: prefill; a run reads
    q [rows, Hq, D] and writes out [rows, Hq, D], lse [rows, Hq])."""
    vals = [ctypes.c_int32() for _ in range(5)]
    _check(_lib.pa_plan_info(plan, *[ctypes.byref(v) for v in vals]), "pa_plan_info")
    return dict(zip(("mode", "rows", "num_qo_heads", "num_kv_heads", "head_dim"),
                    (v.value for v in vals)))


def pa_check_kv_indices(kv_indptr, kv_indices, num_slots: int) -> None:
    """Host-side bounds check of slot lists: raises PAError (PA_ERR_INVALID_ARG,
    naming the request, position and id) if an id is outside [0, num_slots)
    or kv_indptr is not a valid CSR offset array.  kv_indices may be a device
    tensor (copied to the host)."""
    ip = _host_i32(kv_indptr)
    idx = _host_i32(kv_indices)
    if idx.size < int(ip[-1]):
        raise ValueError("kv_indices shorter than kv_indptr[-1]")
    bad = ctypes.c_int64()
    _check(_lib.pa_check_kv_indices(_i32p(ip), ip.size - 1, _i32p(idx), int(num_slots),
                                    ctypes.byref(bad)), "pa_check_kv_indices")


def _check_run_shapes(plan, q, k_pool, v_pool, kv_indices, out, lse, num_slots):
    """Sizes the C ABI cannot see: the tensors must match the last pa_plan
    (rows x Hq x D), the pools must hold num_slots slots, and kv_indices must
    be one packed int32 array."""
    info = pa_plan_info(plan)
    rows, Hq, D = info["rows"], info["num_qo_heads"], info["head_dim"]
    if kv_indices.dtype != torch.int32:
        raise TypeError("kv_indices must be int32")
    if kv_indices.dim() != 1 or not kv_indices.is_contiguous():
        raise ValueError("kv_indices must be a contiguous 1-D tensor")
    if info["mode"] != 0:
        if q.dim() != 3 or tuple(q.shape) != (rows, Hq, D):
            raise ValueError(f"q must be [{rows}, {Hq}, {D}] for this plan, got {tuple(q.shape)}")
        if out.numel() != rows * Hq * D:
            raise ValueError(f"out must hold {rows}x{Hq}x{D} values, has {out.numel()}")
        if lse is not None and lse.numel() != rows * Hq:
            raise ValueError(f"lse must hold {rows}x{Hq} values, has {lse.numel()}")
    if min(k_pool.shape[0], v_pool.shape[0]) < num_slots:
        raise ValueError(f"the pools hold fewer than num_slots={num_slots} slots")


def _run(fn, where, plan, q, k_pool, v_pool, kv_indices, sm_scale, out, lse,
         num_slots, slot_stride, stream):
    head_dim = q.shape[-1]
    if slot_stride is None:
        slot_stride = _pool_stride(k_pool, v_pool, head_dim)
    if num_slots is None:
        num_slots = min(k_pool.shape[0], v_pool.shape[0])
    if out.dtype != torch.float32 or not out.is_contiguous():
        raise TypeError("out must be a contiguous float32 tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise TypeError("lse must be a contiguous float32 tensor")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _check_run_shapes(plan, q, k_pool, v_pool, kv_indices, out, lse, num_slots)
    _check(fn(plan, _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(k_pool, "k_pool", torch.bfloat16),
              _dev_ptr(v_pool, "v_pool", torch.bfloat16), int(num_slots), int(slot_stride),
              _dev_ptr(kv_indices, "kv_indices"), float(sm_scale), _dev_ptr(out, "out"),
              _dev_ptr(lse, "lse"), _stream(stream)), where)


def pa_decode_run(plan, q, k_pool, v_pool, kv_indices, sm_scale, out, lse=None,
                  num_slots=None, slot_stride=None, stream=None) -> None:
    _run(_lib.pa_decode_run, "pa_decode_run", plan, q, k_pool, v_pool, kv_indices, sm_scale,
         out, lse, num_slots, slot_stride, stream)


def _run_fp8(fn, where, plan, q, k_pool, v_pool, kv_indices, sm_scale, k_scale, v_scale, out, lse,
             num_slots, slot_stride, stream):
    head_dim = q.shape[-1]
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise TypeError(f"{name} must hold E4M3 codes (float8_e4m3fn or uint8)")
    if slot_stride is None:
        slot_stride = _pool_stride(k_pool, v_pool, head_dim)
    if num_slots is None:
        num_slots = min(k_pool.shape[0], v_pool.shape[0])
    if out.dtype != torch.float32 or not out.is_contiguous():
        raise TypeError("out must be a contiguous float32 tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise TypeError("lse must be a contiguous float32 tensor")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _check_run_shapes(plan, q, k_pool, v_pool, kv_indices, out, lse, num_slots)
    _check(fn(plan, _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(k_pool, "k_pool"),
              _dev_ptr(v_pool, "v_pool"), int(num_slots), int(slot_stride),
              _dev_ptr(kv_indices, "kv_indices"), float(sm_scale), float(k_scale),
              float(v_scale), _dev_ptr(out, "out"), _dev_ptr(lse, "lse"),
              _stream(stream)), where)


def pa_decode_run_fp8(plan, q, k_pool, v_pool, kv_indices, sm_scale, k_scale, v_scale, out, lse=None,
                      num_slots=None, slot_stride=None, stream=None) -> None:
    """Decode over E4M3 pools (torch.float8_e4m3fn or uint8 [slots, Hkv, D])."""
    _run_fp8(_lib.pa_decode_run_fp8, "pa_decode_run_fp8", plan, q, k_pool, v_pool, kv_indices, sm_scale,
             k_scale, v_scale, out, lse, num_slots, slot_stride, stream)


def pa_decode_run_noalloc(q, k_pool, v_pool, kv_indptr, kv_indices, sm_scale, out, lse=None,
                          num_kv_heads=None, num_slots=None, slot_stride=None, stream=None) -> None:
    """Decode without a plan and without allocation: kv_indptr is a device
    int32 tensor [B + 1]; the split is computed on the device into the
    library's own workspace.  q [B, Hq, D] bf16, pools [slots, Hkv, D] bf16."""
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, D]")
    B, Hq, D = q.shape
    if num_kv_heads is None:
        num_kv_heads = k_pool.shape[-2]
    if slot_stride is None:
        slot_stride = _pool_stride(k_pool, v_pool, D)
    if num_slots is None:
        num_slots = min(k_pool.shape[0], v_pool.shape[0])
    for name, t in (("kv_indptr", kv_indptr), ("kv_indices", kv_indices)):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous 1-D int32 tensor")
    if kv_indptr.numel() != B + 1:
        raise ValueError(f"kv_indptr must hold batch + 1 = {B + 1} offsets")
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != B * Hq * D:
        raise ValueError(f"out must be a contiguous float32 tensor of {B}x{Hq}x{D} values")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * Hq):
        raise ValueError(f"lse must be a contiguous float32 tensor of {B}x{Hq} values")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if min(k_pool.shape[0], v_pool.shape[0]) < num_slots:
        raise ValueError(f"the pools hold fewer than num_slots={num_slots} slots")
    _check(_lib.pa_decode_run_noalloc(
        _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(k_pool, "k_pool", torch.bfloat16),
        _dev_ptr(v_pool, "v_pool", torch.bfloat16), int(num_slots), int(slot_stride),
        _dev_ptr(kv_indptr, "kv_indptr"), _dev_ptr(kv_indices, "kv_indices"), int(B), int(Hq),
        int(num_kv_heads), int(D), float(sm_scale), _dev_ptr(out, "out"), _dev_ptr(lse, "lse"),
        _stream(stream)), "pa_decode_run_noalloc")


def pa_prefill_chunk_run(plan, q, k_pool, v_pool, kv_indices, sm_scale, out, lse=None,
                         num_slots=None, slot_stride=None, stream=None) -> None:
    _run(_lib.pa_prefill_chunk_run, "pa_prefill_chunk_run", plan, q, k_pool, v_pool,
         kv_indices, sm_scale, out, lse, num_slots, slot_stride, stream)


def pa_prefill_chunk_run_fp8(plan, q, k_pool, v_pool, kv_indices, sm_scale, k_scale, v_scale, out,
                             lse=None, num_slots=None, slot_stride=None, stream=None) -> None:
    """Chunked prefill over E4M3 pools (torch.float8_e4m3fn or uint8 [slots, Hkv, D])."""
    _run_fp8(_lib.pa_prefill_chunk_run_fp8, "pa_prefill_chunk_run_fp8", plan, q, k_pool, v_pool, kv_indices,
             sm_scale, k_scale, v_scale, out, lse, num_slots, slot_stride, stream)


def _append_shapes(k_new, v_new, out_loc, positions, q):
    """(T, Hq, Hkv, D) of an append call, after the shape and dtype checks."""
    T, Hkv, D = k_new.shape
    if tuple(v_new.shape) != (T, Hkv, D):
        raise ValueError("v_new must have the shape of k_new")
    for name, t in (("k_new", k_new), ("v_new", v_new), ("q", q)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    Hq = Hkv
    if q is not None:
        if q.dim() != 3 or q.shape[0] != T or q.shape[2] != D:
            raise ValueError("q must be [T, Hq, D]")
        Hq = q.shape[1]
    for name, t in (("out_loc", out_loc), ("positions", positions)):
        if t is not None and (t.dtype != torch.int32 or t.numel() != T):
            raise TypeError(f"{name} must be int32 with one entry per token")
    return T, Hq, Hkv, D


def pa_kv_append(k_new, v_new, out_loc, k_pool, v_pool, positions=None, rope_theta: float = 0.0,
                 q=None, num_slots=None, slot_stride=None, stream=None) -> None:
    """Write the new tokens' K/V rows [T, Hkv, D] to slots out_loc [T] of the
    pools, K rotated by RoPE (and q [T, Hq, D] rotated in place, if given)
    when rope_theta > 0."""
    T, Hq, Hkv, D = _append_shapes(k_new, v_new, out_loc, positions, q)
    if slot_stride is None:
        slot_stride = _pool_stride(k_pool, v_pool, D)
    if num_slots is None:
        num_slots = min(k_pool.shape[0], v_pool.shape[0])
    _check(_lib.pa_kv_append(_dev_ptr(k_new, "k_new", torch.bfloat16), _dev_ptr(v_new, "v_new", torch.bfloat16),
                             _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(positions, "positions"),
                             _dev_ptr(out_loc, "out_loc"), T, Hq, Hkv, D, float(rope_theta),
                             _dev_ptr(k_pool, "k_pool", torch.bfloat16),
                             _dev_ptr(v_pool, "v_pool", torch.bfloat16), int(num_slots),
                             int(slot_stride), _stream(stream)), "pa_kv_append")


def pa_kv_append_fp8(k_new, v_new, out_loc, k_pool, v_pool, k_scale: float, v_scale: float,
                     positions=None, rope_theta: float = 0.0, q=None, num_slots=None,
                     slot_stride=None, stream=None) -> None:
    """pa_kv_append into E4M3 pools (torch.float8_e4m3fn or uint8
    [slots, Hkv, D]): K rotated in double precision and stored as the code
    nearest to value / k_scale, V as the code nearest to value / v_scale."""
    T, Hq, Hkv, D = _append_shapes(k_new, v_new, out_loc, positions, q)
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise TypeError(f"{name} must hold E4M3 codes (float8_e4m3fn or uint8)")
    if slot_stride is None:
        slot_stride = _pool_stride(k_pool, v_pool, D)
    if num_slots is None:
        num_slots = min(k_pool.shape[0], v_pool.shape[0])
    _check(_lib.pa_kv_append_fp8(_dev_ptr(k_new, "k_new", torch.bfloat16),
                                 _dev_ptr(v_new, "v_new", torch.bfloat16),
                                 _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(positions, "positions"),
                                 _dev_ptr(out_loc, "out_loc"), T, Hq, Hkv, D, float(rope_theta),
                                 float(k_scale), float(v_scale), _dev_ptr(k_pool, "k_pool"),
                                 _dev_ptr(v_pool, "v_pool"), int(num_slots), int(slot_stride),
                                 _stream(stream)), "pa_kv_append_fp8")


def pa_plan_destroy(plan) -> None:
    _lib.pa_plan_destroy(plan)


def pa_partition(kv_indptr, qo_indptr, num_qo_heads: int, num_kv_heads: int, head_dim: int,
                 flags: int = 0, max_workgroups: int = 0, xcd_weights=None, wg_weights=None):
    """Host-only: the partition pa_plan would upload (pa_partition_weighted:
    xcd_weights one weight per XCD, wg_weights one per workgroup id).

    Returns (wg_offsets int32 [n_workgroups + 1], units, merges, n_partials);
    workgroup w runs units[wg_offsets[w]:wg_offsets[w + 1]].
    """
    kv = _host_i32(kv_indptr)
    qo = _host_i32(qo_indptr)
    def _f32(a):
        if a is None:
            return None, 0, None
        arr = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
        return arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), int(arr.size), arr
    wp, nw, _keep_x = _f32(xcd_weights)
    gp, ng, _keep_g = _f32(wg_weights)
    n_w, n_u, n_m, n_p = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    counts = (ctypes.byref(n_w), ctypes.byref(n_u), ctypes.byref(n_m), ctypes.byref(n_p))
    st = _lib.pa_partition_weighted(_i32p(kv), _i32p(qo), kv.size - 1, num_qo_heads, num_kv_heads,
                                    head_dim, flags, max_workgroups, wp, nw, gp, ng, None, 0,
                                    None, 0, None, 0, *counts)
    if st not in (PA_OK, PA_ERR_CAPACITY):
        _check(st, "pa_partition")
    offs = np.zeros(n_w.value + 1, np.int32)
    units = (pa_work_unit * max(1, n_u.value))()
    merges = (pa_merge_unit * max(1, n_m.value))()
    _check(_lib.pa_partition_weighted(_i32p(kv), _i32p(qo), kv.size - 1, num_qo_heads,
                                      num_kv_heads, head_dim, flags, max_workgroups, wp, nw, gp,
                                      ng, _i32p(offs), offs.size, units, n_u.value, merges,
                                      n_m.value, *counts), "pa_partition")
    u = np.frombuffer(bytes(units), dtype=WORK_UNIT_DTYPE)[: n_u.value].copy()
    m = np.frombuffer(bytes(merges), dtype=MERGE_UNIT_DTYPE)[: n_m.value].copy()
    return offs, u, m, n_p.value


def pa_partition_cascade(kv_indptr, group_indptr, prefix_len, num_qo_heads: int,
                         num_kv_heads: int, head_dim: int, flags: int = 0,
                         max_workgroups: int = 0):
    """Host-only: the partition pa_plan_cascade would upload.

    Returns (wg_offsets, units, merges, n_partials, prefix_units).
    """
    kv = _host_i32(kv_indptr)
    gi = _host_i32(group_indptr)
    pl = _host_i32(prefix_len)
    ng = 0 if gi is None else gi.size - 1
    cnt = [ctypes.c_int32() for _ in range(5)]
    refs = [ctypes.byref(c) for c in cnt]
    st = _lib.pa_partition_cascade(_i32p(kv), kv.size - 1, _i32p(gi), ng, _i32p(pl), num_qo_heads,
                                   num_kv_heads, head_dim, flags, max_workgroups, None, 0, None, 0,
                                   None, 0, None, 0, *refs)
    if st not in (PA_OK, PA_ERR_CAPACITY):
        _check(st, "pa_partition_cascade")
    n_w, n_u, n_m, n_p, n_x = (c.value for c in cnt)
    offs = np.zeros(n_w + 1, np.int32)
    units = (pa_work_unit * max(1, n_u))()
    merges = (pa_merge_unit * max(1, n_m))()
    pre = (pa_work_unit * max(1, n_x))()
    _check(_lib.pa_partition_cascade(_i32p(kv), kv.size - 1, _i32p(gi), ng, _i32p(pl), num_qo_heads,
                                     num_kv_heads, head_dim, flags, max_workgroups, _i32p(offs),
                                     offs.size, units, n_u, merges, n_m, pre, n_x, *refs),
           "pa_partition_cascade")
    u = np.frombuffer(bytes(units), dtype=WORK_UNIT_DTYPE)[:n_u].copy()
    m = np.frombuffer(bytes(merges), dtype=MERGE_UNIT_DTYPE)[:n_m].copy()
    x = np.frombuffer(bytes(pre), dtype=WORK_UNIT_DTYPE)[:n_x].copy()
    return offs, u, m, cnt[3].value, x


def pa_plan_xcd_weights(plan) -> np.ndarray:
    """The per-XCD weights the plan's next automatic decode partition uses."""
    n = ctypes.c_int32()
    _check(_lib.pa_plan_xcd_weights(plan, None, 0, ctypes.byref(n)), "pa_plan_xcd_weights")
    w = np.zeros(n.value, np.float32)
    _check(_lib.pa_plan_xcd_weights(plan, w.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                    w.size, ctypes.byref(n)), "pa_plan_xcd_weights")
    return w


def pa_plan_workgroup_weights(plan) -> np.ndarray:
    """The per-workgroup-id weights measured by PA_PLAN_SPEED_FEEDBACK (id w
    weighs what its compute unit w % C does)."""
    n = ctypes.c_int32()
    _check(_lib.pa_plan_workgroup_weights(plan, None, 0, ctypes.byref(n)),
           "pa_plan_workgroup_weights")
    w = np.zeros(n.value, np.float32)
    _check(_lib.pa_plan_workgroup_weights(plan, w.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                          w.size, ctypes.byref(n)), "pa_plan_workgroup_weights")
    return w


def pa_plan_set_xcd_weights(plan, weights) -> None:
    w = np.ascontiguousarray(np.asarray(weights, dtype=np.float32))
    _check(_lib.pa_plan_set_xcd_weights(plan, w.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                        int(w.size)), "pa_plan_set_xcd_weights")


def pa_plan_host_timing(plan):
    """-> (host microseconds of the last pa_plan call, of which waiting for an
    earlier upload)."""
    tot, wait = ctypes.c_double(), ctypes.c_double()
    _check(_lib.pa_plan_host_timing(plan, ctypes.byref(tot), ctypes.byref(wait)),
           "pa_plan_host_timing")
    return tot.value, wait.value


def pa_profile_begin(plan, capacity: int) -> None:
    _check(_lib.pa_profile_begin(plan, int(capacity)), "pa_profile_begin")


def pa_profile_end(plan):
    """-> (total kernel milliseconds, number of timed launches)."""
    ms, n = ctypes.c_double(), ctypes.c_int32()
    _check(_lib.pa_profile_end(plan, ctypes.byref(ms), ctypes.byref(n)), "pa_profile_end")
    return ms.value, n.value


class Plan:
    """Owns one pa_plan_t (workspace allocated once; pa_plan once per step)."""

    def __init__(self, max_batch: int, max_kv_total: int, num_qo_heads: int, num_kv_heads: int,
                 head_dim: int, max_q_total: int = 0):
        self.num_qo_heads, self.num_kv_heads, self.head_dim = num_qo_heads, num_kv_heads, head_dim
        self.handle = pa_plan_create(max_batch, max_kv_total, max_q_total, num_qo_heads,
                                     num_kv_heads, head_dim)

    def plan(self, kv_indptr, qo_indptr=None, flags: int = 0, stream=None) -> None:
        pa_plan(self.handle, kv_indptr, qo_indptr, flags, stream)
        self._kv_indptr = _host_i32(kv_indptr) if CHECK_INDICES else None

    def info(self) -> dict:
        return pa_plan_info(self.handle)

    def _debug_check(self, kv_indices, k_pool, kw) -> None:
        if CHECK_INDICES and getattr(self, "_kv_indptr", None) is not None:
            n = kw.get("num_slots")
            pa_check_kv_indices(self._kv_indptr, kv_indices, k_pool.shape[0] if n is None else n)

    def xcd_weights(self) -> np.ndarray:
        return pa_plan_xcd_weights(self.handle)

    def set_xcd_weights(self, weights) -> None:
        pa_plan_set_xcd_weights(self.handle, weights)

    def workgroup_weights(self) -> np.ndarray:
        return pa_plan_workgroup_weights(self.handle)

    def plan_cascade(self, kv_indptr, group_indptr, prefix_len, flags: int = 0,
                     stream=None) -> None:
        pa_plan_cascade(self.handle, kv_indptr, group_indptr, prefix_len, flags, stream)
        self._kv_indptr = _host_i32(kv_indptr) if CHECK_INDICES else None

    def decode(self, q, k_pool, v_pool, kv_indices, sm_scale, out, lse=None, **kw) -> None:
        self._debug_check(kv_indices, k_pool, kw)
        pa_decode_run(self.handle, q, k_pool, v_pool, kv_indices, sm_scale, out, lse, **kw)

    def decode_fp8(self, q, k_pool, v_pool, kv_indices, sm_scale, k_scale, v_scale, out, lse=None,
                   **kw) -> None:
        self._debug_check(kv_indices, k_pool, kw)
        pa_decode_run_fp8(self.handle, q, k_pool, v_pool, kv_indices, sm_scale, k_scale, v_scale, out,
                          lse, **kw)

    def prefill(self, q, k_pool, v_pool, kv_indices, sm_scale, out, lse=None, **kw) -> None:
        self._debug_check(kv_indices, k_pool, kw)
        pa_prefill_chunk_run(self.handle, q, k_pool, v_pool, kv_indices, sm_scale, out, lse, **kw)

    def launch_shape(self):
        return pa_plan_launch_shape(self.handle)

    def prefill_fp8(self, q, k_pool, v_pool, kv_indices, sm_scale, k_scale, v_scale, out, lse=None,
                    **kw) -> None:
        self._debug_check(kv_indices, k_pool, kw)
        pa_prefill_chunk_run_fp8(self.handle, q, k_pool, v_pool, kv_indices, sm_scale, k_scale, v_scale, out,
                                 lse, **kw)

    def close(self) -> None:
        if self.handle is not None and self.handle.value:
            pa_plan_destroy(self.handle)
        self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
