"""fp64 CPU oracle for paged grouped-query decode attention (and the rotary
position embedding and 8-bit encoding of the rows appended to the pool).

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only code that may import this
package.  The product library never loads it, and it shares no code with the
GPU path.

The arithmetic lives in ``pa_oracle.c`` (plain C, double precision, OpenMP over
query rows); this module only builds/loads that library and marshals numpy
arrays.  What is computed, with the passages of the source pages it follows,
is stated at the top of ``pa_oracle.c``.

Inputs are bf16 bit patterns (``numpy.uint16``), so the oracle reads the very
bits the GPU reads.  Outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "pa_oracle.c")
LIBRARY = os.path.join(HERE, "libpa_oracle.so")

STATUS = {
    0: "ok",
    1: "bad shape",
    2: "bad indptr",
    3: "slot id out of range",
    4: "chunk longer than its slot list",
    5: "out of memory",
}


class OracleError(RuntimeError):
    pass


def build(source: str = SOURCE, output: str = LIBRARY,
          extra_flags: Sequence[str] = ()) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           *extra_flags, source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


_i32p = ctypes.POINTER(ctypes.c_int32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)


def _ptr(a: np.ndarray, kind):
    return a.ctypes.data_as(kind)


def _as(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


class Oracle:
    """Handle on one build of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.pa_oracle_decode.restype = ctypes.c_int
        lib.pa_oracle_decode.argtypes = [
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            _u16p, _u16p, _u16p, ctypes.c_int64, ctypes.c_int64,
            _i32p, _i32p, ctypes.c_float, _f64p, _f64p, _i32p, ctypes.c_int64]
        lib.pa_oracle_prefill.restype = ctypes.c_int
        lib.pa_oracle_prefill.argtypes = [
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            _u16p, _u16p, _u16p, ctypes.c_int64, ctypes.c_int64,
            _i32p, _i32p, _i32p, ctypes.c_float, _f64p, _f64p, _i32p, ctypes.c_int64]
        lib.pa_oracle_merge.restype = ctypes.c_int
        lib.pa_oracle_merge.argtypes = [ctypes.c_int32, ctypes.c_int32, _f64p, _f64p, _f64p, _f64p]
        lib.pa_oracle_rope.restype = ctypes.c_int
        lib.pa_oracle_rope.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _u16p, _i32p,
                                       ctypes.c_double, _f64p]
        _u8p = ctypes.POINTER(ctypes.c_uint8)
        lib.pa_oracle_e4m3_to_bf16.restype = ctypes.c_int
        lib.pa_oracle_e4m3_to_bf16.argtypes = [ctypes.c_int64, _u8p, _u16p]
        lib.pa_oracle_e4m3_values.restype = ctypes.c_int
        lib.pa_oracle_e4m3_values.argtypes = [ctypes.c_int64, _u8p, _f64p]
        lib.pa_oracle_e4m3_encode.restype = ctypes.c_int
        lib.pa_oracle_e4m3_encode.argtypes = [ctypes.c_int64, _f64p, ctypes.c_float, _u8p]
        lib.pa_oracle_decode_e4m3.restype = ctypes.c_int
        lib.pa_oracle_decode_e4m3.argtypes = [
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            _u16p, _u8p, _u8p, ctypes.c_int64, ctypes.c_int64,
            _i32p, _i32p, ctypes.c_float, ctypes.c_float, ctypes.c_float,
            _f64p, _f64p, _i32p, ctypes.c_int64]
        lib.pa_oracle_prefill_e4m3.restype = ctypes.c_int
        lib.pa_oracle_prefill_e4m3.argtypes = [
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            _u16p, _u8p, _u8p, ctypes.c_int64, ctypes.c_int64,
            _i32p, _i32p, _i32p, ctypes.c_float, ctypes.c_float, ctypes.c_float,
            _f64p, _f64p, _i32p, ctypes.c_int64]
        lib.pa_oracle_num_threads.restype = ctypes.c_int
        lib.pa_oracle_num_threads.argtypes = []
        self._lib = lib

    @staticmethod
    def _check(rc: int):
        if rc != 0:
            raise OracleError(f"oracle status {rc}: {STATUS.get(rc, '?')}")

    def num_threads(self) -> int:
        return int(self._lib.pa_oracle_num_threads())

    def decode(self, q_bits, k_bits, v_bits, kv_indptr, kv_indices, sm_scale: float,
               num_kv_heads: int, sel: Optional[Sequence[int]] = None):
        """Decode attention.

        q_bits: uint16 [B, Hq, D]; k_bits / v_bits: uint16 [N, Hkv, D] (or any
        array whose leading axis is the slot and whose per-slot row holds the
        Hkv*D head rows first); kv_indptr int32 [B+1]; kv_indices int32.
        sel: optional flat rows b*Hq+h to compute (others are NaN in the result).
        Returns (out float64 [B, Hq, D], lse float64 [B, Hq]).
        """
        q = _as(q_bits, np.uint16)
        k = _as(k_bits, np.uint16)
        v = _as(v_bits, np.uint16)
        B, Hq, D = q.shape
        num_slots = k.shape[0]
        slot_stride = int(np.prod(k.shape[1:])) if k.ndim > 1 else 0
        if v.shape != k.shape:
            raise OracleError("k and v pools differ in shape")
        indptr = _as(kv_indptr, np.int32)
        indices = _as(kv_indices, np.int32)
        if indptr.shape != (B + 1,):
            raise OracleError("kv_indptr must have batch+1 entries")
        if indices.shape[0] < indptr[-1]:
            raise OracleError("kv_indices shorter than kv_indptr[-1]")
        if indices.size == 0:
            indices = np.zeros(1, np.int32)
        out = np.full((B, Hq, D), np.nan)
        lse = np.full((B, Hq), np.nan)
        if sel is None:
            sel_arr, n_sel, sel_p = None, 0, None
        else:
            sel_arr = _as(sel, np.int32)
            n_sel = sel_arr.size
            sel_p = _ptr(sel_arr, _i32p)
        rc = self._lib.pa_oracle_decode(
            B, Hq, num_kv_heads, D, _ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p),
            num_slots, slot_stride, _ptr(indptr, _i32p), _ptr(indices, _i32p),
            ctypes.c_float(sm_scale), _ptr(out, _f64p), _ptr(lse, _f64p), sel_p, n_sel)
        self._check(rc)
        return out, lse

    def prefill(self, q_bits, k_bits, v_bits, qo_indptr, kv_indptr, kv_indices,
                sm_scale: float, num_kv_heads: int, sel: Optional[Sequence[int]] = None):
        """Chunked prefill over a paged context (chunk = last C list entries).

        q_bits uint16 [T, Hq, D]; qo_indptr int32 [B+1] with qo_indptr[-1] == T.
        Returns (out float64 [T, Hq, D], lse float64 [T, Hq]).
        """
        q = _as(q_bits, np.uint16)
        k = _as(k_bits, np.uint16)
        v = _as(v_bits, np.uint16)
        T, Hq, D = q.shape
        num_slots = k.shape[0]
        slot_stride = int(np.prod(k.shape[1:])) if k.ndim > 1 else 0
        if v.shape != k.shape:
            raise OracleError("k and v pools differ in shape")
        qo = _as(qo_indptr, np.int32)
        indptr = _as(kv_indptr, np.int32)
        indices = _as(kv_indices, np.int32)
        B = indptr.shape[0] - 1
        if qo.shape != (B + 1,) or qo[-1] != T:
            raise OracleError("qo_indptr must have batch+1 entries ending at T")
        if indices.size == 0:
            indices = np.zeros(1, np.int32)
        out = np.full((T, Hq, D), np.nan)
        lse = np.full((T, Hq), np.nan)
        if sel is None:
            sel_arr, n_sel, sel_p = None, 0, None
        else:
            sel_arr = _as(sel, np.int32)
            n_sel = sel_arr.size
            sel_p = _ptr(sel_arr, _i32p)
        rc = self._lib.pa_oracle_prefill(
            B, Hq, num_kv_heads, D, _ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p),
            num_slots, slot_stride, _ptr(qo, _i32p), _ptr(indptr, _i32p), _ptr(indices, _i32p),
            ctypes.c_float(sm_scale), _ptr(out, _f64p), _ptr(lse, _f64p), sel_p, n_sel)
        self._check(rc)
        return out, lse

    def rope(self, x_bits, positions, theta: float) -> np.ndarray:
        """Rotary position embedding (rotate-half pairs i, i + D/2) of bf16 rows.

        x_bits: uint16 [T, H, D]; positions: int32 [T].  Returns float64
        [T, H, D], not rounded.
        """
        x = _as(x_bits, np.uint16)
        T, H, D = x.shape
        pos = _as(positions, np.int32)
        if pos.shape != (T,):
            raise OracleError("positions must hold one entry per token")
        y = np.zeros((T, H, D), np.float64)
        self._check(self._lib.pa_oracle_rope(T, H, D, _ptr(x, _u16p), _ptr(pos, _i32p),
                                             float(theta), _ptr(y, _f64p)))
        return y

    def e4m3_values(self, codes) -> np.ndarray:
        """float64 values of OCP FP8 E4M3 codes (uint8)."""
        c = _as(codes, np.uint8)
        out = np.zeros(c.shape, np.float64)
        self._check(self._lib.pa_oracle_e4m3_values(c.size, c.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                                    _ptr(out, _f64p)))
        return out

    def e4m3_to_bf16(self, codes) -> np.ndarray:
        """bf16 bit patterns (uint16) of the values of E4M3 codes (exact)."""
        c = _as(codes, np.uint8)
        out = np.zeros(c.shape, np.uint16)
        self._check(self._lib.pa_oracle_e4m3_to_bf16(c.size, c.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                                     _ptr(out, _u16p)))
        return out

    def e4m3_encode(self, x, scale: float = 1.0) -> np.ndarray:
        """E4M3 codes (uint8) of float64 values divided by a float32 scale:
        round to nearest even among the finite codes (saturating at +-448),
        NaN -> 0x7F."""
        xs = _as(x, np.float64)
        out = np.zeros(xs.shape, np.uint8)
        self._check(self._lib.pa_oracle_e4m3_encode(xs.size, _ptr(xs, _f64p), ctypes.c_float(scale),
                                                    out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))))
        return out

    def append_e4m3(self, k_bits, v_bits, positions, theta: float, k_scale: float, v_scale: float):
        """The rows an append writes into 8-bit pools: K (bf16 [T, Hkv, D])
        rotated as by ``rope`` when theta > 0 (widened unrotated otherwise),
        then encoded under k_scale; V (bf16) widened and encoded under
        v_scale.  Returns (k_codes, v_codes, k_values) with k_values the
        float64 K rows before encoding."""
        kb = _as(k_bits, np.uint16)
        vb = _as(v_bits, np.uint16)
        if kb.shape != vb.shape or kb.ndim != 3:
            raise OracleError("k and v rows must both be [T, Hkv, D]")
        if theta > 0:
            k_values = self.rope(kb, positions, theta)
        else:
            k_values = (kb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        v_values = (vb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return self.e4m3_encode(k_values, k_scale), self.e4m3_encode(v_values, v_scale), k_values

    def decode_fp8(self, q_bits, k_codes, v_codes, kv_indptr, kv_indices, sm_scale: float,
                   k_scale: float, v_scale: float, num_kv_heads: int, sel=None):
        """Decode over E4M3 pools with per-pool scales: the attention of
        ``decode`` on the row values k_scale * value(code) and
        v_scale * value(code), formed in double precision from the codes
        (uint8 [N, Hkv, D]); the three scales are float32 values, widened.
        Returns (out float64 [B, Hq, D], lse float64 [B, Hq])."""
        q = _as(q_bits, np.uint16)
        k = _as(k_codes, np.uint8)
        v = _as(v_codes, np.uint8)
        B, Hq, D = q.shape
        if v.shape != k.shape:
            raise OracleError("k and v pools differ in shape")
        num_slots = k.shape[0]
        slot_stride = int(np.prod(k.shape[1:])) if k.ndim > 1 else 0
        indptr = _as(kv_indptr, np.int32)
        indices = _as(kv_indices, np.int32)
        if indptr.shape != (B + 1,):
            raise OracleError("kv_indptr must have batch+1 entries")
        if indices.shape[0] < indptr[-1]:
            raise OracleError("kv_indices shorter than kv_indptr[-1]")
        if indices.size == 0:
            indices = np.zeros(1, np.int32)
        out = np.full((B, Hq, D), np.nan)
        lse = np.full((B, Hq), np.nan)
        if sel is None:
            sel_arr, n_sel, sel_p = None, 0, None
        else:
            sel_arr = _as(sel, np.int32)
            n_sel = sel_arr.size
            sel_p = _ptr(sel_arr, _i32p)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        rc = self._lib.pa_oracle_decode_e4m3(
            B, Hq, num_kv_heads, D, _ptr(q, _u16p), _ptr(k, u8p), _ptr(v, u8p),
            num_slots, slot_stride, _ptr(indptr, _i32p), _ptr(indices, _i32p),
            ctypes.c_float(sm_scale), ctypes.c_float(k_scale), ctypes.c_float(v_scale),
            _ptr(out, _f64p), _ptr(lse, _f64p), sel_p, n_sel)
        self._check(rc)
        return out, lse

    def prefill_fp8(self, q_bits, k_codes, v_codes, qo_indptr, kv_indptr, kv_indices, sm_scale: float,
                    k_scale: float, v_scale: float, num_kv_heads: int, sel=None):
        """Chunked prefill (as ``prefill``) over E4M3 pools with per-pool
        scales (the values of ``decode_fp8``).  Returns (out float64
        [T, Hq, D], lse float64 [T, Hq])."""
        q = _as(q_bits, np.uint16)
        k = _as(k_codes, np.uint8)
        v = _as(v_codes, np.uint8)
        T, Hq, D = q.shape
        if v.shape != k.shape:
            raise OracleError("k and v pools differ in shape")
        num_slots = k.shape[0]
        slot_stride = int(np.prod(k.shape[1:])) if k.ndim > 1 else 0
        qo = _as(qo_indptr, np.int32)
        indptr = _as(kv_indptr, np.int32)
        indices = _as(kv_indices, np.int32)
        B = indptr.shape[0] - 1
        if qo.shape != (B + 1,) or qo[-1] != T:
            raise OracleError("qo_indptr must have batch+1 entries ending at T")
        if indices.size == 0:
            indices = np.zeros(1, np.int32)
        out = np.full((T, Hq, D), np.nan)
        lse = np.full((T, Hq), np.nan)
        if sel is None:
            sel_arr, n_sel, sel_p = None, 0, None
        else:
            sel_arr = _as(sel, np.int32)
            n_sel = sel_arr.size
            sel_p = _ptr(sel_arr, _i32p)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        rc = self._lib.pa_oracle_prefill_e4m3(
            B, Hq, num_kv_heads, D, _ptr(q, _u16p), _ptr(k, u8p), _ptr(v, u8p),
            num_slots, slot_stride, _ptr(qo, _i32p), _ptr(indptr, _i32p), _ptr(indices, _i32p),
            ctypes.c_float(sm_scale), ctypes.c_float(k_scale), ctypes.c_float(v_scale),
            _ptr(out, _f64p), _ptr(lse, _f64p), sel_p, n_sel)
        self._check(rc)
        return out, lse

    def merge(self, o_parts, lse_parts):
        """Log-sum-exp merge of partial results of one row: o_parts [n, D], lse_parts [n]."""
        o = _as(o_parts, np.float64)
        l = _as(lse_parts, np.float64)
        n, D = o.shape
        out = np.zeros(D)
        lse = np.zeros(1)
        rc = self._lib.pa_oracle_merge(n, D, _ptr(o, _f64p), _ptr(l, _f64p),
                                       _ptr(out, _f64p), _ptr(lse, _f64p))
        self._check(rc)
        return out, float(lse[0])


_default: Optional[Oracle] = None


def load() -> Oracle:
    """The oracle built from ``pa_oracle.c`` next to this file (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIBRARY)
    return _default
