"""The C-ABI library loads without a GPU, exports every function include/pa.h
declares, and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_gqa_decode_pa_amd as pa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)) - {"pa_plan_t"})


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("pa_plan_create", "pa_plan", "pa_decode_run", "pa_prefill_chunk_run",
                     "pa_plan_destroy", "pa_strerror", "pa_last_error_detail", "pa_partition",
                     "pa_version", "pa_decode_run_fp8", "pa_prefill_chunk_run_fp8", "pa_kv_append",
                     "pa_kv_append_fp8", "pa_plan_cascade", "pa_decode_run_noalloc"):
        assert required in names


@pytest.mark.parametrize("name", declared_functions())
def test_symbol_exported(name):
    lib = ctypes.CDLL(pa.LIBRARY)
    assert hasattr(lib, name), f"{name} declared in pa.h but not exported"


def test_status_strings():
    assert pa.pa_strerror(pa.PA_OK) == "ok"
    seen = {pa.pa_strerror(s) for s in range(6)}
    assert len(seen) == 6
    assert pa.pa_strerror(99) == "unknown status"
    assert pa.pa_version() >= 100


@pytest.mark.parametrize("args,status", [
    ((4, 1000, 0, 32, 6, 128), pa.PA_ERR_UNSUPPORTED),    # Hq % Hkv != 0
    ((4, 1000, 0, 48, 4, 128), pa.PA_ERR_UNSUPPORTED),    # group 12
    ((4, 1000, 0, 32, 8, 64), pa.PA_ERR_UNSUPPORTED),     # head_dim 64
    ((4, 1000, 0, 0, 8, 128), pa.PA_ERR_INVALID_ARG),
    ((-1, 1000, 0, 32, 8, 128), pa.PA_ERR_INVALID_ARG),
    ((4, -5, 0, 32, 8, 128), pa.PA_ERR_INVALID_ARG),
    ((4, 1 << 40, 0, 32, 8, 128), pa.PA_ERR_INVALID_ARG),
    ((4, pa.PA_MAX_KV_TOTAL + 1, 0, 32, 8, 128), pa.PA_ERR_INVALID_ARG),
])
def test_plan_create_rejects_on_host(args, status):
    with pytest.raises(pa.PAError) as e:
        pa.pa_plan_create(*args)
    assert e.value.status == status
    assert e.value.detail


def test_null_plan_rejected():
    null = ctypes.c_void_p(0)
    assert pa._lib.pa_decode_run(null, None, None, None, 0, 0, None, 1.0, None, None, None) \
        == pa.PA_ERR_INVALID_ARG
    assert pa._lib.pa_plan(null, None, None, 0, 0, None) == pa.PA_ERR_INVALID_ARG
    pa.pa_plan_destroy(null)  # no-op


@pytest.mark.parametrize("lang,std", [("c", "c99"), ("c++", "c++17")])
def test_header_compiles_standalone(lang, std, tmp_path):
    """include/pa.h is a plain C header: it compiles on its own, warning-free,
    as C99 and as C++17 (no HIP or torch types in the signatures)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    r = subprocess.run([cc, "-fsyntax-only", "-x", lang, f"-std={std}", "-Wall", "-Wextra",
                        "-pedantic", "-Werror", HEADER], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_check_kv_indices_accepts_valid_lists():
    ip = np.array([0, 3, 3, 7], np.int32)
    idx = np.array([0, 9, 4, 1, 2, 3, 9], np.int32)
    pa.pa_check_kv_indices(ip, idx, 10)
    pa.pa_check_kv_indices(np.array([0], np.int32), np.zeros(0, np.int32), 0)   # empty batch


@pytest.mark.parametrize("bad_pos,bad_id", [(0, -1), (4, 10), (6, 1 << 30), (2, -2147483648)])
def test_check_kv_indices_reports_the_first_bad_id(bad_pos, bad_id):
    ip = np.array([0, 3, 3, 7], np.int32)
    idx = np.array([0, 9, 4, 1, 2, 3, 9], np.int32)
    idx[bad_pos] = bad_id
    with pytest.raises(pa.PAError) as e:
        pa.pa_check_kv_indices(ip, idx, 10)
    assert e.value.status == pa.PA_ERR_INVALID_ARG
    assert f"kv_indices[{bad_pos}]" in e.value.detail and str(bad_id) in e.value.detail
    first = ctypes.c_int64()
    st = pa._lib.pa_check_kv_indices(pa._i32p(ip), 3, pa._i32p(idx), 10, ctypes.byref(first))
    assert st == pa.PA_ERR_INVALID_ARG and first.value == bad_pos


@pytest.mark.parametrize("ip", [[1, 3], [0, 3, 2]])
def test_check_kv_indices_rejects_bad_offsets(ip):
    ip = np.asarray(ip, np.int32)
    first = ctypes.c_int64(99)
    idx = np.zeros(8, np.int32)
    st = pa._lib.pa_check_kv_indices(pa._i32p(ip), ip.size - 1, pa._i32p(idx), 10, ctypes.byref(first))
    assert st == pa.PA_ERR_INVALID_ARG and first.value == -1


def test_plan_info_null_plan():
    assert pa._lib.pa_plan_info(ctypes.c_void_p(0), None, None, None, None, None) == pa.PA_ERR_INVALID_ARG


def test_import_fails_loudly_without_library(tmp_path):
    """No fallback path: a copy of the package without libpa.so refuses to
    import, naming the missing library (checked in a child process)."""
    import shutil
    import subprocess
    import sys
    pkg = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "paged_gqa_decode_pa_amd")
    dst = tmp_path / "paged_gqa_decode_pa_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    assert not (dst / "libpa.so").exists()
    r = subprocess.run([sys.executable, "-c", "import paged_gqa_decode_pa_amd"], cwd=tmp_path,
                       capture_output=True, text=True, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libpa.so is missing" in r.stderr, r.stderr[-500:]
