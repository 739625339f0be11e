"""The C-ABI library loads without a GPU, exports every function include/pa.h
declares, and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

import paged_gqa_decode_pa_amd as pa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)) - {"pa_plan_t"})


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("pa_plan_create", "pa_plan", "pa_decode_run", "pa_prefill_chunk_run",
                     "pa_plan_destroy", "pa_strerror", "pa_last_error_detail", "pa_partition",
                     "pa_version"):
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
