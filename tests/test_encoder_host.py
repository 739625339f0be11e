"""The append kernel's E4M3 encoder (e4m3_from_double in csrc/append.hip),
compiled for the host from the kernel source as it stands, against the
oracle's encoder (a plain nearest-value search) on every midpoint between
codes, one double step either side of each, the subnormal and saturation
edges, special values and 2 x 10^5 log-uniform doubles.  The function is
plain C++ on doubles (frexp, rint, ldexp), so a host build runs the same
arithmetic as the device build.  CPU only."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "paged_gqa_decode_pa_amd", "csrc", "append.hip")


@pytest.fixture(scope="module")
def kernel_encoder(tmp_path_factory):
    text = open(SRC).read()
    m = re.search(r"__device__ __forceinline__ uint32_t e4m3_from_double\(double y\) \{.*?\n\}\n", text, re.S)
    assert m, "e4m3_from_double not found in append.hip"
    body = m.group(0).replace("__device__ __forceinline__ ", 'extern "C" ', 1)
    d = tmp_path_factory.mktemp("enc")
    cpp, so = d / "enc.cpp", d / "libenc.so"
    cpp.write_text("#include <cmath>\n#include <cstdint>\nusing namespace std;\n" + body)
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", str(cpp), "-o", str(so)], check=True)
    lib = ctypes.CDLL(str(so))
    lib.e4m3_from_double.restype = ctypes.c_uint32
    lib.e4m3_from_double.argtypes = [ctypes.c_double]
    return lib.e4m3_from_double


def _inputs():
    ref = oracle.load()
    fin = ref.e4m3_values(np.arange(0x7F, dtype=np.uint8))
    mids = (fin[:-1] + fin[1:]) / 2
    rng = np.random.default_rng(91)
    mag = np.exp2(rng.uniform(-14, 10, 200000))
    edges = [448.0, 464.0, 470.0, 480.0, 1e300, np.inf, -np.inf, np.nan, 0.0, -0.0, 2.0 ** -6,
             2.0 ** -6 * (1 - 2.0 ** -40), 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11, 5e-324, 1e-300]
    x = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf), fin, edges,
                        mag * rng.choice([-1.0, 1.0], mag.size)])
    return np.concatenate([x, -x])


def test_kernel_encoder_matches_oracle(kernel_encoder):
    x = _inputs()
    want = oracle.load().e4m3_encode(x)
    got = np.fromiter((kernel_encoder(float(v)) for v in x), dtype=np.uint32, count=x.size)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} of {x.size} differ, e.g. x={x[bad[:4]]} kernel={got[bad[:4]]} oracle={want[bad[:4]]}"
