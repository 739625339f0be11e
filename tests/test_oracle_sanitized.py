"""The oracle under AddressSanitizer and UBSan: pa_oracle.c built with both,
every pin run against that build in a child process with the ASan runtime
preloaded; any sanitizer report fails the test.  CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

SCRIPT = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
from oracle_pins import ALL_PINS
o = oracle.Oracle({lib!r})
for pin in ALL_PINS:
    pin(o)
print("pins ok", len(ALL_PINS))
"""


def test_oracle_pins_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("needs gcc")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no ASan runtime")
    lib = str(tmp_path / "libpa_oracle_asan.so")
    oracle.build(oracle.SOURCE, lib, extra_flags=["-g", "-fsanitize=address,undefined",
                                                  "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"])
    env = {**os.environ, "LD_PRELOAD": asan, "ASAN_OPTIONS": "detect_leaks=0"}
    code = SCRIPT.format(root=os.path.dirname(HERE), tests=HERE, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600, env=env)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-3000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-3000:]
    assert "pins ok" in r.stdout
