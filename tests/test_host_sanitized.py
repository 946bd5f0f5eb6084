"""The host planner under the address and undefined-behaviour sanitizers (CPU).

The planner does pointer arithmetic into pinned staging buffers sized at plan
creation. Here it is built alone with a plain C++ compiler and both sanitizers
(no GPU code is linked: every launcher is a stub), and the whole host-only suite
(``tests/test_host_cpu.py``: 1200 random plans against the oracle's tables, every
host-forcible error, cached-prefix buckets, prefill plans) runs against that
build in a child process with the sanitizer runtimes preloaded. Any report
fails the test.
"""

import os
import shutil
import subprocess
import sys

import pytest

from beam_search_shared_amd import build as bsp_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_suite_passes_under_asan_and_ubsan(tmp_path):
    if shutil.which(os.environ.get("CXX", "g++")) is None:
        pytest.skip("no host C++ compiler")
    lib = bsp_build.build_host_sanitized(str(tmp_path))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": ":".join(bsp_build.sanitizer_runtimes()),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "BSP_LIBRARY": lib,
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "tests/test_host_cpu.py", "-q", "-x",
                          "-s", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
