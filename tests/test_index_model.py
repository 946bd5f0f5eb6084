"""The shared-key kernel's addressing, checked on the CPU (no GPU needed).

``tests/index_model/index_model.cpp`` drives the kernel's loops through the same
offset functions the kernel uses (``csrc/tile_index.h``) for every instantiation
the launchers use, over the beam, cached-prefix and prefill shapes of the tests
and the bench (whole prompts and prompts split into chunks), and checks every
LDS offset against its array and every global offset against its buffer. The
second run covers the head_dim 256, two-block, 64-key, two-stage variant that
was dropped unbuilt after a memory fault in its first GPU test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    out = str(tmp_path_factory.mktemp("index_model") / "index_model")
    src = os.path.join(ROOT, "tests", "index_model", "index_model.cpp")
    res = subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", src,
                          "-o", out], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return out


@pytest.mark.parametrize("which", ["shipped", "dropped-d256"])
def test_every_offset_in_range(model, which):
    args = [model] + (["--dropped-d256"] if which != "shipped" else [])
    res = subprocess.run(args, capture_output=True, text=True, timeout=600)
    last = res.stdout.strip().splitlines()[-1]
    assert res.returncode == 0 and last.endswith(" 0 out of range"), res.stdout[-3000:]
    assert int(last.split()[0]) > 1_000_000  # the model really enumerated the loops
