"""Helpers shared by the GPU tests: tolerances and comparison against the oracle."""

import sys

import numpy as np
import torch

# Output / LSE tolerances (max abs error) by storage dtype.
TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3), "f16": (2e-2, 1e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """Element-by-element check; -inf LSE must match exactly where the oracle has it."""
    to, tl = TOL[dtype]
    o = o_gpu.detach().float().cpu().numpy().astype(np.float64)
    l = lse_gpu.detach().float().cpu().numpy().astype(np.float64)
    o_ref = np.asarray(o_ref, np.float64).reshape(o.shape)
    lse_ref = np.asarray(lse_ref, np.float64).reshape(l.shape)
    assert not np.isnan(o).any(), f"{what}: NaN in output"
    assert not np.isnan(l).any(), f"{what}: NaN in lse"
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l), ninf), f"{what}: empty-set rows differ"
    if (~ninf).any():
        dl = np.abs(l[~ninf] - lse_ref[~ninf]).max()
        assert dl <= tl, f"{what}: max |dLSE| = {dl:.3g} > {tl}"
    do = np.abs(o - o_ref).max() if o.size else 0.0
    assert do <= to, f"{what}: max |dO| = {do:.3g} > {to}"
    return do
