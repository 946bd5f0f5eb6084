"""Seeded synthetic inputs for cascade beam-decode attention.

This package draws random tensors and places them in a paged KV pool. It holds
none of the attention arithmetic, so both the fp64 oracle and the HIP path can
consume what it produces without sharing any computation.
"""

from .generator import (  # noqa: F401
    BEAM_CONFIGS,
    BeamConfig,
    BeamStepInputs,
    CachedPrefixInputs,
    PrefillInputs,
    make_beam_step,
    make_cached_prefix,
    make_prefill,
    round_to_dtype,
)
