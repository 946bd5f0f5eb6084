"""CPU checks of the measurement helpers in bench.py: the layer rotation that
keeps each step's prompt out of the last-level cache, and the algorithmic byte
and FLOP counts the roofline fractions divide by."""

import numpy as np
import pytest

import bench
import oracle
import synth


@pytest.mark.parametrize("step_bytes", [1e6, 42.5e6, 164e6, 229e6, 579e6, 1158e6, 1858e6, 4e9])
def test_rotation_puts_enough_other_reads_between_reuses(step_bytes):
    """Between two steps on the same layer copy, the other copies' steps read at
    least FLUSH_BYTES (at least two copies always)."""
    n = bench.rotation_layers(step_bytes)
    assert n >= 2
    assert (n - 1) * step_bytes >= bench.FLUSH_BYTES
    assert bench.rotation_layers(step_bytes, forced=7) == 7


@pytest.mark.parametrize("cfg,seed", [("tiny", 0), ("qwen3_0p6b", 1), ("nsample", 2)])
def test_algorithmic_bytes_against_the_oracle_index_function(cfg, seed):
    """The step's algorithmic bytes recounted from the oracle's tail-slot
    function: prompt K+V once per request, each distinct tail (page, row) once,
    Q read, O written, the current tokens' K/V written."""
    inp = synth.make_beam_step(cfg, seed, batch=4 if cfg != "tiny" else None)
    step, prefix_kernel = bench.algorithmic_bytes(inp)
    e = bench.EBYTES[inp.dtype]
    row = inp.num_kv_heads * inp.head_dim * e * 2
    pad = int((inp.seq_len - inp.prefix_len).max())
    slots = oracle.tail_slots(inp.prefix_len, inp.seq_len, inp.block_tables,
                              inp.cache_indirection, inp.page_size, max(pad, 1))
    distinct = sum(len(set(slots[b][slots[b] >= 0].tolist())) for b in range(inp.batch))
    rows = inp.batch * inp.beam
    q = rows * inp.num_q_heads * inp.head_dim * e
    want = int(inp.prefix_len.sum()) * row + distinct * row + 2 * q + len(inp.slots) * row
    assert step == want
    assert prefix_kernel == (int(inp.prefix_len.sum()) * row + q
                             + rows * inp.num_q_heads * (inp.head_dim + 1) * 4)


def test_cached_work_closed_forms():
    """One new row over L cached rows attends L + 1 keys; Sq causal new rows attend
    L * Sq + Sq (Sq + 1) / 2 keys; 4 FLOPs per key, query head and dimension."""
    flops, nbytes = bench.cached_work(10368, 1, 24, 8, 128, 2)
    assert flops == 4 * (10368 + 1) * 24 * 128
    assert nbytes == (10368 + 1) * 8 * 128 * 2 * 2 + 1 * 8 * 128 * 2 * 2 + 2 * 24 * 128 * 2
    flops, _ = bench.cached_work(100, 3, 2, 1, 64, 2)
    assert flops == 4 * (100 * 3 + 6) * 2 * 64
