"""bsp_plan_static (the plan's workspace in the library's static device scratch,
for callers that cannot allocate) against bsp_plan with a caller workspace:
the same fused step, bit for bit and within the oracle's tolerance, on two
plans in a row on the same scratch, the second with a smaller batch; and a
plan too large for the scratch is rejected before anything runs."""

import numpy as np
import pytest
import torch

import oracle
import synth
from beam_search_shared_amd import _binding as B
from beam_search_shared_amd import step as S
from tests.gpu_util import assert_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _applied(inp):
    inp.k_pool, inp.v_pool = oracle.write_kv(inp.k_pool, inp.v_pool, inp.slots, inp.k_new,
                                             inp.v_new, inp.page_size)
    return inp


@pytest.mark.parametrize("split", ["128", "0"])
def test_static_plan_matches_caller_workspace(split, monkeypatch):
    need_gpu()
    monkeypatch.setenv("BSP_SPLIT", split)  # "128": counters and partial states in the scratch
    kw = dict(batch=6, prefix_range=(100, 1200))
    inp = synth.make_beam_step("qwen3_0p6b", 11, **kw)
    fo, fl = oracle.beam_decode_attention(_applied(synth.make_beam_step("qwen3_0p6b", 11, **kw)))
    a = S.upload_beam_step(inp, "cuda")   # caller workspace
    b = S.upload_beam_step(inp, "cuda")   # the library's static scratch
    W = inp.beam
    for nb in (6, 3):
        bt = np.ascontiguousarray(inp.block_tables[:nb])
        say(f"static plan split={split} batch={nb}")
        B.bsp_plan(a.plan, nb, W, 1, inp.prefix_len[:nb], inp.seq_len[:nb], bt, a.workspace)
        B.bsp_plan_static(b.plan, nb, W, 1, inp.prefix_len[:nb], inp.seq_len[:nb], bt)
        if split != "0":
            assert (B.bsp_debug_plan_items(b.plan)[:, 3] > 1).any()
        S.run_decode_step(a)
        S.run_decode_step(b)
        B.bsp_check(a.plan)
        B.bsp_check(b.plan)
        torch.cuda.synchronize()
        rows = nb * W
        assert torch.equal(a.out[:rows], b.out[:rows])
        assert torch.equal(a.lse_out[:rows], b.lse_out[:rows])
        assert_close(b.out[:rows], b.lse_out[:rows], fo[:nb], fl[:nb], "bf16",
                     f"static plan batch {nb}")
        assert torch.equal(a.k_pool, b.k_pool) and torch.equal(a.v_pool, b.v_pool)


def test_static_plan_rejects_a_plan_larger_than_the_scratch():
    need_gpu()
    desc = B.make_desc(16, 8, 128, 32, 1 << 20, "bf16")
    plan = B.Plan(desc, max_requests=4096, max_beam=4, max_blocks_per_seq=4096,
                  max_seq_len=4096 * 32, max_q_len=1)
    assert plan.workspace_bytes > (32 << 20)
    P = np.array([64], np.int32)
    bt = np.zeros((1, 1, 4096), np.int32)
    with pytest.raises(B.BspError) as ei:
        B.bsp_plan_static(plan, 1, 1, 1, P, P, bt)
    assert ei.value.name == "BSP_ERR_WORKSPACE"
