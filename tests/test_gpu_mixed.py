"""GPU parity of the mixed step: the context requests' ragged causal prefill
(bsp_plan_prefill + bsp_write_kv + bsp_prefill_attn) against the fp64 oracle,
row by row, and a whole mixed step (prefill beside the fused beam step, on two
streams) against the oracle for both kinds of request."""

import numpy as np
import pytest
import torch

import oracle
import synth
from beam_search_shared_amd import _binding as B
from beam_search_shared_amd import step as S
from synth import BeamConfig
from tests.gpu_util import TOL, assert_close, need_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _check_prefill(inp, what):
    c = S.upload_prefill(inp, DEV)
    S.plan_prefill(c)
    S.run_prefill(c)
    B.bsp_check(c.plan)
    torch.cuda.synchronize()
    kp, vp = oracle.write_kv(inp.k_pool, inp.v_pool, inp.slots, inp.new_k, inp.new_v,
                             inp.page_size)
    assert torch.equal(c.k_pool.cpu(), S.to_device(kp, inp.dtype, "cpu")), what
    assert torch.equal(c.v_pool.cpu(), S.to_device(vp, inp.dtype, "cpu")), what
    fo, fl = oracle.prefill_attention(inp)
    return assert_close(c.out, c.lse_out, fo, fl, inp.dtype, f"{what} prefill")


PREFILL_CASES = {
    # qwen3-0.6B heads, chunks of a medium prompt, some requests with cached rows
    "d128_g2_bf16": dict(cfg="qwen3_0p6b", batch=4, chunk_range=(1, 600), cached_range=(0, 700)),
    "d128_g4_f16": dict(cfg="qwen3_4b", batch=3, chunk_range=(100, 500), cached_range=(0, 300)),
    "d64_g4_f16": dict(cfg="qwen3_4b", batch=3, head_dim=64, chunk_range=(1, 400),
                       cached_range=(0, 200)),
    "d256_g4_bf16": dict(cfg="qwen3_4b", batch=2, head_dim=256, dtype="bf16",
                         chunk_range=(50, 300), cached_range=(0, 100)),
    "one_row_chunks": dict(cfg="qwen3_0p6b", batch=6, chunk_range=(1, 1), cached_range=(0, 900)),
    "fresh_prompts": dict(cfg="qwen3_0p6b", batch=3, chunk_range=(64, 700)),
    # sized so that the plan takes 128-row (MB 2) and 192-row (MB 3) work items
    "mb2_tiles_bf16": dict(cfg="qwen3_0p6b", batch=8, chunk_range=(580, 620), cached_range=(0, 64)),
    "mb3_tiles_d64_f16": dict(cfg="qwen3_4b", batch=3, head_dim=64, chunk_range=(1100, 1200),
                              cached_range=(0, 100)),
}


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_prefill_matches_oracle(case):
    kw = dict(PREFILL_CASES[case])
    cfg = kw.pop("cfg")
    inp = synth.make_prefill(cfg, 2, **kw)
    say(f"prefill {case} Sq={inp.q_len.tolist()} L={inp.cached_len.tolist()}")
    say(f"  max |dO| = {_check_prefill(inp, case):.3g}")


@pytest.mark.parametrize("g,dt", [(1, "bf16"), (3, "f16"), (8, "bf16")])
def test_prefill_group_sizes(g, dt):
    """Query rows per position = group size: tiles end mid-position when 192 % g != 0."""
    cfg = BeamConfig(f"pf{g}", 1, 1, 2 * g, 2, 128, dt, 16, (0, 0), (0, 0), True)
    inp = synth.make_prefill(cfg, 9, batch=3, chunk_range=(1, 260), cached_range=(0, 150))
    say(f"prefill group {g} Sq={inp.q_len.tolist()} L={inp.cached_len.tolist()}")
    _check_prefill(inp, f"group {g}")


def test_prefill_and_beam_entry_points_need_their_own_plans():
    inp = synth.make_prefill("qwen3_0p6b", 1, batch=2, chunk_range=(5, 40), garbage="unit")
    c = S.upload_prefill(inp, DEV)
    with pytest.raises(B.BspError) as ei:
        B.bsp_prefill_attn(c.plan, c.q, c.k_pool, c.v_pool, c.out, c.lse_out)
    assert ei.value.name == "BSP_ERR_STALE_PLAN"
    S.plan_prefill(c)
    rows = c.rows
    o_part = torch.zeros((1, rows, c.num_q_heads, c.head_dim), device=DEV)
    lse_part = torch.zeros((1, rows, c.num_q_heads), device=DEV)
    with pytest.raises(B.BspError) as ei:
        B.bsp_prefix_attn(c.plan, c.q, c.k_pool, c.v_pool, o_part, lse_part)
    assert ei.value.name == "BSP_ERR_ARG"
    S.run_prefill(c)
    B.bsp_check(c.plan)
    torch.cuda.synchronize()


def test_mixed_step_on_two_streams():
    """Context requests (chunks of new prompts) beside a beam step of generation
    requests: prefill on a second stream, the fused step on the main one; each
    matches the oracle, and repeating the step gives the same outputs."""
    ctx_inp = synth.make_prefill("qwen3_0p6b", 4, batch=4, chunk_range=(100, 600),
                                 cached_range=(0, 300))
    gen_inp = synth.make_beam_step("qwen3_0p6b", 4, batch=6)
    say(f"mixed: ctx Sq={ctx_inp.q_len.tolist()} gen P={gen_inp.prefix_len.tolist()}")
    c = S.upload_prefill(ctx_inp, DEV)
    g = S.upload_beam_step(gen_inp, DEV)
    S.plan_prefill(c)
    S.plan_beam_step(g)
    side = torch.cuda.Stream()
    fo_c, fl_c = oracle.prefill_attention(ctx_inp)
    ref = synth.make_beam_step("qwen3_0p6b", 4, batch=6)
    kp, vp = oracle.write_kv(ref.k_pool, ref.v_pool, ref.slots, ref.k_new, ref.v_new,
                             ref.page_size)
    ref.k_pool, ref.v_pool = kp, vp
    fo_g, fl_g = oracle.beam_decode_attention(ref)
    for rep in range(2):
        S.run_mixed_step(c, g, ctx_stream=side)
        B.bsp_check(c.plan)
        B.bsp_check(g.plan)
        torch.cuda.synchronize()
        e1 = assert_close(c.out, c.lse_out, fo_c, fl_c, ctx_inp.dtype, f"mixed ctx {rep}")
        e2 = assert_close(g.out, g.lse_out, fo_g, fl_g, gen_inp.dtype, f"mixed gen {rep}")
        say(f"  launch {rep}: ctx {e1:.3g} gen {e2:.3g}")


def test_full_size_prefill_sampled():
    """Eight 2k-token prompts of the qwen3-0.6B layer in one launch, sampled rows."""
    inp = synth.make_prefill("qwen3_0p6b", 0, batch=8, chunk_range=(1500, 2500),
                             cached_range=(0, 0), garbage="unit")
    c = S.upload_prefill(inp, DEV)
    S.plan_prefill(c)
    S.run_prefill(c)
    B.bsp_check(c.plan)
    torch.cuda.synchronize()
    out = c.out.float().cpu().numpy()
    lse = c.lse_out.cpu().numpy()
    rng = np.random.default_rng(5)
    to, tl = TOL[inp.dtype]
    off = inp.q_off
    for b in range(inp.batch):
        n = int(inp.q_len[b])
        for i in [0, n - 1, int(rng.integers(0, n))]:
            fo, fl = oracle.prefill_attention_one(inp, b, i)
            r = int(off[b]) + i
            assert np.abs(out[r] - fo).max() <= to, (b, i)
            assert np.abs(lse[r] - fl).max() <= tl, (b, i)


@pytest.mark.parametrize("name,page_size,kw", [
    ("single_key", 16, dict(batch=1, chunk_range=(1, 1), cached_range=(0, 0))),
    ("page_size_1", 1, dict(batch=3, chunk_range=(1, 120), cached_range=(0, 90))),
    ("page_size_1024", 1024, dict(batch=3, chunk_range=(100, 700), cached_range=(0, 900))),
])
def test_prefill_degenerate_shapes(name, page_size, kw):
    cfg = BeamConfig(name, 1, 1, 8, 2, 128, "bf16", page_size, (0, 0), (0, 0), True)
    inp = synth.make_prefill(cfg, 13, **kw)
    say(f"prefill {name} Sq={inp.q_len.tolist()} L={inp.cached_len.tolist()}")
    _check_prefill(inp, name)


def _mixed_refs(ctx_inp, gen_cfg, seed, **gen_kw):
    fo_c, fl_c = oracle.prefill_attention(ctx_inp)
    ref = synth.make_beam_step(gen_cfg, seed, **gen_kw)
    ref.k_pool, ref.v_pool = oracle.write_kv(ref.k_pool, ref.v_pool, ref.slots, ref.k_new,
                                             ref.v_new, ref.page_size)
    return fo_c, fl_c, ref


@pytest.mark.parametrize("gen_cfg,gen_kw,one_launch", [
    ("qwen3_0p6b", dict(batch=6), True),            # W*G = 60 rows: one query block per wave
    ("qwen3_4b", dict(batch=3), False),             # 120 rows: two blocks, two launches
    ("nsample", dict(batch=5), True),               # 32 rows over four waves
])
def test_mixed_step_entry_point(gen_cfg, gen_kw, one_launch):
    """bsp_mixed_step: context workgroups beside beam-step workgroups in one launch
    (or two where the shapes do not allow it); both parts match the oracle on two
    launches in a row, and the beam step's token write is bit-exact."""
    ctx_inp = synth.make_prefill(gen_cfg, 6, batch=4, chunk_range=(100, 600), cached_range=(0, 300))
    gen_inp = synth.make_beam_step(gen_cfg, 6, **gen_kw)
    say(f"mixed entry {gen_cfg}: ctx Sq={ctx_inp.q_len.tolist()} gen P={gen_inp.prefix_len.tolist()}")
    c = S.upload_prefill(ctx_inp, DEV)
    g = S.upload_beam_step(gen_inp, DEV)
    S.plan_prefill(c)
    S.plan_beam_step(g)
    fo_c, fl_c, ref = _mixed_refs(ctx_inp, gen_cfg, 6, **gen_kw)
    fo_g, fl_g = oracle.beam_decode_attention(ref)
    for rep in range(2):
        S.run_mixed_step_fused(c, g)
        B.bsp_check(c.plan)
        B.bsp_check(g.plan)
        torch.cuda.synchronize()
        assert_close(c.out, c.lse_out, fo_c, fl_c, ctx_inp.dtype, f"mixed ctx {rep}")
        assert_close(g.out, g.lse_out, fo_g, fl_g, gen_inp.dtype, f"mixed gen {rep}")
    assert torch.equal(g.k_pool.cpu(), S.to_device(ref.k_pool, gen_inp.dtype, "cpu"))
    assert torch.equal(g.v_pool.cpu(), S.to_device(ref.v_pool, gen_inp.dtype, "cpu"))


def test_full_size_mixed_step_sampled():
    """The bench's mixed step in one launch: 64 x 30 beams (512 beam-step
    workgroups) beside four ~500-token prompts (~500 context workgroups); the
    chunks of the two kinds alternate. Sampled rows of both against the oracle."""
    ctx_inp = synth.make_prefill("qwen3_0p6b", 1, batch=4, chunk_range=(400, 600), garbage="unit")
    gen_inp = synth.make_beam_step("qwen3_0p6b", 0, garbage="unit")
    c = S.upload_prefill(ctx_inp, DEV)
    g = S.upload_beam_step(gen_inp, DEV)
    S.plan_prefill(c)
    S.plan_beam_step(g)
    S.run_mixed_step_fused(c, g)
    B.bsp_check(c.plan)
    B.bsp_check(g.plan)
    torch.cuda.synchronize()
    ref = gen_inp
    ref.k_pool, ref.v_pool = oracle.write_kv(ref.k_pool, ref.v_pool, ref.slots, ref.k_new,
                                             ref.v_new, ref.page_size)
    to, tl = TOL["bf16"]
    out = g.out.float().cpu().numpy().reshape(64, 30, 16, 128)
    lse = g.lse_out.cpu().numpy().reshape(64, 30, 16)
    rng = np.random.default_rng(4)
    for b, k in [(0, 0), (63, 29)] + [(int(x), int(y)) for x, y in
                                      zip(rng.integers(0, 64, 8), rng.integers(0, 30, 8))]:
        fo, fl = oracle.beam_attention_one(ref, b, k)
        assert np.abs(out[b, k] - fo[0]).max() <= to, (b, k)
        assert np.abs(lse[b, k] - fl[0]).max() <= tl, (b, k)
    cout = c.out.float().cpu().numpy()
    clse = c.lse_out.cpu().numpy()
    for b in range(ctx_inp.batch):
        n = int(ctx_inp.q_len[b])
        for i in [0, n - 1, int(rng.integers(0, n))]:
            fo, fl = oracle.prefill_attention_one(ctx_inp, b, i)
            r = int(ctx_inp.q_off[b]) + i
            assert np.abs(cout[r] - fo).max() <= to, (b, i)
            assert np.abs(clse[r] - fl).max() <= tl, (b, i)
