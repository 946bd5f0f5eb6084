"""GPU parity: every entry point against the fp64 oracle, element by element.

Sizes are the configs' own shapes with fewer requests (several MFMA tiles and
a ragged last tile per request), plus the edge cases: fp32 at 1e-5, empty
tails, group sizes 1..8, head_dim 64/128/256, shuffled and strided page ids,
fixed padded tails, bad device-side indices, and the cached-prefix variant at
its edge lengths.
"""

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


def _applied(inp):
    kp, vp = oracle.write_kv(inp.k_pool, inp.v_pool, inp.slots, inp.k_new, inp.v_new,
                             inp.page_size)
    inp.k_pool, inp.v_pool = kp, vp
    return inp


# ------------------------------------------------------------------ merge

@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n_parts", [1, 2, 5, 13, 55, 64, 65, 130])
def test_merge_matches_oracle(out_dtype, n_parts, D):
    """Both merge kernels: per-element (<= 8 parts) and per (row, head) workgroup,
    its register form (<= 64 parts) and its looping form (more)."""
    say(f"merge out={out_dtype} parts={n_parts} D={D}")
    rng = np.random.default_rng(n_parts)
    rows, heads = 37, 6
    o = rng.standard_normal((n_parts, rows, heads, D)).astype(np.float32)
    lse = (rng.standard_normal((n_parts, rows, heads)) * 3).astype(np.float32)
    lse[0, :5] = -np.inf                   # some parts empty
    lse[:, 5:7] = -np.inf                  # every part empty for two rows
    o[0, :5] = 0.0
    o[:, 5:7] = 0.0
    ref_o, ref_l = oracle.merge_states(list(o), list(lse))
    o[0, :5] = np.nan                      # an empty part's o is never used
    o[:, 5:7] = np.inf
    og = torch.from_numpy(o).to(DEV)
    lg = torch.from_numpy(lse).to(DEV)
    out = torch.empty((rows, heads, D), device=DEV, dtype=S.TORCH_DTYPE[out_dtype])
    lout = torch.empty((rows, heads), device=DEV)
    B.bsp_merge(rows, heads, D, n_parts, og, lg, rows * heads * D, rows * heads, out, out_dtype,
                lout)
    torch.cuda.synchronize()
    tol_o = TOL[out_dtype][0]
    o_gpu = out.float().cpu().numpy()
    assert np.abs(o_gpu - ref_o).max() <= tol_o
    l_gpu = lout.cpu().numpy()
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isneginf(l_gpu), ~fin)
    assert np.abs(l_gpu[fin] - ref_l[fin]).max() <= 1e-5


@pytest.mark.parametrize("D,n_parts", [(64, 20), (96, 41), (128, 54), (256, 20)])
def test_merge_one_row_many_parts(D, n_parts):
    """A split one-row decode: 1 row x 24 heads and dozens of parts (the
    workgroup-per-head merge), empty parts holding NaN."""
    rng = np.random.default_rng(D + n_parts)
    o = rng.standard_normal((n_parts, 1, 24, D)).astype(np.float32)
    lse = (rng.standard_normal((n_parts, 1, 24)) * 3).astype(np.float32)
    lse[::3, :, :5] = -np.inf
    lse[:, :, 7] = -np.inf                 # every part empty for one head
    o[lse == -np.inf] = 0.0
    ref_o, ref_l = oracle.merge_states(list(o), list(lse))
    o[lse == -np.inf] = np.nan
    og = torch.from_numpy(o).to(DEV)
    lg = torch.from_numpy(lse).to(DEV)
    out = torch.empty((1, 24, D), device=DEV, dtype=torch.bfloat16)
    lout = torch.empty((1, 24), device=DEV)
    B.bsp_merge(1, 24, D, n_parts, og, lg, 24 * D, 24, out, "bf16", lout)
    torch.cuda.synchronize()
    assert np.abs(out.float().cpu().numpy() - ref_o).max() <= TOL["bf16"][0]
    l_gpu = lout.cpu().numpy()
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isneginf(l_gpu), ~fin)
    assert np.abs(l_gpu[fin] - ref_l[fin]).max() <= 1e-5


# ----------------------------------------------------------------- KV write

@pytest.mark.parametrize("cfg", ["tiny", "qwen3_0p6b", "qwen3_4b"])
def test_write_kv_is_bit_exact(cfg):
    inp = synth.make_beam_step(cfg, 3, batch=3 if cfg != "tiny" else None)
    say(f"write_kv {cfg} n={len(inp.slots)}")
    ref_k, ref_v = oracle.write_kv(inp.k_pool, inp.v_pool, inp.slots, inp.k_new, inp.v_new,
                                   inp.page_size)
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    S.write_current_tokens(s)
    B.bsp_check(s.plan)
    assert torch.equal(s.k_pool.cpu(), S.to_device(ref_k, inp.dtype, "cpu"))
    assert torch.equal(s.v_pool.cpu(), S.to_device(ref_v, inp.dtype, "cpu"))


def test_write_kv_skips_and_reports_bad_slots():
    inp = synth.make_beam_step("qwen3_0p6b", 4, batch=2, tail_range=(2, 4))
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    before_k = s.k_pool.clone()
    slots = s.slots.clone()
    slots[1] = inp.num_pages * inp.page_size          # one past the pool
    slots[3] = -5
    good = torch.ones(len(slots), dtype=torch.bool)
    good[[1, 3]] = False
    B.bsp_write_kv(s.plan, s.k_new, s.v_new, s.num_kv_heads * s.head_dim, slots,
                   len(slots), s.k_pool, s.v_pool)
    with pytest.raises(B.BspError) as ei:
        B.bsp_check(s.plan)
    assert ei.value.name == "BSP_ERR_DEVICE_INDEX"
    B.bsp_check(s.plan)  # the error word was cleared
    ref_k, _ = oracle.write_kv(inp.k_pool, inp.v_pool, inp.slots[good.numpy()],
                               inp.k_new[good.numpy()], inp.v_new[good.numpy()], inp.page_size)
    assert torch.equal(s.k_pool.cpu(), S.to_device(ref_k, inp.dtype, "cpu"))
    assert not torch.equal(s.k_pool, before_k)


@pytest.mark.parametrize("cfg,dtype", [("tiny", None), ("qwen3_4b", None), ("qwen3_0p6b", "f32")])
def test_write_kv_desc_is_bit_exact_without_a_plan(cfg, dtype):
    """bsp_write_kv_desc from the layer descriptor alone (no plan object at all):
    bit-exact against the oracle's write, and skipped slots counted in the
    caller's fault word."""
    kw = {"batch": 3} if cfg != "tiny" else {}
    if dtype:
        kw["dtype"] = dtype
    inp = synth.make_beam_step(cfg, 8, **kw)
    k_pool = S.to_device(inp.k_pool, inp.dtype, DEV)
    v_pool = S.to_device(inp.v_pool, inp.dtype, DEV)
    k_new = S.to_device(inp.k_new, inp.dtype, DEV).reshape(len(inp.slots), -1).contiguous()
    v_new = S.to_device(inp.v_new, inp.dtype, DEV).reshape(len(inp.slots), -1).contiguous()
    slots = torch.as_tensor(inp.slots, dtype=torch.int32, device=DEV)
    desc = B.make_desc(inp.num_q_heads, inp.num_kv_heads, inp.head_dim, inp.page_size,
                       inp.num_pages, inp.dtype)
    faults = torch.zeros(3, dtype=torch.int32, device=DEV)
    B.bsp_write_kv_desc(desc, k_new, v_new, inp.num_kv_heads * inp.head_dim, slots, len(slots),
                        k_pool, v_pool, faults)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.write_kv(inp.k_pool, inp.v_pool, inp.slots, inp.k_new, inp.v_new,
                                   inp.page_size)
    assert torch.equal(k_pool.cpu(), S.to_device(ref_k, inp.dtype, "cpu"))
    assert torch.equal(v_pool.cpu(), S.to_device(ref_v, inp.dtype, "cpu"))
    assert faults.tolist() == [0, 0, 0]
    # two bad slots: skipped, counted, the good ones written
    bad = slots.clone()
    bad[0] = inp.num_pages * inp.page_size
    bad[-1] = -3
    k2 = S.to_device(inp.k_pool, inp.dtype, DEV)
    v2 = S.to_device(inp.v_pool, inp.dtype, DEV)
    B.bsp_write_kv_desc(desc, k_new, v_new, inp.num_kv_heads * inp.head_dim, bad, len(bad),
                        k2, v2, faults)
    torch.cuda.synchronize()
    f = faults.tolist()
    assert f[0] != 0 and f[1] == 2 and f[2] in (inp.num_pages * inp.page_size, -3)
    good = np.ones(len(inp.slots), dtype=bool)
    good[[0, -1]] = False
    ref_k2, _ = oracle.write_kv(inp.k_pool, inp.v_pool, inp.slots[good], inp.k_new[good],
                                inp.v_new[good], inp.page_size)
    assert torch.equal(k2.cpu(), S.to_device(ref_k2, inp.dtype, "cpu"))
    # with no fault word the bad slots are skipped all the same
    k3 = S.to_device(inp.k_pool, inp.dtype, DEV)
    v3 = S.to_device(inp.v_pool, inp.dtype, DEV)
    B.bsp_write_kv_desc(desc, k_new, v_new, inp.num_kv_heads * inp.head_dim, bad, len(bad),
                        k3, v3, None)
    torch.cuda.synchronize()
    assert torch.equal(k3, k2) and torch.equal(v3, v2)


# ----------------------------------------------------------- index resolution

def _tail_slots_gpu(s, pad):
    out = torch.full((s.batch, s.beam, max(pad, 1)), -7, dtype=torch.int32, device=DEV)
    B.bsp_debug_tail_slots(s.plan, s.block_tables, s.cache_indirection, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()[:, :, :pad]


@pytest.mark.parametrize("seed", range(6))
def test_tail_slots_bit_exact(seed):
    cfgs = [BeamConfig("idx", 3, 5, 4, 2, 64, "bf16", ps, (1, 40), (0, 9), bool(seed % 2))
            for ps in (4, 8, 16)]
    for cfg in cfgs:
        inp = synth.make_beam_step(cfg, seed, page_stride=1 + seed % 2)
        say(f"tail slots seed={seed} ps={cfg.page_size}")
        s = S.upload_beam_step(inp, DEV)
        S.plan_beam_step(s)
        pad = s.plan.tail_len
        ref = oracle.tail_slots(inp.prefix_len, inp.seq_len, inp.block_tables,
                                inp.cache_indirection, inp.page_size, pad)
        assert np.array_equal(_tail_slots_gpu(s, pad), ref)


def test_tail_slots_bit_exact_1200_random_batches():
    """The device's tail-slot resolution against the oracle's index function over
    1200 random batches: page sizes 1..1024, page ids at stride 1 or 2 (pages at
    even ids only), shuffled or in order, prompts that end exactly at a page
    boundary (a full last prompt page) or one row into a page, empty tails and
    tails that end at a page boundary."""
    rng = np.random.default_rng(1200)
    n_full_last = n_one_row = 0
    for trial in range(1200):
        ps = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]))
        kind = trial % 4
        if kind == 0:    # prompts that fill their last page
            pr = (ps * int(rng.integers(0, 3)),) * 2
        elif kind == 1:  # prompts one row into their last page
            pr = (ps * int(rng.integers(0, 3)) + 1,) * 2
        else:
            pr = (0, int(rng.integers(1, 3 * ps + 2)))
        cfg = BeamConfig("idx1200", batch=int(rng.integers(1, 5)), beam=int(rng.integers(1, 7)),
                         num_q_heads=2, num_kv_heads=1, head_dim=64, dtype="bf16", page_size=ps,
                         prefix_range=pr, tail_range=(0, int(rng.integers(1, 2 * ps + 3))),
                         shuffle_pages=bool(rng.integers(0, 2)))
        inp = synth.make_beam_step(cfg, trial, page_stride=int(rng.integers(1, 3)), garbage="unit")
        n_full_last += int(((inp.prefix_len % ps) == 0).sum())
        n_one_row += int(((inp.prefix_len % ps) == 1).sum())
        s = S.upload_beam_step(inp, DEV)
        S.plan_beam_step(s)
        pad = s.plan.tail_len
        ref = oracle.tail_slots(inp.prefix_len, inp.seq_len, inp.block_tables,
                                inp.cache_indirection, inp.page_size, pad)
        got = _tail_slots_gpu(s, pad)
        if not np.array_equal(got, ref):
            say(f"mismatch trial={trial} ps={ps} P={inp.prefix_len.tolist()} "
                f"S={inp.seq_len.tolist()}")
        assert np.array_equal(got, ref), trial
        B.bsp_check(s.plan)
    say(f"1200 batches: {n_full_last} prompts ending on a page boundary, "
        f"{n_one_row} one row into a page")
    assert n_full_last > 100 and n_one_row > 100


def _fused_slots_gpu(s, pad):
    out = torch.full((s.batch, s.num_kv_heads, s.beam, max(pad, 1)), -7, dtype=torch.int32,
                     device=DEV)
    B.bsp_debug_fused_slots(s.plan, s.q, s.k_new_beams, s.v_new_beams,
                            s.num_kv_heads * s.head_dim, s.k_pool, s.v_pool, s.block_tables,
                            s.cache_indirection, s.out, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_fused_slots(inp, got, pad):
    """The fused kernel's table entry (b, g, beam, t) against oracle.tail_slots:
    a pool row ((page * Hkv + g) * ps + row) whose page * ps + row is the
    oracle's slot, and for the current token (t = S - P - 1) the beam whose
    new-token row it reads, cache_indirection[b, beam, S - 1], the beam the
    oracle's slot for that position is taken from."""
    ps, hkv = inp.page_size, inp.num_kv_heads
    shift = ps.bit_length() - 1
    ref = oracle.tail_slots(inp.prefix_len, inp.seq_len, inp.block_tables,
                            inp.cache_indirection, ps, pad)
    for b in range(inp.batch):
        P, S_ = int(inp.prefix_len[b]), int(inp.seq_len[b])
        T = S_ - P
        assert (got[b, :, :, T:] == -7).all(), b
        if T == 0:  # no tail (and no current token past the prompt)
            continue
        e = got[b, :, :, :T - 1].astype(np.int64)
        assert (e >= 0).all(), b
        ph = e >> shift
        assert (ph % hkv == np.arange(hkv)[:, None, None]).all(), b
        assert ((ph // hkv) * ps + (e & (ps - 1)) == ref[b][None, :, :T - 1]).all(), b
        src = -2 - got[b, :, :, T - 1].astype(np.int64)
        assert (src == inp.cache_indirection[b, :, S_ - 1][None, :]).all(), b


def test_fused_slot_table_bit_exact_random_batches(monkeypatch):
    """bsp_decode_step's LDS tail-slot table, dumped by the kernel itself, bit for
    bit against the oracle's index function over 600 random batches: page sizes
    1..1024 at stride 1 or 2, prompts that fill their last page or end one row
    into it, beams spread over two query tiles, and prompts split into chunks
    (the table is then built by the last chunk to finish)."""
    rng = np.random.default_rng(600)
    n_split = n_tiles = n_full_last = 0
    for trial in range(600):
        ps = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]))
        kind = trial % 5
        beam = int(rng.integers(1, 7))
        if kind == 0:
            pr = (ps * int(rng.integers(1, 3)),) * 2
        elif kind == 1:
            pr = (ps * int(rng.integers(0, 3)) + 1,) * 2
        elif kind == 2:    # more than 64 query rows: two query tiles
            pr, beam = (1, 200), int(rng.integers(33, 60))
        else:
            pr = (1, int(rng.integers(2, 3 * ps + 3)))
        split = kind == 4 and trial % 10 == 4
        if split:
            pr = (300, 900)
            monkeypatch.setenv("BSP_SPLIT", "64")
        else:
            monkeypatch.delenv("BSP_SPLIT", raising=False)
        cfg = BeamConfig("fslots", batch=int(rng.integers(1, 5)), beam=beam, num_q_heads=4,
                         num_kv_heads=2, head_dim=64, dtype="bf16" if trial % 2 else "f16",
                         page_size=ps, prefix_range=pr, tail_range=(0, int(rng.integers(1, 60))),
                         shuffle_pages=bool(rng.integers(0, 2)))
        inp = synth.make_beam_step(cfg, trial, page_stride=int(rng.integers(1, 3)), garbage="unit")
        s = S.upload_beam_step(inp, DEV)
        S.plan_beam_step(s)
        items = B.bsp_debug_plan_items(s.plan)
        n_split += int(split and (items[:, 3] > 1).any())
        n_tiles += int(beam * 2 > 64)
        n_full_last += int(((inp.prefix_len % ps) == 0).sum())
        pad = s.plan.tail_len
        got = _fused_slots_gpu(s, pad)
        B.bsp_check(s.plan)
        try:
            _check_fused_slots(inp, got, pad)
        except AssertionError:
            say(f"mismatch trial={trial} ps={ps} W={beam} split={split} "
                f"P={inp.prefix_len.tolist()} S={inp.seq_len.tolist()}")
            raise
    say(f"600 batches: {n_split} with split prompts, {n_tiles} with two query tiles, "
        f"{n_full_last} prompts ending on a page boundary")
    assert n_split >= 50 and n_tiles >= 100 and n_full_last >= 100


def test_fused_slot_table_dump_leaves_outputs_and_pool():
    """The dump launch writes only the table: the output and the pools are untouched."""
    inp = synth.make_beam_step("qwen3_0p6b", 3, batch=3)
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    s.out.fill_(7)
    k0, v0 = s.k_pool.clone(), s.v_pool.clone()
    got = _fused_slots_gpu(s, s.plan.tail_len)
    B.bsp_check(s.plan)
    _check_fused_slots(inp, got, s.plan.tail_len)
    assert (s.out == 7).all()
    assert torch.equal(s.k_pool, k0) and torch.equal(s.v_pool, v0)


def test_bad_cache_indirection_is_skipped_and_reported():
    inp = synth.make_beam_step("qwen3_0p6b", 5, batch=2, tail_range=(3, 4))
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    P = int(inp.prefix_len[1])
    s.cache_indirection[1, 4, P + 1] = inp.beam      # parent beam out of range
    S.run_beam_step(s)
    with pytest.raises(B.BspError) as ei:
        B.bsp_check(s.plan)
    assert ei.value.name == "BSP_ERR_DEVICE_INDEX"
    assert not torch.isnan(s.out.float()).any()


# ---------------------------------------------------------- whole beam step

STEP_CASES = {
    "tiny_f32": dict(cfg="tiny"),
    "qwen3_0p6b_bf16": dict(cfg="qwen3_0p6b", batch=3),
    "wide_beam_bf16": dict(cfg="wide_beam", batch=2),
    "wide_beam_fixed_tail8": dict(cfg="wide_beam", batch=2, tail_range=(8, 8)),
    "qwen3_4b_f16_d128": dict(cfg="qwen3_4b", batch=2),
    "qwen3_4b_f16_d64": dict(cfg="qwen3_4b", batch=2, head_dim=64),
    "qwen3_4b_f16_d256": dict(cfg="qwen3_4b", batch=2, head_dim=256),
    "no_tails_bf16": dict(cfg="qwen3_0p6b", batch=3, tail_range=(0, 0)),
    "strided_pages_bf16": dict(cfg="qwen3_0p6b", batch=2, page_stride=2, shuffle_pages=True),
    "f32_d128": dict(cfg="qwen3_0p6b", batch=2, dtype="f32", prefix_range=(30, 90)),
    "f32_d256": dict(cfg="qwen3_4b", batch=1, dtype="f32", head_dim=256, prefix_range=(50, 90)),
    "nsample_bf16": dict(cfg="nsample", batch=3),
    "nsample_f16_d64": dict(cfg="nsample", batch=2, dtype="f16", head_dim=64, beam=40),
}
GROUP_CASES = {f"group{g}_{dt}": (g, dt) for g, dt in
               [(1, "bf16"), (2, "f16"), (3, "f16"), (4, "bf16"), (6, "bf16"), (8, "f16")]}


def _run_and_check(inp, what, max_tail=None):
    s = S.upload_beam_step(inp, DEV, max_tail=max_tail)
    S.plan_beam_step(s)
    S.run_beam_step(s)
    B.bsp_check(s.plan)
    torch.cuda.synchronize()
    ref = _applied(inp)
    po, pl = oracle.beam_partial_attention(ref, "prefix")
    to, tl = oracle.beam_partial_attention(ref, "tail")
    fo, fl = oracle.beam_decode_attention(ref)
    assert_close(s.o_part[0], s.lse_part[0], po, pl, "f32" if inp.dtype == "f32" else inp.dtype,
                 f"{what} prefix partial")
    assert_close(s.o_part[1], s.lse_part[1], to, tl, "f32" if inp.dtype == "f32" else inp.dtype,
                 f"{what} tail partial")
    return assert_close(s.out, s.lse_out, fo, fl, inp.dtype, f"{what} output")


@pytest.mark.parametrize("case", list(STEP_CASES))
@pytest.mark.parametrize("seed", [0, 1])
def test_beam_step_matches_oracle(case, seed):
    kw = dict(STEP_CASES[case])
    cfg = kw.pop("cfg")
    inp = synth.make_beam_step(cfg, seed, **kw)
    say(f"beam step {case} seed={seed} B={inp.batch} W={inp.beam} D={inp.head_dim} "
        f"P={inp.prefix_len.tolist()} T={inp.tail_len.tolist()}")
    mt = 8 if "fixed_tail" in case else None
    err = _run_and_check(inp, case, max_tail=mt)
    say(f"  max |dO| = {err:.3g}")


@pytest.mark.parametrize("case", list(GROUP_CASES))
def test_beam_step_group_sizes(case):
    g, dt = GROUP_CASES[case]
    cfg = BeamConfig(case, 2, 7, 2 * g, 2, 128, dt, 16, (70, 150), (0, 5), True)
    inp = synth.make_beam_step(cfg, 11)
    say(f"group size {g} {dt} M={7 * g}")
    _run_and_check(inp, case)


def test_naive_comparator_matches_oracle():
    inp = synth.make_beam_step("qwen3_0p6b", 2, batch=2)
    say("naive comparator")
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    S.write_current_tokens(s)
    out = torch.empty_like(s.out)
    lout = torch.empty_like(s.lse_out)
    B.bsp_naive_beam_attn(s.plan, s.q, s.k_pool, s.v_pool, s.block_tables, s.cache_indirection,
                          out, lout)
    B.bsp_check(s.plan)
    fo, fl = oracle.beam_decode_attention(_applied(inp))
    assert_close(out, lout, fo, fl, inp.dtype, "naive")


# ------------------------------------------------- cached prefix (beam 1)

CACHED_L = [0, 1, 255, 256, 257, 1000, 5184, 10240, 10241, 10368]


def _cached_small(seed, L, q_len, **kw):
    # Same geometry as the Phi-4 shape with a 1024-row allocation so the oracle is quick
    # for prefill; decode runs at the full 10368 rows.
    return synth.make_cached_prefix(seed, valid_rows=L, q_len=q_len, **kw)


@pytest.mark.parametrize("split", [256, -1])
@pytest.mark.parametrize("L", CACHED_L)
def test_cached_prefix_decode_matches_oracle(L, split):
    """Fixed 256-key chunks, and the chunk the plan picks (kv_split = -1)."""
    R = oracle.bucket_rows(L, 256, 10368)
    inp = synth.make_cached_prefix(L % 7, valid_rows=L, q_len=1, nan_from_row=R)
    c = S.upload_cached_prefix(inp, DEV, kv_split=split)
    S.plan_cached_prefix(c)
    sk = c.plan_cache.split_keys
    say(f"cached decode L={L} R={R} split={split}: {c.n_split} chunks of {sk} keys")
    if split > 0:
        assert sk == split
    S.run_cached_prefix(c)
    B.bsp_check(c.plan_cache)
    B.bsp_check(c.plan_new)
    o, lse = oracle.cached_prefix_attention(inp, causal=True)
    assert_close(c.out.reshape(1, 24, 128), c.lse_out.reshape(1, 24), o, lse, "f16",
                 f"decode L={L}")
    # every split partial against the oracle's partial over the same key chunk
    step = sk if sk > 0 else max(L, 1)
    for sp in range(c.n_split):
        po, pl = oracle.cached_prefix_partial(inp, "cache", key_range=(step * sp, step * (sp + 1)))
        assert_close(c.o_part[sp], c.lse_part[sp], po, pl, "f16", f"decode L={L} split {sp}")


# 16 seeded draws of the valid length over the whole allocation, beside the edges
RANDOM_L = [int(x) for x in np.random.default_rng(10368).integers(0, 10369, 16)]


@pytest.mark.parametrize("L", RANDOM_L)
def test_cached_prefix_decode_random_lengths(L):
    """A one-row decode at the full 10368-row allocation, valid length drawn
    uniformly: the output and every chunk's partial against the oracle."""
    R = oracle.bucket_rows(L, 256, 10368)
    inp = synth.make_cached_prefix(L % 13, valid_rows=L, q_len=1, nan_from_row=R)
    c = S.upload_cached_prefix(inp, DEV)
    S.plan_cached_prefix(c)
    sk = c.plan_cache.split_keys
    say(f"cached decode random L={L} R={R}: {c.n_split} chunks of {sk} keys")
    S.run_cached_prefix(c)
    B.bsp_check(c.plan_cache)
    B.bsp_check(c.plan_new)
    o, lse = oracle.cached_prefix_attention(inp, causal=True)
    assert_close(c.out.reshape(1, 24, 128), c.lse_out.reshape(1, 24), o, lse, "f16",
                 f"decode L={L}")
    step = sk if sk > 0 else max(L, 1)
    for sp in range(c.n_split):
        po, pl = oracle.cached_prefix_partial(inp, "cache", key_range=(step * sp, step * (sp + 1)))
        assert_close(c.o_part[sp], c.lse_part[sp], po, pl, "f16", f"decode L={L} split {sp}")


@pytest.mark.parametrize("L", CACHED_L + RANDOM_L[:8])
def test_cached_decode_one_launch(L):
    """The one-row decode in one launch (bsp_cached_decode) against the oracle at
    the edge and random valid lengths of the 10368-row allocation, twice in a
    row (the last chunk resets each counter for the next launch): the output
    within tolerance, the new row written at its slot bit for bit, and the
    result equal to that of the four-launch call."""
    R = oracle.bucket_rows(L, 256, 10368)
    inp = synth.make_cached_prefix(L % 5, valid_rows=L, q_len=1, nan_from_row=R)
    c = S.upload_cached_prefix(inp, DEV)
    S.plan_cached_prefix(c)
    say(f"one-launch cached decode L={L}: {c.n_split} chunks of {c.plan_cache.split_keys} keys")
    o, lse = oracle.cached_prefix_attention(inp, causal=True)
    outs = []
    for rep in range(2):
        S.run_cached_decode(c)
        B.bsp_check(c.plan_cache)
        torch.cuda.synchronize()
        assert_close(c.out.reshape(1, 24, 128), c.lse_out.reshape(1, 24), o, lse, "f16",
                     f"one-launch decode L={L} launch {rep}")
        outs.append((c.out.clone(), c.lse_out.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    page, row = divmod(int(c.slots[0]), c.page_size)
    assert torch.equal(c.k_pool[page, :, row].cpu(), S.to_device(inp.new_k[0], "f16", "cpu"))
    assert torch.equal(c.v_pool[page, :, row].cpu(), S.to_device(inp.new_v[0], "f16", "cpu"))
    S.run_cached_prefix(c)  # the four-launch call
    B.bsp_check(c.plan_cache)
    B.bsp_check(c.plan_new)
    torch.cuda.synchronize()
    assert (c.out.float() - outs[0][0].float()).abs().max().item() <= 2e-3
    assert (c.lse_out - outs[0][1]).abs().max().item() <= 1e-5


@pytest.mark.parametrize("L,split", [(10368, 64), (5000, 64), (777, 64), (10368, 128)])
def test_cached_decode_one_launch_many_chunks(L, split):
    """Forced small chunks, so each merging thread folds its chunks over several
    batches of loads (more than 32 chunks per slice of threads): against the
    oracle and the four-launch call."""
    R = oracle.bucket_rows(L, 256, 10368)
    inp = synth.make_cached_prefix(11 + L % 7, valid_rows=L, q_len=1, nan_from_row=R)
    c = S.upload_cached_prefix(inp, DEV, kv_split=split)
    S.plan_cached_prefix(c)
    say(f"one-launch cached decode L={L}: {c.n_split} chunks of {c.plan_cache.split_keys} keys")
    if L >= 5000:
        assert c.n_split > 64  # more than 32 chunks per slice at 2 slices
    o, lse = oracle.cached_prefix_attention(inp, causal=True)
    S.run_cached_decode(c)
    B.bsp_check(c.plan_cache)
    torch.cuda.synchronize()
    assert_close(c.out.reshape(1, 24, 128), c.lse_out.reshape(1, 24), o, lse, "f16",
                 f"one-launch decode L={L} split {split}")
    one = (c.out.clone(), c.lse_out.clone())
    S.run_cached_prefix(c)
    B.bsp_check(c.plan_cache)
    B.bsp_check(c.plan_new)
    torch.cuda.synchronize()
    assert (c.out.float() - one[0].float()).abs().max().item() <= 2e-3
    assert (c.lse_out - one[1]).abs().max().item() <= 1e-5


@pytest.mark.parametrize("hq,hkv,d,dtype,L", [(16, 4, 64, "bf16", 3000), (8, 4, 256, "f16", 2000),
                                              (32, 4, 128, "bf16", 4100), (16, 4, 256, "bf16", 777),
                                              (8, 8, 64, "f16", 1)])
def test_cached_decode_one_launch_other_shapes(hq, hkv, d, dtype, L):
    """bsp_cached_decode at the other head sizes and group sizes its merge takes
    (query heads per KV head x head_dim / 4 up to 256), in both 16-bit dtypes:
    against the oracle, the new row written bit for bit, and equal to the
    four-launch call within rounding."""
    R = oracle.bucket_rows(L, 256, 4608)
    inp = synth.make_cached_prefix(L % 11, valid_rows=L, q_len=1, num_q_heads=hq,
                                   num_kv_heads=hkv, head_dim=d, dtype=dtype,
                                   max_cache_rows=4608, nan_from_row=R)
    c = S.upload_cached_prefix(inp, DEV)
    S.plan_cached_prefix(c)
    say(f"one-launch cached decode {hq}/{hkv} heads d={d} {dtype} L={L}: {c.n_split} chunks")
    o, lse = oracle.cached_prefix_attention(inp, causal=True)
    S.run_cached_decode(c)
    B.bsp_check(c.plan_cache)
    torch.cuda.synchronize()
    assert_close(c.out.reshape(1, hq, d), c.lse_out.reshape(1, hq), o, lse, dtype,
                 f"one-launch decode {hq}/{hkv} d={d} {dtype}")
    one = (c.out.clone(), c.lse_out.clone())
    page, row = divmod(int(c.slots[0]), c.page_size)
    assert torch.equal(c.k_pool[page, :, row].cpu(), S.to_device(inp.new_k[0], dtype, "cpu"))
    assert torch.equal(c.v_pool[page, :, row].cpu(), S.to_device(inp.new_v[0], dtype, "cpu"))
    S.run_cached_prefix(c)
    B.bsp_check(c.plan_cache)
    B.bsp_check(c.plan_new)
    torch.cuda.synchronize()
    assert (c.out.float() - one[0].float()).abs().max().item() <= TOL[dtype][0]
    assert (c.lse_out - one[1]).abs().max().item() <= 1e-5


@pytest.mark.parametrize("L", CACHED_L + RANDOM_L[8:])
def test_cached_decode_two_launches(L):
    """The one-row decode as the cache chunks plus bsp_cached_decode_merge (the
    merge folded with the call's row, which it also writes into its page), at
    the edge and random valid lengths of the 10368-row allocation, twice in a
    row: against the oracle, the new row bit for bit, and equal to the
    four-launch call within rounding."""
    R = oracle.bucket_rows(L, 256, 10368)
    inp = synth.make_cached_prefix(L % 7, valid_rows=L, q_len=1, nan_from_row=R)
    c = S.upload_cached_prefix(inp, DEV)
    S.plan_cached_prefix(c)
    say(f"two-launch cached decode L={L}: {c.n_split} chunks of {c.plan_cache.split_keys} keys")
    o, lse = oracle.cached_prefix_attention(inp, causal=True)
    outs = []
    for rep in range(2):
        S.run_cached_decode_two(c)
        B.bsp_check(c.plan_cache)
        torch.cuda.synchronize()
        assert_close(c.out.reshape(1, 24, 128), c.lse_out.reshape(1, 24), o, lse, "f16",
                     f"two-launch decode L={L} launch {rep}")
        outs.append((c.out.clone(), c.lse_out.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    page, row = divmod(int(c.slots[0]), c.page_size)
    assert torch.equal(c.k_pool[page, :, row].cpu(), S.to_device(inp.new_k[0], "f16", "cpu"))
    assert torch.equal(c.v_pool[page, :, row].cpu(), S.to_device(inp.new_v[0], "f16", "cpu"))
    S.run_cached_prefix(c)  # the four-launch call
    B.bsp_check(c.plan_cache)
    B.bsp_check(c.plan_new)
    torch.cuda.synchronize()
    assert (c.out.float() - outs[0][0].float()).abs().max().item() <= 2e-3
    assert (c.lse_out - outs[0][1]).abs().max().item() <= 1e-5


@pytest.mark.parametrize("hq,hkv,d,dtype,L,split", [
    (16, 4, 64, "bf16", 3000, 0), (8, 4, 256, "f16", 2000, 0), (32, 4, 128, "bf16", 4100, 0),
    (16, 2, 256, "bf16", 777, 0), (8, 8, 64, "f16", 1, 0),
    (24, 8, 128, "f16", 4608, 64),   # 72 chunks: more than the 64 held in registers
    (24, 8, 128, "bf16", 4500, 64)])  # 71 chunks
def test_cached_decode_two_launches_other_shapes(hq, hkv, d, dtype, L, split):
    """bsp_cached_decode_merge at other head and group sizes (groups of eight at
    head_dim 256 too), both 16-bit dtypes, and with more chunks than its merge
    holds in registers: against the oracle, the row written bit for bit."""
    R = oracle.bucket_rows(L, 256, 4608)
    inp = synth.make_cached_prefix(L % 11, valid_rows=L, q_len=1, num_q_heads=hq,
                                   num_kv_heads=hkv, head_dim=d, dtype=dtype,
                                   max_cache_rows=4608, nan_from_row=R)
    c = S.upload_cached_prefix(inp, DEV, kv_split=split if split else -1)
    S.plan_cached_prefix(c)
    say(f"two-launch cached decode {hq}/{hkv} heads d={d} {dtype} L={L}: {c.n_split} chunks")
    if split:
        assert c.n_split > 64
    o, lse = oracle.cached_prefix_attention(inp, causal=True)
    S.run_cached_decode_two(c)
    B.bsp_check(c.plan_cache)
    torch.cuda.synchronize()
    assert_close(c.out.reshape(1, hq, d), c.lse_out.reshape(1, hq), o, lse, dtype,
                 f"two-launch decode {hq}/{hkv} d={d} {dtype}")
    page, row = divmod(int(c.slots[0]), c.page_size)
    assert torch.equal(c.k_pool[page, :, row].cpu(), S.to_device(inp.new_k[0], dtype, "cpu"))
    assert torch.equal(c.v_pool[page, :, row].cpu(), S.to_device(inp.new_v[0], dtype, "cpu"))


def test_cached_decode_two_launches_bad_slot_is_skipped_and_reported():
    """A slot outside the pool: the row is not written, bsp_check reports the
    fault, and the output (which never reads the row from the pool) is right."""
    inp = synth.make_cached_prefix(4, valid_rows=900, q_len=1)
    c = S.upload_cached_prefix(inp, DEV)
    S.plan_cached_prefix(c)
    before_k, before_v = c.k_pool.clone(), c.v_pool.clone()
    c.slots.fill_(int(c.k_pool.shape[0]) * c.page_size)  # one past the pool
    S.run_cached_decode_two(c)
    with pytest.raises(B.BspError):
        B.bsp_check(c.plan_cache)
    torch.cuda.synchronize()
    # bit patterns: the pools hold NaN past the valid rows
    assert torch.equal(c.k_pool.view(torch.int16), before_k.view(torch.int16))
    assert torch.equal(c.v_pool.view(torch.int16), before_v.view(torch.int16))
    o, lse = oracle.cached_prefix_attention(inp, causal=True)
    assert_close(c.out.reshape(1, 24, 128), c.lse_out.reshape(1, 24), o, lse, "f16", "bad slot")


def test_cached_decode_two_launches_rejects_other_plans():
    inp = synth.make_cached_prefix(3, valid_rows=300, q_len=4)
    c = S.upload_cached_prefix(inp, DEV)
    S.plan_cached_prefix(c)
    with pytest.raises(B.BspError) as ei:
        B.bsp_cached_decode_merge(c.plan_cache, c.q, c.new_k, c.new_v, c.num_kv_heads * c.head_dim,
                                  c.slots, c.k_pool, c.v_pool, c.o_part, c.lse_part, c.out,
                                  c.lse_out)
    assert ei.value.name == "BSP_ERR_UNSUPPORTED"


def test_cached_decode_one_launch_rejects_too_wide_groups():
    """Eight query heads per KV head at head_dim 256 (512 row-chunk pairs) are more
    than the merge's 256 threads: refused before any launch."""
    inp = synth.make_cached_prefix(2, valid_rows=500, q_len=1, num_q_heads=16, num_kv_heads=2,
                                   head_dim=256, dtype="f16", max_cache_rows=1024)
    c = S.upload_cached_prefix(inp, DEV)
    S.plan_cached_prefix(c)
    with pytest.raises(B.BspError) as ei:
        S.run_cached_decode(c)
    assert ei.value.name == "BSP_ERR_UNSUPPORTED"


def test_cached_decode_one_launch_rejects_other_plans():
    inp = synth.make_cached_prefix(3, valid_rows=300, q_len=4)
    c = S.upload_cached_prefix(inp, DEV)
    S.plan_cached_prefix(c)
    with pytest.raises(B.BspError) as ei:
        S.run_cached_decode(c)
    assert ei.value.name == "BSP_ERR_UNSUPPORTED"
    beam = S.upload_beam_step(synth.make_beam_step("qwen3_0p6b", 1, batch=2), DEV)
    S.plan_beam_step(beam)
    with pytest.raises(B.BspError) as ei:
        B.bsp_cached_decode(beam.plan, beam.q, beam.k_new, beam.v_new, 1024, beam.slots,
                            beam.k_pool, beam.v_pool, beam.o_part[0], beam.lse_part[0], beam.out)
    assert ei.value.name == "BSP_ERR_UNSUPPORTED"


@pytest.mark.parametrize("draw", range(16))
def test_cached_prefix_prefill_random_lengths(draw):
    """A prefill at the full 10368-row allocation with the valid length drawn from
    U{0..10368} and the prompt from U{500..2000}: sampled query rows (first, last,
    tile edges, random) against the oracle."""
    rng = np.random.default_rng(7000 + draw)
    L = int(rng.integers(0, 10369))
    Sq = int(rng.integers(500, 2001))
    R = oracle.bucket_rows(L, 256, 10368)
    inp = synth.make_cached_prefix(draw, valid_rows=L, q_len=Sq, nan_from_row=R)
    c = S.upload_cached_prefix(inp, DEV)
    S.plan_cached_prefix(c)
    say(f"cached prefill random L={L} Sq={Sq}: {c.n_split} chunks of {c.plan_cache.split_keys} keys")
    S.run_cached_prefix(c)
    B.bsp_check(c.plan_cache)
    B.bsp_check(c.plan_new)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 63, 64, Sq // 2, Sq - 2, Sq - 1} |
                  {int(r) for r in rng.integers(0, Sq, 5)})
    o, lse = oracle.cached_prefix_attention(inp, causal=True, rows=rows)
    idx = torch.tensor(rows, device=DEV)
    assert_close(c.out[idx], c.lse_out[idx], o, lse, "f16", f"prefill L={L} Sq={Sq}")


@pytest.mark.parametrize("L,Sq,causal,split", [(0, 37, True, 0), (300, 64, True, 0),
                                                (777, 200, True, 0), (1024, 130, False, 0),
                                                (513, 1, True, 256), (777, 200, True, -1),
                                                (1024, 130, False, -1), (900, 3, True, -1)])
def test_cached_prefix_prefill_matches_oracle(L, Sq, causal, split):
    R = oracle.bucket_rows(L, 256, 1024)
    inp = synth.make_cached_prefix(Sq, valid_rows=L, q_len=Sq, max_cache_rows=1024,
                                   nan_from_row=R)
    c = S.upload_cached_prefix(inp, DEV, kv_split=split, causal=causal)
    say(f"cached prefill L={L} Sq={Sq} causal={causal} split={split}")
    S.plan_cached_prefix(c)
    S.run_cached_prefix(c)
    B.bsp_check(c.plan_cache)
    o, lse = oracle.cached_prefix_attention(inp, causal=causal)
    assert_close(c.out, c.lse_out, o, lse, "f16", f"prefill L={L} Sq={Sq}")


@pytest.mark.parametrize("L,Sq", [(10368, 1), (5000, 1), (0, 1), (777, 200)])
def test_prefix_attn_two_equals_two_calls(L, Sq):
    """bsp_prefix_attn_two writes exactly what two bsp_prefix_attn calls write: one
    launch for a one-row decode (both segments in 64-row tiles), one per plan for a
    prefill whose cache segment takes taller tiles."""
    rows_alloc = 10368 if Sq == 1 else 1024
    inp = synth.make_cached_prefix(L % 11, valid_rows=L, q_len=Sq, max_cache_rows=rows_alloc)
    say(f"prefix_attn_two L={L} Sq={Sq}")
    outs = []
    for two in (False, True):
        c = S.upload_cached_prefix(inp, DEV)
        S.plan_cached_prefix(c)
        c.o_part.fill_(7.0)
        c.lse_part.fill_(7.0)
        S.run_cached_prefix(c, two_launches=not two)
        B.bsp_check(c.plan_cache)
        B.bsp_check(c.plan_new)
        torch.cuda.synchronize()
        outs.append((c.o_part.clone(), c.lse_part.clone(), c.out.clone(), c.lse_out.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    o, lse = oracle.cached_prefix_attention(inp, causal=True)
    assert_close(outs[1][2], outs[1][3], o, lse, "f16", f"two-plan L={L} Sq={Sq}")


def test_prefix_attn_two_rejects_mismatched_plans():
    inp = synth.make_cached_prefix(3, valid_rows=300, q_len=1)
    c = S.upload_cached_prefix(inp, DEV)
    S.plan_cached_prefix(c)
    ns = c.n_split
    with pytest.raises(RuntimeError):  # the same plan twice
        B.bsp_prefix_attn_two(c.plan_cache, c.plan_cache, c.q, c.k_pool, c.v_pool, c.o_part[:ns],
                              c.lse_part[:ns], c.o_part[ns], c.lse_part[ns])
    other = synth.make_cached_prefix(3, valid_rows=300, q_len=4)
    d = S.upload_cached_prefix(other, DEV)
    S.plan_cached_prefix(d)
    with pytest.raises(RuntimeError):  # different query rows
        B.bsp_prefix_attn_two(c.plan_cache, d.plan_new, c.q, c.k_pool, c.v_pool, c.o_part[:ns],
                              c.lse_part[:ns], c.o_part[ns], c.lse_part[ns])


def test_full_size_cached_prefill_sampled():
    """The bench's cached-prefix prefill: 10368 valid cached rows + 2000 causal new rows,
    the automatic key split; sampled query rows (first, last, tile edges, random)."""
    inp = synth.make_cached_prefix(0, valid_rows=10368, q_len=2000)
    c = S.upload_cached_prefix(inp, DEV)
    S.plan_cached_prefix(c)
    say(f"full-size cached prefill: {c.n_split} chunks of {c.plan_cache.split_keys} keys")
    S.run_cached_prefix(c)
    B.bsp_check(c.plan_cache)
    B.bsp_check(c.plan_new)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = sorted({0, 1, 21, 63, 64, 191, 192, 1000, 1998, 1999} |
                  {int(r) for r in rng.integers(0, 2000, 10)})
    o, lse = oracle.cached_prefix_attention(inp, causal=True, rows=rows)
    idx = torch.tensor(rows, device=DEV)
    assert_close(c.out[idx], c.lse_out[idx], o, lse, "f16", "full-size cached prefill")


def test_cached_prefix_garbage_rows_do_not_matter():
    L = 700
    a = synth.make_cached_prefix(1, valid_rows=L, q_len=1)
    b = synth.make_cached_prefix(1, valid_rows=L, q_len=1, nan_from_row=L)
    outs = []
    for inp in (a, b):
        c = S.upload_cached_prefix(inp, DEV)
        S.plan_cached_prefix(c)
        S.run_cached_prefix(c)
        torch.cuda.synchronize()
        outs.append((c.out.clone(), c.lse_out.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


# ------------------------------------------- full size, sampled outputs

def test_full_size_qwen3_0p6b_sampled():
    """64 requests x 30 beams, bf16, in the launch configuration the bench times."""
    inp = synth.make_beam_step("qwen3_0p6b", 0)
    say(f"full-size qwen3_0p6b: pages={inp.num_pages}")
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    S.run_beam_step(s)
    B.bsp_check(s.plan)
    torch.cuda.synchronize()
    ref = _applied(inp)
    rng = np.random.default_rng(0)
    picks = [(int(b), int(k)) for b, k in zip(rng.integers(0, 64, 24), rng.integers(0, 30, 24))]
    picks += [(0, 0), (63, 29)]
    out = s.out.float().cpu().numpy().reshape(64, 30, 16, 128)
    lse = s.lse_out.cpu().numpy().reshape(64, 30, 16)
    to, tl = TOL["bf16"]
    for b, k in picks:
        fo, fl = oracle.beam_attention_one(ref, b, k)
        assert np.abs(out[b, k] - fo[0]).max() <= to
        assert np.abs(lse[b, k] - fl[0]).max() <= tl


# ------------------------------------------- fused decode step (one launch)

def _run_fused_and_check(inp, what, max_tail=None):
    s = S.upload_beam_step(inp, DEV, max_tail=max_tail)
    S.plan_beam_step(s)
    S.run_decode_step(s)
    B.bsp_check(s.plan)
    torch.cuda.synchronize()
    ref = _applied(inp)
    # the token write is bit-exact
    assert torch.equal(s.k_pool.cpu(), S.to_device(ref.k_pool, inp.dtype, "cpu")), what
    assert torch.equal(s.v_pool.cpu(), S.to_device(ref.v_pool, inp.dtype, "cpu")), what
    fo, fl = oracle.beam_decode_attention(ref)
    return assert_close(s.out, s.lse_out, fo, fl, inp.dtype, f"{what} fused output")


FUSED_CASES = [c for c in STEP_CASES if "f32" not in c]


@pytest.mark.parametrize("case", FUSED_CASES)
@pytest.mark.parametrize("seed", [0, 1])
def test_decode_step_matches_oracle(case, seed):
    kw = dict(STEP_CASES[case])
    cfg = kw.pop("cfg")
    inp = synth.make_beam_step(cfg, seed, **kw)
    say(f"fused step {case} seed={seed} P={inp.prefix_len.tolist()} T={inp.tail_len.tolist()}")
    mt = 8 if "fixed_tail" in case else None
    say(f"  max |dO| = {_run_fused_and_check(inp, case, max_tail=mt):.3g}")


# Current-token rows at one or two query blocks per wave (head_dim <= 128, no
# split) are loaded in the prologue when each thread has at most 4 (MB = 1) or
# 2 (MB = 2) of a tile's 16-byte tasks, else loaded at the end; each case sits
# on one side of that line (tasks = beams in the tile x head_dim / 8).
TOKEN_ROW_CASES = {
    # MB = 1 (64 rows), 64 beams x 16 tasks = 1024 = 256 x 4: prologue
    "mb1_d128_at_limit": (BeamConfig("tw1", 2, 64, 2, 2, 128, "bf16", 16, (70, 150), (1, 5), True), None),
    # MB = 2 (100 rows), 100 beams x 16 tasks = 1600 > 512: loaded at the end
    "mb2_d128_g1_late": (BeamConfig("tw2", 2, 100, 2, 2, 128, "bf16", 16, (70, 150), (1, 5), True), None),
    # MB = 2 (100 rows), 50 beams x 8 tasks = 400 <= 512: prologue
    "mb2_d64_g2_early": (BeamConfig("tw3", 2, 50, 4, 2, 64, "f16", 16, (70, 150), (1, 5), True), None),
    # MB = 2 (128 rows), 64 beams x 8 tasks = 512 = 256 x 2: prologue
    "mb2_d64_g2_at_limit": (BeamConfig("tw4", 2, 64, 4, 2, 64, "bf16", 16, (70, 150), (1, 5), False), None),
    # head_dim 256 (MB = 1): loaded at the end
    "mb1_d256_late": (BeamConfig("tw5", 2, 30, 4, 2, 256, "bf16", 16, (70, 150), (1, 5), True), None),
    # a split request (chunks of 64 keys): loaded at the end by the finishing chunk
    "mb1_d128_split": (BeamConfig("tw6", 2, 30, 4, 2, 128, "bf16", 16, (150, 300), (1, 5), True), 64),
}


@pytest.mark.parametrize("case", list(TOKEN_ROW_CASES))
def test_decode_step_token_rows_early_and_late(case, monkeypatch):
    cfg, split = TOKEN_ROW_CASES[case]
    if split is not None:
        monkeypatch.setenv("BSP_SPLIT", str(split))
    inp = synth.make_beam_step(cfg, 13)
    say(f"fused token rows {case} P={inp.prefix_len.tolist()} T={inp.tail_len.tolist()}")
    assert (inp.tail_len > 0).all()  # every beam writes its current token
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    items = B.bsp_debug_plan_items(s.plan)
    assert (items[:, 3] > 1).any() == (split is not None), items
    S.run_decode_step(s)
    B.bsp_check(s.plan)
    torch.cuda.synchronize()
    ref = _applied(inp)
    assert torch.equal(s.k_pool.cpu(), S.to_device(ref.k_pool, inp.dtype, "cpu")), case
    assert torch.equal(s.v_pool.cpu(), S.to_device(ref.v_pool, inp.dtype, "cpu")), case
    fo, fl = oracle.beam_decode_attention(ref)
    say(f"  max |dO| = {assert_close(s.out, s.lse_out, fo, fl, inp.dtype, case):.3g}")


@pytest.mark.parametrize("case", list(GROUP_CASES))
def test_decode_step_group_sizes(case):
    g, dt = GROUP_CASES[case]
    cfg = BeamConfig(case, 2, 7, 2 * g, 2, 128, dt, 16, (70, 150), (0, 5), True)
    say(f"fused group size {g} {dt}")
    _run_fused_and_check(synth.make_beam_step(cfg, 12), case)


@pytest.mark.parametrize("G,W,dt", [(5, 90, "bf16"), (4, 100, "f16"), (2, 150, "bf16")])
def test_decode_step_query_tiles(G, W, dt):
    """W * G above one workgroup's 192 rows: several query tiles per (request, KV head),
    beams straddling tiles when 192 % G != 0; every token written exactly once."""
    cfg = BeamConfig("qtiles", 2, W, 2 * G, 2, 64, dt, 16, (40, 90), (1, 6), True)
    inp = synth.make_beam_step(cfg, 3)
    say(f"fused query tiles G={G} W={W} rows={W * G}")
    _run_fused_and_check(inp, f"qtiles G={G}")


def test_decode_step_long_tails_resolved_on_the_fly():
    """More tail slots per tile than the LDS table holds (192 beams x 20 positions)."""
    cfg = BeamConfig("longtail", 1, 192, 2, 2, 64, "bf16", 16, (30, 60), (17, 20), True)
    inp = synth.make_beam_step(cfg, 4)
    say(f"fused long tails T={inp.tail_len.tolist()}")
    _run_fused_and_check(inp, "long tails")


def _growing_scores(inp, tail_dominates=False):
    """Queries along one unit vector and prompt keys growing along it with position,
    so that every 32-key tile raises the row max by more than 2^8 (the online
    softmax must rescale on every tile); optionally current tokens far above the
    prompt, so the rescale also happens inside the tail."""
    D, ps = inp.head_dim, inp.page_size
    u = np.full(D, 1.0 / np.sqrt(D), np.float32)
    inp.q[...] = u
    for b in range(inp.batch):
        for j in range(int(inp.prefix_len[b])):
            page = inp.block_tables[b, 0, j // ps]
            inp.k_pool[page, :, j % ps, :] = u * (0.5 + 2.5 * j)
    if tail_dominates:
        inp.k_new[...] = u * (2.5 * inp.prefix_len.max() + 400.0)
    for a in (inp.q, inp.k_pool, inp.k_new):
        synth.round_to_dtype(a, inp.dtype, inplace=True)
    return inp


@pytest.mark.parametrize("cfg,batch", [("qwen3_0p6b", 2), ("wide_beam", 1), ("qwen3_4b", 1)])
@pytest.mark.parametrize("tail_dominates", [False, True])
def test_decode_step_rescales_on_every_tile(cfg, batch, tail_dominates):
    """The lazy running-max update taken on every prompt tile (and in the tail)."""
    inp = _growing_scores(synth.make_beam_step(cfg, 5, batch=batch, tail_range=(2, 4)), tail_dominates)
    say(f"fused growing scores {cfg} tail_dominates={tail_dominates} P={inp.prefix_len.tolist()}")
    _run_fused_and_check(inp, f"growing scores {cfg}")


def test_decode_step_rejects_unsupported():
    inp = synth.make_beam_step("tiny", 0)
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    with pytest.raises(B.BspError) as ei:
        S.run_decode_step(s)
    assert ei.value.name == "BSP_ERR_UNSUPPORTED"


def test_decode_step_bad_parent_is_skipped_and_reported():
    inp = synth.make_beam_step("qwen3_0p6b", 6, batch=2, tail_range=(3, 4))
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    P = int(inp.prefix_len[0])
    s.cache_indirection[0, 2, P] = -3
    S.run_decode_step(s)
    with pytest.raises(B.BspError) as ei:
        B.bsp_check(s.plan)
    assert ei.value.name == "BSP_ERR_DEVICE_INDEX"
    assert not torch.isnan(s.out.float()).any()


def test_full_size_nsample_fused_sampled():
    """64 prompts x 16 parallel samples (own tails of 8-32 tokens), the fused step."""
    inp = synth.make_beam_step("nsample", 0, garbage="unit")
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    S.run_decode_step(s)
    B.bsp_check(s.plan)
    torch.cuda.synchronize()
    ref = _applied(inp)
    rng = np.random.default_rng(2)
    W = inp.beam
    picks = [(int(b), int(k)) for b, k in zip(rng.integers(0, inp.batch, 10), rng.integers(0, W, 10))]
    picks += [(0, 0), (inp.batch - 1, W - 1)]
    out = s.out.float().cpu().numpy().reshape(inp.batch, W, inp.num_q_heads, inp.head_dim)
    lse = s.lse_out.cpu().numpy().reshape(inp.batch, W, inp.num_q_heads)
    to, tl = TOL["bf16"]
    for b, k in picks:
        fo, fl = oracle.beam_attention_one(ref, b, k)
        assert np.abs(out[b, k] - fo[0]).max() <= to, (b, k)
        assert np.abs(lse[b, k] - fl[0]).max() <= tl, (b, k)


def test_full_size_wide_beam_fused_sampled():
    """128 requests x 96 beams, bf16, shuffled pages, the fused step the bench times."""
    inp = synth.make_beam_step("wide_beam", 0, garbage="unit")
    say(f"full-size wide_beam: pages={inp.num_pages}")
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    S.run_decode_step(s)
    B.bsp_check(s.plan)
    torch.cuda.synchronize()
    ref = _applied(inp)
    rng = np.random.default_rng(1)
    picks = [(int(b), int(k)) for b, k in zip(rng.integers(0, 128, 12), rng.integers(0, 96, 12))]
    picks += [(0, 0), (127, 95)]
    out = s.out.float().cpu().numpy().reshape(128, 96, 16, 128)
    lse = s.lse_out.cpu().numpy().reshape(128, 96, 16)
    to, tl = TOL["bf16"]
    for b, k in picks:
        fo, fl = oracle.beam_attention_one(ref, b, k)
        assert np.abs(out[b, k] - fo[0]).max() <= to
        assert np.abs(lse[b, k] - fl[0]).max() <= tl


# ------------------------------------ split prompts in the fused step

SPLIT_CASES = {
    "odd_spread_bf16": (dict(cfg="qwen3_0p6b", batch=7, prefix_range=(0, 1200)), 128),
    "two_bf16": (dict(cfg="qwen3_0p6b", batch=2, prefix_range=(32, 1500)), 192),
    "equal_bf16": (dict(cfg="qwen3_0p6b", batch=4, prefix_range=(512, 512)), 256),
    "no_tails_bf16": (dict(cfg="qwen3_0p6b", batch=4, prefix_range=(0, 900), tail_range=(0, 0)), 64),
    "mb2_d128_f16": (dict(cfg="qwen3_4b", batch=5, prefix_range=(64, 3000)), 512),
    "mb2_d64_f16": (dict(cfg="qwen3_4b", batch=4, head_dim=64, prefix_range=(100, 2400)), 320),
    "mb3_wide_bf16": (dict(cfg="wide_beam", batch=3, prefix_range=(100, 1000)), 256),
    "d256_f16": (dict(cfg="qwen3_4b", batch=3, head_dim=256, prefix_range=(100, 900)), 128),
    "nsample_bf16": (dict(cfg="nsample", batch=5, prefix_range=(30, 1000)), 128),
    "query_tiles_bf16": (dict(cfg=BeamConfig("qt", 2, 90, 10, 2, 64, "bf16", 16, (40, 400), (1, 6), True)), 64),
    "long_tails_bf16": (dict(cfg=BeamConfig("lt", 1, 192, 2, 2, 64, "bf16", 16, (100, 300), (17, 20), True)), 64),
    "page_size_1_bf16": (dict(cfg=BeamConfig("p1", 2, 6, 4, 2, 128, "bf16", 1, (40, 400), (1, 5), True)), 64),
}


@pytest.mark.parametrize("case", list(SPLIT_CASES))
def test_decode_step_split_prompts(case, monkeypatch):
    """Prompts split into chunks (BSP_SPLIT forces the chunk): each chunk's
    workgroup leaves its partial state and the last to arrive merges them and
    finishes the request. Two launches in a row match the oracle (the last
    arrival resets each counter for the next launch), the token write is
    bit-exact, and the same step unsplit matches too."""
    kw, chunk = dict(SPLIT_CASES[case][0]), SPLIT_CASES[case][1]
    cfg = kw.pop("cfg")
    monkeypatch.setenv("BSP_SPLIT", str(chunk))
    inp = synth.make_beam_step(cfg, 5, **kw)
    P = inp.prefix_len
    say(f"split {case} chunk={chunk} P={P.tolist()} T={inp.tail_len.tolist()}")
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    items = B.bsp_debug_plan_items(s.plan)
    assert (items[:, 3] > 1).any(), items
    say(f"  items={len(items)} split={(items[:, 3] > 1).sum()}")
    ref = _applied(synth.make_beam_step(cfg, 5, **kw))
    fo, fl = oracle.beam_decode_attention(ref)
    outs = []
    for rep in range(2):
        S.run_decode_step(s)
        B.bsp_check(s.plan)
        torch.cuda.synchronize()
        err = assert_close(s.out, s.lse_out, fo, fl, inp.dtype, f"{case} launch {rep}")
        say(f"  launch {rep}: max |dO| = {err:.3g}")
        outs.append((s.out.clone(), s.lse_out.clone()))
    # the merge runs in chunk order, whichever chunk arrives last: launches agree bit for bit
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(s.k_pool.cpu(), S.to_device(ref.k_pool, inp.dtype, "cpu")), case
    assert torch.equal(s.v_pool.cpu(), S.to_device(ref.v_pool, inp.dtype, "cpu")), case

    monkeypatch.setenv("BSP_SPLIT", "0")
    s2 = S.upload_beam_step(synth.make_beam_step(cfg, 5, **kw), DEV)
    S.plan_beam_step(s2)
    assert (B.bsp_debug_plan_items(s2.plan)[:, 3] == 1).all()
    S.run_decode_step(s2)
    B.bsp_check(s2.plan)
    torch.cuda.synchronize()
    assert_close(s2.out, s2.lse_out, fo, fl, inp.dtype, f"{case} unsplit")


def test_decode_step_split_replanned_between_launches(monkeypatch):
    """One plan and workspace, re-planned between launches for batches of
    different sizes (so the split, the items and the counters' layout change):
    every step matches the oracle."""
    kw = dict(batch=5, prefix_range=(100, 1400))
    ref = _applied(synth.make_beam_step("qwen3_0p6b", 9, **kw))
    fo, fl = oracle.beam_decode_attention(ref)
    monkeypatch.setenv("BSP_SPLIT", "128")
    inp = synth.make_beam_step("qwen3_0p6b", 9, **kw)
    s = S.upload_beam_step(inp, DEV)
    W = inp.beam
    for nb in (5, 3, 5, 2):
        B.bsp_plan(s.plan, nb, W, 1, inp.prefix_len[:nb], inp.seq_len[:nb],
                   np.ascontiguousarray(inp.block_tables[:nb]), s.workspace)
        assert (B.bsp_debug_plan_items(s.plan)[:, 3] > 1).any()
        S.run_decode_step(s)
        B.bsp_check(s.plan)
        torch.cuda.synchronize()
        rows = nb * W
        assert_close(s.out[:rows], s.lse_out[:rows], fo[:nb], fl[:nb], "bf16",
                     f"re-planned batch of {nb}")


@pytest.mark.parametrize("cfg,split_env", [("qwen3_0p6b", None), ("qwen3_0p6b", "256"),
                                           ("qwen3_4b", None), ("qwen3_4b", "512"),
                                           ("wide_beam", "1024")])
def test_full_size_fused_sampled(cfg, split_env, monkeypatch):
    """The bench's full shapes through the fused step, as planned (no split at
    these prompt spreads) and with every prompt split that the plan's partial-
    state reserve allows; sampled beams against the oracle."""
    if split_env is not None:
        monkeypatch.setenv("BSP_SPLIT", split_env)
    else:
        monkeypatch.delenv("BSP_SPLIT", raising=False)
    inp = synth.make_beam_step(cfg, 0, garbage="unit")
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    items = B.bsp_debug_plan_items(s.plan)
    n_split = int((items[:, 3] > 1).sum())
    say(f"full-size fused {cfg}: items={len(items)} split items={n_split}")
    assert (n_split > 0) == (split_env is not None)
    S.run_decode_step(s)
    B.bsp_check(s.plan)
    torch.cuda.synchronize()
    ref = _applied(inp)
    rng = np.random.default_rng(3)
    W, Hq, D = inp.beam, inp.num_q_heads, inp.head_dim
    split_reqs = sorted({int(b) for b, lo, hi, n in items if n > 1})
    a, b = int(np.argmax(inp.prefix_len)), int(np.argmin(inp.prefix_len))
    picks = [(a, 0), (a, W - 1), (b, 1)]
    picks += [(r, int(rng.integers(0, W))) for r in split_reqs[:4]]
    picks += [(int(x), int(k)) for x, k in zip(rng.integers(0, inp.batch, 8), rng.integers(0, W, 8))]
    out = s.out.float().cpu().numpy().reshape(inp.batch, W, Hq, D)
    lse = s.lse_out.cpu().numpy().reshape(inp.batch, W, Hq)
    to, tl = TOL[inp.dtype]
    for x, k in picks:
        fo, fl = oracle.beam_attention_one(ref, x, k)
        assert np.abs(out[x, k] - fo[0]).max() <= to, (x, k)
        assert np.abs(lse[x, k] - fl[0]).max() <= tl, (x, k)


@pytest.mark.parametrize("cfg,batch", [("qwen3_4b", 96), ("qwen3_4b_d64", 140), ("qwen3_0p6b", 128)])
def test_fused_step_above_the_streaming_limit(cfg, batch):
    """A step whose outputs, LSE and token rows exceed 24 MiB is written with
    plain stores instead of streaming ones (one and two query blocks per wave):
    the token rows bit-exact, sampled beams against the oracle."""
    inp = synth.make_beam_step(cfg, 2, batch=batch, prefix_range=(100, 300), tail_range=(1, 4))
    W, Hq, Hkv, D = inp.beam, inp.num_q_heads, inp.num_kv_heads, inp.head_dim
    rows = inp.batch * W
    writes = rows * Hq * (2 * D + 4) + rows * Hkv * D * 2 * 2
    assert writes > 24 << 20, writes
    say(f"large writes {cfg} batch={batch}: {writes / 2**20:.1f} MiB")
    s = S.upload_beam_step(inp, DEV)
    S.plan_beam_step(s)
    S.run_decode_step(s)
    B.bsp_check(s.plan)
    torch.cuda.synchronize()
    ref = _applied(inp)
    assert torch.equal(s.k_pool.cpu(), S.to_device(ref.k_pool, inp.dtype, "cpu")), cfg
    assert torch.equal(s.v_pool.cpu(), S.to_device(ref.v_pool, inp.dtype, "cpu")), cfg
    rng = np.random.default_rng(5)
    out = s.out.float().cpu().numpy().reshape(inp.batch, W, Hq, D)
    lse = s.lse_out.cpu().numpy().reshape(inp.batch, W, Hq)
    to, tl = TOL[inp.dtype]
    picks = [(0, 0), (inp.batch - 1, W - 1)]
    picks += [(int(x), int(k)) for x, k in zip(rng.integers(0, inp.batch, 10), rng.integers(0, W, 10))]
    for x, k in picks:
        fo, fl = oracle.beam_attention_one(ref, x, k)
        assert np.abs(out[x, k] - fo[0]).max() <= to, (x, k)
        assert np.abs(lse[x, k] - fl[0]).max() <= tl, (x, k)


# ------------------------------------------------- degenerate shapes, fused

@pytest.mark.parametrize("name,cfg", [
    # every prompt empty: only the tails are attended
    ("empty_prompts", BeamConfig("e0", 3, 5, 4, 2, 128, "bf16", 16, (0, 0), (1, 6), True)),
    # one request, one beam, MHA (group 1), prompt inside one page
    ("single_mha", BeamConfig("s1", 1, 1, 2, 2, 64, "f16", 32, (1, 20), (1, 1), False)),
    # one-row pages: every key tile spans 32 pages
    ("page_size_1", BeamConfig("p1", 2, 6, 4, 2, 128, "bf16", 1, (40, 200), (1, 5), True)),
    # 1024-row pages: a prompt in one page
    ("page_size_1024", BeamConfig("p1k", 2, 6, 8, 2, 128, "f16", 1024, (300, 900), (1, 5), True)),
])
def test_decode_step_degenerate_shapes(name, cfg):
    inp = synth.make_beam_step(cfg, 21)
    say(f"fused {name} P={inp.prefix_len.tolist()} T={inp.tail_len.tolist()}")
    _run_fused_and_check(inp, name)


def test_plan_returns_without_waiting_for_queued_work():
    """Re-planning stages its tables in pinned host memory and copies them with
    an asynchronous copy ordered on the stream: with about a second of work
    queued ahead on the same stream, two bsp_plan calls (one per staging
    buffer) return while that work still runs, and the step planned behind it
    gives the same output as before."""
    import time
    beam = S.upload_beam_step(synth.make_beam_step("qwen3_0p6b", 5, batch=8), DEV)
    S.plan_beam_step(beam)
    S.run_decode_step(beam)
    B.bsp_check(beam.plan)
    torch.cuda.synchronize()
    ref = beam.out.clone()
    stream = torch.cuda.current_stream()
    x = torch.randn(4096, 4096, device=DEV)
    y = x @ x
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    y = x @ x
    torch.cuda.synchronize()
    one = time.perf_counter() - t0
    n = max(20, min(2000, int(1.0 / max(one, 1e-5))))  # about a second of matrix products
    for _ in range(n):
        y = x @ y * 1e-3
    queued_at = time.perf_counter()
    plan_s = []
    for _ in range(2):
        t0 = time.perf_counter()
        S.plan_beam_step(beam)
        plan_s.append(time.perf_counter() - t0)
    busy = not stream.query()
    say(f"{n} products of {one * 1e3:.2f} ms queued; plan calls {[round(t * 1e3, 3) for t in plan_s]} ms; "
        f"stream busy after them: {busy} ({(time.perf_counter() - queued_at) * 1e3:.1f} ms after queueing)")
    assert busy, "the queued products finished before the plans returned: no evidence either way"
    assert max(plan_s) < 0.1 * n * one
    S.run_decode_step(beam)
    B.bsp_check(beam.plan)
    torch.cuda.synchronize()
    assert torch.equal(beam.out, ref)
