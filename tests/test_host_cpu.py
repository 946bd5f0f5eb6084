"""CPU tier for libbsp: the library loads and exports every declared symbol, and
the host planner (no HIP calls in host-only mode) builds the oracle's page
tables bit for bit and returns the documented status for every host-forcible
error. No kernel is launched here."""

import ctypes
import re
import json
import os

import numpy as np
import pytest

import oracle
import synth
from beam_search_shared_amd import _binding as B
from synth import BeamConfig


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = B.declared_symbols()
    assert len(names) >= 14
    for name in ["bsp_plan_create", "bsp_plan", "bsp_write_kv", "bsp_prefix_attn",
                 "bsp_tail_attn", "bsp_merge", "bsp_check", "bsp_last_error"]:
        assert name in names
    for name in names:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value
    assert lib.bsp_version() >= 100


def _c_kind(decl: str) -> str:
    """The ctypes kind a C parameter or return type maps to."""
    decl = decl.strip()
    if "*" in decl or decl.split()[0] in ("bsp_plan_t", "hipStream_t"):
        return "char*" if decl.replace(" ", "").startswith("constchar*") else "ptr"
    base = decl.replace("const ", "").split()[0]
    return {"bsp_status_t": "i32", "int32_t": "i32", "int64_t": "i64", "uint32_t": "u32",
            "size_t": "size", "void": "void"}[base]


def _ctypes_kind(t) -> str:
    if t is None:
        return "void"
    if t is ctypes.c_char_p:
        return "char*"
    if t is ctypes.c_void_p or (isinstance(t, type) and issubclass(t, ctypes._Pointer)):
        return "ptr"
    return {ctypes.c_int32: "i32", ctypes.c_int64: "i64", ctypes.c_uint32: "u32",
            ctypes.c_size_t: "size"}[t]


def test_binding_signatures_match_the_header():
    """Every function include/bsp.h declares has a binding entry whose return and
    argument kinds (pointer, int32, int64, uint32, size_t) match the declaration
    one for one, so a drifted argument list fails here instead of at a call."""
    text = open(B.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    decls = re.findall(r"^[ \t]*([A-Za-z_][\w \t\*]*?)\b(bsp_\w+)\s*\(([^;{]*?)\)\s*;", text,
                       flags=re.M)
    assert len(decls) == len(B.declared_symbols())
    for ret, name, args in decls:
        assert name in B._SIGS, f"{name} has no binding"
        res, argtypes = B._SIGS[name]
        params = [] if args.strip() in ("", "void") else [x for x in args.split(",")]
        kinds = [_c_kind(x.rsplit(None, 1)[0] if not x.strip().endswith("*") else x) for x in params]
        assert [_ctypes_kind(t) for t in argtypes] == kinds, name
        assert _ctypes_kind(res) == _c_kind(ret), name


def _host_plan(inp, max_tail=0, key_bucket=0, max_cache_rows=0):
    desc = B.make_desc(inp.num_q_heads, inp.num_kv_heads, inp.head_dim, inp.page_size,
                       inp.num_pages, inp.dtype, max_tail=max_tail, key_bucket=key_bucket,
                       max_cache_rows=max_cache_rows)
    return B.Plan(desc, inp.batch, inp.beam, inp.max_blocks, inp.max_seq_len, 1, host_only=True)


def _check_plan_against_oracle(inp, plan):
    B.bsp_plan(plan, inp.batch, inp.beam, 1, inp.prefix_len, inp.seq_len, inp.block_tables)
    indptr, pages, n_keys, valid, tail = B.bsp_debug_plan_tables(plan, inp.batch)
    o_indptr, o_pages = oracle.prefix_page_table(inp.prefix_len, inp.block_tables, inp.page_size)
    assert np.array_equal(indptr, o_indptr) and np.array_equal(pages, o_pages)
    assert np.array_equal(n_keys, inp.prefix_len) and np.array_equal(valid, inp.prefix_len)
    assert np.array_equal(tail, inp.seq_len - inp.prefix_len)


def test_planner_matches_oracle_on_1200_random_batches():
    rng = np.random.default_rng(1234)
    for trial in range(1200):
        ps = int(rng.choice([1, 2, 4, 8, 16, 32]))
        cfg = BeamConfig("rand", batch=int(rng.integers(1, 5)), beam=int(rng.integers(1, 6)),
                         num_q_heads=2, num_kv_heads=1, head_dim=64, dtype="f32", page_size=ps,
                         prefix_range=(0, int(rng.integers(1, 70))),
                         tail_range=(0, int(rng.integers(0, 9))),
                         shuffle_pages=bool(rng.integers(0, 2)))
        inp = synth.make_beam_step(cfg, trial, page_stride=int(rng.integers(1, 3)))
        inp.k_pool = inp.v_pool = None  # not needed on the host
        _check_plan_against_oracle(inp, _host_plan(inp))


def test_planner_golden_page_tables(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "prefix_pages.json")))
    ps = g["page_size"]
    cases = g["cases"]
    Bn, W, nb = len(cases), 3, 5
    bt = np.array([[[100 * r + 10 * k + i for i in range(nb)] for k in range(W)]
                   for r in range(Bn)], dtype=np.int32)
    P = np.array([c["prefix_len"] for c in cases], np.int32)
    desc = B.make_desc(2, 1, 64, ps, 1000, "bf16")
    plan = B.Plan(desc, Bn, W, nb, nb * ps, 1, host_only=True)
    B.bsp_plan(plan, Bn, W, 1, P, P, bt)
    indptr, pages, n_keys, _, _ = B.bsp_debug_plan_tables(plan, Bn)
    for r, c in enumerate(cases):
        assert pages[indptr[r]:indptr[r + 1]].tolist() == c["expected_pages"]
        assert n_keys[r] == c["expected_keys"]


def test_planner_bucket_rows_match_printed_rule(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "bucket_rows.json")))
    cap, gran, ps = g["cap"], g["granularity"], 32
    L = np.array([c[0] for c in g["rule_256_cases"]], np.int32)
    nb = cap // ps
    bt = np.tile(np.arange(nb, dtype=np.int32), (len(L), 1, 1))
    desc = B.make_desc(24, 8, 128, ps, nb, "f16", key_bucket=gran, max_cache_rows=cap)
    plan = B.Plan(desc, len(L), 1, nb, cap, 1, host_only=True)
    B.bsp_plan(plan, len(L), 1, 1, L, L, bt)
    _, _, n_keys, valid, _ = B.bsp_debug_plan_tables(plan, len(L))
    assert n_keys.tolist() == [c[1] for c in g["rule_256_cases"]]
    assert n_keys.tolist() == [oracle.bucket_rows(int(x), gran, cap) for x in L]
    assert valid.tolist() == L.tolist()


PLAN_CFG = BeamConfig("errs", batch=3, beam=4, num_q_heads=4, num_kv_heads=2, head_dim=64,
                      dtype="bf16", page_size=8, prefix_range=(9, 30), tail_range=(1, 5),
                      shuffle_pages=False)


def _status(fn):
    with pytest.raises(B.BspError) as ei:
        fn()
    return ei.value.name, str(ei.value)


def test_plan_rejects_bad_prompt_page_without_clamping():
    inp = synth.make_beam_step(PLAN_CFG, 0)
    plan = _host_plan(inp)
    bt = inp.block_tables.copy()
    bt[1, 0, 0] = inp.num_pages  # one past the pool
    name, msg = _status(lambda: B.bsp_plan(plan, inp.batch, inp.beam, 1, inp.prefix_len,
                                           inp.seq_len, bt))
    assert name == "BSP_ERR_PAGE_INDEX" and "request 1" in msg
    bt[1, 0, 0] = -1
    assert _status(lambda: B.bsp_plan(plan, inp.batch, inp.beam, 1, inp.prefix_len,
                                      inp.seq_len, bt))[0] == "BSP_ERR_PAGE_INDEX"


def test_plan_rejects_bad_tail_page_of_any_beam():
    inp = synth.make_beam_step(PLAN_CFG, 1)
    plan = _host_plan(inp)
    bt = inp.block_tables.copy()
    b = 2
    last_blk = (int(inp.seq_len[b]) - 1) // inp.page_size
    bt[b, 3, last_blk] = inp.num_pages + 7
    assert _status(lambda: B.bsp_plan(plan, inp.batch, inp.beam, 1, inp.prefix_len,
                                      inp.seq_len, bt))[0] == "BSP_ERR_PAGE_INDEX"


def test_plan_tail_overflow_in_fixed_mode():
    inp = synth.make_beam_step(PLAN_CFG, 2)
    T = int((inp.seq_len - inp.prefix_len).max())
    ok = _host_plan(inp, max_tail=T)
    B.bsp_plan(ok, inp.batch, inp.beam, 1, inp.prefix_len, inp.seq_len, inp.block_tables)
    assert ok.tail_len == T
    bad = _host_plan(inp, max_tail=T - 1)
    name, msg = _status(lambda: B.bsp_plan(bad, inp.batch, inp.beam, 1, inp.prefix_len,
                                           inp.seq_len, inp.block_tables))
    assert name == "BSP_ERR_TAIL_OVERFLOW" and str(T) in msg


def test_plan_length_checks_and_stale_plan():
    inp = synth.make_beam_step(PLAN_CFG, 3)
    plan = _host_plan(inp)
    B.bsp_plan(plan, inp.batch, inp.beam, 1, inp.prefix_len, inp.seq_len, inp.block_tables)
    assert plan.num_splits == 1
    P = inp.prefix_len.copy()
    P[0] = inp.seq_len[0] + 1  # prefix longer than the sequence
    assert _status(lambda: B.bsp_plan(plan, inp.batch, inp.beam, 1, P, inp.seq_len,
                                      inp.block_tables))[0] == "BSP_ERR_ARG"
    # the failed call dropped the previous plan
    assert plan.num_splits == -1
    assert _status(lambda: B.bsp_debug_plan_tables(plan, inp.batch))[0] == "BSP_ERR_STALE_PLAN"
    S = inp.seq_len.copy()
    S[1] = inp.max_seq_len + 1
    assert _status(lambda: B.bsp_plan(plan, inp.batch, inp.beam, 1, inp.prefix_len, S,
                                      inp.block_tables))[0] == "BSP_ERR_ARG"
    assert _status(lambda: B.bsp_plan(plan, inp.batch + 1, inp.beam, 1, inp.prefix_len,
                                      inp.seq_len, inp.block_tables))[0] == "BSP_ERR_ARG"


def test_kernel_entry_points_refuse_unplanned_plan_before_any_launch():
    inp = synth.make_beam_step(PLAN_CFG, 4)
    plan = _host_plan(inp)
    fake = 1 << 20  # never dereferenced: the status is returned before any launch
    assert _status(lambda: B.bsp_prefix_attn(plan, fake, fake, fake, fake, fake, stream=0))[0] \
        == "BSP_ERR_STALE_PLAN"
    assert _status(lambda: B.bsp_tail_attn(plan, fake, fake, fake, fake, fake, fake, fake,
                                           stream=0))[0] == "BSP_ERR_STALE_PLAN"
    assert _status(lambda: B.bsp_write_kv(plan, fake, fake, 128, fake, 1, fake, fake,
                                          stream=0))[0] == "BSP_ERR_STALE_PLAN"
    B.bsp_plan(plan, inp.batch, inp.beam, 1, inp.prefix_len, inp.seq_len, inp.block_tables)
    # a host-only plan never launches
    assert _status(lambda: B.bsp_prefix_attn(plan, fake, fake, fake, fake, fake, stream=0))[0] \
        == "BSP_ERR_ARG"


def test_prefix_attn_two_checks_its_plans_before_any_launch():
    inp = synth.make_beam_step(PLAN_CFG, 5)
    a, b = _host_plan(inp), _host_plan(inp)
    fake = 1 << 20  # never dereferenced: the status is returned before any launch
    two = lambda x, y: _status(lambda: B.bsp_prefix_attn_two(  # noqa: E731
        x, y, fake, fake, fake, fake, fake, fake, fake, stream=0))[0]
    assert two(a, a) == "BSP_ERR_ARG"                   # the same plan twice
    assert two(a, b) == "BSP_ERR_STALE_PLAN"            # neither planned
    B.bsp_plan(b, inp.batch, inp.beam, 1, inp.prefix_len, inp.seq_len, inp.block_tables)
    assert two(a, b) == "BSP_ERR_STALE_PLAN"            # the first not planned
    B.bsp_plan(a, inp.batch, inp.beam, 1, inp.prefix_len, inp.seq_len, inp.block_tables)
    assert two(a, b) == "BSP_ERR_ARG"                   # host-only plans never launch


def test_plan_create_rejects_bad_geometry():
    def create(**kw):
        base = dict(num_q_heads=4, num_kv_heads=2, head_dim=128, page_size=32, num_pages=10,
                    dtype="bf16")
        base.update(kw)
        return B.Plan(B.make_desc(**base), 1, 1, 4, 100, 1, host_only=True)
    assert _status(lambda: create(head_dim=96))[0] == "BSP_ERR_UNSUPPORTED"
    assert _status(lambda: create(page_size=24))[0] == "BSP_ERR_UNSUPPORTED"
    assert _status(lambda: create(num_q_heads=3))[0] == "BSP_ERR_ARG"
    assert _status(lambda: create(kv_split=100))[0] == "BSP_ERR_ARG"
    bad = B.make_desc(4, 2, 128, 32, 10, "bf16")
    bad.dtype = 7
    assert _status(lambda: B.Plan(bad, 1, 1, 4, 100, 1, host_only=True))[0] == "BSP_ERR_DTYPE"
    assert _status(lambda: B.Plan(B.make_desc(4, 2, 128, 32, 10, "bf16"), 1, 1, 2, 100, 1,
                                  host_only=True))[0] == "BSP_ERR_ARG"


def test_write_kv_desc_checks_before_any_launch(lib):
    """bsp_write_kv_desc validates the descriptor and arguments on the host and
    returns a status before any launch; n == 0 succeeds without one."""
    fake = 1 << 20
    d = B.make_desc(4, 2, 128, 32, 10, "bf16")

    def call(desc, n=4, stride=256, k=fake, faults=None):
        return B.bsp_write_kv_desc(desc, k, fake, stride, fake, n, fake, fake, faults, stream=0)
    assert _status(lambda: B.bsp_write_kv_desc(None, fake, fake, 256, fake, 4, fake, fake,
                                               stream=0))[0] == "BSP_ERR_ARG"
    bad = B.make_desc(4, 2, 128, 32, 10, "bf16")
    bad.dtype = 7
    assert _status(lambda: call(bad))[0] == "BSP_ERR_DTYPE"
    assert _status(lambda: call(B.make_desc(4, 2, 96, 32, 10, "bf16")))[0] == "BSP_ERR_UNSUPPORTED"
    assert _status(lambda: call(B.make_desc(4, 2, 128, 24, 10, "bf16")))[0] == "BSP_ERR_UNSUPPORTED"
    assert _status(lambda: call(B.make_desc(4, 2, 128, 32, 0, "bf16")))[0] == "BSP_ERR_ARG"
    assert _status(lambda: call(d, n=-1))[0] == "BSP_ERR_ARG"
    assert _status(lambda: call(d, stride=255))[0] == "BSP_ERR_ARG"   # < Hkv * D
    assert _status(lambda: call(d, k=fake + 2))[0] == "BSP_ERR_ARG"   # misaligned
    assert _status(lambda: call(d, k=0))[0] == "BSP_ERR_ARG"          # null
    assert _status(lambda: call(d, faults=fake + 2))[0] == "BSP_ERR_ARG"
    call(d, n=0)  # nothing to write: no launch


def test_merge_argument_checks(lib):
    fake = 1 << 20
    assert _status(lambda: B.bsp_merge(4, 2, 6, 2, fake, fake, 48, 8, fake, "bf16",
                                       stream=0))[0] == "BSP_ERR_ARG"  # head_dim % 4
    assert _status(lambda: B.bsp_merge(4, 2, 8, 2, fake, fake, 10, 8, fake, "bf16",
                                       stream=0))[0] == "BSP_ERR_ARG"  # stride < part
    B.bsp_merge(0, 2, 8, 2, fake, fake, 64, 8, fake, "bf16", stream=0)  # empty: no launch


def test_check_mode_requires_shared_prompt_blocks(monkeypatch):
    monkeypatch.setenv("BSP_CHECK", "1")
    inp = synth.make_beam_step(PLAN_CFG, 5, prefix_range=(24, 30))
    plan = _host_plan(inp)
    B.bsp_plan(plan, inp.batch, inp.beam, 1, inp.prefix_len, inp.seq_len, inp.block_tables)
    bt = inp.block_tables.copy()
    bt[0, 2, 0] = bt[0, 0, 1]  # beam 2 no longer shares prompt block 0
    name, msg = _status(lambda: B.bsp_plan(plan, inp.batch, inp.beam, 1, inp.prefix_len,
                                           inp.seq_len, bt))
    assert name == "BSP_ERR_ARG" and "share prompt block" in msg


# ------------------------------------- fused-step work items and splits (host plan)

def _item_plan(B_, W, G, D, dtype, prefix, key_bucket=0, hkv=8, tails=3):
    ps = 32
    nb = -(-(max(prefix) + 8) // ps)
    desc = B.make_desc(hkv * G, hkv, D, ps, 1 << 20, dtype, key_bucket=key_bucket,
                       max_cache_rows=nb * ps if key_bucket else 0)
    plan = B.Plan(desc, B_, W, nb, nb * ps, 1, host_only=True)
    P = np.asarray(prefix, np.int32)
    bt = np.arange(B_ * W * nb, dtype=np.int32).reshape(B_, W, nb) % (1 << 20)
    bt[:, :, :] = bt[:, :1, :]  # every beam shares its request's blocks
    S = P if key_bucket else P + np.asarray(tails, np.int32)
    B.bsp_plan(plan, B_, W, 1, P, S.astype(np.int32), bt)
    return B.bsp_debug_plan_items(plan)


def _deal_cost(items, P, W, G, D, hkv=8, tails=3):
    """The order items are dealt in: keys, plus W rows per tail position on a
    request's last chunk when the items fill more than one round of 512
    workgroups (per KV head and query tile: 64 rows per 16-row block, up to
    three blocks per wave, one at head_dim 256)."""
    P = np.asarray(P, np.int64)
    T = np.broadcast_to(np.asarray(tails, np.int64), P.shape)
    lens = (items[:, 2] - items[:, 1]).astype(np.int64)
    last = items[:, 2] == P[items[:, 0]]
    return lens + np.where(_several_rounds(items, W, G, D, hkv) & last, W * T[items[:, 0]], 0)


def _several_rounds(items, W, G, D, hkv=8):
    rows = W * G
    mb = min(max(-(-rows // 64), 1), 1 if D == 256 else 3)
    return len(items) > max(1, 512 // (hkv * -(-rows // (64 * mb))))


def _check_items(items, P, chunk=None, *, deal):
    """Each request's items are contiguous, disjoint chunks covering [0, P_b)
    (one item [0, P_b) when unsplit), listed in dealing order by
    `_deal_cost(items, P, *deal)`: longest first over several rounds; in one
    round the longer half longest first, then the shorter half shortest first."""
    cost = _deal_cost(items, P, *deal)
    if _several_rounds(items, *deal[:3], *deal[3:4]):
        assert np.all(np.diff(cost) <= 0), "items must be listed longest first"
    else:
        h = len(cost) // 2
        assert np.all(np.diff(cost[:h]) <= 0) and np.all(np.diff(cost[h:]) >= 0), cost
        assert h == 0 or cost[:h].min() >= cost[h:].max(), cost
    for b, Pb in enumerate(P):
        mine = items[items[:, 0] == b]
        mine = mine[np.argsort(mine[:, 1])]
        n = len(mine)
        assert n >= 1 and np.all(mine[:, 3] == n)
        assert mine[0, 1] == 0 and mine[-1, 2] == Pb
        assert np.all(mine[1:, 1] == mine[:-1, 2])
        if n > 1:
            assert np.all(mine[:, 2] > mine[:, 1])
            if chunk is not None:
                assert np.all(mine[:, 1] % chunk == 0)
                assert np.all(mine[:-1, 2] - mine[:-1, 1] == chunk)


def test_items_cover_every_request_once(monkeypatch):
    """Random batches, unsplit, forced chunks and the automatic choice."""
    rng = np.random.default_rng(7)
    for trial in range(300):
        Bn = int(rng.integers(1, 40))
        P = rng.integers(0, 3000, size=Bn)
        mode = trial % 3
        if mode == 0:
            monkeypatch.setenv("BSP_SPLIT", "0")
        elif mode == 1:
            monkeypatch.setenv("BSP_SPLIT", str(int(rng.integers(1, 1200))))
        else:
            monkeypatch.delenv("BSP_SPLIT", raising=False)
        G = int(rng.choice([1, 2, 4]))
        W = int(rng.integers(1, 40))
        items = _item_plan(Bn, W, G, 128, "bf16", P)
        chunk = None
        if mode == 1:
            chunk = -(-int(__import__("os").environ["BSP_SPLIT"]) // 64) * 64
        _check_items(items, P, chunk, deal=(W, G, 128))
        if mode == 0:
            assert np.all(items[:, 3] == 1) and len(items) == Bn


def test_forced_split_respects_the_partial_state_budget(monkeypatch):
    """A forced split of every prompt goes through the requests longest first and
    splits each one whose chunks still fit the plan's partial-state slots; the
    rest stay whole, and the slots in use never exceed the reserve."""
    monkeypatch.setenv("BSP_SPLIT", "64")
    P = np.arange(64, dtype=np.int32) * 40 + 100
    items = _item_plan(64, 96, 2, 128, "bf16", P)  # three 16-row blocks per wave
    _check_items(items, P, 64, deal=(96, 2, 128))
    split = sorted({int(b) for b, lo, hi, n in items if n > 1})
    assert split and len(split) < 64
    used = sum(-(-int(P[b]) // 64) for b in split)
    slot_bytes = 4 * 256 * (8 * 3 * 4 + 6) * 8   # floats of a 48-row state x 256 threads x 8 heads
    assert used <= (24 << 20) // slot_bytes
    whole = [b for b in range(64) if b not in split]
    # the longest whole request did not fit what was left after the longer ones
    longer = [b for b in split if P[b] > P[max(whole, key=lambda x: P[x])]]
    left = (24 << 20) // slot_bytes - sum(-(-int(P[b]) // 64) for b in longer)
    assert -(-int(P[max(whole, key=lambda x: P[x])]) // 64) > left


@pytest.mark.parametrize("what", ["f32", "cached"])
def test_no_items_where_the_fused_step_does_not_run(what, monkeypatch):
    monkeypatch.setenv("BSP_SPLIT", "64")
    kw = dict(B_=4, W=30, G=2, D=128, dtype="bf16", prefix=[2000, 100, 900, 1500])
    assert len(_item_plan(**kw)) > 4
    if what == "f32":
        kw["dtype"] = "f32"
    else:
        kw.update(key_bucket=64, W=1)
    assert len(_item_plan(**kw)) == 0


@pytest.mark.parametrize("name,prefix,split", [
    ("qwen3_0p6b spread 400-600", ("u", 64, 400, 600), False),
    ("qwen3_4b spread 1600-2400", ("u", 64, 1600, 2400), False),
    ("wide beam spread 2800-3200", ("u", 128, 2800, 3200), False),
    ("spread 200-800", ("u", 64, 200, 800), False),
    ("spread 100-1500", ("u", 64, 100, 1500), True),
    ("four long prompts among short ones", ("few",), True),
    ("empty prompts", ("z",), False),
])
def test_split_chosen_only_where_the_model_gains(name, prefix, split, monkeypatch):
    """Without BSP_SPLIT the plan splits only when its model of the step gets
    at least 5% shorter: not on the bench spreads, yes when a few prompts are
    much longer than the rest."""
    monkeypatch.delenv("BSP_SPLIT", raising=False)
    rng = np.random.default_rng(3)
    if prefix[0] == "u":
        P = rng.integers(prefix[2], prefix[3] + 1, prefix[1])
    elif prefix[0] == "few":
        P = np.full(64, 300)
        P[:4] = 3000
    else:
        P = np.zeros(16, np.int64)
    W, G = (96, 2) if prefix[0] == "u" and prefix[1] == 128 else (30, 2)
    items = _item_plan(len(P), W, G, 128, "bf16", P)
    _check_items(items, P, deal=(W, G, 128))
    assert bool((items[:, 3] > 1).any()) == split, name
    monkeypatch.setenv("BSP_SPLIT", "0")
    assert not (_item_plan(len(P), W, G, 128, "bf16", P)[:, 3] > 1).any()


def test_items_dealt_with_tails_only_over_several_rounds(monkeypatch):
    """Tail rows count in the dealing order only when the items fill more than
    one round: 128 requests x beam 96 (two rounds) with tails 0-8 put a short
    prompt with a long tail ahead of a longer prompt without one; 64 requests
    (one round) are ordered by their prompts alone (longer half first)."""
    monkeypatch.delenv("BSP_SPLIT", raising=False)
    rng = np.random.default_rng(11)
    for Bn in (128, 64):
        P = rng.integers(2800, 3201, Bn)
        T = rng.integers(0, 9, Bn)
        items = _item_plan(Bn, 96, 2, 128, "bf16", P, tails=T)
        assert np.all(items[:, 3] == 1)
        _check_items(items, P, deal=(96, 2, 128, 8, T))
        keys = P[items[:, 0]]
        by_keys = np.all(np.diff(keys) <= 0) or (
            np.all(np.diff(keys[:Bn // 2]) <= 0) and np.all(np.diff(keys[Bn // 2:]) >= 0))
        assert by_keys == (Bn == 64), Bn


# ------------------------------------------------ prefill plans (mixed steps)

def _prefill_host_plan(inp, max_q_len=None):
    desc = B.make_desc(inp.num_q_heads, inp.num_kv_heads, inp.head_dim, inp.page_size,
                       inp.num_pages, inp.dtype)
    return B.Plan(desc, inp.batch, 1, inp.max_blocks, inp.max_seq_len,
                  max_q_len or inp.max_q_len, host_only=True)


@pytest.mark.parametrize("seed", range(5))
def test_prefill_plan_tables(seed):
    """Page CSR from each request's block table over cached + chunk rows, keys
    and query rows per request (bit-exact against the generator's layout)."""
    inp = synth.make_prefill("qwen3_0p6b", seed, batch=5, chunk_range=(1, 300),
                             cached_range=(0, 400), garbage="unit")
    plan = _prefill_host_plan(inp)
    B.bsp_plan_prefill(plan, inp.batch, inp.q_len, inp.cached_len, inp.block_tables)
    indptr, pages, n_keys, valid, tail = B.bsp_debug_plan_tables(plan, inp.batch)
    ps = inp.page_size
    nblk = -(-(inp.cached_len + inp.q_len) // ps)
    assert np.array_equal(np.diff(indptr), nblk)
    want = np.concatenate([inp.block_tables[b, :nblk[b]] for b in range(inp.batch)])
    assert np.array_equal(pages, want)
    assert np.array_equal(n_keys, inp.cached_len + inp.q_len)
    assert np.array_equal(valid, inp.cached_len + inp.q_len)
    assert np.array_equal(tail, inp.q_len)


def test_prefill_plan_rejects_bad_input():
    inp = synth.make_prefill("qwen3_0p6b", 1, batch=3, chunk_range=(1, 50), cached_range=(0, 60),
                             garbage="unit")
    plan = _prefill_host_plan(inp)

    def status(fn):
        try:
            fn()
        except B.BspError as e:
            return e.name
        return "BSP_OK"

    ql = inp.q_len.copy()
    ql[1] = 51  # above max_q_len
    assert status(lambda: B.bsp_plan_prefill(plan, 3, ql, inp.cached_len, inp.block_tables)) == \
        "BSP_ERR_ARG"
    ql[1] = 0
    assert status(lambda: B.bsp_plan_prefill(plan, 3, ql, inp.cached_len, inp.block_tables)) == \
        "BSP_ERR_ARG"
    bt = inp.block_tables.copy()
    bt[2, 0] = inp.num_pages
    assert status(lambda: B.bsp_plan_prefill(plan, 3, inp.q_len, inp.cached_len, bt)) == \
        "BSP_ERR_PAGE_INDEX"
    cl = inp.cached_len.copy()
    cl[0] = inp.max_seq_len
    assert status(lambda: B.bsp_plan_prefill(plan, 3, inp.q_len, cl, inp.block_tables)) == \
        "BSP_ERR_ARG"
    assert status(lambda: B.bsp_plan_prefill(plan, 4, inp.q_len, inp.cached_len,
                                             inp.block_tables)) == "BSP_ERR_ARG"
    B.bsp_plan_prefill(plan, 3, inp.q_len, inp.cached_len, inp.block_tables)


# ------------------------------------------ automatic key split (kv_split = -1)

@pytest.mark.parametrize("L,Sq,want", [
    (10368, 1, 54),    # 192-key chunks: 54 x 8 KV heads = 432 items <= 512
    (2000, 1, 32),     # 64-key chunks fill 256 items; none smaller exists
    (100, 1, 2),
    (64, 1, 1),        # no chunk is shorter than the whole range
    (0, 1, 1),
    (10368, 2000, 2),  # 2000 x 3 rows = 32 tiles of 192 per KV head: 2 chunks
])
def test_auto_split_fills_one_round(L, Sq, want):
    """kv_split = -1: the smallest multiple of 64 keys whose (request, KV head,
    chunk, query tile) items fit 512 workgroups."""
    desc = B.make_desc(24, 8, 128, 32, 400, "f16", key_bucket=256, max_cache_rows=10368,
                       kv_split=-1)
    nb = 10368 // 32
    plan = B.Plan(desc, 1, 1, nb, 10368, 2000, host_only=True)
    bt = (np.arange(nb, dtype=np.int32) % 400).reshape(1, 1, nb)
    Lh = np.array([L], np.int32)
    B.bsp_plan(plan, 1, 1, Sq, Lh, Lh, bt)
    assert plan.num_splits == want
