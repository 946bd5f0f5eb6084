"""Pins of the fp64 oracle to things other than itself (CPU only).

* brute force: an independent scalar evaluation at 50 significant digits
  (mpmath), over each beam's sequence rebuilt from the generator's logical draws
  (prompt rows plus the parent beams' own rows), never from page tables;
* a library routine: torch's scaled_dot_product_attention in float64 for the
  cases that reduce to plain (masked) attention;
* closed forms: zero query, identical keys, a single key;
* invariants: the cascade merge equals unsplit attention, garbage in masked
  rows and NaN past the bound do not change the result, page relabelling and
  beam relabelling;
* printed values: the bucket rule and the bound-row cases of the Phi-4 PR, the
  page-table cases of the cascade PR, the slot rule of the KV-write PR.
"""

import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import BeamConfig

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

PIN_CFG = BeamConfig("pin", batch=2, beam=3, num_q_heads=4, num_kv_heads=2, head_dim=8,
                     dtype="f32", page_size=4, prefix_range=(5, 11), tail_range=(0, 4),
                     shuffle_pages=True)


def _applied(inp):
    """Return the step inputs with the current-token write applied (oracle write)."""
    kp, vp = oracle.write_kv(inp.k_pool, inp.v_pool, inp.slots, inp.k_new, inp.v_new,
                             inp.page_size)
    inp.k_pool, inp.v_pool = kp, vp
    return inp


def _logical_sequence(inp, b, k):
    """Beam k's K/V sequence from the generator's logical draws, no page tables."""
    P, S = int(inp.prefix_len[b]), int(inp.seq_len[b])
    ks, vs = [inp.prompt_k[b][j] for j in range(P)], [inp.prompt_v[b][j] for j in range(P)]
    for j in range(P, S):
        src = int(inp.cache_indirection[b, k, j])
        ks.append(inp.own_k[b][src, j - P])
        vs.append(inp.own_v[b][src, j - P])
    D, Hkv = inp.head_dim, inp.num_kv_heads
    if not ks:
        return np.zeros((0, Hkv, D)), np.zeros((0, Hkv, D))
    return np.stack(ks).astype(np.float64), np.stack(vs).astype(np.float64)


def _mp_attention(q, K, V, scale):
    """Scalar softmax attention at 50 digits: q [D], K [n, D], V [n, D]."""
    mpmath.mp.dps = 50
    n, D = K.shape
    if n == 0:
        return [mpmath.mpf(0)] * V.shape[1], mpmath.mpf("-inf")
    s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(q[d])) * mpmath.mpf(float(K[j, d]))
                                         for d in range(D)) for j in range(n)]
    m = max(s)
    z = mpmath.fsum(mpmath.exp(x - m) for x in s)
    lse = m + mpmath.log(z)
    o = [mpmath.fsum(mpmath.exp(s[j] - lse) * mpmath.mpf(float(V[j, d])) for j in range(n))
         for d in range(V.shape[1])]
    return o, lse


# ---------------------------------------------------------------- index pins

@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_sequence_slots_rebuild_logical_sequences(seed):
    """Page-table walk + write == what the generator placed at each position."""
    inp = _applied(synth.make_beam_step(PIN_CFG, seed, keep_logical=True, page_stride=2))
    for b in range(inp.batch):
        for k in range(inp.beam):
            pages, rows = oracle.sequence_slots(b, k, inp.prefix_len, inp.seq_len,
                                                inp.block_tables, inp.cache_indirection,
                                                inp.page_size)
            K = inp.k_pool[pages, :, rows, :]
            V = inp.v_pool[pages, :, rows, :]
            Kl, Vl = _logical_sequence(inp, b, k)
            assert np.array_equal(K, Kl) and np.array_equal(V, Vl)


def test_write_kv_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "write_kv_slots.json")))
    ps, n = g["page_size"], len(g["slots"])
    kp = np.zeros((g["num_pages"], 1, ps, 2))
    kn = np.array([[[i + 1.0, -(i + 1.0)]] for i in range(n)])
    k2, v2 = oracle.write_kv(kp, kp, g["slots"], kn, -kn, ps)
    expect = np.zeros_like(kp)
    for i, (page, row) in enumerate(g["expected_page_row"]):
        expect[page, 0, row] = kn[i, 0]
    assert np.array_equal(k2, expect) and np.array_equal(v2, -expect)
    assert not kp.any(), "inputs must not be modified"


def test_prefix_page_table_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "prefix_pages.json")))
    ps = g["page_size"]
    cases = g["cases"]
    B, W, nb = len(cases), 3, 5
    bt = np.array([[[100 * r + 10 * k + i for i in range(nb)] for k in range(W)]
                   for r in range(B)])
    P = [c["prefix_len"] for c in cases]
    indptr, pages = oracle.prefix_page_table(P, bt, ps)
    for r, c in enumerate(cases):
        got = pages[indptr[r]:indptr[r + 1]].tolist()
        assert got == c["expected_pages"]
        assert P[r] == c["expected_keys"]
        if got:  # the keys end inside the last page: (count - 1) * ps < P <= count * ps
            assert (len(got) - 1) * ps < P[r] <= len(got) * ps


def test_tail_slots_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tail_slots.json")))
    got = oracle.tail_slots(g["prefix_len"], g["seq_len"], np.array(g["block_tables"]),
                            np.array(g["cache_indirection"]), g["page_size"], g["tail_pad"])
    assert got.tolist() == g["expected_slots"]


def test_tail_slots_match_sequence_slots():
    inp = synth.make_beam_step(PIN_CFG, 5, page_stride=2)
    pad = int(inp.tail_len.max())
    ts = oracle.tail_slots(inp.prefix_len, inp.seq_len, inp.block_tables,
                           inp.cache_indirection, inp.page_size, pad)
    for b in range(inp.batch):
        P, S = int(inp.prefix_len[b]), int(inp.seq_len[b])
        for k in range(inp.beam):
            pages, rows = oracle.sequence_slots(b, k, inp.prefix_len, inp.seq_len,
                                                inp.block_tables, inp.cache_indirection,
                                                inp.page_size, range(P, S))
            assert ts[b, k, :S - P].tolist() == (pages * inp.page_size + rows).tolist()
            assert (ts[b, k, S - P:] == -1).all()


# -------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", [0, 1])
def test_beam_decode_matches_50_digit_brute_force(seed):
    inp = _applied(synth.make_beam_step(PIN_CFG, seed, keep_logical=True))
    o, lse = oracle.beam_decode_attention(inp)
    scale = 1.0 / math.sqrt(inp.head_dim)
    G = inp.num_q_heads // inp.num_kv_heads
    worst = 0.0
    for b in range(inp.batch):
        for k in range(inp.beam):
            K, V = _logical_sequence(inp, b, k)
            for h in range(inp.num_q_heads):
                g = h // G
                mo, ml = _mp_attention(inp.q[b, k, 0, h], K[:, g], V[:, g], scale)
                assert abs(float(ml) - lse[b, k, 0, h]) <= 1e-12
                worst = max(worst, max(abs(float(x) - y) for x, y in zip(mo, o[b, k, 0, h])))
    assert worst <= 1e-12


def test_self_parents_read_only_own_rows():
    """n parallel samples of one prompt (parents = self): each sample's sequence is
    the shared prompt followed by its own rows, and the oracle matches brute force."""
    inp = _applied(synth.make_beam_step(PIN_CFG, 4, keep_logical=True, parents="self",
                                        tail_range=(2, 4)))
    o, lse = oracle.beam_decode_attention(inp)
    scale = 1.0 / math.sqrt(inp.head_dim)
    G = inp.num_q_heads // inp.num_kv_heads
    for b in range(inp.batch):
        P, S = int(inp.prefix_len[b]), int(inp.seq_len[b])
        assert (inp.cache_indirection[b, :, P:S] == np.arange(inp.beam)[:, None]).all()
        for k in range(inp.beam):
            K, V = _logical_sequence(inp, b, k)
            assert np.array_equal(K[P:], inp.own_k[b][k].astype(np.float64))
            for h in range(inp.num_q_heads):
                mo, ml = _mp_attention(inp.q[b, k, 0, h], K[:, h // G], V[:, h // G], scale)
                assert abs(float(ml) - lse[b, k, 0, h]) <= 1e-12
                assert max(abs(float(x) - y) for x, y in zip(mo, o[b, k, 0, h])) <= 1e-12


def test_cached_prefix_matches_50_digit_brute_force():
    inp = synth.make_cached_prefix(3, valid_rows=6, q_len=4, num_q_heads=4, num_kv_heads=2,
                                   head_dim=8, dtype="f32", max_cache_rows=16)
    scale = 1.0 / math.sqrt(8)
    for causal in (True, False):
        o, lse = oracle.cached_prefix_attention(inp, causal=causal)
        for i in range(4):
            new = range(i + 1) if causal else range(4)
            for h in range(4):
                g = h // 2
                K = np.concatenate([inp.cache_k[:6, g], inp.new_k[list(new), g]])
                V = np.concatenate([inp.cache_v[:6, g], inp.new_v[list(new), g]])
                mo, ml = _mp_attention(inp.q[i, h], K, V, scale)
                assert abs(float(ml) - lse[i, h]) <= 1e-12
                assert max(abs(float(x) - y) for x, y in zip(mo, o[i, h])) <= 1e-12


# ----------------------------------------------------------- library routine

def _sdpa(q, k, v, mask=None, scale=None):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=None if mask is None else torch.from_numpy(mask), scale=scale).numpy()


def test_plain_attention_matches_torch_sdpa():
    """Beam 1 with no tail is plain GQA attention over the prompt."""
    cfg = BeamConfig("sdpa", 3, 1, 8, 2, 16, "f32", 8, (1, 40), (0, 0), True)
    inp = synth.make_beam_step(cfg, 11, keep_logical=True)
    o, _ = oracle.beam_decode_attention(inp)
    G = 4
    for b in range(inp.batch):
        q = inp.q[b, 0, 0].astype(np.float64)[:, None, :]                # [Hq, 1, D]
        K = np.repeat(inp.prompt_k[b].astype(np.float64).transpose(1, 0, 2), G, axis=0)
        V = np.repeat(inp.prompt_v[b].astype(np.float64).transpose(1, 0, 2), G, axis=0)
        ref = _sdpa(q, K, V)[:, 0, :]
        assert np.abs(ref - o[b, 0, 0]).max() <= 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_cached_prefix_matches_torch_sdpa_with_explicit_mask(causal):
    """Keys = bound cache rows then the new rows; mask hides rows >= L (and the future)."""
    inp = synth.make_cached_prefix(4, valid_rows=37, q_len=5, num_q_heads=6, num_kv_heads=2,
                                   head_dim=16, dtype="f32", max_cache_rows=64)
    L, Sq, G = 37, 5, 3
    R = oracle.bucket_rows(L, 16, 64)
    o, _ = oracle.cached_prefix_attention(inp, causal=causal)
    K = np.concatenate([inp.cache_k[:R], inp.new_k]).astype(np.float64)   # [R+Sq, Hkv, D]
    V = np.concatenate([inp.cache_v[:R], inp.new_v]).astype(np.float64)
    mask = np.zeros((Sq, R + Sq), dtype=bool)
    mask[:, :L] = True
    for i in range(Sq):
        mask[i, R:R + (i + 1 if causal else Sq)] = True
    Kh = np.repeat(K.transpose(1, 0, 2), G, axis=0)
    Vh = np.repeat(V.transpose(1, 0, 2), G, axis=0)
    ref = _sdpa(inp.q.astype(np.float64).transpose(1, 0, 2), Kh, Vh, mask[None])
    assert np.abs(ref.transpose(1, 0, 2) - o).max() <= 1e-12


# -------------------------------------------------------------- closed forms

def test_zero_query_gives_mean_value_and_log_count():
    inp = _applied(synth.make_beam_step(PIN_CFG, 7, keep_logical=True))
    inp.q[:] = 0.0
    o, lse = oracle.beam_decode_attention(inp)
    G = inp.num_q_heads // inp.num_kv_heads
    for b in range(inp.batch):
        S = int(inp.seq_len[b])
        for k in range(inp.beam):
            _, V = _logical_sequence(inp, b, k)
            for h in range(inp.num_q_heads):
                assert abs(lse[b, k, 0, h] - math.log(S)) <= 1e-12
                assert np.abs(o[b, k, 0, h] - V[:, h // G].mean(axis=0)).max() <= 1e-12


def test_identical_keys_and_single_key():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((3, 8))
    kr = rng.standard_normal(8)
    V = rng.standard_normal((5, 8))
    o, lse = oracle.attend(q, np.tile(kr, (5, 1)), V, 0.5)
    s = 0.5 * q @ kr
    assert np.abs(lse - (s + math.log(5))).max() <= 1e-12
    assert np.abs(o - V.mean(axis=0)).max() <= 1e-12
    o1, lse1 = oracle.attend(q, kr[None], V[:1], 0.5)
    assert np.abs(lse1 - s).max() <= 1e-12 and np.abs(o1 - V[0]).max() <= 1e-15


def test_empty_key_set():
    o, lse = oracle.attend(np.ones((2, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert (o == 0).all() and np.isneginf(lse).all()


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cascade_merge_equals_unsplit(seed):
    inp = _applied(synth.make_beam_step(PIN_CFG, seed))
    full_o, full_l = oracle.beam_decode_attention(inp)
    po, pl = oracle.beam_partial_attention(inp, "prefix")
    to, tl = oracle.beam_partial_attention(inp, "tail")
    mo, ml = oracle.merge_states([po, to], [pl, tl])
    assert np.abs(mo - full_o).max() <= 1e-12
    assert np.abs(ml - full_l).max() <= 1e-12


def test_merge_every_split_point_and_nway():
    rng = np.random.default_rng(3)
    q, K, V = rng.standard_normal((4, 16)), rng.standard_normal((23, 16)), rng.standard_normal((23, 16))
    full_o, full_l = oracle.attend(q, K, V, 0.25)
    for cut in range(0, 24):
        a = oracle.attend(q, K[:cut], V[:cut], 0.25)
        b = oracle.attend(q, K[cut:], V[cut:], 0.25)
        for parts in ([a, b], [b, a]):
            mo, ml = oracle.merge_states([p[0] for p in parts], [p[1] for p in parts])
            assert np.abs(mo - full_o).max() <= 1e-12 and np.abs(ml - full_l).max() <= 1e-12
    cuts = [0, 5, 5, 11, 17, 23]
    parts = [oracle.attend(q, K[a:b], V[a:b], 0.25) for a, b in zip(cuts[:-1], cuts[1:])]
    mo, ml = oracle.merge_states([p[0] for p in parts], [p[1] for p in parts])
    assert np.abs(mo - full_o).max() <= 1e-12 and np.abs(ml - full_l).max() <= 1e-12
    # pairwise merging in another association order gives the same state
    left = oracle.merge_states([parts[0][0], parts[1][0]], [parts[0][1], parts[1][1]])
    right = oracle.merge_states([p[0] for p in parts[2:]], [p[1] for p in parts[2:]])
    mo2, ml2 = oracle.merge_states([left[0], right[0]], [left[1], right[1]])
    assert np.abs(mo2 - full_o).max() <= 1e-12 and np.abs(ml2 - full_l).max() <= 1e-12


def test_merge_with_empty_parts():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((3, 8))
    lse = rng.standard_normal(3)
    z, ninf = np.zeros((3, 8)), np.full(3, -np.inf)
    mo, ml = oracle.merge_states([o, z], [lse, ninf])
    assert np.array_equal(mo, o) and np.array_equal(ml, lse)
    mo, ml = oracle.merge_states([z, z], [ninf, ninf])
    assert (mo == 0).all() and np.isneginf(ml).all() and not np.isnan(mo).any()


def test_masked_rows_and_nan_past_bound_do_not_change_result():
    L, cap = 300, 1024
    R = oracle.bucket_rows(L, 256, cap)
    a = synth.make_cached_prefix(9, valid_rows=L, q_len=3, num_q_heads=6, num_kv_heads=2,
                                 head_dim=16, dtype="f16", max_cache_rows=cap)
    b = synth.make_cached_prefix(9, valid_rows=L, q_len=3, num_q_heads=6, num_kv_heads=2,
                                 head_dim=16, dtype="f16", max_cache_rows=cap, nan_from_row=R)
    rng = np.random.default_rng(1)
    b.cache_k[L:R] = rng.standard_normal(b.cache_k[L:R].shape) * 10
    b.cache_v[L:R] = rng.standard_normal(b.cache_v[L:R].shape) * 10
    for causal in (True, False):
        oa, la = oracle.cached_prefix_attention(a, causal=causal)
        ob, lb = oracle.cached_prefix_attention(b, causal=causal)
        assert np.array_equal(oa, ob) and np.array_equal(la, lb) and not np.isnan(ob).any()


def test_bound_rows_printed_cases_equal_whole_cache(golden_dir):
    """The Phi-4 PR's tiny-model cases: any bound >= valid rows gives the whole-cache result.

    Evaluated with the library attention over exactly ``bound + Sq`` key
    columns (cache rows beyond the valid prefix masked), against the oracle.
    """
    g = json.load(open(os.path.join(golden_dir, "bucket_rows.json")))
    rows = g["tiny_cache_rows"]
    runs = [(g["tiny_prefill"]["q_len"], c) for c in g["tiny_prefill"]["cases"]]
    runs += [(1, c) for c in g["tiny_decode"]["cases"]]
    for Sq, (L, bound) in runs:
        inp = synth.make_cached_prefix(L + 17, valid_rows=L, q_len=Sq, num_q_heads=4,
                                       num_kv_heads=2, head_dim=8, dtype="f32",
                                       max_cache_rows=rows)
        o, _ = oracle.cached_prefix_attention(inp, causal=True)
        for width in (bound, rows):
            K = np.concatenate([inp.cache_k[:width], inp.new_k]).astype(np.float64)
            V = np.concatenate([inp.cache_v[:width], inp.new_v]).astype(np.float64)
            mask = np.zeros((Sq, width + Sq), dtype=bool)
            mask[:, :L] = True
            for i in range(Sq):
                mask[i, width:width + i + 1] = True
            ref = _sdpa(inp.q.astype(np.float64).transpose(1, 0, 2),
                        np.repeat(K.transpose(1, 0, 2), 2, axis=0),
                        np.repeat(V.transpose(1, 0, 2), 2, axis=0), mask[None])
            assert np.abs(ref.transpose(1, 0, 2) - o).max() <= 1e-12


def test_bucket_rule_printed_values(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "bucket_rows.json")))
    for L, R in g["rule_256_cases"]:
        assert oracle.bucket_rows(L, g["granularity"], g["cap"]) == R
    for L, R in g["tiny_decode"]["cases"]:
        assert oracle.bucket_rows(L, 16, g["tiny_cache_rows"]) == R
    with pytest.raises(ValueError):
        oracle.bucket_rows(-1)


def test_page_relabelling_is_bit_identical():
    inp = _applied(synth.make_beam_step(PIN_CFG, 8))
    o1, l1 = oracle.beam_decode_attention(inp)
    perm = np.random.default_rng(2).permutation(inp.num_pages)
    kp, vp = np.empty_like(inp.k_pool), np.empty_like(inp.v_pool)
    kp[perm], vp[perm] = inp.k_pool, inp.v_pool
    inp.k_pool, inp.v_pool = kp, vp
    inp.block_tables = np.where(inp.block_tables >= 0, perm[np.maximum(inp.block_tables, 0)], -1)
    o2, l2 = oracle.beam_decode_attention(inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_beam_relabelling_permutes_outputs():
    inp = _applied(synth.make_beam_step(PIN_CFG, 9))
    o1, l1 = oracle.beam_decode_attention(inp)
    sigma = np.array([2, 0, 1])          # new beam k is old beam sigma[k]
    inv = np.argsort(sigma)
    inp.q = inp.q[:, sigma]
    inp.block_tables = inp.block_tables[:, sigma]
    ci = inp.cache_indirection[:, sigma]
    inp.cache_indirection = np.where(ci >= 0, inv[np.maximum(ci, 0)], -1).astype(np.int32)
    o2, l2 = oracle.beam_decode_attention(inp)
    assert np.array_equal(o2, o1[:, sigma]) and np.array_equal(l2, l1[:, sigma])


def test_input_slips_change_the_result():
    """A wrong parent or a missing current-token write moves the result well past tolerance."""
    inp = _applied(synth.make_beam_step(PIN_CFG, 0, keep_logical=True))
    o, lse = oracle.beam_decode_attention(inp)
    # a prefix read through the beam's own table instead of beam 0 is identical by
    # construction of the shared blocks, so plant the wrong parent instead:
    bad = synth.make_beam_step(PIN_CFG, 0)
    bad = _applied(bad)
    t = bad.tail_len
    b = int(np.argmax(t))
    assert t[b] > 0
    P = int(bad.prefix_len[b])
    bad.cache_indirection[b, :, P] = (bad.cache_indirection[b, :, P] + 1) % bad.beam
    o2, _ = oracle.beam_decode_attention(bad)
    assert np.abs(o2 - o).max() > 1e-3
    # a missing current-token write leaves N(0,100) garbage in the sequence
    raw = synth.make_beam_step(PIN_CFG, 0)
    o3, _ = oracle.beam_decode_attention(raw)
    assert np.abs(o3 - o).max() > 1e-3


# ------------------------------------------- context requests of a mixed step

PREFILL_CFG = BeamConfig("pf", batch=1, beam=1, num_q_heads=6, num_kv_heads=2, head_dim=16,
                         dtype="f32", page_size=4, prefix_range=(0, 0), tail_range=(0, 0),
                         shuffle_pages=True)


def test_prefill_without_cache_is_torch_causal_attention():
    """No cached rows: each request is plain causal GQA attention (torch's is_causal)."""
    inp = synth.make_prefill(PREFILL_CFG, 3, batch=3, chunk_range=(1, 23))
    o, lse = oracle.prefill_attention(inp)
    G = 3
    for b in range(inp.batch):
        r0, n = int(inp.q_off[b]), int(inp.q_len[b])
        q = inp.q[r0:r0 + n].astype(np.float64).transpose(1, 0, 2)            # [Hq, n, D]
        K = np.repeat(inp.new_k[r0:r0 + n].astype(np.float64).transpose(1, 0, 2), G, axis=0)
        V = np.repeat(inp.new_v[r0:r0 + n].astype(np.float64).transpose(1, 0, 2), G, axis=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(K), torch.from_numpy(V), is_causal=True).numpy()
        assert np.abs(ref.transpose(1, 0, 2) - o[r0:r0 + n]).max() <= 1e-12


def test_prefill_with_cache_matches_torch_sdpa_with_explicit_mask():
    """Cached rows then the chunk: key j is visible to chunk row i iff j <= L + i."""
    inp = synth.make_prefill(PREFILL_CFG, 4, batch=3, chunk_range=(1, 9), cached_range=(0, 30))
    o, _ = oracle.prefill_attention(inp)
    G = 3
    for b in range(inp.batch):
        r0, n, L = int(inp.q_off[b]), int(inp.q_len[b]), int(inp.cached_len[b])
        K = np.concatenate([inp.cache_k[b], inp.new_k[r0:r0 + n]]).astype(np.float64)
        V = np.concatenate([inp.cache_v[b], inp.new_v[r0:r0 + n]]).astype(np.float64)
        mask = np.arange(L + n)[None, :] <= (L + np.arange(n))[:, None]       # [n, L + n]
        Kh = np.repeat(K.transpose(1, 0, 2), G, axis=0)
        Vh = np.repeat(V.transpose(1, 0, 2), G, axis=0)
        ref = _sdpa(inp.q[r0:r0 + n].astype(np.float64).transpose(1, 0, 2), Kh, Vh, mask[None])
        assert np.abs(ref.transpose(1, 0, 2) - o[r0:r0 + n]).max() <= 1e-12


def test_prefill_row_matches_50_digit_brute_force():
    inp = synth.make_prefill(PREFILL_CFG, 5, batch=2, chunk_range=(3, 5), cached_range=(2, 6))
    b, i, h = 1, 2, 4
    o, lse = oracle.prefill_attention_one(inp, b, i)
    r0, L = int(inp.q_off[b]), int(inp.cached_len[b])
    g = h // 3
    K = np.concatenate([inp.cache_k[b][:, g], inp.new_k[r0:r0 + i + 1, g]]).astype(np.float64)
    V = np.concatenate([inp.cache_v[b][:, g], inp.new_v[r0:r0 + i + 1, g]]).astype(np.float64)
    assert K.shape[0] == L + i + 1
    mo, ml = _mp_attention(inp.q[r0 + i, h], K, V, 1 / math.sqrt(16))
    assert abs(float(ml) - lse[h]) <= 1e-12
    assert max(abs(float(x) - y) for x, y in zip(mo, o[h])) <= 1e-12


def test_prefill_in_two_chunks_equals_one_chunk():
    """Chunked prefill: the second chunk, with the first one cached, gives the
    same rows as the whole chunk at once."""
    inp = synth.make_prefill(PREFILL_CFG, 6, batch=1, chunk_range=(12, 12), cached_range=(5, 5))
    o, lse = oracle.prefill_attention(inp)
    cut = 7
    second = synth.PrefillInputs(**{**inp.__dict__,
                                    "q_len": np.array([12 - cut]),
                                    "cached_len": np.array([5 + cut]),
                                    "q": inp.q[cut:], "new_k": inp.new_k[cut:],
                                    "new_v": inp.new_v[cut:],
                                    "cache_k": [np.concatenate([inp.cache_k[0], inp.new_k[:cut]])],
                                    "cache_v": [np.concatenate([inp.cache_v[0], inp.new_v[:cut]])]})
    o2, lse2 = oracle.prefill_attention(second)
    assert np.abs(o2 - o[cut:]).max() <= 1e-13 and np.abs(lse2 - lse[cut:]).max() <= 1e-13


def test_prefill_pool_and_slots_hold_the_logical_rows():
    """After the KV write through ``slots``, the request's pages read in block
    order give its cached rows followed by the chunk's rows."""
    inp = synth.make_prefill(PREFILL_CFG, 7, batch=3, chunk_range=(1, 9), cached_range=(0, 13))
    kp, vp = oracle.write_kv(inp.k_pool, inp.v_pool, inp.slots, inp.new_k, inp.new_v,
                             inp.page_size)
    ps = inp.page_size
    for b in range(inp.batch):
        r0, n, L = int(inp.q_off[b]), int(inp.q_len[b]), int(inp.cached_len[b])
        want = np.concatenate([inp.cache_k[b], inp.new_k[r0:r0 + n]])
        got = np.stack([kp[inp.block_tables[b, j // ps], :, j % ps] for j in range(L + n)])
        assert np.array_equal(got, want)


def test_cached_prefix_row_subset_is_the_full_result_restricted():
    """Asking for some query rows gives exactly those rows of the full result."""
    inp = synth.make_cached_prefix(5, valid_rows=300, q_len=40, max_cache_rows=512)
    o, lse = oracle.cached_prefix_attention(inp, causal=True)
    rows = [39, 0, 17, 18]
    so, sl = oracle.cached_prefix_attention(inp, causal=True, rows=rows)
    assert np.array_equal(so, o[rows]) and np.array_equal(sl, lse[rows])


# --------------------------- pins of the partial-state and sampling helpers

def test_beam_attention_one_equals_the_full_result_bit_for_bit():
    """Every beam's ``beam_attention_one`` is exactly that beam's slice of
    ``beam_decode_attention`` (the full-size GPU tests compare sampled beams
    against it)."""
    inp = _applied(synth.make_beam_step(PIN_CFG, 12, keep_logical=True, page_stride=2))
    o, lse = oracle.beam_decode_attention(inp)
    for b in range(inp.batch):
        for k in range(inp.beam):
            ob, lb = oracle.beam_attention_one(inp, b, k)
            assert np.array_equal(ob, o[b, k]) and np.array_equal(lb, lse[b, k])


def test_beam_attention_one_matches_50_digit_brute_force():
    """One beam against an independent evaluation over its logical sequence: a
    wrong key count (``range(seq_len)`` off by one) would drop or add a key."""
    inp = _applied(synth.make_beam_step(PIN_CFG, 13, keep_logical=True, tail_range=(2, 4)))
    scale = 1.0 / math.sqrt(inp.head_dim)
    G = inp.num_q_heads // inp.num_kv_heads
    for b, k in ((0, 0), (inp.batch - 1, inp.beam - 1), (1, 1)):
        K, V = _logical_sequence(inp, b, k)
        assert K.shape[0] == int(inp.seq_len[b])
        ob, lb = oracle.beam_attention_one(inp, b, k)
        for h in range(inp.num_q_heads):
            mo, ml = _mp_attention(inp.q[b, k, 0, h], K[:, h // G], V[:, h // G], scale)
            assert abs(float(ml) - lb[0, h]) <= 1e-12
            assert max(abs(float(x) - y) for x, y in zip(mo, ob[0, h])) <= 1e-12


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_beam_partial_attention_matches_brute_force_on_each_side_of_the_prompt_end(seed):
    """The prefix part is the prompt rows ``j < P_b`` and the tail part the rows
    ``P_b <= j < S_b`` read through the parents, both rebuilt from the
    generator's logical draws (no page table): a boundary off by one at ``P_b``
    moves a key from one part to the other and fails both checks, although the
    merge of the two would still equal the whole."""
    inp = _applied(synth.make_beam_step(PIN_CFG, seed, keep_logical=True, tail_range=(1, 4)))
    po, pl = oracle.beam_partial_attention(inp, "prefix")
    to, tl = oracle.beam_partial_attention(inp, "tail")
    scale = 1.0 / math.sqrt(inp.head_dim)
    G = inp.num_q_heads // inp.num_kv_heads
    for b in range(inp.batch):
        P = int(inp.prefix_len[b])
        for k in range(inp.beam):
            K, V = _logical_sequence(inp, b, k)
            for h in range(inp.num_q_heads):
                g = h // G
                for part_o, part_l, rows in ((po, pl, slice(0, P)), (to, tl, slice(P, None))):
                    mo, ml = _mp_attention(inp.q[b, k, 0, h], K[rows, g], V[rows, g], scale)
                    if K[rows].shape[0] == 0:
                        assert np.isneginf(part_l[b, k, 0, h])
                        assert (part_o[b, k, 0, h] == 0).all()
                        continue
                    assert abs(float(ml) - part_l[b, k, 0, h]) <= 1e-12
                    assert max(abs(float(x) - y)
                               for x, y in zip(mo, part_o[b, k, 0, h])) <= 1e-12


def test_beam_partial_attention_prompt_part_ignores_the_tail():
    """Changing every tail row (and the current token) leaves the prefix part
    bit-identical and changes the tail part: the two parts really split at P_b."""
    a = _applied(synth.make_beam_step(PIN_CFG, 4, tail_range=(2, 4)))
    b = _applied(synth.make_beam_step(PIN_CFG, 4, tail_range=(2, 4)))
    for r in range(b.batch):
        P, S = int(b.prefix_len[r]), int(b.seq_len[r])
        for k in range(b.beam):
            pages, rows = oracle.sequence_slots(r, k, b.prefix_len, b.seq_len, b.block_tables,
                                                b.cache_indirection, b.page_size, range(P, S))
            b.k_pool[pages, :, rows, :] += 1.0
            b.v_pool[pages, :, rows, :] -= 1.0
    pa = oracle.beam_partial_attention(a, "prefix")
    pb = oracle.beam_partial_attention(b, "prefix")
    assert np.array_equal(pa[0], pb[0]) and np.array_equal(pa[1], pb[1])
    ta = oracle.beam_partial_attention(a, "tail")
    tb = oracle.beam_partial_attention(b, "tail")
    assert np.abs(ta[0] - tb[0]).max() > 0.1


def _mp_cached_rows(inp, i, h, rows, new_rows, scale):
    g = h // (inp.num_q_heads // inp.num_kv_heads)
    K = np.concatenate([inp.cache_k[list(rows), g], inp.new_k[list(new_rows), g]]).astype(np.float64)
    V = np.concatenate([inp.cache_v[list(rows), g], inp.new_v[list(new_rows), g]]).astype(np.float64)
    return _mp_attention(inp.q[i, h], K, V, scale)


@pytest.mark.parametrize("causal", [True, False])
def test_cached_prefix_partial_matches_50_digit_brute_force(causal):
    """The cache segment over explicit key ranges (including ranges that cross
    the valid length, start past it, or hold one row) and the new-row segment,
    each against an independent evaluation over the rows the definition names:
    cache rows ``lo <= r < min(hi, L)`` and new rows ``i' <= i`` (causal) or all."""
    L, Sq = 13, 4
    inp = synth.make_cached_prefix(21, valid_rows=L, q_len=Sq, num_q_heads=4, num_kv_heads=2,
                                   head_dim=8, dtype="f32", max_cache_rows=32)
    scale = 1.0 / math.sqrt(8)
    ranges = [None, (0, 5), (5, 13), (12, 13), (4, 20), (13, 32), (0, 1)]
    for kr in ranges:
        o, lse = oracle.cached_prefix_partial(inp, "cache", causal=causal, key_range=kr)
        lo, hi = (0, L) if kr is None else (kr[0], min(kr[1], L))
        rows = range(lo, hi)
        for i in range(Sq):
            for h in range(4):
                if len(rows) == 0:
                    assert np.isneginf(lse[i, h]) and (o[i, h] == 0).all()
                    continue
                mo, ml = _mp_cached_rows(inp, i, h, rows, [], scale)
                assert abs(float(ml) - lse[i, h]) <= 1e-12, (kr, i, h)
                assert max(abs(float(x) - y) for x, y in zip(mo, o[i, h])) <= 1e-12
    o, lse = oracle.cached_prefix_partial(inp, "new", causal=causal)
    for i in range(Sq):
        new = range(i + 1) if causal else range(Sq)
        for h in range(4):
            mo, ml = _mp_cached_rows(inp, i, h, [], new, scale)
            assert abs(float(ml) - lse[i, h]) <= 1e-12
            assert max(abs(float(x) - y) for x, y in zip(mo, o[i, h])) <= 1e-12


@pytest.mark.parametrize("L,cuts", [(0, [0, 256]), (1, [0, 64, 128]), (300, [0, 64, 256, 512]),
                                    (777, [0, 192, 384, 576, 768, 960]),
                                    (1024, [0, 256, 512, 768, 1024])])
def test_cached_prefix_partials_merge_to_the_whole_call(L, cuts):
    """Splitting the cache segment at chunk boundaries and merging every chunk's
    partial with the new-row segment gives the whole call (to rounding), for
    chunks that end inside, at or past the valid length."""
    inp = synth.make_cached_prefix(L + 3, valid_rows=L, q_len=5, num_q_heads=6, num_kv_heads=2,
                                   head_dim=16, dtype="f16", max_cache_rows=1024)
    for causal in (True, False):
        full_o, full_l = oracle.cached_prefix_attention(inp, causal=causal)
        parts = [oracle.cached_prefix_partial(inp, "cache", causal=causal, key_range=(a, b))
                 for a, b in zip(cuts[:-1], cuts[1:])]
        parts.append(oracle.cached_prefix_partial(inp, "new", causal=causal))
        mo, ml = oracle.merge_states([p[0] for p in parts], [p[1] for p in parts])
        assert np.abs(mo - full_o).max() <= 1e-12 and np.abs(ml - full_l).max() <= 1e-12
