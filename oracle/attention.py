"""Plain fp64 attention for one beam-search decode step and for cached-prefix calls.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method splits a beam decode step into a shared-prompt part and a per-beam
tail and merges the two with their log-sum-exp; the pages state that the merge
is exact (TensorRT-LLM PR #21738, "Add opt-in cascade attention for wide beam
search on KVCM V2": Description, Solution; first commit message). So the oracle
does not compute the cascade: it computes the plain definition the cascade
reaches, softmax attention of each beam over its own whole cached sequence, and
separately the same formula over any subset of keys (for checking partial
results) plus the fp64 merge of partial states.

Conventions (readings of points the pages leave open):
* softmax scale ``1/sqrt(D)`` unless given;
* query head ``h`` reads KV head ``h // (Hq // Hkv)`` (dense GQA, consecutive
  query heads share a KV head; MHA when the ratio is 1);
* LSE is the natural logarithm of the softmax denominator including the scale:
  ``LSE = ln sum_j exp(scale * q.k_j)``;
* an empty key set gives ``O = 0`` and ``LSE = -inf``.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

NEG_INF = float("-inf")


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Softmax attention of query rows over one key set, in fp64.

    ``q [n_q, D]``, ``k [n_k, D]``, ``v [n_k, D]`` -> ``o [n_q, D]``, ``lse [n_q]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, d = q.shape
    if k.shape[0] == 0:
        return np.zeros((n_q, v.shape[1] if v.ndim == 2 else d)), np.full(n_q, NEG_INF)
    s = scale * (q @ k.T)                       # [n_q, n_k]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    denom = w.sum(axis=1, keepdims=True)
    lse = (m + np.log(denom))[:, 0]
    o = (w / denom) @ v
    return o, lse


def merge_states(os: Sequence[np.ndarray], lses: Sequence[np.ndarray]):
    """Exact merge of partial attention states over disjoint key sets.

    Each part ``i`` is ``(o_i, lse_i)`` with ``o_i [..., D]`` normalised over its
    own keys. The merged state is ``lse = ln sum_i exp(lse_i)`` and
    ``o = sum_i exp(lse_i - lse) * o_i`` (the log-sum-exp combination named in the
    Solution section of TensorRT-LLM PR #21738). Parts with ``lse = -inf`` carry
    no keys and drop out; if every part is empty the result is ``(0, -inf)``.
    """
    lse_stack = np.stack([np.asarray(x, dtype=np.float64) for x in lses])   # [n, ...]
    o_stack = np.stack([np.asarray(x, dtype=np.float64) for x in os])       # [n, ..., D]
    m = lse_stack.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_stack), np.exp(lse_stack - m_safe), 0.0)  # [n, ...]
    denom = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, denom, 1.0)), NEG_INF)
    safe = np.where(finite, denom, 1.0)
    o = (w[..., None] * o_stack).sum(axis=0) / safe[..., None]
    o = np.where(finite[..., None], o, 0.0)
    return o, lse


def sequence_slots(b: int, k: int, prefix_len, seq_len, block_tables, cache_indirection,
                   page_size: int, positions: Optional[Iterable[int]] = None):
    """(page, row) of each cached position of beam ``k`` of request ``b``.

    Positions ``j < P_b`` are the shared prompt, read through beam 0's block
    table (the KV-cache-manager-V2 commit of PR #21738 takes the prompt page
    table from beam 0). Positions ``P_b <= j < S_b`` are the beam's generated
    tail, read from the beam that ``cache_indirection[b, k, j]`` names
    (Solution section: the tail is gathered through cache_indirection).
    The row inside a page is ``j mod page_size``.
    """
    P, S = int(prefix_len[b]), int(seq_len[b])
    pos = range(S) if positions is None else positions
    pages, rows = [], []
    for j in pos:
        src = 0 if j < P else int(cache_indirection[b, k, j])
        pages.append(int(block_tables[b, src, j // page_size]))
        rows.append(j % page_size)
    return np.asarray(pages, dtype=np.int64), np.asarray(rows, dtype=np.int64)


def _one_beam(inp, b: int, k: int, positions, scale: float):
    """Attention of beam ``k`` of request ``b`` over the given sequence positions."""
    q = inp.q
    q_len, Hq, D = q.shape[2], q.shape[3], q.shape[4]
    Hkv = inp.k_pool.shape[1]
    G = Hq // Hkv
    pages, rows = sequence_slots(b, k, inp.prefix_len, inp.seq_len, inp.block_tables,
                                 inp.cache_indirection, inp.page_size, list(positions))
    K = inp.k_pool[pages, :, rows, :].astype(np.float64)   # [n, Hkv, D]
    V = inp.v_pool[pages, :, rows, :].astype(np.float64)
    o = np.zeros((q_len, Hq, D))
    lse = np.full((q_len, Hq), NEG_INF)
    for i in range(q_len):
        for g in range(Hkv):             # query heads g*G .. g*G+G-1 read KV head g
            heads = slice(g * G, (g + 1) * G)
            oo, ll = attend(q[b, k, i, heads], K[:, g, :], V[:, g, :], scale)
            o[i, heads] = oo
            lse[i, heads] = ll
    return o, lse


def _beam_attention(inp, positions_of, scale):
    B, W = inp.block_tables.shape[:2]
    q = inp.q
    q_len, Hq, D = q.shape[2], q.shape[3], q.shape[4]
    o = np.zeros((B, W, q_len, Hq, D))
    lse = np.full((B, W, q_len, Hq), NEG_INF)
    for b in range(B):
        for k in range(W):
            o[b, k], lse[b, k] = _one_beam(inp, b, k, positions_of(b), scale)
    return o, lse


def beam_attention_one(inp, b: int, k: int, scale: Optional[float] = None):
    """``beam_decode_attention`` of a single beam: ``o [q_len, Hq, D]``, ``lse [q_len, Hq]``.

    Used to check sampled outputs of full-size runs.
    """
    sc = default_scale(inp.q.shape[-1]) if scale is None else scale
    return _one_beam(inp, b, k, range(int(inp.seq_len[b])), sc)


def beam_decode_attention(inp, scale: Optional[float] = None):
    """Per-beam full softmax attention over each beam's reconstructed sequence.

    ``inp`` carries ``q [B, W, q_len, Hq, D]``, the pools ``[pages, Hkv, ps, D]``,
    ``block_tables``, ``cache_indirection``, ``prefix_len``, ``seq_len`` and
    ``page_size`` (the current-token write must already be applied to the
    pools; see ``write_kv``). Returns ``o [B, W, q_len, Hq, D]`` and
    ``lse [B, W, q_len, Hq]`` in fp64.
    """
    sc = default_scale(inp.q.shape[-1]) if scale is None else scale
    return _beam_attention(inp, lambda b: range(int(inp.seq_len[b])), sc)


def beam_partial_attention(inp, part: str, scale: Optional[float] = None):
    """The same formula over one part of each sequence.

    ``part="prefix"``: positions ``j < P_b`` (the shared prompt);
    ``part="tail"``: positions ``P_b <= j < S_b`` (the beam's own tail).
    """
    sc = default_scale(inp.q.shape[-1]) if scale is None else scale
    if part == "prefix":
        return _beam_attention(inp, lambda b: range(int(inp.prefix_len[b])), sc)
    if part == "tail":
        return _beam_attention(
            inp, lambda b: range(int(inp.prefix_len[b]), int(inp.seq_len[b])), sc)
    raise ValueError(part)


def write_kv(k_pool, v_pool, slots, k_new, v_new, page_size: int):
    """Scatter new K/V rows into copies of the pools.

    Token ``i`` goes to page ``slots[i] // page_size``, row ``slots[i] %
    page_size``, for every KV head (the MiniMax-M3 fused KV-write PR,
    TensorRT-LLM #18614, Description: page and in-page row are derived from
    the flat slot). Returns the new pools; the inputs are not modified.
    """
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    for i, slot in enumerate(np.asarray(slots).tolist()):
        page, row = divmod(int(slot), page_size)
        kp[page, :, row, :] = k_new[i]
        vp[page, :, row, :] = v_new[i]
    return kp, vp


def bucket_rows(valid_rows: int, granularity: int = 256, cap: Optional[int] = None) -> int:
    """Number of cache rows bound for a valid prefix of ``valid_rows`` rows.

    The valid prefix rounded up to a multiple of ``granularity``, capped at the
    allocation, and one (masked) row for an empty cache (Phi-4 cached-prefix PR,
    TensorRT-Model-Connect #2202: Exit Criteria; Implementation, kv_cache
    paragraph; Notes For Future Readers).
    """
    if valid_rows < 0:
        raise ValueError("valid_rows < 0")
    if valid_rows == 0:
        return 1
    r = -(-valid_rows // granularity) * granularity
    return r if cap is None else min(r, cap)


def _cached_visible(i: int, L: int, q_len: int, causal: bool):
    """Visible keys of query row ``i``: cache rows ``< L`` and new rows."""
    new = range(i + 1) if causal else range(q_len)
    return list(range(L)), list(new)


def cached_prefix_attention(inp, causal: bool = True, scale: Optional[float] = None,
                            rows: Optional[list] = None):
    """Beam-1 attention over the valid cached prefix plus this call's rows.

    Keys are the concatenation of the bound cache rows and the ``Sq`` new rows
    (Phi-4 cached-prefix PR, Implementation: the graph concatenates the cache and
    prompt rows; the masks are ``[Sq, rows + Sq]`` with the prompt columns after
    the cache rows, and ``[1, rows + 1]`` for one-token decode). Cache rows at or
    past the valid length ``L`` are masked, so only rows ``< L`` count; new row
    ``i'`` is visible to query ``i`` when ``i' <= i`` (causal, the "batched"
    mask) or always (bidirectional).

    ``inp`` carries ``q [Sq, Hq, D]``, ``cache_k/cache_v [rows, Hkv, D]``,
    ``valid_rows`` and ``new_k/new_v [Sq, Hkv, D]``. Returns ``o [Sq, Hq, D]``,
    ``lse [Sq, Hq]``; with ``rows`` (query row indices) only those rows, in that
    order, ``o [len(rows), Hq, D]`` and ``lse [len(rows), Hq]``.
    """
    q = inp.q
    Sq, Hq, D = q.shape
    Hkv = inp.cache_k.shape[1]
    G = Hq // Hkv
    sc = default_scale(D) if scale is None else scale
    L = int(inp.valid_rows)
    which = list(range(Sq)) if rows is None else [int(i) for i in rows]
    o = np.zeros((len(which), Hq, D))
    lse = np.full((len(which), Hq), NEG_INF)
    for n, i in enumerate(which):
        crow, nrow = _cached_visible(i, L, Sq, causal)
        for g in range(Hkv):             # query heads g*G .. g*G+G-1 read KV head g
            heads = slice(g * G, (g + 1) * G)
            K = np.concatenate([inp.cache_k[crow, g, :], inp.new_k[nrow, g, :]]).astype(np.float64)
            V = np.concatenate([inp.cache_v[crow, g, :], inp.new_v[nrow, g, :]]).astype(np.float64)
            oo, ll = attend(q[i, heads], K, V, sc)
            o[n, heads] = oo
            lse[n, heads] = ll
    return o, lse


def cached_prefix_partial(inp, segment: str, causal: bool = True,
                          key_range: Optional[tuple] = None, scale: Optional[float] = None):
    """The cached-prefix formula over one key segment.

    ``segment="cache"``: the valid cache rows only, optionally restricted to
    rows ``key_range = (lo, hi)`` (a split of the cache segment);
    ``segment="new"``: this call's rows only, with the same self mask.
    """
    q = inp.q
    Sq, Hq, D = q.shape
    Hkv = inp.cache_k.shape[1]
    G = Hq // Hkv
    sc = default_scale(D) if scale is None else scale
    L = int(inp.valid_rows)
    o = np.zeros((Sq, Hq, D))
    lse = np.full((Sq, Hq), NEG_INF)
    for i in range(Sq):
        crow, nrow = _cached_visible(i, L, Sq, causal)
        if segment == "cache":
            if key_range is not None:
                crow = [r for r in crow if key_range[0] <= r < key_range[1]]
            src_k, src_v, rows = inp.cache_k, inp.cache_v, crow
        elif segment == "new":
            src_k, src_v, rows = inp.new_k, inp.new_v, nrow
        else:
            raise ValueError(segment)
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)
            oo, ll = attend(q[i, heads], src_k[rows, g, :], src_v[rows, g, :], sc)
            o[i, heads] = oo
            lse[i, heads] = ll
    return o, lse


def prefill_attention_one(inp, b: int, i: int, scale: Optional[float] = None):
    """Causal attention of chunk row ``i`` of context request ``b``: ``o [Hq, D]``, ``lse [Hq]``.

    The context requests of a mixed step go through an ordinary causal prefill
    (TensorRT-LLM PR #21738, mixed-batches commit: the generation rows of a
    step that also carries context requests use the cascade, the context rows
    the regular attention). The row at sequence position ``L_b + i`` sees the
    request's cached rows ``0 .. L_b - 1`` and the chunk's rows ``0 .. i``,
    and nothing after itself.
    """
    Hq, D = inp.q.shape[1], inp.q.shape[2]
    Hkv = inp.new_k.shape[1]
    G = Hq // Hkv
    sc = default_scale(D) if scale is None else scale
    r0 = int(inp.q_off[b])
    o = np.zeros((Hq, D))
    lse = np.full(Hq, NEG_INF)
    for g in range(Hkv):
        K = np.concatenate([inp.cache_k[b][:, g, :], inp.new_k[r0:r0 + i + 1, g, :]])
        V = np.concatenate([inp.cache_v[b][:, g, :], inp.new_v[r0:r0 + i + 1, g, :]])
        heads = slice(g * G, (g + 1) * G)
        o[heads], lse[heads] = attend(inp.q[r0 + i, heads], K, V, sc)
    return o, lse


def prefill_attention(inp, scale: Optional[float] = None):
    """``prefill_attention_one`` for every packed row: ``o [R, Hq, D]``, ``lse [R, Hq]``."""
    R, Hq, D = inp.q.shape
    o = np.zeros((R, Hq, D))
    lse = np.full((R, Hq), NEG_INF)
    for b in range(inp.batch):
        r0 = int(inp.q_off[b])
        for i in range(int(inp.q_len[b])):
            o[r0 + i], lse[r0 + i] = prefill_attention_one(inp, b, i, scale)
    return o, lse
