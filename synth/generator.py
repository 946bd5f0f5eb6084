"""Seeded synthetic workloads shaped like the pages' beam-search and cached-prefix runs.

Everything here is random drawing, rounding of the draws to the storage dtype,
and placement of the draws into a paged KV pool. No attention arithmetic lives
here: the oracle and the HIP path both take these arrays as given.

Paged pool layout (shared by every consumer): ``[num_pages, num_kv_heads,
page_size, head_dim]``, K and V in separate arrays of the same geometry. Block
tables are ``int32 [batch, beam, max_blocks]`` and ``cache_indirection`` is
``int32 [batch, beam, max_seq_len]``; entries that are never meant to be read
hold -1.

Placement rules (the workload shapes come from the TensorRT-LLM PR #21738
"Add opt-in cascade attention for wide beam search on KVCM V2", Description >
Performance table; the page ownership is the plainest reading of its commit
notes on prompt pages and tail gathering):

* every beam of a request points at the same page ids for the full prompt
  blocks;
* each beam owns its own copy of the block holding the end of the prompt (the
  prompt rows in it are identical copies) and of every later block, where its
  own generated rows live;
* ``cache_indirection[b, k, j]`` for a tail position ``P_b <= j < S_b`` names
  the beam whose pages hold that position for beam ``k``; it is drawn
  uniformly from the request's beams (beam search), or is ``k`` itself for
  n parallel samples of one prompt (``parents="self"``);
* the last tail position (the current token, when the tail is not empty) holds
  large garbage in the pool until the step's KV write puts ``k_new``/``v_new``
  there through ``slots``;
* every pool row that nothing references holds N(0, 100) garbage (or NaN when
  asked), so a read of the wrong row shows up in the results.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")


def _round_bf16_inplace(x: np.ndarray) -> None:
    """Round-to-nearest-even of float32 values to bf16, in place, in chunks.

    Finite values cannot wrap in uint32 (the largest magnitude rounds to an
    infinity at most); NaNs are restored afterwards.
    """
    flat = x.reshape(-1)
    bits = flat.view(np.uint32)
    step = 1 << 18
    for lo in range(0, flat.size, step):
        f = flat[lo:lo + step]
        nan = np.isnan(f)
        u = bits[lo:lo + step]
        lsb = u >> np.uint32(16)
        lsb &= np.uint32(1)
        u += np.uint32(0x7FFF)
        u += lsb
        u &= np.uint32(0xFFFF0000)
        if nan.any():
            f[nan] = np.float32(np.nan)


def round_to_dtype(x: np.ndarray, dtype: str, inplace: bool = False) -> np.ndarray:
    """Round float32 draws once, to nearest-even, to the storage dtype.

    Returns float32 arrays whose every value is exactly representable in
    ``dtype`` so that a later cast to that dtype is exact.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = x if inplace else x.copy()
    if dtype == "f32":
        return out
    if dtype == "f16":
        flat = out.reshape(-1)
        step = 1 << 20
        for lo in range(0, flat.size, step):
            flat[lo:lo + step] = flat[lo:lo + step].astype(np.float16)
        return out
    if dtype == "bf16":
        _round_bf16_inplace(out)
        return out
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass(frozen=True)
class BeamConfig:
    """One beam-decode workload: lengths are drawn per request, inclusive ranges."""

    name: str
    batch: int
    beam: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    page_size: int
    prefix_range: tuple
    tail_range: tuple
    shuffle_pages: bool
    max_tail: int = 0  # fixed padded tail length for graph-style plans (0: per step)
    # tail parents: "uniform" (beam search: each tail position of each beam names a
    # beam drawn uniformly) or "self" (n parallel samples of one prompt: every
    # sample reads only its own generated rows)
    parents: str = "uniform"

    @property
    def max_seq_len(self) -> int:
        return self.prefix_range[1] + self.tail_range[1]


BEAM_CONFIGS = {
    # 1 request, beam 4, GQA 2:1, head_dim 64, fp32, 128-token prompt in 16-token
    # pages, 3 tail tokens per beam.
    "tiny": BeamConfig("tiny", 1, 4, 2, 1, 64, "f32", 16, (128, 128), (3, 3), False),
    # Qwen3-0.6B-like layer, workload B "medium" prompts.
    "qwen3_0p6b": BeamConfig("qwen3_0p6b", 64, 30, 16, 8, 128, "bf16", 32,
                             (400, 600), (0, 4), False),
    # Wide-beam recommendation shape, workload A; pages shuffled in the pool.
    "wide_beam": BeamConfig("wide_beam", 128, 96, 16, 8, 128, "bf16", 32,
                            (2800, 3200), (0, 8), True, max_tail=8),
    # Qwen3-4B-like layer (head_dim 64/256 variants via make_beam_step(head_dim=...)).
    "qwen3_4b": BeamConfig("qwen3_4b", 64, 30, 32, 8, 128, "f16", 32,
                           (1600, 2400), (1, 4), False),
    # the same layer at head_dim 64 and 256 (same token counts)
    "qwen3_4b_d64": BeamConfig("qwen3_4b_d64", 64, 30, 32, 8, 64, "f16", 32,
                               (1600, 2400), (1, 4), False),
    "qwen3_4b_d256": BeamConfig("qwen3_4b_d256", 64, 30, 32, 8, 256, "f16", 32,
                                (1600, 2400), (1, 4), False),
    # n-sample prefix sharing (parallel sampling): 16 samples of each prompt,
    # each attending the shared prompt and its own 8-32 generated tokens.
    "nsample": BeamConfig("nsample", 64, 16, 16, 8, 128, "bf16", 32,
                          (400, 600), (8, 32), False, parents="self"),
}


@dataclass
class BeamStepInputs:
    """One decode step of one layer, before the current-token KV write."""

    config: str
    dtype: str
    batch: int
    beam: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    max_blocks: int
    max_seq_len: int
    max_tail: int
    q: np.ndarray                 # float32 [B, W, 1, Hq, D]
    k_pool: np.ndarray            # float32 [num_pages, Hkv, ps, D]
    v_pool: np.ndarray
    block_tables: np.ndarray      # int32 [B, W, max_blocks]
    cache_indirection: np.ndarray  # int32 [B, W, max_seq_len]
    prefix_len: np.ndarray        # int32 [B]
    seq_len: np.ndarray           # int32 [B]   (prefix + tail, current token included)
    k_new: np.ndarray             # float32 [N, Hkv, D]  current tokens of beams with a tail
    v_new: np.ndarray
    slots: np.ndarray             # int32 [N]  flat pool slot (page * ps + row) of each
    # Logical draws, kept only when asked: what each beam's own rows are, by position.
    prompt_k: Optional[list] = field(default=None, repr=False)   # [b] -> [P_b, Hkv, D]
    prompt_v: Optional[list] = field(default=None, repr=False)
    own_k: Optional[list] = field(default=None, repr=False)      # [b] -> [W, T_b, Hkv, D]
    own_v: Optional[list] = field(default=None, repr=False)

    @property
    def tail_len(self) -> np.ndarray:
        return (self.seq_len - self.prefix_len).astype(np.int32)


def _pool_fill(rng, shape, garbage: str) -> np.ndarray:
    """A pool of unreferenced-row garbage, filled in place page by page."""
    out = np.empty(shape, dtype=np.float32)
    if garbage == "nan":
        out.fill(np.nan)
        return out
    if garbage not in ("normal", "unit"):
        raise ValueError(f"unknown garbage mode {garbage!r}")
    rows = max(1, (1 << 22) // max(1, int(np.prod(shape[1:]))))
    for p0 in range(0, shape[0], rows):
        chunk = out[p0:p0 + rows]
        rng.standard_normal(dtype=np.float32, out=chunk)
        if garbage == "normal":  # N(0, 100): standard deviation 10
            chunk *= np.float32(10.0)
    return out


def make_beam_step(config, seed: int = 0, *, batch: Optional[int] = None,
                   beam: Optional[int] = None, head_dim: Optional[int] = None,
                   dtype: Optional[str] = None, prefix_range: Optional[tuple] = None,
                   tail_range: Optional[tuple] = None, garbage: str = "normal",
                   spare_frac: float = 0.05, shuffle_pages: Optional[bool] = None,
                   page_stride: int = 1, keep_logical: bool = False,
                   parents: Optional[str] = None) -> BeamStepInputs:
    """Draw one beam-decode step of ``config`` with ``numpy.random.default_rng(seed)``.

    ``config`` is a name in ``BEAM_CONFIGS`` or a ``BeamConfig``.
    Keyword overrides shrink or vary a config for tests (e.g. ``batch=2``) while
    keeping its other shapes and distributions. ``page_stride=2`` leaves every
    other page id unused (pages only at even ids). ``garbage`` fills
    unreferenced pool rows: "normal" N(0, 100), "unit" N(0, 1), "nan". With
    "unit" (and no ``keep_logical``) the pool draw itself supplies the
    referenced rows, which is much faster for the large configs. ``parents``
    overrides the config's tail-parent mode ("uniform" or "self").
    """
    spec = BEAM_CONFIGS[config] if isinstance(config, str) else config
    B = batch if batch is not None else spec.batch
    W = beam if beam is not None else spec.beam
    D = head_dim if head_dim is not None else spec.head_dim
    dt = dtype if dtype is not None else spec.dtype
    p_lo, p_hi = prefix_range if prefix_range is not None else spec.prefix_range
    t_lo, t_hi = tail_range if tail_range is not None else spec.tail_range
    shuffle = spec.shuffle_pages if shuffle_pages is None else shuffle_pages
    parent_mode = spec.parents if parents is None else parents
    assert parent_mode in ("uniform", "self")
    Hq, Hkv, ps = spec.num_q_heads, spec.num_kv_heads, spec.page_size
    assert Hq % Hkv == 0 and dt in DTYPES

    rng = np.random.default_rng(seed)
    P = rng.integers(p_lo, p_hi + 1, size=B).astype(np.int64)
    T = rng.integers(t_lo, t_hi + 1, size=B).astype(np.int64)
    S = P + T
    max_seq_len = p_hi + t_hi
    max_blocks = -(-max_seq_len // ps)

    n_full = P // ps                    # prompt blocks shared by every beam
    n_blk = -(-S // ps)                 # blocks each beam's table uses
    n_own = n_blk - n_full              # blocks each beam owns
    used = int(np.sum(n_full + W * n_own))
    n_slots = int(np.ceil(used * (1.0 + spare_frac))) + 1
    num_pages = n_slots * page_stride
    ids = np.arange(0, num_pages, page_stride, dtype=np.int64)
    if shuffle:
        ids = ids[rng.permutation(len(ids))]

    block_tables = np.full((B, W, max_blocks), -1, dtype=np.int32)
    cursor = 0
    for b in range(B):
        shared = ids[cursor:cursor + n_full[b]]
        cursor += n_full[b]
        block_tables[b, :, :n_full[b]] = shared[None, :]
        for k in range(W):
            own = ids[cursor:cursor + n_own[b]]
            cursor += n_own[b]
            block_tables[b, k, n_full[b]:n_blk[b]] = own

    k_pool = _pool_fill(rng, (num_pages, Hkv, ps, D), garbage)
    v_pool = _pool_fill(rng, (num_pages, Hkv, ps, D), garbage)

    prompt_k, prompt_v, own_k, own_v = [], [], [], []
    # With N(0, 1) garbage and no logical copies wanted, the pool draw itself
    # supplies every referenced row: only the end of the prompt has to be made
    # identical in every beam's own block (copied from beam 0's block).
    fast = garbage == "unit" and not keep_logical
    for b in range(B):
        nf, full_rows = int(n_full[b]), int(n_full[b]) * ps
        rest = int(P[b]) - full_rows
        if fast:
            if rest and W > 1:
                src = int(block_tables[b, 0, nf])
                pages = block_tables[b, 1:, nf]
                k_pool[pages, :, :rest, :] = k_pool[src, :, :rest, :][None]
                v_pool[pages, :, :rest, :] = v_pool[src, :, :rest, :][None]
            continue
        pk = rng.standard_normal((P[b], Hkv, D), dtype=np.float32)
        pv = rng.standard_normal((P[b], Hkv, D), dtype=np.float32)
        ok = rng.standard_normal((W, T[b], Hkv, D), dtype=np.float32)
        ov = rng.standard_normal((W, T[b], Hkv, D), dtype=np.float32)
        if nf:                  # full prompt blocks: one shared copy
            pages = block_tables[b, 0, :nf]
            k_pool[pages] = pk[:full_rows].reshape(nf, ps, Hkv, D).transpose(0, 2, 1, 3)
            v_pool[pages] = pv[:full_rows].reshape(nf, ps, Hkv, D).transpose(0, 2, 1, 3)
        if rest:                # end of the prompt: a copy in every beam's own block
            pages = block_tables[b, :, nf]
            k_pool[pages, :, :rest, :] = pk[full_rows:].transpose(1, 0, 2)[None]
            v_pool[pages, :, :rest, :] = pv[full_rows:].transpose(1, 0, 2)[None]
        for t in range(int(T[b]) - 1):  # own generated rows, except the current token
            blk, row = divmod(int(P[b] + t), ps)
            pages = block_tables[b, :, blk]
            k_pool[pages, :, row, :] = ok[:, t]
            v_pool[pages, :, row, :] = ov[:, t]
        prompt_k.append(pk)
        prompt_v.append(pv)
        own_k.append(ok)
        own_v.append(ov)

    ci = np.full((B, W, max_seq_len), -1, dtype=np.int32)
    for b in range(B):
        if T[b] > 0:
            if parent_mode == "self":
                ci[b, :, P[b]:S[b]] = np.arange(W, dtype=np.int32)[:, None]
            else:
                ci[b, :, P[b]:S[b]] = rng.integers(0, W, size=(W, T[b]))

    # Current token of each beam (last tail position), written during the step.
    k_new, v_new, slots = [], [], []
    for b in range(B):
        if T[b] == 0:
            continue
        j = int(S[b] - 1)
        blk, row = divmod(j, ps)
        for k in range(W):
            slots.append(int(block_tables[b, k, blk]) * ps + row)
            if not fast:
                k_new.append(own_k[b][k, T[b] - 1])
                v_new.append(own_v[b][k, T[b] - 1])
    if fast:
        k_new = rng.standard_normal((len(slots), Hkv, D), dtype=np.float32)
        v_new = rng.standard_normal((len(slots), Hkv, D), dtype=np.float32)
    elif slots:
        k_new = np.stack(k_new).astype(np.float32)
        v_new = np.stack(v_new).astype(np.float32)
    else:
        k_new = np.zeros((0, Hkv, D), np.float32)
        v_new = np.zeros((0, Hkv, D), np.float32)

    q = rng.standard_normal((B, W, 1, Hq, D), dtype=np.float32)

    rd = lambda a: round_to_dtype(a, dt)  # noqa: E731
    round_to_dtype(k_pool, dt, inplace=True)
    round_to_dtype(v_pool, dt, inplace=True)
    out = BeamStepInputs(
        config=spec.name, dtype=dt, batch=B, beam=W, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=D, page_size=ps, num_pages=num_pages, max_blocks=max_blocks,
        max_seq_len=max_seq_len, max_tail=spec.max_tail,
        q=rd(q), k_pool=k_pool, v_pool=v_pool, block_tables=block_tables,
        cache_indirection=ci, prefix_len=P.astype(np.int32), seq_len=S.astype(np.int32),
        k_new=rd(k_new), v_new=rd(v_new), slots=np.asarray(slots, dtype=np.int32),
    )
    if keep_logical:
        out.prompt_k = [rd(a) for a in prompt_k]
        out.prompt_v = [rd(a) for a in prompt_v]
        out.own_k = [rd(a) for a in own_k]
        out.own_v = [rd(a) for a in own_v]
    return out


@dataclass
class CachedPrefixInputs:
    """Beam-1 attention over a cache allocation with a valid prefix of L rows.

    ``cache_k``/``cache_v`` are the whole allocation, ``[max_cache_rows, Hkv, D]``;
    rows ``>= L`` hold N(0, 100) garbage, and rows ``>= nan_from_row`` hold NaN.
    ``new_k``/``new_v`` are the ``Sq`` rows of this call (one for decode).
    """

    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_cache_rows: int
    valid_rows: int
    q: np.ndarray        # float32 [Sq, Hq, D]
    cache_k: np.ndarray  # float32 [max_cache_rows, Hkv, D]
    cache_v: np.ndarray
    new_k: np.ndarray    # float32 [Sq, Hkv, D]
    new_v: np.ndarray

    @property
    def q_len(self) -> int:
        return int(self.q.shape[0])


def make_cached_prefix(seed: int = 0, *, valid_rows: Optional[int] = None,
                       q_len: int = 1, num_q_heads: int = 24, num_kv_heads: int = 8,
                       head_dim: int = 128, dtype: str = "f16",
                       max_cache_rows: int = 10368, nan_from_row: Optional[int] = None,
                       garbage: str = "normal") -> CachedPrefixInputs:
    """Draw one cached-prefix call (the Phi-4-multimodal shape by default).

    ``valid_rows`` defaults to a uniform draw in ``[0, max_cache_rows]``.
    """
    rng = np.random.default_rng(seed)
    L = int(rng.integers(0, max_cache_rows + 1)) if valid_rows is None else int(valid_rows)
    assert 0 <= L <= max_cache_rows
    shape = (max_cache_rows, num_kv_heads, head_dim)
    ck = _pool_fill(rng, shape, garbage)
    cv = _pool_fill(rng, shape, garbage)
    ck[:L] = rng.standard_normal((L, num_kv_heads, head_dim), dtype=np.float32)
    cv[:L] = rng.standard_normal((L, num_kv_heads, head_dim), dtype=np.float32)
    if nan_from_row is not None:
        ck[nan_from_row:] = np.nan
        cv[nan_from_row:] = np.nan
    q = rng.standard_normal((q_len, num_q_heads, head_dim), dtype=np.float32)
    nk = rng.standard_normal((q_len, num_kv_heads, head_dim), dtype=np.float32)
    nv = rng.standard_normal((q_len, num_kv_heads, head_dim), dtype=np.float32)
    rd = lambda a: round_to_dtype(a, dtype)  # noqa: E731
    return CachedPrefixInputs(dtype=dtype, num_q_heads=num_q_heads,
                              num_kv_heads=num_kv_heads, head_dim=head_dim,
                              max_cache_rows=max_cache_rows, valid_rows=L, q=rd(q),
                              cache_k=rd(ck), cache_v=rd(cv), new_k=rd(nk), new_v=rd(nv))


@dataclass
class PrefillInputs:
    """The context requests of a mixed step: one chunk of new rows per request.

    Request ``b`` has ``cached_len[b] = L_b`` rows already in its pages and
    ``q_len[b] = Sq_b`` new rows at positions ``L_b .. L_b + Sq_b - 1``. Query,
    new-K and new-V rows are packed request after request (``q_off``). The pool
    holds the cached rows at their pages; the chunk's positions hold garbage
    until the step's KV write puts ``new_k``/``new_v`` there through ``slots``.
    """

    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    max_blocks: int
    max_seq_len: int
    max_q_len: int
    q_len: np.ndarray         # int64 [C]
    cached_len: np.ndarray    # int64 [C]
    q: np.ndarray             # float32 [R, Hq, D], R = sum q_len
    new_k: np.ndarray         # float32 [R, Hkv, D]
    new_v: np.ndarray
    cache_k: list             # per request float32 [L_b, Hkv, D]
    cache_v: list
    k_pool: np.ndarray        # float32 [num_pages, Hkv, page_size, D]
    v_pool: np.ndarray
    block_tables: np.ndarray  # int32 [C, max_blocks], -1 past each request's blocks
    slots: np.ndarray         # int32 [R]: page * page_size + row of each new row

    @property
    def batch(self) -> int:
        return int(self.q_len.shape[0])

    @property
    def q_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_len)[:-1]]).astype(np.int64)


def make_prefill(config, seed: int = 0, *, batch: int = 4, chunk_range: tuple = (1, 600),
                 cached_range: tuple = (0, 0), head_dim: Optional[int] = None,
                 dtype: Optional[str] = None, garbage: str = "normal",
                 spare_frac: float = 0.05, max_q_len: Optional[int] = None) -> PrefillInputs:
    """Draw the context requests of a mixed step with the heads, dtype and page
    size of beam config ``config``: per request a chunk length in
    ``chunk_range`` and a cached length in ``cached_range`` (inclusive), pages
    drawn without replacement from a shuffled pool."""
    spec = BEAM_CONFIGS[config] if isinstance(config, str) else config
    D = head_dim if head_dim is not None else spec.head_dim
    dt = dtype if dtype is not None else spec.dtype
    Hq, Hkv, ps = spec.num_q_heads, spec.num_kv_heads, spec.page_size
    rng = np.random.default_rng(seed)
    C = batch
    Sq = rng.integers(chunk_range[0], chunk_range[1] + 1, size=C).astype(np.int64)
    L = rng.integers(cached_range[0], cached_range[1] + 1, size=C).astype(np.int64)
    max_seq_len = int(cached_range[1] + chunk_range[1])
    max_blocks = -(-max_seq_len // ps)
    nblk = -(-(L + Sq) // ps)
    used = int(nblk.sum())
    num_pages = used + max(1, int(used * spare_frac))
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((C, max_blocks), -1, np.int32)
    off = 0
    for b in range(C):
        bt[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += int(nblk[b])
    shape = (num_pages, Hkv, ps, D)
    kp = _pool_fill(rng, shape, garbage)
    vp = _pool_fill(rng, shape, garbage)
    rd = lambda a: round_to_dtype(a, dt)  # noqa: E731
    ck, cv = [], []
    for b in range(C):
        k = rd(rng.standard_normal((int(L[b]), Hkv, D), dtype=np.float32))
        v = rd(rng.standard_normal((int(L[b]), Hkv, D), dtype=np.float32))
        ck.append(k)
        cv.append(v)
        for j in range(int(L[b])):
            kp[bt[b, j // ps], :, j % ps, :] = k[j]
            vp[bt[b, j // ps], :, j % ps, :] = v[j]
    R = int(Sq.sum())
    q = rd(rng.standard_normal((R, Hq, D), dtype=np.float32))
    nk = rd(rng.standard_normal((R, Hkv, D), dtype=np.float32))
    nv = rd(rng.standard_normal((R, Hkv, D), dtype=np.float32))
    slots = np.empty(R, np.int32)
    r = 0
    for b in range(C):
        for i in range(int(Sq[b])):
            j = int(L[b]) + i
            slots[r] = bt[b, j // ps] * ps + j % ps
            r += 1
    return PrefillInputs(dtype=dt, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                         num_pages=num_pages, max_blocks=max_blocks, max_seq_len=max_seq_len,
                         max_q_len=int(max_q_len if max_q_len is not None else chunk_range[1]),
                         q_len=Sq, cached_len=L, q=q, new_k=nk, new_v=nv, cache_k=ck, cache_v=cv,
                         k_pool=kp, v_pool=vp, block_tables=bt, slots=slots)
