"""One decode step of one layer, composed from the C entry points.

torch is used for device memory and streams only: every arithmetic step runs in
libbsp's kernels. A beam step is

    bsp_write_kv     current token of every beam -> its own page
    bsp_prefix_attn  all beams' query rows x the shared prompt, once per request
    bsp_tail_attn    each beam's tail through cache_indirection
    bsp_merge        exact LSE merge of the two partial states

or, fused into one launch, ``bsp_decode_step``;
and a cached-prefix call (beam 1) is

    bsp_write_kv     this call's rows -> scratch pages
    bsp_prefix_attn  the bound cache rows (valid rows only), split into chunks
    bsp_prefix_attn  this call's rows, causal
    bsp_merge        n-way merge of all the partial states

or, for a one-row decode, all four in one launch (``bsp_cached_decode``);

and a mixed step (context requests beside generation requests) is

    bsp_write_kv     the context chunks' rows -> their requests' pages
    bsp_prefill_attn causal attention of every context row (ragged, one launch)
    bsp_decode_step  the generation requests' beam step

with the context part on a second stream when one is given.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _binding as B

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload float32 values (already representable in ``dtype``) exactly."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device).to(TORCH_DTYPE[dtype])


def _i32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


@dataclass
class BeamStepDevice:
    dtype: str
    batch: int
    beam: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    plan: B.Plan
    prefix_len: np.ndarray
    seq_len: np.ndarray
    block_tables_h: np.ndarray
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_tables: torch.Tensor
    cache_indirection: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    slots: torch.Tensor
    workspace: torch.Tensor
    o_part: torch.Tensor     # float [2, rows, Hq, D]: part 0 prefix, part 1 tail
    lse_part: torch.Tensor   # float [2, rows, Hq]
    out: torch.Tensor        # dtype [rows, Hq, D]
    lse_out: torch.Tensor    # float [rows, Hq]
    k_new_beams: torch.Tensor = None  # dtype [B*W, Hkv, D]: current token by beam (fused step)
    v_new_beams: torch.Tensor = None

    @property
    def rows(self) -> int:
        return self.batch * self.beam


def upload_beam_step(inp, device="cuda", max_tail: Optional[int] = None,
                     sm_scale: float = 0.0) -> BeamStepDevice:
    """Copy a ``synth.BeamStepInputs`` to the GPU and create its plan."""
    mt = inp.max_tail if max_tail is None else max_tail
    desc = B.make_desc(inp.num_q_heads, inp.num_kv_heads, inp.head_dim, inp.page_size,
                       inp.num_pages, inp.dtype, sm_scale=sm_scale, max_tail=mt)
    plan = B.Plan(desc, max_requests=inp.batch, max_beam=inp.beam,
                  max_blocks_per_seq=inp.max_blocks, max_seq_len=inp.max_seq_len, max_q_len=1)
    rows, Hq, D = inp.batch * inp.beam, inp.num_q_heads, inp.head_dim
    f32 = dict(device=device, dtype=torch.float32)
    # The fused step reads every beam's current token as row b * W + k; the
    # generator lists them only for requests with a tail, request-major.
    beam_rows = [b * inp.beam + k for b in range(inp.batch) if inp.tail_len[b] > 0
                 for k in range(inp.beam)]
    knb = np.zeros((rows, inp.num_kv_heads, D), np.float32)
    vnb = np.zeros((rows, inp.num_kv_heads, D), np.float32)
    if beam_rows:
        knb[beam_rows] = inp.k_new
        vnb[beam_rows] = inp.v_new
    return BeamStepDevice(
        dtype=inp.dtype, batch=inp.batch, beam=inp.beam, num_q_heads=Hq,
        num_kv_heads=inp.num_kv_heads, head_dim=D, plan=plan,
        prefix_len=inp.prefix_len.copy(), seq_len=inp.seq_len.copy(),
        block_tables_h=inp.block_tables.copy(),
        q=to_device(inp.q, inp.dtype, device),
        k_pool=to_device(inp.k_pool, inp.dtype, device),
        v_pool=to_device(inp.v_pool, inp.dtype, device),
        block_tables=_i32(inp.block_tables, device),
        cache_indirection=_i32(inp.cache_indirection, device),
        k_new=to_device(inp.k_new, inp.dtype, device),
        v_new=to_device(inp.v_new, inp.dtype, device),
        slots=_i32(inp.slots, device),
        workspace=torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=device),
        o_part=torch.zeros((2, rows, Hq, D), **f32),
        lse_part=torch.zeros((2, rows, Hq), **f32),
        out=torch.zeros((rows, Hq, D), device=device, dtype=TORCH_DTYPE[inp.dtype]),
        lse_out=torch.zeros((rows, Hq), **f32),
        k_new_beams=to_device(knb, inp.dtype, device),
        v_new_beams=to_device(vnb, inp.dtype, device),
    )


def plan_beam_step(s: BeamStepDevice, stream=None) -> None:
    B.bsp_plan(s.plan, s.batch, s.beam, 1, s.prefix_len, s.seq_len, s.block_tables_h,
               s.workspace, stream)


def write_current_tokens(s: BeamStepDevice, stream=None) -> None:
    n = int(s.slots.numel())
    B.bsp_write_kv(s.plan, s.k_new, s.v_new, s.num_kv_heads * s.head_dim, s.slots, n,
                   s.k_pool, s.v_pool, stream)


def run_beam_step(s: BeamStepDevice, stream=None, write: bool = True) -> None:
    """write_kv + prefix + tail + merge for the current plan (plan_beam_step first)."""
    if write:
        write_current_tokens(s, stream)
    B.bsp_prefix_attn(s.plan, s.q, s.k_pool, s.v_pool, s.o_part[0], s.lse_part[0], stream)
    B.bsp_tail_attn(s.plan, s.q, s.k_pool, s.v_pool, s.block_tables, s.cache_indirection,
                    s.o_part[1], s.lse_part[1], stream)
    rows = s.rows
    B.bsp_merge(rows, s.num_q_heads, s.head_dim, 2, s.o_part, s.lse_part,
                rows * s.num_q_heads * s.head_dim, rows * s.num_q_heads, s.out, s.dtype,
                s.lse_out, stream)


def run_decode_step(s: BeamStepDevice, stream=None) -> None:
    """The whole step in one launch (bsp_decode_step): token write + prefix + tail."""
    B.bsp_decode_step(s.plan, s.q, s.k_new_beams, s.v_new_beams, s.num_kv_heads * s.head_dim,
                      s.k_pool, s.v_pool, s.block_tables, s.cache_indirection, s.out,
                      s.lse_out, stream)


def paged_from_rows(rows: np.ndarray, page_size: int, num_pages: int,
                    fill: float = float("nan")) -> np.ndarray:
    """Lay a row array ``[n, Hkv, D]`` out as identity pages ``[num_pages, Hkv, ps, D]``
    (host-side layout before the upload, no arithmetic on the values): page p
    holds rows ``p*ps .. p*ps+ps-1``; rows past ``n`` hold ``fill``."""
    n, hkv, d = rows.shape
    assert num_pages * page_size >= n
    out = np.full((num_pages * page_size, hkv, d), fill, dtype=np.float32)
    out[:n] = rows
    return np.ascontiguousarray(out.reshape(num_pages, page_size, hkv, d).transpose(0, 2, 1, 3))


@dataclass
class CachedPrefixDevice:
    dtype: str
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    cache_pages: int
    plan_cache: B.Plan
    plan_new: B.Plan
    valid_rows: int
    bt_cache: np.ndarray
    bt_new: np.ndarray
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    new_k: torch.Tensor
    new_v: torch.Tensor
    slots: torch.Tensor
    ws_cache: torch.Tensor
    ws_new: torch.Tensor
    o_part: Optional[torch.Tensor] = None
    lse_part: Optional[torch.Tensor] = None
    out: Optional[torch.Tensor] = None
    lse_out: Optional[torch.Tensor] = None
    n_split: int = 1


def upload_cached_prefix(inp, device="cuda", page_size: int = 32, key_bucket: int = 256,
                         kv_split: Optional[int] = None, causal: bool = True,
                         pool_fill: float = float("nan")) -> CachedPrefixDevice:
    """Lay a ``synth.CachedPrefixInputs`` out as identity pages plus scratch pages.

    The cache allocation ``[max_cache_rows, Hkv, D]`` becomes pages
    ``0 .. cache_pages-1`` (page p holds rows p*ps .. p*ps+ps-1); this call's
    rows go to scratch pages after them through ``bsp_write_kv``.
    ``kv_split`` defaults to -1: the plan picks the chunk per step (the
    smallest multiple of 64 keys whose work items fill one round of the chip).
    """
    ps = page_size
    Sq, Hq, D = inp.q.shape
    Hkv = inp.cache_k.shape[1]
    rows = inp.max_cache_rows
    cache_pages = -(-rows // ps)
    new_pages = -(-Sq // ps)
    num_pages = cache_pages + new_pages
    split = -1 if kv_split is None else kv_split
    mk = lambda **kw: B.make_desc(Hq, Hkv, D, ps, num_pages, inp.dtype, **kw)  # noqa: E731
    d_cache = mk(key_bucket=key_bucket, max_cache_rows=rows, kv_split=split)
    d_new = mk(mask=B.BSP_MASK_CAUSAL if causal else B.BSP_MASK_NONE)
    plan_cache = B.Plan(d_cache, 1, 1, cache_pages, rows, Sq)
    plan_new = B.Plan(d_new, 1, 1, new_pages, Sq, Sq)
    kpool = paged_from_rows(inp.cache_k, ps, num_pages, fill=pool_fill)
    vpool = paged_from_rows(inp.cache_v, ps, num_pages, fill=pool_fill)
    bt_cache = np.arange(cache_pages, dtype=np.int32).reshape(1, 1, -1)
    bt_new = (cache_pages + np.arange(new_pages, dtype=np.int32)).reshape(1, 1, -1)
    slots = (cache_pages * ps + np.arange(Sq)).astype(np.int32)
    return CachedPrefixDevice(
        dtype=inp.dtype, q_len=Sq, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
        cache_pages=cache_pages, plan_cache=plan_cache, plan_new=plan_new,
        valid_rows=int(inp.valid_rows), bt_cache=bt_cache, bt_new=bt_new,
        q=to_device(inp.q.reshape(1, 1, Sq, Hq, D), inp.dtype, device),
        k_pool=to_device(kpool, inp.dtype, device), v_pool=to_device(vpool, inp.dtype, device),
        new_k=to_device(inp.new_k, inp.dtype, device), new_v=to_device(inp.new_v, inp.dtype, device),
        slots=_i32(slots, device),
        ws_cache=torch.zeros(plan_cache.workspace_bytes, dtype=torch.uint8, device=device),
        ws_new=torch.zeros(plan_new.workspace_bytes, dtype=torch.uint8, device=device),
    )


def plan_cached_prefix(c: CachedPrefixDevice, stream=None) -> None:
    L = np.array([c.valid_rows], np.int32)
    Sq = np.array([c.q_len], np.int32)
    B.bsp_plan(c.plan_cache, 1, 1, c.q_len, L, L, c.bt_cache, c.ws_cache, stream)
    B.bsp_plan(c.plan_new, 1, 1, c.q_len, Sq, Sq, c.bt_new, c.ws_new, stream)
    n_split = c.plan_cache.num_splits
    if c.o_part is None or c.n_split != n_split:
        dev = c.q.device
        rows, Hq, D = c.q_len, c.num_q_heads, c.head_dim
        c.n_split = n_split
        c.o_part = torch.zeros((n_split + 1, rows, Hq, D), device=dev, dtype=torch.float32)
        c.lse_part = torch.zeros((n_split + 1, rows, Hq), device=dev, dtype=torch.float32)
        c.out = torch.zeros((rows, Hq, D), device=dev, dtype=TORCH_DTYPE[c.dtype])
        c.lse_out = torch.zeros((rows, Hq), device=dev, dtype=torch.float32)


def run_cached_prefix(c: CachedPrefixDevice, stream=None, two_launches: bool = False) -> None:
    """write new rows + cache segment and new-row segment (one launch when both take
    64-row tiles, as in a one-row decode; ``two_launches`` forces one launch each)
    + n-way merge."""
    Hkv, D = c.num_kv_heads, c.head_dim
    B.bsp_write_kv(c.plan_new, c.new_k, c.new_v, Hkv * D, c.slots, c.q_len, c.k_pool, c.v_pool,
                   stream)
    ns = c.n_split
    if two_launches:
        B.bsp_prefix_attn(c.plan_cache, c.q, c.k_pool, c.v_pool, c.o_part[:ns], c.lse_part[:ns],
                          stream)
        B.bsp_prefix_attn(c.plan_new, c.q, c.k_pool, c.v_pool, c.o_part[ns], c.lse_part[ns],
                          stream)
    else:
        B.bsp_prefix_attn_two(c.plan_cache, c.plan_new, c.q, c.k_pool, c.v_pool, c.o_part[:ns],
                              c.lse_part[:ns], c.o_part[ns], c.lse_part[ns], stream)
    rows = c.q_len
    B.bsp_merge(rows, c.num_q_heads, D, ns + 1, c.o_part, c.lse_part, rows * c.num_q_heads * D,
                rows * c.num_q_heads, c.out, c.dtype, c.lse_out, stream)


def run_cached_decode(c: CachedPrefixDevice, stream=None) -> None:
    """A one-row cached-prefix decode call in one launch (bsp_cached_decode): the
    cache chunks, the merge with this call's row and the row's write into its
    page."""
    ns = c.n_split
    B.bsp_cached_decode(c.plan_cache, c.q, c.new_k, c.new_v, c.num_kv_heads * c.head_dim, c.slots,
                        c.k_pool, c.v_pool, c.o_part[:ns], c.lse_part[:ns], c.out, c.lse_out,
                        stream)


def run_cached_decode_two(c: CachedPrefixDevice, stream=None) -> None:
    """A one-row cached-prefix decode call in two launches: the cache chunks
    (bsp_prefix_attn), then their merge with this call's row and the row's write
    into its page (bsp_cached_decode_merge)."""
    ns = c.n_split
    B.bsp_prefix_attn(c.plan_cache, c.q, c.k_pool, c.v_pool, c.o_part[:ns], c.lse_part[:ns], stream)
    B.bsp_cached_decode_merge(c.plan_cache, c.q, c.new_k, c.new_v, c.num_kv_heads * c.head_dim,
                              c.slots, c.k_pool, c.v_pool, c.o_part[:ns], c.lse_part[:ns], c.out,
                              c.lse_out, stream)


@dataclass
class PrefillDevice:
    """The context requests of a mixed step on the device, with their plan."""

    dtype: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    plan: B.Plan
    q_len: np.ndarray
    cached_len: np.ndarray
    block_tables_h: np.ndarray
    q: torch.Tensor          # dtype [R, Hq, D], packed by request
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    new_k: torch.Tensor      # dtype [R, Hkv, D]
    new_v: torch.Tensor
    slots: torch.Tensor      # int32 [R]
    workspace: torch.Tensor
    out: torch.Tensor        # dtype [R, Hq, D]
    lse_out: torch.Tensor    # float [R, Hq]

    @property
    def rows(self) -> int:
        return int(self.q_len.sum())


def upload_prefill(inp, device="cuda", plan_desc_kw: Optional[dict] = None) -> PrefillDevice:
    """Copy a ``synth.PrefillInputs`` to the GPU and create its plan."""
    desc = B.make_desc(inp.num_q_heads, inp.num_kv_heads, inp.head_dim, inp.page_size,
                       inp.num_pages, inp.dtype, **(plan_desc_kw or {}))
    plan = B.Plan(desc, max_requests=inp.batch, max_beam=1, max_blocks_per_seq=inp.max_blocks,
                  max_seq_len=inp.max_seq_len, max_q_len=inp.max_q_len)
    R, Hq, D = inp.q.shape
    return PrefillDevice(
        dtype=inp.dtype, batch=inp.batch, num_q_heads=Hq, num_kv_heads=inp.num_kv_heads,
        head_dim=D, plan=plan, q_len=inp.q_len.astype(np.int32),
        cached_len=inp.cached_len.astype(np.int32), block_tables_h=inp.block_tables.copy(),
        q=to_device(inp.q, inp.dtype, device),
        k_pool=to_device(inp.k_pool, inp.dtype, device),
        v_pool=to_device(inp.v_pool, inp.dtype, device),
        new_k=to_device(inp.new_k, inp.dtype, device),
        new_v=to_device(inp.new_v, inp.dtype, device),
        slots=_i32(inp.slots, device),
        workspace=torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=device),
        out=torch.zeros((R, Hq, D), device=device, dtype=TORCH_DTYPE[inp.dtype]),
        lse_out=torch.zeros((R, Hq), device=device, dtype=torch.float32),
    )


def plan_prefill(c: PrefillDevice, stream=None) -> None:
    B.bsp_plan_prefill(c.plan, c.batch, c.q_len, c.cached_len, c.block_tables_h, c.workspace,
                       stream)


def run_prefill(c: PrefillDevice, stream=None, write: bool = True) -> None:
    """The context phase: write the chunks' rows, then causal attention of every row."""
    if write:
        B.bsp_write_kv(c.plan, c.new_k, c.new_v, c.num_kv_heads * c.head_dim, c.slots, c.rows,
                       c.k_pool, c.v_pool, stream)
    B.bsp_prefill_attn(c.plan, c.q, c.k_pool, c.v_pool, c.out, c.lse_out, stream)


def run_mixed_step_fused(ctx: PrefillDevice, gen: BeamStepDevice, stream=None) -> None:
    """One mixed step through bsp_mixed_step: the context chunks' KV write, then
    the prefill and the beam step in one launch (two when the shapes do not
    allow it)."""
    B.bsp_write_kv(ctx.plan, ctx.new_k, ctx.new_v, ctx.num_kv_heads * ctx.head_dim, ctx.slots,
                   ctx.rows, ctx.k_pool, ctx.v_pool, stream)
    B.bsp_mixed_step(gen.plan, ctx.plan, gen.q, gen.k_new_beams, gen.v_new_beams,
                     gen.num_kv_heads * gen.head_dim, gen.k_pool, gen.v_pool, gen.block_tables,
                     gen.cache_indirection, gen.out, gen.lse_out, ctx.q, ctx.k_pool, ctx.v_pool,
                     ctx.out, ctx.lse_out, stream)


def run_mixed_step(ctx: PrefillDevice, gen: BeamStepDevice, stream=None,
                   ctx_stream=None) -> None:
    """One mixed step: the context requests' prefill and the generation requests'
    fused beam step. The two touch disjoint pages; with ``ctx_stream`` the
    prefill (matrix-core heavy) runs beside the beam step (HBM heavy) and
    ``stream`` waits for it at the end."""
    if ctx_stream is None:
        run_prefill(ctx, stream)
        run_decode_step(gen, stream)
        return
    main = torch.cuda.current_stream() if stream is None else stream
    ready = torch.cuda.Event()
    ready.record(main)
    ctx_stream.wait_event(ready)
    run_prefill(ctx, ctx_stream)
    run_decode_step(gen, main)
    done = torch.cuda.Event()
    done.record(ctx_stream)
    main.wait_event(done)
