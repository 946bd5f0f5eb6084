"""Index functions of a beam decode step, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The planner and the tail gather on the HIP side must reproduce these integers
bit for bit.
"""

from __future__ import annotations

import numpy as np


def prefix_page_table(prefix_len, block_tables, page_size: int, key_rows=None):
    """Pages holding each request's shared keys, as a CSR over requests.

    The shared prompt of request ``b`` is read through beam 0's block table
    (TensorRT-LLM PR #21738, KV-cache-manager-V2 commit), and its last page may
    be only partly used: a prompt of ``P`` rows in pages of ``ps`` rows spans
    ``ceil(P / ps)`` pages, so a last page holding one row gives
    ``P = (pages - 1) * ps + 1`` (review thread on ``prefix_request_tables``).

    ``key_rows[b]`` overrides the number of rows to cover (the bound row count of
    a cached prefix); it defaults to ``prefix_len``.
    Returns ``indptr int64 [B + 1]`` and ``pages int64 [indptr[-1]]``.
    """
    prefix_len = np.asarray(prefix_len)
    rows = prefix_len if key_rows is None else np.asarray(key_rows)
    counts = [-(-int(r) // page_size) for r in rows]
    indptr = np.zeros(len(counts) + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(counts)
    pages = []
    for b, c in enumerate(counts):
        pages.extend(int(p) for p in block_tables[b, 0, :c])
    return indptr, np.asarray(pages, dtype=np.int64)


def tail_slots(prefix_len, seq_len, block_tables, cache_indirection, page_size: int,
               tail_pad: int):
    """Flat pool slot of every tail key of every beam, padded with -1.

    Tail position ``t`` of beam ``k`` of request ``b`` is sequence position
    ``j = P_b + t``; it is read from beam ``src = cache_indirection[b, k, j]``,
    page ``block_tables[b, src, j // ps]``, row ``j % ps`` (Solution section of
    PR #21738: each beam's generated tokens are gathered through
    cache_indirection). The slot is ``page * ps + row``. Positions ``t >=
    S_b - P_b`` (padding up to ``tail_pad``) are -1.
    Returns ``int64 [B, W, tail_pad]``.
    """
    B, W = block_tables.shape[:2]
    out = np.full((B, W, tail_pad), -1, dtype=np.int64)
    for b in range(B):
        P, S = int(prefix_len[b]), int(seq_len[b])
        for k in range(W):
            for t in range(min(S - P, tail_pad)):
                j = P + t
                src = int(cache_indirection[b, k, j])
                page = int(block_tables[b, src, j // page_size])
                out[b, k, t] = page * page_size + j % page_size
    return out
