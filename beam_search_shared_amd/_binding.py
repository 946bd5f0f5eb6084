"""ctypes binding of libbsp (include/bsp.h): argument marshalling only.

Every function here has the name of the C entry point it calls and does no
computation of its own: it converts tensors to raw pointers, arrays to int32
host buffers and the current torch stream to a hipStream_t, then raises
``BspError`` on a non-zero status. If the HIP library is not built, loading
fails loudly; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# BSP_LIBRARY names another build of the same ABI (the sanitized host-only build
# the CPU tests load); by default the in-tree gfx950 library.
LIB_PATH = os.environ.get("BSP_LIBRARY") or os.path.join(HERE, "libbsp.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "bsp.h")

BSP_F32, BSP_F16, BSP_BF16 = 0, 1, 2
BSP_MASK_NONE, BSP_MASK_CAUSAL = 0, 1
BSP_PLAN_HOST_ONLY = 1

STATUS = {
    0: "BSP_OK", 1: "BSP_ERR_ARG", 2: "BSP_ERR_PAGE_INDEX", 3: "BSP_ERR_TAIL_OVERFLOW",
    4: "BSP_ERR_DTYPE", 5: "BSP_ERR_UNSUPPORTED", 6: "BSP_ERR_STALE_PLAN",
    7: "BSP_ERR_WORKSPACE", 8: "BSP_ERR_DEVICE_INDEX", 9: "BSP_ERR_HIP",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

DTYPE_CODE = {"f32": BSP_F32, "f16": BSP_F16, "bf16": BSP_BF16}


class BspError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("max_tail", ctypes.c_int32),
        ("key_bucket", ctypes.c_int32),
        ("max_cache_rows", ctypes.c_int32),
        ("mask", ctypes.c_int32),
        ("kv_split", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64

_SIGS = {
    "bsp_last_error": (ctypes.c_char_p, []),
    "bsp_version": (_I32, []),
    "bsp_plan_create": (_I32, [ctypes.POINTER(LayerDesc), _I32, _I32, _I32, _I32, _I32,
                               ctypes.c_uint32, ctypes.POINTER(_P)]),
    "bsp_plan_workspace_bytes": (ctypes.c_size_t, [_P]),
    "bsp_plan_destroy": (None, [_P]),
    "bsp_plan": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "bsp_plan_static": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P, _P]),
    "bsp_plan_num_splits": (_I32, [_P]),
    "bsp_plan_split_keys": (_I32, [_P]),
    "bsp_plan_tail_len": (_I32, [_P]),
    "bsp_write_kv": (_I32, [_P, _P, _P, _I64, _P, _I32, _P, _P, _P]),
    "bsp_prefix_attn": (_I32, [_P, _P, _P, _P, _P, _P, _P]),
    "bsp_prefix_attn_two": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "bsp_cached_decode": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "bsp_cached_decode_merge": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "bsp_tail_attn": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "bsp_merge": (_I32, [_I32, _I32, _I32, _I32, _P, _P, _I64, _I64, _P, _I32, _P, _P]),
    "bsp_naive_beam_attn": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "bsp_decode_step": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "bsp_plan_prefill": (_I32, [_P, _I32, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "bsp_mixed_step": (_I32, [_P, _P, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              _P, _P]),
    "bsp_prefill_attn": (_I32, [_P, _P, _P, _P, _P, _P, _P]),
    "bsp_check": (_I32, [_P, _P]),
    "bsp_debug_plan_tables": (_I32, [_P, _P, _P, _P, _P, _P]),
    "bsp_debug_plan_items": (_I32, [_P, _P, _P]),
    "bsp_debug_tail_slots": (_I32, [_P, _P, _P, _P, _P]),
    "bsp_write_kv_desc": (_I32, [_P, _P, _P, _I64, _P, _I32, _P, _P, _P, _P]),
    "bsp_debug_fused_slots": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbsp.so (built by ``python -m beam_search_shared_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libbsp.so is not built ({path}); run "
                           "`python -m beam_search_shared_amd.build` first")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def declared_symbols(header: str = HEADER_PATH) -> list:
    """Names of the functions include/bsp.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsp_\w+)\s*\(", text)))


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().bsp_last_error().decode(errors="replace")
        raise BspError(status, msg)


def _ptr(x) -> Optional[int]:
    """Raw address of a tensor / ndarray / int; None stays null."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _host_i32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a


class Plan:
    """Owner of a ``bsp_plan_t`` handle (destroyed with the object)."""

    def __init__(self, desc: LayerDesc, max_requests: int, max_beam: int,
                 max_blocks_per_seq: int, max_seq_len: int, max_q_len: int = 1,
                 host_only: bool = False):
        lib = load_library()
        self.desc = desc
        self.handle = ctypes.c_void_p()
        flags = BSP_PLAN_HOST_ONLY if host_only else 0
        _check(lib.bsp_plan_create(ctypes.byref(desc), max_requests, max_beam,
                                   max_blocks_per_seq, max_seq_len, max_q_len, flags,
                                   ctypes.byref(self.handle)))
        self.host_only = host_only
        self.max_requests = max_requests
        self.max_beam = max_beam
        self.max_blocks = max_blocks_per_seq
        self.max_seq_len = max_seq_len
        self._keep = []  # host arrays of the current plan, kept alive for the copy

    @property
    def workspace_bytes(self) -> int:
        return int(load_library().bsp_plan_workspace_bytes(self.handle))

    @property
    def num_splits(self) -> int:
        return int(load_library().bsp_plan_num_splits(self.handle))

    @property
    def split_keys(self) -> int:
        return int(load_library().bsp_plan_split_keys(self.handle))

    @property
    def tail_len(self) -> int:
        return int(load_library().bsp_plan_tail_len(self.handle))

    def close(self) -> None:
        if self.handle:
            load_library().bsp_plan_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def make_desc(num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
              num_pages: int, dtype: str, sm_scale: float = 0.0, max_tail: int = 0,
              key_bucket: int = 0, max_cache_rows: int = 0, mask: int = BSP_MASK_NONE,
              kv_split: int = 0) -> LayerDesc:
    return LayerDesc(num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                     DTYPE_CODE[dtype], sm_scale, max_tail, key_bucket, max_cache_rows, mask,
                     kv_split)


def bsp_plan(plan: Plan, B: int, W: int, q_len: int, prefix_len, seq_len, block_tables,
             workspace=None, stream=None) -> None:
    pl = _host_i32(prefix_len)
    sl = _host_i32(seq_len)
    bt = _host_i32(block_tables)
    plan._keep = [pl, sl, bt]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = None if plan.host_only else _stream(stream)
    _check(load_library().bsp_plan(plan.handle, B, W, q_len, _ptr(pl), _ptr(sl), _ptr(bt),
                                   _ptr(workspace), nbytes, st))


def bsp_plan_static(plan: Plan, B: int, W: int, q_len: int, prefix_len, seq_len, block_tables,
                    stream=None) -> None:
    pl = _host_i32(prefix_len)
    sl = _host_i32(seq_len)
    bt = _host_i32(block_tables)
    plan._keep = [pl, sl, bt]
    _check(load_library().bsp_plan_static(plan.handle, B, W, q_len, _ptr(pl), _ptr(sl), _ptr(bt),
                                          _stream(stream)))


def bsp_write_kv(plan: Plan, k_new, v_new, src_row_stride: int, slots, n: int, k_pool, v_pool,
                 stream=None) -> None:
    _check(load_library().bsp_write_kv(plan.handle, _ptr(k_new), _ptr(v_new), src_row_stride,
                                       _ptr(slots), n, _ptr(k_pool), _ptr(v_pool),
                                       _stream(stream)))


def bsp_prefix_attn(plan: Plan, q, k_pool, v_pool, o_part, lse_part, stream=None) -> None:
    _check(load_library().bsp_prefix_attn(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                          _ptr(o_part), _ptr(lse_part), _stream(stream)))


def bsp_prefix_attn_two(plan_a: Plan, plan_b: Plan, q, k_pool, v_pool, o_part_a, lse_part_a,
                        o_part_b, lse_part_b, stream=None) -> None:
    _check(load_library().bsp_prefix_attn_two(plan_a.handle, plan_b.handle, _ptr(q), _ptr(k_pool),
                                              _ptr(v_pool), _ptr(o_part_a), _ptr(lse_part_a),
                                              _ptr(o_part_b), _ptr(lse_part_b), _stream(stream)))


def bsp_cached_decode(plan: Plan, q, k_new, v_new, new_row_stride: int, slots, k_pool, v_pool,
                      o_part, lse_part, o_out, lse_out=None, stream=None) -> None:
    _check(load_library().bsp_cached_decode(plan.handle, _ptr(q), _ptr(k_new), _ptr(v_new),
                                            new_row_stride, _ptr(slots), _ptr(k_pool),
                                            _ptr(v_pool), _ptr(o_part), _ptr(lse_part),
                                            _ptr(o_out), _ptr(lse_out), _stream(stream)))


def bsp_cached_decode_merge(plan: Plan, q, k_new, v_new, new_row_stride: int, slots, k_pool,
                            v_pool, o_part, lse_part, o_out, lse_out=None, stream=None) -> None:
    _check(load_library().bsp_cached_decode_merge(plan.handle, _ptr(q), _ptr(k_new), _ptr(v_new),
                                                  new_row_stride, _ptr(slots), _ptr(k_pool),
                                                  _ptr(v_pool), _ptr(o_part), _ptr(lse_part),
                                                  _ptr(o_out), _ptr(lse_out), _stream(stream)))


def bsp_tail_attn(plan: Plan, q, k_pool, v_pool, block_tables, cache_indirection, o_tail,
                  lse_tail, stream=None) -> None:
    _check(load_library().bsp_tail_attn(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                        _ptr(block_tables), _ptr(cache_indirection),
                                        _ptr(o_tail), _ptr(lse_tail), _stream(stream)))


def bsp_merge(rows: int, heads: int, head_dim: int, n_parts: int, o_parts, lse_parts,
              o_part_stride: int, lse_part_stride: int, o_out, out_dtype: str, lse_out=None,
              stream=None) -> None:
    _check(load_library().bsp_merge(rows, heads, head_dim, n_parts, _ptr(o_parts),
                                    _ptr(lse_parts), o_part_stride, lse_part_stride,
                                    _ptr(o_out), DTYPE_CODE[out_dtype], _ptr(lse_out),
                                    _stream(stream)))


def bsp_naive_beam_attn(plan: Plan, q, k_pool, v_pool, block_tables, cache_indirection, o_out,
                        lse_out=None, stream=None) -> None:
    _check(load_library().bsp_naive_beam_attn(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                              _ptr(block_tables), _ptr(cache_indirection),
                                              _ptr(o_out), _ptr(lse_out), _stream(stream)))


def bsp_decode_step(plan: Plan, q, k_new, v_new, new_row_stride: int, k_pool, v_pool,
                    block_tables, cache_indirection, o_out, lse_out=None, stream=None) -> None:
    _check(load_library().bsp_decode_step(plan.handle, _ptr(q), _ptr(k_new), _ptr(v_new),
                                          new_row_stride, _ptr(k_pool), _ptr(v_pool),
                                          _ptr(block_tables), _ptr(cache_indirection),
                                          _ptr(o_out), _ptr(lse_out), _stream(stream)))


def bsp_plan_prefill(plan: Plan, C: int, q_len, cached_len, block_tables, workspace=None,
                     stream=None) -> None:
    ql = _host_i32(q_len)
    cl = _host_i32(cached_len)
    bt = _host_i32(block_tables)
    plan._keep = [ql, cl, bt]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = None if plan.host_only else _stream(stream)
    _check(load_library().bsp_plan_prefill(plan.handle, C, _ptr(ql), _ptr(cl), _ptr(bt),
                                           _ptr(workspace), nbytes, st))


def bsp_prefill_attn(plan: Plan, q, k_pool, v_pool, o_out, lse_out=None, stream=None) -> None:
    _check(load_library().bsp_prefill_attn(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                           _ptr(o_out), _ptr(lse_out), _stream(stream)))


def bsp_mixed_step(gen: Plan, ctx: Plan, q, k_new, v_new, new_row_stride: int, k_pool, v_pool,
                   block_tables, cache_indirection, o_out, lse_out, q_ctx, k_pool_ctx, v_pool_ctx,
                   o_ctx, lse_ctx=None, stream=None) -> None:
    _check(load_library().bsp_mixed_step(gen.handle, ctx.handle, _ptr(q), _ptr(k_new),
                                         _ptr(v_new), new_row_stride, _ptr(k_pool), _ptr(v_pool),
                                         _ptr(block_tables), _ptr(cache_indirection), _ptr(o_out),
                                         _ptr(lse_out), _ptr(q_ctx), _ptr(k_pool_ctx),
                                         _ptr(v_pool_ctx), _ptr(o_ctx), _ptr(lse_ctx),
                                         _stream(stream)))


def bsp_check(plan: Plan, stream=None) -> None:
    _check(load_library().bsp_check(plan.handle, _stream(stream)))


def bsp_debug_plan_tables(plan: Plan, B: int):
    """Host copy of the plan tables: indptr, pages, n_keys, valid, tail (int32 arrays)."""
    lib = load_library()
    indptr = np.zeros(B + 1, np.int32)
    n_keys = np.zeros(B, np.int32)
    valid = np.zeros(B, np.int32)
    tail = np.zeros(B, np.int32)
    _check(lib.bsp_debug_plan_tables(plan.handle, _ptr(indptr), None, _ptr(n_keys), _ptr(valid),
                                     _ptr(tail)))
    pages = np.zeros(max(int(indptr[B]), 1), np.int32)
    _check(lib.bsp_debug_plan_tables(plan.handle, None, _ptr(pages), None, None, None))
    return indptr, pages[:int(indptr[B])], n_keys, valid, tail


def bsp_debug_plan_items(plan: Plan):
    """The fused step's work items as an int32 array [n_items][4] = (request,
    first key, end key, chunks of that request), in dispatch order."""
    lib = load_library()
    n = np.zeros(1, np.int32)
    _check(lib.bsp_debug_plan_items(plan.handle, _ptr(n), None))
    items = np.zeros((max(int(n[0]), 1), 4), np.int32)
    _check(lib.bsp_debug_plan_items(plan.handle, _ptr(n), _ptr(items)))
    return items[:int(n[0])]


def bsp_write_kv_desc(desc: LayerDesc, k_new, v_new, src_row_stride: int, slots, n: int,
                      k_pool, v_pool, faults=None, stream=None) -> None:
    _check(load_library().bsp_write_kv_desc(None if desc is None else ctypes.byref(desc),
                                            _ptr(k_new), _ptr(v_new),
                                            src_row_stride, _ptr(slots), n, _ptr(k_pool),
                                            _ptr(v_pool), _ptr(faults), _stream(stream)))


def bsp_debug_tail_slots(plan: Plan, block_tables, cache_indirection, slots_out,
                         stream=None) -> None:
    _check(load_library().bsp_debug_tail_slots(plan.handle, _ptr(block_tables),
                                               _ptr(cache_indirection), _ptr(slots_out),
                                               _stream(stream)))


def bsp_debug_fused_slots(plan: Plan, q, k_new, v_new, new_row_stride: int, k_pool, v_pool,
                          block_tables, cache_indirection, o_out, slots_out,
                          stream=None) -> None:
    _check(load_library().bsp_debug_fused_slots(plan.handle, _ptr(q), _ptr(k_new), _ptr(v_new),
                                                new_row_stride, _ptr(k_pool), _ptr(v_pool),
                                                _ptr(block_tables), _ptr(cache_indirection),
                                                _ptr(o_out), _ptr(slots_out), _stream(stream)))
