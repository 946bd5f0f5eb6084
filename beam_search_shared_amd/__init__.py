"""Cascade beam-decode attention for AMD MI355X (gfx950).

The work runs in the HIP library ``libbsp.so`` behind the C ABI declared in
``include/bsp.h``; ``_binding`` is a thin ctypes layer with the same names.
``step`` composes the entry points into one decode step of one layer.
"""

from ._binding import (  # noqa: F401
    BSP_BF16,
    BSP_F16,
    BSP_F32,
    BSP_MASK_CAUSAL,
    BSP_MASK_NONE,
    BspError,
    LayerDesc,
    Plan,
    bsp_check,
    bsp_debug_plan_tables,
    bsp_debug_tail_slots,
    bsp_decode_step,
    bsp_merge,
    bsp_naive_beam_attn,
    bsp_plan,
    bsp_prefix_attn,
    bsp_tail_attn,
    bsp_write_kv,
    declared_symbols,
    load_library,
    make_desc,
)
