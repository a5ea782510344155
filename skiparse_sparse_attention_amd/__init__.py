"""Skiparse sparse attention for AMD MI355X (gfx950).

The computation lives in the HIP library ``libskiparse_amd.so`` (C ABI in
include/skiparse.h); this package is its Python binding.  Loading is lazy:
importing the package does not open the library, the first call does, and it
raises if the library has not been built.
"""

from ._lib import (  # noqa: F401
    BF16,
    E_ALIAS,
    E_DEVICE,
    E_DIVISIBILITY,
    E_NULL,
    E_SHAPE,
    E_UNSUPPORTED,
    E_WORKSPACE,
    FP32,
    GROUP,
    LIB_PATH,
    Layer,
    MAX_GRID_SUM,
    OK,
    SINGLE,
    STATIC_DELTA_MAX,
    SkiparseError,
    attn,
    attn8,
    attn_bwd,
    attn_bwd_rotated,
    attn_bwd_rotated_static,
    attn_schedule,
    attn_schedule_rotated,
    attn_bwd_flops,
    attn_flops,
    attn_lse,
    attn_rotated,
    attn_rotated_lse,
    lib,
    probe_mfma,
    probe_stream,
    q8_scope_pitch,
    quant8,
    rearrange,
    reverse,
    rope_qk,
    rope_remap,
    scope_table,
    status_string,
    u_schedule,
    version,
)
