"""fp64 CPU oracle of Skiparse attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and
the oracle imports nothing from the product package.
"""

from . import skiparse_oracle8  # noqa: F401  (8-bit Skiparse attention)
from .skiparse_oracle import (  # noqa: F401
    GROUP,
    ROPE_BASE,
    SINGLE,
    attention,
    attention_backward,
    rearrange,
    reverse,
    reverse_rows,
    rope_3d,
    rope_3d_at,
    rope_3d_transpose_at,
    rope_axis_sizes,
    rope_rearrange,
    scope_table,
    skiparse_attention,
    skiparse_attention_backward,
    skiparse_attention_backward_scope,
    skiparse_backward_flops,
    skiparse_attention_rows,
    skiparse_flops,
    token_positions,
    token_scope,
)
