"""CPU tests of the Python binding's own argument checks (skiparse_sparse_attention_amd._lib).

Every call below is rejected by the binding before it reaches the library, so no device is
involved: shapes that do not match the grid, mismatched or non-contiguous operands, and a
log2-sum-exp vector of the wrong shape or dtype raise ValueError.
"""

import pytest
import torch

import skiparse_sparse_attention_amd as sk

GRID = (2, 4, 8)          # N = 64
SHAPE = (1, 64, 2, 128)


def _t(shape=SHAPE, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_rope_qk_rejects_bad_shapes():
    with pytest.raises(ValueError):
        sk.rope_qk(_t(), _t(), (2, 4, 4))                     # N does not match the grid
    with pytest.raises(ValueError):
        sk.rope_qk(_t(), _t((1, 64, 2, 64)), GRID)            # k differs from q
    with pytest.raises(ValueError):
        sk.rope_qk(_t(), _t(), GRID, outs=(_t(), _t(dtype=torch.float32)))
    with pytest.raises(ValueError):
        sk.rope_qk(_t((1, 64, 128)), _t((1, 64, 128)), GRID)  # not (B, N, heads, d)


def test_attn_rotated_rejects_bad_operands():
    with pytest.raises(ValueError):
        sk.attn_rotated(_t(), _t(), _t(dtype=torch.float32), GRID, 2, sk.SINGLE)
    nc = _t((1, 64, 128, 2)).transpose(2, 3)                   # right shape, not contiguous
    with pytest.raises(ValueError):
        sk.attn_rotated(_t(), nc, _t(), GRID, 2, sk.SINGLE)
    with pytest.raises(ValueError):
        sk.attn_rotated_lse(_t(), _t(), _t((1, 64, 2, 64)), GRID, 2, sk.GROUP)


def test_attn_bwd_rotated_rejects_bad_lse_and_operands():
    q = _t()
    good_lse = torch.zeros((1, 2, 64), dtype=torch.float32)
    with pytest.raises(ValueError):
        sk.attn_bwd_rotated(q, q, q, q, q, good_lse.to(torch.float64), GRID, 2, sk.SINGLE)
    with pytest.raises(ValueError):
        sk.attn_bwd_rotated(q, q, q, q, q, torch.zeros((1, 64, 2), dtype=torch.float32), GRID, 2, sk.SINGLE)
    with pytest.raises(ValueError):
        sk.attn_bwd_rotated(q, q, q, q, _t((1, 64, 2, 64)), good_lse, GRID, 2, sk.SINGLE)
