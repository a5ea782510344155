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


# ---------------------------------------------------------------------------
# Every tensor a wrapper passes is checked (shape, dtype, contiguity, then GPU residence)
# before the library is called.  The library is replaced by a stub whose compute entry
# points fail the test if they are ever reached.
# ---------------------------------------------------------------------------

from skiparse_sparse_attention_amd import _lib as binding   # noqa: E402


class _NoComputeLib:
    """Host-only helpers answer; any other entry point is a test failure."""

    def skiparse_q8_scope_pitch(self, T, H, W, k):
        L = T * H * W // k
        return (L + 63) // 64 * 64

    def __getattr__(self, name):
        def fail(*args, **kwargs):
            raise AssertionError(f"{name} was called although the arguments are invalid")
        return fail


@pytest.fixture
def no_compute(monkeypatch):
    monkeypatch.setattr(binding, "_lib", _NoComputeLib())


F32 = torch.float32
LSE = (1, 2, 64)


def _lse(shape=LSE, dtype=F32):
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.usefixtures("no_compute")
class TestEveryTensorIsChecked:
    def test_host_tensors_are_rejected(self):
        q = _t()
        for call in (lambda: sk.attn(q, q, q, GRID, 2, sk.SINGLE),
                     lambda: sk.attn_lse(q, q, q, GRID, 2, sk.SINGLE),
                     lambda: sk.rope_qk(q, q, GRID),
                     lambda: sk.attn_rotated(q, q, q, GRID, 2, sk.SINGLE),
                     lambda: sk.attn_rotated_lse(q, q, q, GRID, 2, sk.SINGLE),
                     lambda: sk.attn_bwd(q, q, q, q, q, _lse(), GRID, 2, sk.SINGLE),
                     lambda: sk.attn_bwd_rotated(q, q, q, q, q, _lse(), GRID, 2, sk.SINGLE),
                     lambda: sk.rope_remap(q, q, q, GRID, 2, sk.SINGLE),
                     lambda: sk.rearrange(q, GRID, 2, sk.GROUP),
                     lambda: sk.reverse(_t((2, 32, 2, 128)), GRID, 2, sk.SINGLE),
                     lambda: sk.quant8(q, q, q, GRID, 2, sk.SINGLE),
                     lambda: sk.attn_schedule([(q, q, q, _t(), 2, sk.SINGLE)], GRID),
                     lambda: sk.attn_schedule_rotated([(q, q, q, _t(), 2, sk.SINGLE)], GRID)):
            with pytest.raises(ValueError, match="GPU tensor"):
                call()

    def test_forward_outputs_are_checked(self):
        q = _t()
        with pytest.raises(ValueError, match="out has shape"):
            sk.attn(q, q, q, GRID, 2, sk.SINGLE, out=_t((1, 64, 2, 64)))
        with pytest.raises(ValueError, match="out has dtype"):
            sk.attn_rotated(q, q, q, GRID, 2, sk.SINGLE, out=_t(dtype=F32))
        with pytest.raises(ValueError, match="out must be contiguous"):
            sk.attn_lse(q, q, q, GRID, 2, sk.SINGLE, out=_t((1, 64, 128, 2)).transpose(2, 3))
        with pytest.raises(ValueError, match="lse has shape"):
            sk.attn_lse(q, q, q, GRID, 2, sk.SINGLE, lse=_lse((1, 64, 2)))
        with pytest.raises(ValueError, match="lse has dtype"):
            sk.attn_rotated_lse(q, q, q, GRID, 2, sk.SINGLE, lse=_lse(dtype=torch.float64))

    def test_backward_buffers_are_checked(self):
        q = _t()
        for fn in (sk.attn_bwd, sk.attn_bwd_rotated):
            with pytest.raises(ValueError, match="dk has shape"):
                fn(q, q, q, q, q, _lse(), GRID, 2, sk.SINGLE, grads=(_t(), _t((1, 64, 2, 64)), _t()))
            with pytest.raises(ValueError, match="dv has dtype"):
                fn(q, q, q, q, q, _lse(), GRID, 2, sk.SINGLE, grads=(_t(), _t(), _t(dtype=F32)))
            with pytest.raises(ValueError, match="delta has shape"):
                fn(q, q, q, q, q, _lse(), GRID, 2, sk.SINGLE, delta=_lse((1, 64)))
            with pytest.raises(ValueError, match="out has shape"):
                fn(q, q, q, _t((1, 64, 2, 64)), q, _lse(), GRID, 2, sk.SINGLE)
            with pytest.raises(ValueError, match="grads"):
                fn(q, q, q, q, q, _lse(), GRID, 2, sk.SINGLE, grads=(_t(), _t()))

    def test_remap_operands_and_outputs_are_checked(self):
        q = _t()
        with pytest.raises(ValueError, match="k has shape"):
            sk.rope_remap(q, _t((1, 64, 2, 64)), q, GRID, 2, sk.SINGLE)
        with pytest.raises(ValueError, match="v has dtype"):
            sk.rope_remap(q, q, _t(dtype=F32), GRID, 2, sk.SINGLE)
        rs = (2, 32, 2, 128)
        with pytest.raises(ValueError, match="rk has shape"):
            sk.rope_remap(q, q, q, GRID, 2, sk.SINGLE, outs=(_t(rs), _t(SHAPE), _t(rs)))
        with pytest.raises(ValueError, match="out has shape"):
            sk.rearrange(q, GRID, 2, sk.SINGLE, out=_t(SHAPE))
        with pytest.raises(ValueError, match="out has shape"):
            sk.reverse(_t(rs), GRID, 2, sk.SINGLE, out=_t(rs))
        with pytest.raises(ValueError, match="not a sparse_k=2 rearrangement"):
            sk.reverse(_t((3, 32, 2, 128)), GRID, 2, sk.SINGLE)
        with pytest.raises(ValueError, match="not divisible"):
            sk.rearrange(_t((1, 63, 2, 128)), (1, 7, 9), 2, sk.SINGLE)
        with pytest.raises(ValueError, match="sparse_k"):
            sk.rearrange(q, GRID, 0, sk.SINGLE)

    def test_quant8_outputs_and_attn8_operands_are_checked(self):
        q = _t()
        outs = {"q8": _t(dtype=torch.int8), "q_amax": _t((1, 64, 2), F32),
                "k8": _t(dtype=torch.int8), "k_amax": _t((1, 2), F32),
                "vt8": _t((1, 2, 2, 128, 64), torch.uint8), "v_amax": _t((1, 2, 128), F32)}
        bad = dict(outs, vt8=_t((1, 2, 2, 128, 32), torch.uint8))      # pitch must be 64
        with pytest.raises(ValueError, match="vt8 has shape"):
            sk.quant8(q, q, q, GRID, 2, sk.SINGLE, outs=bad)
        bad = dict(outs, k_amax=_t((1, 2), torch.float16))
        with pytest.raises(ValueError, match="k_amax has dtype"):
            sk.quant8(q, q, q, GRID, 2, sk.SINGLE, outs=bad)
        with pytest.raises(ValueError, match="lacks"):
            sk.quant8(q, q, q, GRID, 2, sk.SINGLE, outs={"q8": outs["q8"]})
        bad = dict(outs, q_amax=_t((1, 64, 3), F32))
        with pytest.raises(ValueError, match="q_amax has shape"):
            sk.attn8(bad, GRID, 2, sk.SINGLE)
        with pytest.raises(ValueError, match="out has shape"):
            sk.attn8(outs, GRID, 2, sk.SINGLE, out=_t((1, 64, 2, 64)))
        with pytest.raises(ValueError, match="GPU tensor"):
            sk.attn8(outs, GRID, 2, sk.SINGLE)

    def test_schedule_tensors_are_checked(self):
        q = _t()
        with pytest.raises(ValueError, match="layer 1 out has shape"):
            sk.attn_schedule([(q, q, q, _t(), 2, sk.SINGLE), (q, q, q, _t((1, 64, 2, 64)), 4, sk.GROUP)], GRID)
        with pytest.raises(ValueError, match="scratch kr has dtype"):
            sk.attn_schedule_rotated([(q, q, q, _t(), 2, sk.SINGLE)], GRID, scratch=(_t(), _t(dtype=F32)))
        with pytest.raises(ValueError, match="empty"):
            sk.attn_schedule([], GRID)
