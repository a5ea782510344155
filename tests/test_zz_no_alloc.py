"""GPU test of skiparse_attn_bwd_rotated_static (the backward whose delta workspace is the
library's static per-GPU array) through the C ABI, against skiparse_attn_bwd_rotated with a
caller-owned delta.  Two calls in a row, the second on a smaller input, must both equal the
workspace-argument entry point bit for bit (the same kernels run on the same operands).
"""

import pytest
import torch

import skiparse_sparse_attention_amd as sk
from skiparse_sparse_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    sk.lib()
    yield


def _case(B, T, H, W, heads, k, mode, seed):
    w = wl.Workload("case", B, T, H, W, heads, 128, k, mode)
    q, kk, v = wl.make_inputs(w, seed=seed, device="cuda")
    do = wl.make_output_grad(w, seed=seed + 1, device="cuda")
    qr, kr = sk.rope_qk(q, kk, w.grid)
    out, lse = sk.attn_rotated_lse(qr, kr, v, w.grid, k, mode)
    return w, (qr, kr, v, out, do, lse)


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("first,second", [
    # (B, T, H, W, heads, k, mode): the second call is smaller than the first
    ((2, 4, 10, 12, 3, 2, sk.GROUP), (1, 4, 8, 8, 2, 4, sk.SINGLE)),
    ((1, 24, 22, 40, 24, 4, sk.SINGLE), (1, 6, 10, 12, 2, 4, sk.GROUP)),
])
def test_static_workspace_backward_equals_workspace_argument(first, second):
    for i, shape in enumerate((first, second)):
        print(f"call {i}: B,T,H,W,heads,k,mode = {shape}", flush=True)
        w, args = _case(*shape, seed=10 + i)
        ref = sk.attn_bwd_rotated(*args, w.grid, w.sparse_k, w.mode)
        grads = tuple(torch.full_like(args[0], float("nan")) for _ in range(3))
        got = sk.attn_bwd_rotated_static(*args, w.grid, w.sparse_k, w.mode, grads=grads)
        torch.cuda.synchronize()
        for name, g_, r in zip(("dq", "dk", "dv"), got, ref):
            assert not torch.isnan(g_).any().item(), f"{name}: not every element written"
            assert torch.equal(_bits(g_), _bits(r)), f"{name} differs on call {i}"
