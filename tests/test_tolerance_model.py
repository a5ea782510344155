"""The GPU tests' tolerances, derived from the kernels' arithmetic rather than from their output.

A rounding model replays, in float64, the points where the kernels round to bfloat16:
  forward:  q' = bf16(RoPE(q) log2(e)/sqrt(d)), k' = bf16(RoPE(k)); weights P rounded to bf16
            for the P V product, the row sum taken over the unrounded weights; the output
            rounded to bf16;
  backward: the same q', k'; P rounded to bf16 for dV = P^T dO; dZ = P (dP - D) rounded to
            bf16 for dQ = dZ k' and dK = dZ^T q'; D from the bf16 output the forward stored;
            the gradients rounded to the output dtype.
Everything else (the float32 accumulations, the exponentials) is taken exact, so the model
errors are the part the bf16 operands force.  Each test checks that the bar its GPU test uses
leaves at least a factor 2 over the modelled error on that test's own inputs: the bars follow
from the arithmetic, and a kernel that met only a much looser bar would fail.
  8-bit path, bf16 output: the 8-bit oracle already quantises exactly as the kernel does, so
            the floor is the rounding of its output to bf16; those bars sit 1.5x (RMS) and
            2x (max) above it.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import skiparse_oracle8 as o8
from skiparse_sparse_attention_amd import workloads as wl

import test_gpu_attn8 as gpu_attn8
import test_gpu_backward as gpu_bwd
import test_gpu_parity as gpu_fwd


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).float().to(torch.bfloat16).double().numpy()


def _scope_operands(q, k, T, H, W, sk_, mode):
    """(k*B, heads, L, d) rotated q (scaled to base-2 units, bf16) and k (bf16) per scope."""
    d = q.shape[-1]
    c2 = math.log2(math.e) / math.sqrt(d)
    rq = oracle.rope_rearrange(q, T, H, W, sk_, mode, True).transpose(0, 2, 1, 3)
    rk = oracle.rope_rearrange(k, T, H, W, sk_, mode, True).transpose(0, 2, 1, 3)
    return _bf16(rq * c2), _bf16(rk)


def _model_forward(q, k, v, T, H, W, sk_, mode, out_bf16):
    qs, ks = _scope_operands(q, k, T, H, W, sk_, mode)
    rv = oracle.rope_rearrange(v, T, H, W, sk_, mode, False).transpose(0, 2, 1, 3)
    z = np.matmul(qs, np.swapaxes(ks, -1, -2))                    # base-2 scores
    p = np.exp2(z - z.max(axis=-1, keepdims=True))
    pb = _bf16(p)
    o = np.matmul(pb, rv) / p.sum(axis=-1, keepdims=True)
    if out_bf16:
        o = _bf16(o)
    return oracle.reverse_rows(o.transpose(0, 2, 1, 3), sk_, mode), qs, ks, rv


def _errors(got, want):
    err = np.abs(got - want)
    return float(err.max()), float(err.mean()), float(np.sqrt((err ** 2).sum() / (want ** 2).sum()))


@pytest.mark.parametrize("B,T,H,W,heads,d,k,mode,dtype", gpu_fwd.SMALL)
def test_forward_bars_leave_headroom_over_the_rounding_model(B, T, H, W, heads, d, k, mode, dtype):
    w = wl.Workload("case", B, T, H, W, heads, d, 1, 0, "bf16" if dtype == torch.bfloat16 else "fp32")
    q, kk, v = (x.double().numpy() for x in wl.make_inputs(w, seed=11))
    model, _, _, _ = _model_forward(q, kk, v, T, H, W, k, mode, dtype == torch.bfloat16)
    exact = oracle.skiparse_attention(q, kk, v, T, H, W, k, mode)
    mx, mean, rel = _errors(model, exact)
    assert gpu_fwd.MAX_ABS >= 2 * mx and gpu_fwd.MEAN_ABS >= 2 * mean and gpu_fwd.REL_RMS >= 2 * rel, (mx, mean, rel)


def test_forward_bars_at_the_full_size_scope_length():
    # one scope of the 24x22x40 workload at k = 4 (L = 5280 keys), 64 query rows of one head:
    # the regime of the full-size GPU checks
    w = wl.OSP_SINGLE
    q, kk, v = (x.double().numpy() for x in wl.make_inputs(w, seed=0))
    table = oracle.scope_table(w.N, w.sparse_k, w.mode)
    members = table[1]
    t, h, ww = oracle.token_positions(w.T, w.H, w.W)
    d = w.head_dim
    c2 = math.log2(math.e) / math.sqrt(d)
    sel = lambda x, idx: x[0, idx][:, 0]                         # head 0
    rk = oracle.rope_3d_at(sel(kk, members)[:, None], t[members], h[members], ww[members])[:, 0]
    rows = members[:: len(members) // 64][:64]
    rq = oracle.rope_3d_at(sel(q, rows)[:, None], t[rows], h[rows], ww[rows])[:, 0]
    vv = sel(v, members)
    exact = oracle.attention(rq, rk, vv)
    z = _bf16(rq * c2) @ _bf16(rk).T
    p = np.exp2(z - z.max(axis=-1, keepdims=True))
    model = _bf16((_bf16(p) @ vv) / p.sum(axis=-1, keepdims=True))
    mx, mean, rel = _errors(model, exact)
    assert gpu_fwd.MAX_ABS >= 2 * mx and gpu_fwd.MEAN_ABS >= 2 * mean and gpu_fwd.REL_RMS >= 2 * rel, (mx, mean, rel)


def _model_backward(q, kk, v, do, T, H, W, k, mode, out_bf16):
    """(modelled dq, dk, dv) with the kernels' rounding points, and the exact fp64 gradients."""
    d = q.shape[-1]
    o_b, qs, ks, rv = _model_forward(q, kk, v, T, H, W, k, mode, True)   # the stored bf16 output
    rdo = oracle.rope_rearrange(do, T, H, W, k, mode, False).transpose(0, 2, 1, 3)
    ro = oracle.rope_rearrange(o_b, T, H, W, k, mode, False).transpose(0, 2, 1, 3)
    z = np.matmul(qs, np.swapaxes(ks, -1, -2))
    p = np.exp2(z - z.max(axis=-1, keepdims=True))
    p = p / p.sum(axis=-1, keepdims=True)
    dD = (rdo * ro).sum(axis=-1, keepdims=True)
    dp = np.matmul(rdo, np.swapaxes(rv, -1, -2))
    dz = _bf16(p * (dp - dD))
    dv = np.matmul(np.swapaxes(_bf16(p), -1, -2), rdo)
    ln2 = math.log(2.0)
    dk = np.matmul(np.swapaxes(dz, -1, -2), qs) * ln2             # dZ^T q' with q' in base-2 units
    dq = np.matmul(dz, ks) / math.sqrt(d)
    t, h, ww = oracle.token_positions(T, H, W)
    back = lambda x: oracle.reverse_rows(x.transpose(0, 2, 1, 3), k, mode)
    model = [oracle.rope_3d_transpose_at(back(dq), t, h, ww), oracle.rope_3d_transpose_at(back(dk), t, h, ww),
             back(dv)]
    if out_bf16:
        model = [_bf16(x) for x in model]
    exact = oracle.skiparse_attention_backward(q, kk, v, do, T, H, W, k, mode)
    return model, exact


def _assert_backward_headroom(model, exact, rel_bar, max_bar):
    for name, m, e in zip(("dq", "dk", "dv"), model, exact):
        err = np.abs(m - e)
        rel = float(np.sqrt((err ** 2).sum() / (e ** 2).sum()))
        mrel = float(err.max() / np.abs(e).max())
        assert rel_bar >= 2 * rel and max_bar >= 2 * mrel, (name, rel, mrel)


@pytest.mark.parametrize("B,T,H,W,heads,d,k,mode,dtype", gpu_bwd.CASES)
def test_backward_bars_leave_headroom_over_the_rounding_model(B, T, H, W, heads, d, k, mode, dtype):
    out_bf16 = dtype == torch.bfloat16
    w = wl.Workload("case", B, T, H, W, heads, d, k, mode, "bf16" if out_bf16 else "fp32")
    q, kk, v = (x.double().numpy() for x in wl.make_inputs(w, seed=0))
    do = wl.make_output_grad(w, seed=1).double().numpy()
    model, exact = _model_backward(q, kk, v, do, T, H, W, k, mode, out_bf16)
    _assert_backward_headroom(model, exact, gpu_bwd.REL_RMS, gpu_bwd.MAX_REL)


def test_backward_peaked_bars_leave_headroom_over_the_rounding_model():
    # the GPU test's peaked case (q x PEAKED_SCALE): the same replay on the scaled inputs
    B, T, H, W, heads, d, k, mode = gpu_bwd.PEAKED_CASE
    w = wl.Workload("case", B, T, H, W, heads, d, k, mode, "bf16")
    q, kk, v = (x.double().numpy() for x in wl.make_inputs(w, seed=0))
    q = _bf16(q * gpu_bwd.PEAKED_SCALE)
    do = wl.make_output_grad(w, seed=1).double().numpy()
    model, exact = _model_backward(q, kk, v, do, T, H, W, k, mode, True)
    _assert_backward_headroom(model, exact, gpu_bwd.PEAKED_REL_RMS, gpu_bwd.PEAKED_MAX_REL)


@pytest.mark.parametrize("case", [c for c in gpu_attn8.CASES if c[-1] == torch.bfloat16],
                         ids=lambda c: f"{c[1]}x{c[2]}x{c[3]}_k{c[5]}_m{c[6]}")
def test_attn8_bf16_bars_sit_above_the_output_rounding(case):
    # With bf16 output, the 8-bit kernel's error against the 8-bit oracle is the rounding of
    # its float32 result to bf16 (the float32-output cases show everything else below 4e-5).
    # That rounding, applied to the oracle's float64 output on the test's own inputs, is the
    # floor: 1.65e-3 .. 1.67e-3 relative RMS here.  The bars sit 1.5x (RMS) and >= 2x (max)
    # above it.
    B, T, H, W, heads, k, mode, dtype, out_dtype = case
    w = wl.Workload("case", B, T, H, W, heads, 128, k, mode, "bf16" if dtype == torch.bfloat16 else "fp32")
    q, kk, v = wl.make_inputs(w, seed=0, device="cpu")
    qn, kn, vn = (x.float().numpy() for x in (q, kk, v))
    want = o8.skiparse_attention_8bit(o8.quantize_8bit(qn, kn, vn, T, H, W, k, mode), T, H, W, k, mode)
    floor = torch.from_numpy(want).to(torch.bfloat16).double().numpy()
    err = np.abs(floor - want)
    rel = float(np.sqrt((err ** 2).sum() / (want ** 2).sum()))
    mx = float(err.max() / np.abs(want).max())
    assert gpu_attn8.REL_RMS[torch.bfloat16] >= 1.4 * rel and gpu_attn8.MAX_REL[torch.bfloat16] >= 2 * mx, (rel, mx)
