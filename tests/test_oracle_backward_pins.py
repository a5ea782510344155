"""Pins of the oracle's Skiparse backward (CPU only).

The backward oracle is the chain rule written out (oracle.attention_backward,
oracle.skiparse_attention_backward).  It is pinned here against things that do
not retype that formula:

* central finite differences of the forward oracle (itself pinned in
  test_oracle_pins.py), element by element, on tiny grids in both modes;
* torch autograd (float64, CPU) through the scaled-dot-product attention call
  the Open-Sora Plan page makes, for the dense k = 1 case, with RoPE applied
  as explicit per-token rotation matrices;
* closed forms: with q = 0 the softmax is uniform, so dk is exactly 0 and dv
  of every key is the mean of do over its scope; for any input the dv of a
  scope sums to the do of that scope (softmax rows sum to 1);
* the transposed RoPE is the inverse and the adjoint of RoPE.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _inputs(B, N, heads, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, N, heads, d)) for _ in range(4)]


def _loss(q, k, v, g, T, H, W, sk, mode):
    return float((oracle.skiparse_attention(q, k, v, T, H, W, sk, mode) * g).sum())


@pytest.mark.parametrize("mode,sk,T,H,W,elems", [
    (oracle.SINGLE, 2, 2, 2, 4, None),      # every element
    (oracle.GROUP, 2, 2, 2, 4, 96),         # a random subset of elements per tensor
    (oracle.SINGLE, 1, 1, 2, 4, 96),
    (oracle.GROUP, 2, 1, 4, 4, 96),
])
def test_backward_matches_finite_differences(mode, sk, T, H, W, elems):
    B, heads, d = 1, 2, 16
    N = T * H * W
    q, k, v, g = _inputs(B, N, heads, d, seed=7 + sk + 3 * mode)
    dq, dk, dv = oracle.skiparse_attention_backward(q, k, v, g, T, H, W, sk, mode)
    rng = np.random.default_rng(11)
    eps = 1e-6
    for which, (x, grad) in enumerate(((q, dq), (k, dk), (v, dv))):
        flat = x.reshape(-1)
        idx = np.arange(flat.size) if elems is None else rng.choice(flat.size, elems, replace=False)
        for i in idx:
            keep = flat[i]
            flat[i] = keep + eps
            args = [q, k, v]
            lp = _loss(*args, g, T, H, W, sk, mode)
            flat[i] = keep - eps
            lm = _loss(*args, g, T, H, W, sk, mode)
            flat[i] = keep
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.reshape(-1)[i]) <= 1e-6 * max(1.0, abs(fd)), (which, i, fd, grad.reshape(-1)[i])


def _rotation_matrices(T, H, W, d):
    """Per-token RoPE matrices R[n] (d x d) with rope(x)[n] = R[n] x[n], from the pinned forward."""
    N = T * H * W
    eye = np.broadcast_to(np.eye(d), (N, d, d)).copy()        # (N, d basis vectors, d)
    t, h, w = oracle.token_positions(T, H, W)
    # rope_3d_at rotates the last axis of (..., ntok, heads, d): basis vectors play the heads
    cols = oracle.rope_3d_at(eye, t, h, w)                      # (N, basis, d): R[n] e_b
    return np.transpose(cols, (0, 2, 1))                        # R[n][:, b] = R[n] e_b


def test_dense_k1_backward_matches_torch_autograd():
    T, H, W, heads, d = 2, 2, 4, 2, 16
    N = T * H * W
    q, k, v, g = _inputs(1, N, heads, d, seed=3)
    R = torch.from_numpy(_rotation_matrices(T, H, W, d))
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    rq = torch.einsum("nij,bnhj->bnhi", R, tq)
    rk = torch.einsum("nij,bnhj->bnhi", R, tk)
    o = torch.nn.functional.scaled_dot_product_attention(
        rq.transpose(1, 2), rk.transpose(1, 2), tv.transpose(1, 2)).transpose(1, 2)
    (o * torch.from_numpy(g)).sum().backward()
    dq, dk, dv = oracle.skiparse_attention_backward(q, k, v, g, T, H, W, 1, oracle.SINGLE)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("mode,sk", [(oracle.SINGLE, 2), (oracle.GROUP, 2), (oracle.SINGLE, 4)])
def test_uniform_softmax_closed_form(mode, sk):
    T, H, W, heads, d = 4, 4, 4, 2, 16
    N = T * H * W
    L = N // sk
    _, k, v, g = _inputs(1, N, heads, d, seed=5)
    q = np.zeros_like(k)
    _, dk, dv = oracle.skiparse_attention_backward(q, k, v, g, T, H, W, sk, mode)
    assert np.array_equal(dk, np.zeros_like(dk))     # dk = dS^T q / sqrt(d) with q = 0
    table = oracle.scope_table(N, sk, mode)
    for s in range(sk):
        members = table[s]
        want = g[0, members].sum(axis=0) / L          # every weight is exactly 1/L
        np.testing.assert_allclose(dv[0, members], np.broadcast_to(want, dv[0, members].shape), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mode,sk", [(oracle.SINGLE, 4), (oracle.GROUP, 2)])
def test_dv_of_a_scope_sums_to_its_do(mode, sk):
    T, H, W, heads, d = 2, 4, 8, 3, 16
    N = T * H * W
    q, k, v, g = _inputs(2, N, heads, d, seed=9)
    _, _, dv = oracle.skiparse_attention_backward(q * 3, k, v, g, T, H, W, sk, mode)
    table = oracle.scope_table(N, sk, mode)
    for b in range(2):
        for s in range(sk):
            m = table[s]
            np.testing.assert_allclose(dv[b, m].sum(axis=0), g[b, m].sum(axis=0), rtol=1e-10, atol=1e-10)


def test_rope_transpose_is_inverse_and_adjoint():
    T, H, W, heads, d = 3, 4, 5, 2, 32
    t, h, w = oracle.token_positions(T, H, W)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, T * H * W, heads, d))
    y = rng.standard_normal((1, T * H * W, heads, d))
    rx = oracle.rope_3d_at(x, t, h, w)
    np.testing.assert_allclose(oracle.rope_3d_transpose_at(rx, t, h, w), x, rtol=0, atol=1e-12)
    lhs = (rx * y).sum()
    rhs = (x * oracle.rope_3d_transpose_at(y, t, h, w)).sum()
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


@pytest.mark.parametrize("mode,sk", [(oracle.SINGLE, 4), (oracle.GROUP, 2)])
def test_scope_backward_matches_full_backward(mode, sk):
    T, H, W, heads, d = 2, 4, 8, 3, 16
    N = T * H * W
    q, k, v, g = _inputs(2, N, heads, d, seed=13)
    dq, dk, dv = oracle.skiparse_attention_backward(q, k, v, g, T, H, W, sk, mode)
    for b in range(2):
        for s in range(sk):
            toks, sq, skk, sv = oracle.skiparse_attention_backward_scope(q, k, v, g, T, H, W, sk, mode, b, s, [2, 0])
            np.testing.assert_allclose(sq, dq[b, toks][:, [2, 0]], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(skk, dk[b, toks][:, [2, 0]], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(sv, dv[b, toks][:, [2, 0]], rtol=1e-12, atol=1e-12)


def test_backward_flops_are_twice_the_forward():
    assert oracle.skiparse_backward_flops(1, 21120, 24, 128, 4) == 2 * oracle.skiparse_flops(1, 21120, 24, 128, 4)
    assert oracle.skiparse_backward_flops(2, 64, 3, 64, 8) == 8.0 * 2 * 3 * 64 * 8 * 64
