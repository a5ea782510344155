"""Plain fp64 CPU oracle for Skiparse attention.

TEST INFRASTRUCTURE ONLY.  This module is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``;
nothing on the product path may import or call it.  It shares no code with
the HIP library (no headers, tables, helpers or constants): it is written
directly from the pages so that a reader can check it by eye.

What it computes, and where each step comes from
-----------------------------------------------
Open-Sora Plan documentation, section "Skiparse Attention":

* The attention sequence of a Full-3D-attention block is split into ``k``
  scopes; attention runs inside each scope only.  Only the attention part of
  the transformer block changes.
* "Single Skip Mode": a token shares its scope with the tokens k positions
  away from it, so token ``n`` is in scope ``n mod k``.
* "Group Skip Mode": runs of ``k`` adjacent tokens form groups, and a group
  shares its scope with the groups k groups away from it, so group
  ``j = n div k`` (and each of its tokens) is in scope ``j mod k``.
* Inside a scope the tokens keep their original order; the page's code puts
  the scope axis in front of the batch axis of the rearranged tensor
  (row ``s*B + b`` holds scope ``s`` of batch ``b``).
* Implementation note: RoPE is applied to q and k *before* the rearrange,
  because the rearrange loses the original positions.
* The forward snippet runs ``F.scaled_dot_product_attention(q, k, v)`` on the
  rearranged tensors: non-causal softmax attention, no mask, no dropout.

``add_rope`` is used but never defined on the pages (the vidax page notes
that 3D-RoPE conventions differ per model family).  The reading taken here:
base 10000; head_dim split over the t/h/w axes in the ratio 2:3:3
(16/24/24 at d=64, 32/48/48 at d=128), in that order; inside each axis chunk
the pairs are rotate-half pairs (j, j + d_a/2) with angle
pos_a * base**(-2j/d_a); integer positions from 0.

Multi-head reading: the rearrange acts on the token axis of (B, N, C) with
C = heads*head_dim, so it is the same for every head; attention is per head
with scale 1/sqrt(head_dim).

Token flattening: n = (t*H + h)*W + w (Wan 2.1 report, section 4.2.1
"Video Diffusion Transformer": the patchified latent is flattened into a
(B, L, D) sequence).

The backward (gradients of a loss through the whole forward) follows the same
steps in reverse, by the chain rule: scatter the output gradient into the
scopes, differentiate softmax attention inside each scope, rotate the q and k
gradients back with the transposed RoPE rotation, and scatter them to their
original tokens.  Open-Sora Plan's page says Skiparse exists to speed up
training, which is what needs these gradients.

Every pin of this module lives in ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import math

import numpy as np

ROPE_BASE = 10000.0


# ---------------------------------------------------------------------------
# Positions
# ---------------------------------------------------------------------------

def token_positions(T: int, H: int, W: int):
    """(t, h, w) of every token n = (t*H + h)*W + w, as int64 arrays of length T*H*W.

    Wan 2.1 report, section 4.2.1: the (T, H, W) latent grid is flattened
    into one token sequence, frame-major.
    """
    n = np.arange(T * H * W, dtype=np.int64)
    t = n // (H * W)
    h = (n // W) % H
    w = n % W
    return t, h, w


# ---------------------------------------------------------------------------
# 3D RoPE
# ---------------------------------------------------------------------------

def rope_axis_sizes(head_dim: int):
    """Chunk sizes (d_t, d_h, d_w) of head_dim for the t, h, w axes (ratio 2:3:3)."""
    if head_dim % 16 != 0:
        raise ValueError("3D RoPE split 2:3:3 into even chunks needs head_dim % 16 == 0")
    return head_dim // 4, 3 * head_dim // 8, 3 * head_dim // 8


def rope_3d_at(x, t, h, w, base: float = ROPE_BASE):
    """Rotate the last axis of ``x`` (..., ntok, heads, d) by 3D RoPE.

    ``t, h, w`` give the grid position of each of the ``ntok`` tokens.
    For axis a with chunk offset o, size d_a and position pos, and for
    j in [0, d_a/2):
        theta = pos * base**(-2j/d_a)
        x1 = x[o+j], x2 = x[o+j+d_a/2]
        out[o+j]        = x1*cos(theta) - x2*sin(theta)
        out[o+j+d_a/2]  = x2*cos(theta) + x1*sin(theta)
    Computed in float64.  (Open-Sora Plan docs, "Skiparse Attention",
    implementation note: RoPE goes on q and k in the original token order.)
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    sizes = rope_axis_sizes(d)
    out = x.copy()
    offset = 0
    for pos, d_a in zip((t, h, w), sizes):
        half = d_a // 2
        j = np.arange(half, dtype=np.float64)
        freq = base ** (-2.0 * j / d_a)                      # (half,)
        theta = np.asarray(pos, dtype=np.float64)[:, None] * freq[None, :]   # (ntok, half)
        cos = np.cos(theta)[:, None, :]                      # broadcast over heads
        sin = np.sin(theta)[:, None, :]
        x1 = x[..., offset:offset + half]
        x2 = x[..., offset + half:offset + d_a]
        out[..., offset:offset + half] = x1 * cos - x2 * sin
        out[..., offset + half:offset + d_a] = x2 * cos + x1 * sin
        offset += d_a
    return out


def rope_3d(x, T: int, H: int, W: int, base: float = ROPE_BASE):
    """3D RoPE of a full (B, N, heads, d) tensor laid out on the T x H x W grid."""
    t, h, w = token_positions(T, H, W)
    return rope_3d_at(x, t, h, w, base)


def rope_3d_transpose_at(x, t, h, w, base: float = ROPE_BASE):
    """The transpose of :func:`rope_3d_at`: every rotate-half pair turned by -theta.

    RoPE rotates each pair (x1, x2) by the angle theta, i.e. multiplies it by
    [[cos, -sin], [sin, cos]]; the transpose of that matrix is the rotation by
    -theta.  Since theta = pos * freq is linear in the position, turning by
    -theta is RoPE at the negated positions.  This is what carries a gradient
    with respect to rotated q or k back to the unrotated input.
    """
    return rope_3d_at(x, -np.asarray(t), -np.asarray(h), -np.asarray(w), base)


# ---------------------------------------------------------------------------
# Scope map (Open-Sora Plan documentation, "Skiparse Attention": Single Skip
# Mode, Group Skip Mode)
# ---------------------------------------------------------------------------

SINGLE = 0
GROUP = 1


def token_scope(n, k: int, mode: int):
    """Scope index of token(s) ``n`` (int64 array or int).

    Single Skip: token n is in scope n mod k.  Group Skip: token n belongs to
    group n div k, and that group is in scope (n div k) mod k.
    """
    n = np.asarray(n, dtype=np.int64)
    if mode == SINGLE:
        return n % k
    if mode == GROUP:
        return (n // k) % k
    raise ValueError("mode must be SINGLE (0) or GROUP (1)")


def _check_divisible(N: int, k: int, mode: int):
    # Every scope must hold the same number of tokens; Group Skip also needs whole
    # groups in every scope (the page's code rejects other lengths).
    if mode == SINGLE and N % k:
        raise ValueError("single skip needs N % k == 0")
    if mode == GROUP and N % (k * k):
        raise ValueError("group skip needs N % k**2 == 0")


def scope_table(N: int, k: int, mode: int):
    """int64 (k, N/k): row s lists the tokens of scope s in their original order.

    Entry [s, p] is the token at in-scope position p of scope s.
    """
    _check_divisible(N, k, mode)
    n = np.arange(N, dtype=np.int64)
    s = token_scope(n, k, mode)
    return np.stack([n[s == i] for i in range(k)])


def rearrange(x, k: int, mode: int):
    """(B, N, C) -> (k*B, N/k, C): row s*B + b, position p holds x[b, table[s, p]]."""
    x = np.asarray(x)
    B, N, C = x.shape
    table = scope_table(N, k, mode)                 # (k, L)
    gathered = x[:, table, :]                       # (B, k, L, C)
    return np.ascontiguousarray(gathered.transpose(1, 0, 2, 3)).reshape(k * B, N // k, C)


def reverse(x, k: int, mode: int):
    """Inverse of :func:`rearrange`: (k*B, N/k, C) -> (B, N, C), each row back to its token."""
    x = np.asarray(x)
    kB, L, C = x.shape
    B, N = kB // k, L * k
    table = scope_table(N, k, mode)
    out = np.empty((B, N, C), dtype=x.dtype)
    out[:, table, :] = x.reshape(k, B, L, C).transpose(1, 0, 2, 3)
    return out


# ---------------------------------------------------------------------------
# Attention inside a scope
# ---------------------------------------------------------------------------

def attention(q, k, v):
    """softmax(q k^T / sqrt(d)) v over the last two axes, one (L, d) problem per leading index.

    ``q``: (..., Lq, d); ``k``, ``v``: (..., Lk, d).  float64, non-causal,
    no mask, no dropout (the defaults of the scaled-dot-product attention
    call on the Open-Sora Plan page).  The row maximum is subtracted before
    the exponential.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(d)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.matmul(p, v)


def attention_backward(q, k, v, do):
    """Gradients of sum(attention(q, k, v) * do) with respect to q, k and v, float64.

    One (L, d) problem per leading index, as in :func:`attention`.  The chain
    rule written out, with S = q k^T / sqrt(d), P = softmax(S) row-wise and
    O = P v:
        dv = P^T do
        dP = do v^T
        dS = P * (dP - rowsum(dP * P))      (the softmax Jacobian, row by row)
        dq = dS k / sqrt(d)
        dk = dS^T q / sqrt(d)
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    d = q.shape[-1]
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(d)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
    dq = np.matmul(ds, k) / math.sqrt(d)
    dk = np.matmul(np.swapaxes(ds, -1, -2), q) / math.sqrt(d)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# The full Skiparse forward
# ---------------------------------------------------------------------------

def rope_rearrange(x, T, H, W, sparse_k, mode, apply_rope=True, base=ROPE_BASE):
    """(B, N, heads, d) -> (k*B, N/k, heads, d): optional 3D RoPE, then the Skiparse rearrange.

    Row s*B + b of the result holds scope s of batch b, its tokens in their
    original order (the layout of the page's rearranged tensors).
    """
    x = np.asarray(x, dtype=np.float64)
    B, N, heads, d = x.shape
    if apply_rope:
        x = rope_3d(x, T, H, W, base)
    r = rearrange(x.reshape(B, N, heads * d), sparse_k, mode)
    return r.reshape(r.shape[0], r.shape[1], heads, d)


def reverse_rows(x, sparse_k, mode):
    """(k*B, N/k, heads, d) -> (B, N, heads, d): the Skiparse reverse."""
    kB, L, heads, d = x.shape
    r = reverse(np.asarray(x).reshape(kB, L, heads * d), sparse_k, mode)
    return r.reshape(r.shape[0], r.shape[1], heads, d)


def skiparse_attention(q, k, v, T, H, W, sparse_k, mode, base=ROPE_BASE):
    """Skiparse attention forward, float64.  q, k, v: (B, N, heads, d) with N = T*H*W.

    RoPE on q and k at every token's own grid position (the implementation
    note: before the tokens are regrouped); then, for every batch, head and
    scope, softmax attention of the scope's queries over the scope's keys and
    values; each output row lands on the token its query came from.  With
    sparse_k == 1 there is one scope and this is dense full-3D attention.
    """
    q = np.asarray(q, dtype=np.float64)
    B, N, heads, d = q.shape
    if N != T * H * W:
        raise ValueError("N must equal T*H*W")
    rq = rope_3d(q, T, H, W, base)
    rk = rope_3d(np.asarray(k, dtype=np.float64), T, H, W, base)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(rq)
    for members in scope_table(N, sparse_k, mode):
        # (B, L, heads, d) -> (B, heads, L, d): one attention problem per (batch, head)
        tr = lambda x: x[:, members].transpose(0, 2, 1, 3)
        out[:, members] = attention(tr(rq), tr(rk), tr(v)).transpose(0, 2, 1, 3)
    return out


def skiparse_attention_rows(q, k, v, T, H, W, sparse_k, mode, batch_idx, token_idx,
                            base=ROPE_BASE):
    """Skiparse attention output of selected (batch, token) rows only, float64.

    Returns (len(token_idx), heads, d).  For each requested token n of batch
    b: its scope is the row of :func:`scope_table` that contains n; its
    query is RoPE(q[b, n]) at n's own grid position; its keys and values are
    RoPE(k[b, m]) and v[b, m] for every member m of that scope; the output is
    softmax attention over them.  This is the same definition as
    :func:`skiparse_attention`, evaluated row by row so that very large
    inputs can be checked on a sample.
    """
    batch_idx = np.asarray(batch_idx, dtype=np.int64)
    token_idx = np.asarray(token_idx, dtype=np.int64)
    B, N, heads, d = q.shape
    table = scope_table(N, sparse_k, mode)
    scope_of = np.empty(N, dtype=np.int64)
    for s in range(sparse_k):
        scope_of[table[s]] = s
    t_all, h_all, w_all = token_positions(T, H, W)
    out = np.empty((len(token_idx), heads, d), dtype=np.float64)
    keys = sorted(set(zip(batch_idx.tolist(), scope_of[token_idx].tolist())))
    for b, s in keys:
        members = table[s]
        sel = np.nonzero((batch_idx == b) & (scope_of[token_idx] == s))[0]
        toks = token_idx[sel]
        kk = rope_3d_at(np.asarray(k[b, members], dtype=np.float64),
                        t_all[members], h_all[members], w_all[members], base)
        vv = np.asarray(v[b, members], dtype=np.float64)
        qq = rope_3d_at(np.asarray(q[b, toks], dtype=np.float64),
                        t_all[toks], h_all[toks], w_all[toks], base)
        o = attention(qq.transpose(1, 0, 2), kk.transpose(1, 0, 2), vv.transpose(1, 0, 2))
        out[sel] = o.transpose(1, 0, 2)
    return out


def skiparse_attention_backward(q, k, v, do, T, H, W, sparse_k, mode, base=ROPE_BASE):
    """Gradients (dq, dk, dv) of sum(skiparse_attention(q, k, v) * do), float64.

    All arrays (B, N, heads, d).  The forward's steps taken backwards: the
    output gradient of a token belongs to the scope its query is in; softmax
    attention is differentiated per batch, head and scope
    (:func:`attention_backward`), each gradient row landing on its own token
    (no token is in two scopes); the q and k gradients are then rotated back
    by the transposed RoPE (:func:`rope_3d_transpose_at`).
    """
    q = np.asarray(q, dtype=np.float64)
    B, N, heads, d = q.shape
    if N != T * H * W:
        raise ValueError("N must equal T*H*W")
    rq = rope_3d(q, T, H, W, base)
    rk = rope_3d(np.asarray(k, dtype=np.float64), T, H, W, base)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    dq, dk, dv = np.empty_like(rq), np.empty_like(rq), np.empty_like(rq)
    for members in scope_table(N, sparse_k, mode):
        tr = lambda x: x[:, members].transpose(0, 2, 1, 3)
        gq, gk, gv = attention_backward(tr(rq), tr(rk), tr(v), tr(do))
        dq[:, members] = gq.transpose(0, 2, 1, 3)
        dk[:, members] = gk.transpose(0, 2, 1, 3)
        dv[:, members] = gv.transpose(0, 2, 1, 3)
    t, h, w = token_positions(T, H, W)
    return rope_3d_transpose_at(dq, t, h, w, base), rope_3d_transpose_at(dk, t, h, w, base), dv


def skiparse_attention_backward_scope(q, k, v, do, T, H, W, sparse_k, mode, b, s, heads_idx,
                                      base=ROPE_BASE):
    """Gradients of every member token of scope ``s`` of batch ``b``, selected heads only.

    Returns (tokens, dq, dk, dv): ``tokens`` are the scope's member token
    indices in in-scope order, and dq/dk/dv are (L, len(heads_idx), d).  The
    gradients of a scope depend only on that scope's rows (no token belongs
    to two scopes), so this is :func:`skiparse_attention_backward` restricted
    to one scope, for checking large inputs on a sample.
    """
    heads_idx = np.asarray(heads_idx, dtype=np.int64)
    B, N, heads, d = np.shape(q)
    members = scope_table(N, sparse_k, mode)[s]
    t_all, h_all, w_all = token_positions(T, H, W)
    tm, hm, wm = t_all[members], h_all[members], w_all[members]
    sel = lambda x: np.asarray(x[b][members][:, heads_idx], dtype=np.float64)
    qq = rope_3d_at(sel(q), tm, hm, wm, base)
    kk = rope_3d_at(sel(k), tm, hm, wm, base)
    tr = lambda x: x.transpose(1, 0, 2)
    dq, dk, dv = attention_backward(tr(qq), tr(kk), tr(sel(v)), tr(sel(do)))
    dq = rope_3d_transpose_at(tr(dq), tm, hm, wm, base)
    dk = rope_3d_transpose_at(tr(dk), tm, hm, wm, base)
    return members, dq, dk, tr(dv)


def skiparse_backward_flops(B, N, heads, head_dim, sparse_k):
    """Backward attention FLOPs counted for a Skiparse call: 8 * B * heads * N * (N/k) * d.

    Wan 2.1 report, section 4.3.1: the backward pass of attention costs twice
    the forward (beta = 8 against 4), applied to k scopes of length N/k.
    """
    return 8.0 * B * heads * N * (N // sparse_k) * head_dim


def skiparse_flops(B, N, heads, head_dim, sparse_k):
    """Forward attention FLOPs counted for a Skiparse call: 4 * B * heads * N * (N/k) * d.

    Wan 2.1 report, section 4.3.1 "Workload Analysis": non-causal attention
    costs beta*b*s^2*h with beta = 4 in the forward pass; Skiparse runs it
    on k scopes of length N/k, i.e. k * 4 * (N/k)^2 * d per batch and head.
    """
    return 4.0 * B * heads * N * (N // sparse_k) * head_dim
