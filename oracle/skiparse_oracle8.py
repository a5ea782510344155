"""CPU oracle of 8-bit Skiparse attention -- TEST INFRASTRUCTURE ONLY.

Like :mod:`oracle.skiparse_oracle`, this module is imported only by
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``; it shares no code with the HIP library.

What the pages fix
------------------
Wan 2.1 report, section 4.4.3 "Quantization", paragraph "8-Bit
FlashAttention":

* S = Q K^T is computed from Int8 operands, O = P V from FP8 (E4M3)
  operands (their "mixed 8-bit" strategy);
* the PV products of one key block are reduced on the matrix cores, and the
  sum across blocks is carried in float32 registers, fused with the rescale of
  O when the running maximum moves.

Everything else about the attention is the exact Skiparse attention of
:mod:`oracle.skiparse_oracle` (3D RoPE before the rearrange, Single/Group Skip
scopes, softmax with scale 1/sqrt(head_dim), reverse).

What the pages leave open, and the reading taken
------------------------------------------------
* Quantisation grains (the same section applies per-token scales to
  activations in its FP8 GEMMs; FlashAttention-3's FP8 path, which the
  report adapts, takes one descale per (batch, head)):
  - q' (q after RoPE): symmetric int8, one scale per (batch, token, head):
    amax = max |q'| over head_dim, code = round-half-even(q' * (127 / amax));
  - k' (k after RoPE): symmetric int8, one scale per (batch, head): amax over
    every token and channel of that head;
  - v: E4M3, one scale per (batch, head, channel): amax over every token,
    code = E4M3(v * (448 / amax)); 448 is the largest finite E4M3 value.
  A zero amax gives all-zero codes.
* The int8 codes are integers that floating point decides, so they are taken
  in the precision the kernel uses: RoPE in float32 from a float32 cos/sin
  table (angles and their cosines evaluated in float64, then rounded), one
  rounding per multiply and per add (no fused multiply-add); the reciprocal
  127/amax and the product x * (127/amax) each rounded to float32.
* P's quantisation: the softmax weights are taken against an integer
  reference M = ceil(max_j z_j) of the row's scores in base-2 units,
  z = S * log2(e) / sqrt(d), and scaled by 2^8: P_j = 2^(z_j - M + 8), so
  every weight lies in (0, 256] (inside E4M3's range) and a kernel that moves
  its reference during the scan rescales by exact powers of two.  The PV
  operand is E4M3(P_j); the row sum l = sum_j P_j uses the unquantised
  weights (the softmax itself stays in float32).
* O_i = (sum_j E4M3(P_ij) * V~_j) * (v_amax / 448) / l_i, where V~ are the
  decoded E4M3 codes.

Layouts (the library's boundary uses the same ones)
---------------------------------------------------
q8, k8: int8 (B, N, heads, d) in the original token order; q_amax: float32
(B, N, heads); k_amax: float32 (B, heads); v_amax: float32 (B, heads, d);
vt8: uint8 E4M3 codes (B, heads, sparse_k, d, Lp) -- V of every scope
transposed (channel-major) in scope-position order, each channel row padded
with zero codes to Lp = L rounded up to a multiple of 64.

Every pin of this module lives in ``tests/test_oracle8_pins.py``.
"""

from __future__ import annotations

import math

import numpy as np

from . import skiparse_oracle as base

E4M3_MAX = 448.0
INT8_MAX = 127
P_HEADROOM_LOG2 = 8      # largest softmax weight fed to E4M3 is 2^8
VT_PAD = 64              # channel rows of vt8 are padded to a multiple of this many keys


# ---------------------------------------------------------------------------
# E4M3 (OCP 8-bit float: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
# no infinities, S.1111.111 is NaN, largest finite value 448)
# ---------------------------------------------------------------------------

def e4m3_decode(codes):
    """float64 values of uint8 E4M3 codes (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(x):
    """uint8 E4M3 codes of finite values, round to nearest, ties to even.

    The spacing of E4M3 values in [2^E, 2^(E+1)) is 2^(E-3) for E >= -6 and
    2^-9 below 2^-6 (subnormals).  A magnitude that rounds above 448 is an
    error here: the method never produces one.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.isfinite(x).all():
        raise ValueError("e4m3_encode takes finite values only")
    a = np.abs(x)
    _, ex = np.frexp(a)                     # a = f * 2^ex, f in [0.5, 1)
    E = np.maximum(ex - 1, -6)              # floor(log2 a), clamped to the subnormal exponent
    quantum = np.exp2(E.astype(np.float64) - 3.0)
    n = np.rint(a / quantum)                # exact division by a power of two; rint ties to even
    val = n * quantum
    if (val > E4M3_MAX).any():
        raise ValueError("value rounds beyond the E4M3 range")
    # value -> code
    _, ev = np.frexp(val)
    Ev = ev - 1
    normal = val >= 2.0 ** -6
    exp_field = np.where(normal, Ev + 7, 0)
    mant = np.where(normal, val / np.exp2(Ev.astype(np.float64)) * 8.0 - 8.0, val / 2.0 ** -9)
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(val == 0, 0, code)
    code = code | np.where(np.signbit(x), 0x80, 0)      # the sign survives rounding to zero (-0 is 0x80)
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# Quantisation (float32 arithmetic, one rounding per operation)
# ---------------------------------------------------------------------------

def rope_table_f32(axis_len: int, d_a: int, rope_base: float = base.ROPE_BASE):
    """float32 (cos, sin) of pos * rope_base**(-2j/d_a), pos < axis_len, j < d_a/2.

    The angle and its cosine/sine are evaluated in float64, then rounded once.
    """
    j = np.arange(d_a // 2, dtype=np.float64)
    freq = rope_base ** (-2.0 * j / d_a)
    theta = np.arange(axis_len, dtype=np.float64)[:, None] * freq[None, :]
    return np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)


def rope_3d_f32(x, T: int, H: int, W: int):
    """3D RoPE of (B, N, heads, d) in float32 with the pairs of oracle.rope_3d_at.

    x1' = x1*c - x2*s and x2' = x2*c + x1*s, every product and sum rounded to
    float32 (numpy float32 arithmetic), cos/sin from :func:`rope_table_f32`.
    """
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    t, h, w = base.token_positions(T, H, W)
    out = x.copy()
    offset = 0
    for pos, n_pos, d_a in zip((t, h, w), (T, H, W), base.rope_axis_sizes(d)):
        half = d_a // 2
        cos, sin = rope_table_f32(n_pos, d_a)
        c = cos[pos][:, None, :]            # (N, 1, half)
        s = sin[pos][:, None, :]
        x1 = x[..., offset:offset + half]
        x2 = x[..., offset + half:offset + d_a]
        out[..., offset:offset + half] = (x1 * c) - (x2 * s)
        out[..., offset + half:offset + d_a] = (x2 * c) + (x1 * s)
        offset += d_a
    return out


def quantize_int8(x32, amax32):
    """int8 codes round-half-even(x * (127/amax)), float32 arithmetic; amax == 0 gives 0."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax32 = np.asarray(amax32, dtype=np.float32)
    safe = np.where(amax32 > 0, amax32, np.float32(1.0)).astype(np.float32)
    r = (np.float32(INT8_MAX) / safe).astype(np.float32)
    y = (x32 * r).astype(np.float32)
    codes = np.clip(np.rint(y), -INT8_MAX, INT8_MAX)
    return np.where(amax32 > 0, codes, 0).astype(np.int8)


def padded_scope_len(L: int) -> int:
    return (L + VT_PAD - 1) // VT_PAD * VT_PAD


def quantize_8bit(q, k, v, T: int, H: int, W: int, sparse_k: int, mode: int):
    """The 8-bit operands of Skiparse attention (readings in the module docstring).

    q, k, v: (B, N, heads, d), values exactly representable in float32.
    Returns a dict with q8, q_amax, k8, k_amax, vt8, v_amax in the layouts of
    the module docstring.
    """
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    B, N, heads, d = q.shape
    if N != T * H * W:
        raise ValueError("N must equal T*H*W")
    rq = rope_3d_f32(q, T, H, W)
    rk = rope_3d_f32(k, T, H, W)
    q_amax = np.abs(rq).max(axis=-1)                          # (B, N, heads)
    q8 = quantize_int8(rq, q_amax[..., None])
    k_amax = np.abs(rk).max(axis=(1, 3))                      # (B, heads)
    k8 = quantize_int8(rk, k_amax[:, None, :, None])
    v_amax = np.abs(v).max(axis=1)                            # (B, heads, d)
    safe = np.where(v_amax > 0, v_amax, np.float32(1.0)).astype(np.float32)
    rv = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    vs = (v * rv[:, None, :, :]).astype(np.float32)
    vq = np.where(v_amax[:, None, :, :] > 0, e4m3_encode(vs), 0).astype(np.uint8)
    table = base.scope_table(N, sparse_k, mode)                # (k, L)
    L = N // sparse_k
    Lp = padded_scope_len(L)
    vt8 = np.zeros((B, heads, sparse_k, d, Lp), dtype=np.uint8)
    # vq[b, table[s, p], h, c] -> vt8[b, h, s, c, p]
    vt8[..., :L] = vq[:, table].transpose(0, 3, 1, 4, 2)
    return {"q8": q8, "q_amax": q_amax.astype(np.float32), "k8": k8,
            "k_amax": k_amax.astype(np.float32), "vt8": vt8, "v_amax": v_amax.astype(np.float32)}


# ---------------------------------------------------------------------------
# 8-bit attention inside each scope
# ---------------------------------------------------------------------------

def attention_8bit_scope(q8, q_amax, k8, k_amax, vt, v_amax):
    """One (batch, head, scope) problem, float64 except where the method rounds.

    q8: (Lq, d) int8 codes of the query rows, q_amax: (Lq,);
    k8: (L, d) int8 codes of the scope's keys, k_amax: scalar;
    vt: (d, L) E4M3 codes of the scope's values (transposed), v_amax: (d,).
    """
    d = q8.shape[-1]
    acc = np.asarray(q8, dtype=np.int64) @ np.asarray(k8, dtype=np.int64).T      # exact
    scale = (np.asarray(q_amax, np.float64) / INT8_MAX) * (float(k_amax) / INT8_MAX)
    z = acc * (scale * math.log2(math.e) / math.sqrt(d))[:, None]
    M = np.ceil(z.max(axis=-1, keepdims=True))
    p = np.exp2(z - M + P_HEADROOM_LOG2)
    pq = e4m3_decode(e4m3_encode(p))
    l = p.sum(axis=-1, keepdims=True)
    vdec = e4m3_decode(vt).T                                   # (L, d)
    return (pq @ vdec) * (np.asarray(v_amax, np.float64) / E4M3_MAX)[None, :] / l


def skiparse_attention_8bit(qz, T: int, H: int, W: int, sparse_k: int, mode: int):
    """8-bit Skiparse attention of the operands from :func:`quantize_8bit`: (B, N, heads, d) float64."""
    q8, k8 = qz["q8"], qz["k8"]
    B, N, heads, d = q8.shape
    table = base.scope_table(N, sparse_k, mode)
    L = N // sparse_k
    out = np.zeros((B, N, heads, d), dtype=np.float64)
    for b in range(B):
        for hd in range(heads):
            for s in range(sparse_k):
                toks = table[s]
                out[b, toks, hd] = attention_8bit_scope(
                    q8[b, toks, hd], qz["q_amax"][b, toks, hd], k8[b, toks, hd], qz["k_amax"][b, hd],
                    qz["vt8"][b, hd, s, :, :L], qz["v_amax"][b, hd])
    return out


def skiparse_attention_8bit_rows(qz, T: int, H: int, W: int, sparse_k: int, mode: int,
                                 b: int, s: int, positions, heads_idx):
    """Output rows of scope s of batch b at the given scope positions, for the given heads.

    Returns (tokens, out) with out of shape (len(positions), len(heads_idx), d).
    """
    q8, k8 = qz["q8"], qz["k8"]
    N, d = q8.shape[1], q8.shape[3]
    table = base.scope_table(N, sparse_k, mode)
    L = N // sparse_k
    toks = table[s]
    rows = toks[np.asarray(positions)]
    out = np.stack([attention_8bit_scope(q8[b, rows, hd], qz["q_amax"][b, rows, hd], k8[b, toks, hd],
                                         qz["k_amax"][b, hd], qz["vt8"][b, hd, s, :, :L], qz["v_amax"][b, hd])
                    for hd in heads_idx], axis=1)
    return rows, out
