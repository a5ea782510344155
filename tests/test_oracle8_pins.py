"""Pins of the 8-bit Skiparse attention oracle (CPU only).

oracle.skiparse_oracle8 is pinned against things that do not retype it:

* E4M3: every one of the 256 codes decoded, and random and tie-breaking values
  encoded, against torch's float8_e4m3fn conversion (a library routine);
* int8 quantisation: against torch.round (half to even) of the same float32
  product, and its defining bounds (the row's largest magnitude maps to +-127,
  the error is at most half a step);
* float32 RoPE: against the float64 RoPE of the main oracle (itself pinned);
* the vt8 layout: against scope membership written from the pages' prose with
  plain loops;
* the attention: the q = 0 closed form (uniform weights: the output is the
  scope mean of the dequantised values, exactly), plain-loop brute force on
  tiny inputs, and the exact (unquantised) Skiparse attention within the
  quantisation error the readings imply.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import skiparse_oracle8 as o8


def _bf16(rng, shape, scale=1.0):
    x = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(torch.bfloat16)
    return x.float().numpy()


# ---------------------------------------------------------------------------
# E4M3
# ---------------------------------------------------------------------------

def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = o8.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_and_round_trips():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * 40.0, rng.standard_normal(50000) * 1e-2,
                        rng.uniform(-448.0, 448.0, 50000)]).astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o8.e4m3_encode(x), ref)
    codes = np.arange(256, dtype=np.uint8)
    vals = o8.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(o8.e4m3_encode(vals[fin]), codes[fin])


def test_e4m3_ties_go_to_even():
    # 1 + 1/16 lies halfway between 1 (mantissa 0) and 1.125 (mantissa 1): even is 1
    assert o8.e4m3_decode(o8.e4m3_encode(np.array([1.0 + 1 / 16]))) == 1.0
    # 1.125 + 1/16 lies between mantissa 1 and 2: even is 1.25
    assert o8.e4m3_decode(o8.e4m3_encode(np.array([1.125 + 1 / 16]))) == 1.25
    # subnormal tie 1.5 * 2^-9 -> 2 * 2^-9
    assert o8.e4m3_decode(o8.e4m3_encode(np.array([1.5 * 2.0 ** -9]))) == 2.0 * 2.0 ** -9
    # the midpoint between 448 and the (missing) 480 must not be produced by the method
    with pytest.raises(ValueError):
        o8.e4m3_encode(np.array([470.0]))


# ---------------------------------------------------------------------------
# int8 quantisation and float32 RoPE
# ---------------------------------------------------------------------------

def test_int8_quantisation_matches_torch_round_and_bounds():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((500, 64)) * rng.uniform(0.01, 10.0, (500, 1))).astype(np.float32)
    amax = np.abs(x).max(axis=1, keepdims=True)
    codes = o8.quantize_int8(x, amax)
    r = torch.tensor(127.0, dtype=torch.float32) / torch.from_numpy(amax)
    ref = torch.round(torch.from_numpy(x) * r).clamp(-127, 127).to(torch.int8).numpy()
    assert np.array_equal(codes, ref)
    assert (np.abs(codes).max(axis=1) == 127).all()
    step = amax / 127.0
    assert (np.abs(codes * step - x) <= 0.5 * step * (1 + 1e-6)).all()
    assert np.array_equal(o8.quantize_int8(np.zeros((2, 8), np.float32), np.zeros((2, 1), np.float32)),
                          np.zeros((2, 8), np.int8))


@pytest.mark.parametrize("d", [64, 128])
def test_float32_rope_matches_float64_rope(d):
    T, H, W = 3, 5, 7
    rng = np.random.default_rng(2)
    x = _bf16(rng, (1, T * H * W, 2, d))
    got = o8.rope_3d_f32(x, T, H, W).astype(np.float64)
    want = oracle.rope_3d(x, T, H, W)
    # float32 table (half an ulp each) and three roundings per output
    assert np.abs(got - want).max() <= 4 * 2.0 ** -24 * (np.abs(x).max() * 2)


# ---------------------------------------------------------------------------
# vt8 layout
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode,sk,T,H,W", [(oracle.SINGLE, 4, 2, 4, 8), (oracle.GROUP, 2, 2, 4, 8),
                                           (oracle.SINGLE, 1, 1, 3, 5)])
def test_vt8_layout_from_the_prose(mode, sk, T, H, W):
    B, heads, d = 2, 2, 16
    N = T * H * W
    rng = np.random.default_rng(3)
    q, k, v = (_bf16(rng, (B, N, heads, d)) for _ in range(3))
    qz = o8.quantize_8bit(q, k, v, T, H, W, sk, mode)
    L = N // sk
    Lp = o8.padded_scope_len(L)
    assert qz["vt8"].shape == (B, heads, sk, d, Lp) and Lp % 64 == 0 and Lp >= L
    amax = np.abs(v).max(axis=1)
    for b in range(B):
        for hd in range(heads):
            for s in range(sk):
                # members of scope s in increasing token order, from the prose: Single Skip
                # takes every k-th token starting at s; Group Skip takes the runs of k adjacent
                # tokens whose run index is s modulo k
                if mode == oracle.SINGLE:
                    members = [n for n in range(N) if n % sk == s]
                else:
                    members = [n for n in range(N) if (n // sk) % sk == s]
                for p, n in enumerate(members):
                    for c in range(d):
                        want = o8.e4m3_encode(np.array([np.float32(v[b, n, hd, c]) *
                                                        np.float32(np.float32(448.0) / amax[b, hd, c])]))[0]
                        assert qz["vt8"][b, hd, s, c, p] == want
                assert not qz["vt8"][b, hd, s, :, L:].any()


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode,sk", [(oracle.SINGLE, 2), (oracle.GROUP, 2), (oracle.SINGLE, 1)])
def test_uniform_weights_give_the_scope_mean(mode, sk):
    T, H, W, B, heads, d = 2, 4, 8, 1, 2, 64
    N = T * H * W
    rng = np.random.default_rng(4)
    k, v = (_bf16(rng, (B, N, heads, d)) for _ in range(2))
    q = np.zeros_like(k)
    qz = o8.quantize_8bit(q, k, v, T, H, W, sk, mode)
    out = o8.skiparse_attention_8bit(qz, T, H, W, sk, mode)
    vdec = o8.e4m3_decode(qz["vt8"])
    table = oracle.scope_table(N, sk, mode)
    L = N // sk
    for hd in range(heads):
        for s in range(sk):
            mean = vdec[0, hd, s, :, :L].mean(axis=1) * qz["v_amax"][0, hd].astype(np.float64) / 448.0
            np.testing.assert_allclose(out[0, table[s], hd], np.broadcast_to(mean, (L, d)), rtol=1e-14, atol=1e-15)


def test_attention_matches_plain_loops():
    T, H, W, B, heads, d, sk = 2, 2, 4, 1, 2, 16, 2
    N = T * H * W
    rng = np.random.default_rng(5)
    q, k, v = (_bf16(rng, (B, N, heads, d), 2.0) for _ in range(3))
    for mode in (oracle.SINGLE, oracle.GROUP):
        qz = o8.quantize_8bit(q, k, v, T, H, W, sk, mode)
        out = o8.skiparse_attention_8bit(qz, T, H, W, sk, mode)
        vdec = o8.e4m3_decode(qz["vt8"])
        for hd in range(heads):
            for s in range(sk):
                members = [n for n in range(N) if (n % sk if mode == oracle.SINGLE else (n // sk) % sk) == s]
                for i, n in enumerate(members):
                    z = []
                    for m in members:
                        dot = sum(int(qz["q8"][0, n, hd, c]) * int(qz["k8"][0, m, hd, c]) for c in range(d))
                        z.append(dot * float(qz["q_amax"][0, n, hd]) / 127 * float(qz["k_amax"][0, hd]) / 127
                                 / math.sqrt(d) * math.log2(math.e))
                    M = math.ceil(max(z))
                    w = [2.0 ** (zz - M + 8) for zz in z]
                    wq = [float(o8.e4m3_decode(o8.e4m3_encode(np.array([x])))[0]) for x in w]
                    for c in range(d):
                        acc = sum(wq[j] * vdec[0, hd, s, c, j] for j in range(len(members)))
                        want = acc * float(qz["v_amax"][0, hd, c]) / 448.0 / sum(w)
                        assert abs(out[0, n, hd, c] - want) <= 1e-12 * max(1.0, abs(want))


@pytest.mark.parametrize("mode,sk,d", [(oracle.SINGLE, 2, 64), (oracle.GROUP, 2, 128), (oracle.SINGLE, 4, 128)])
def test_close_to_exact_attention(mode, sk, d):
    """E4M3 weights and values each carry a relative error of at most 2^-4 (about 2^-4/sqrt(3)
    RMS), int8 scores an error of half a step per operand: the output's relative RMS error
    against the exact fp64 Skiparse attention stays near 5 %; a wrong scale, exponent, sign or
    operand order gives errors of order 100 %."""
    T, H, W, B, heads = 2, 8, 8, 1, 2
    N = T * H * W
    rng = np.random.default_rng(6)
    q, k, v = (_bf16(rng, (B, N, heads, d)) for _ in range(3))
    qz = o8.quantize_8bit(q, k, v, T, H, W, sk, mode)
    got = o8.skiparse_attention_8bit(qz, T, H, W, sk, mode)
    want = oracle.skiparse_attention(q, k, v, T, H, W, sk, mode)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel <= 0.08, rel
    # peaked softmax (q x 4): errors of the same relative size
    qz = o8.quantize_8bit(q * 4, k, v, T, H, W, sk, mode)
    got = o8.skiparse_attention_8bit(qz, T, H, W, sk, mode)
    want = oracle.skiparse_attention(q * 4, k, v, T, H, W, sk, mode)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) <= 0.08


def test_rows_variant_matches_full():
    T, H, W, B, heads, d, sk = 2, 4, 8, 2, 3, 64, 4
    N = T * H * W
    rng = np.random.default_rng(7)
    q, k, v = (_bf16(rng, (B, N, heads, d)) for _ in range(3))
    for mode in (oracle.SINGLE, oracle.GROUP):
        qz = o8.quantize_8bit(q, k, v, T, H, W, sk, mode)
        full = o8.skiparse_attention_8bit(qz, T, H, W, sk, mode)
        rows, part = o8.skiparse_attention_8bit_rows(qz, T, H, W, sk, mode, 1, 3, [0, 5, 15], [2, 0])
        np.testing.assert_allclose(part, full[1][rows][:, [2, 0]], rtol=1e-14, atol=1e-15)
