"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here re-types the oracle's own formulas: each test compares it with
something independent of it -- the pages' literal einops patterns run by the
einops library, scope tables written out by hand from the prose
(``tests/golden/``), torch's scaled-dot-product attention (the call the
Open-Sora Plan page makes), closed forms and invariants, and brute force with
plain Python loops on tiny inputs.
"""

import math
import os

import numpy as np
import pytest
import torch
from einops import rearrange as einops_rearrange

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Permutation: bit-exact pins
# ---------------------------------------------------------------------------

# The pattern strings exactly as the Open-Sora Plan page prints them
# ("Skiparse Attention", Single Skip and Group Skip implementations).
PAGE_SINGLE_FWD = 'b (g k) d -> (k b) g d'
PAGE_SINGLE_REV = '(k b) g d -> b (g k) d'
PAGE_GROUP_FWD = ' b (n m k) d -> (m b) (n k) d'
PAGE_GROUP_REV = '(m b) (n k) d -> b (n m k) d'


def _page_rearrange(x, k, mode):
    if mode == oracle.SINGLE:
        return einops_rearrange(x, PAGE_SINGLE_FWD, k=k)
    return einops_rearrange(x, PAGE_GROUP_FWD, m=k, k=k)


def _page_reverse(x, k, mode):
    if mode == oracle.SINGLE:
        return einops_rearrange(x, PAGE_SINGLE_REV, k=k)
    return einops_rearrange(x, PAGE_GROUP_REV, m=k, k=k)


PERM_CASES = [
    (oracle.SINGLE, 1, 3, 12, 5),
    (oracle.SINGLE, 2, 2, 256, 7),
    (oracle.SINGLE, 4, 3, 64, 3),
    (oracle.SINGLE, 8, 1, 128, 2),
    (oracle.SINGLE, 3, 2, 27, 4),
    (oracle.GROUP, 1, 2, 10, 3),
    (oracle.GROUP, 2, 2, 256, 7),
    (oracle.GROUP, 4, 3, 64, 3),
    (oracle.GROUP, 8, 1, 128, 2),
    (oracle.GROUP, 3, 2, 36, 4),
]


@pytest.mark.parametrize("mode,k,B,N,C", PERM_CASES)
def test_rearrange_matches_page_patterns_bit_exact(mode, k, B, N, C):
    rng = np.random.default_rng(1234 + N + k)
    # arbitrary bit patterns (including NaN payloads) carried as uint32
    x = rng.integers(0, 2**32, size=(B, N, C), dtype=np.uint64).astype(np.uint32)
    got = oracle.rearrange(x, k, mode)
    want = _page_rearrange(x, k, mode)
    assert got.shape == (k * B, N // k, C)
    assert np.array_equal(got, want)
    back = oracle.reverse(got, k, mode)
    assert np.array_equal(back, _page_reverse(want, k, mode))
    assert np.array_equal(back, x)


@pytest.mark.parametrize("mode,k,B,N,C", PERM_CASES)
def test_bf16_payload_round_trip(mode, k, B, N, C):
    gen = torch.Generator().manual_seed(N * 31 + k)
    x = torch.randn(B, N, C, generator=gen).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy()
    assert np.array_equal(oracle.reverse(oracle.rearrange(bits, k, mode), k, mode), bits)


def _read_scope_golden():
    cases = []
    with open(os.path.join(GOLDEN, "scopes_hand_derived.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, body = line.split(":")
            mode, N, k = head.split()
            scopes = [[int(t) for t in part.split()] for part in body.split("|")]
            cases.append((oracle.SINGLE if mode == "single" else oracle.GROUP, int(N), int(k), scopes))
    return cases


@pytest.mark.parametrize("mode,N,k,scopes", _read_scope_golden())
def test_scope_table_matches_hand_derived_golden(mode, N, k, scopes):
    assert oracle.scope_table(N, k, mode).tolist() == scopes


def test_batch_order_matches_hand_derived_golden():
    with open(os.path.join(GOLDEN, "batch_order_hand_derived.txt")) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(lines) == 2
    for line in lines:
        head, body = line.split(":", 1)
        mode_s, B, N, k = head.split()
        B, N, k = int(B), int(N), int(k)
        mode = oracle.SINGLE if mode_s == "single" else oracle.GROUP
        # payload encodes (batch, token) so rows can be read back
        x = np.zeros((B, N, 2), dtype=np.int64)
        x[:, :, 0] = np.arange(B)[:, None]
        x[:, :, 1] = np.arange(N)[None, :]
        r = oracle.rearrange(x, k, mode)
        rows = []
        for part in body.split("|"):
            b, toks = part.strip().split(":")
            rows.append((int(b), [int(t) for t in toks.split()]))
        assert len(rows) == r.shape[0]
        for ri, (b, toks) in enumerate(rows):
            assert (r[ri, :, 0] == b).all()
            assert r[ri, :, 1].tolist() == toks


@pytest.mark.parametrize("N,k", [(256, 1), (256, 2), (256, 4), (256, 8), (21120, 4), (46080, 8), (36864, 4)])
@pytest.mark.parametrize("mode", [oracle.SINGLE, oracle.GROUP])
def test_scope_membership_from_prose_brute_force(N, k, mode):
    if mode == oracle.GROUP and N % (k * k):
        pytest.skip("group skip needs N % k^2 == 0")
    table = oracle.scope_table(N, k, mode)
    assert table.shape == (k, N // k)
    # partition of [0, N)
    assert np.array_equal(np.sort(table.ravel()), np.arange(N))
    for s in range(k):
        members = table[s]
        # in-scope order is increasing token index
        assert (np.diff(members) > 0).all()
        if mode == oracle.SINGLE:
            # every k-th token, starting at s
            assert (members % k == s).all()
        else:
            # groups of k adjacent tokens; group index congruent to s mod k
            assert ((members // k) % k == s).all()
            assert len(members) == N // k


def test_rearrange_rejects_non_divisible_like_einops():
    x = np.zeros((1, 10, 2))
    with pytest.raises(Exception):
        _page_rearrange(x, 4, oracle.SINGLE)
    with pytest.raises(ValueError):
        oracle.rearrange(x, 4, oracle.SINGLE)
    x = np.zeros((1, 24, 2))
    with pytest.raises(Exception):
        _page_rearrange(x, 4, oracle.GROUP)
    with pytest.raises(ValueError):
        oracle.rearrange(x, 4, oracle.GROUP)


# ---------------------------------------------------------------------------
# 3D RoPE: closed forms and invariants
# ---------------------------------------------------------------------------

def test_rope_axis_split_matches_stated_ratio():
    assert oracle.rope_axis_sizes(64) == (16, 24, 24)
    assert oracle.rope_axis_sizes(128) == (32, 48, 48)


def test_rope_identity_at_origin():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 1, 3, 64))
    got = oracle.rope_3d_at(x, [0], [0], [0])
    assert np.array_equal(got, x)


@pytest.mark.parametrize("d", [64, 128])
def test_rope_unit_vector_worked_values(d):
    # A unit vector at the first slot of an axis chunk rotates by angle pos*base^0 = pos
    # into its rotate-half partner d_a/2 slots later, with cos on itself and +sin on the
    # partner; the (j=1) slot rotates by pos*base^(-2/d_a).
    d_t, d_h, d_w = oracle.rope_axis_sizes(d)
    offsets = {"t": 0, "h": d_t, "w": d_t + d_h}
    sizes = {"t": d_t, "h": d_h, "w": d_w}
    for axis, pos in (("t", 3), ("h", 5), ("w", 7)):
        o, da = offsets[axis], sizes[axis]
        grid = {"t": 0, "h": 0, "w": 0}
        grid[axis] = pos
        for j, angle in ((0, float(pos)), (1, pos * 10000.0 ** (-2.0 / da))):
            x = np.zeros((1, 1, 1, d))
            x[..., o + j] = 1.0
            y = oracle.rope_3d_at(x, [grid["t"]], [grid["h"]], [grid["w"]])[0, 0, 0]
            expect = np.zeros(d)
            expect[o + j] = math.cos(angle)
            expect[o + j + da // 2] = math.sin(angle)
            assert np.allclose(y, expect, atol=1e-15, rtol=0)
            # the partner slot rotates the other way: e_{partner} -> -sin on the first slot
            x = np.zeros((1, 1, 1, d))
            x[..., o + j + da // 2] = 1.0
            y = oracle.rope_3d_at(x, [grid["t"]], [grid["h"]], [grid["w"]])[0, 0, 0]
            expect = np.zeros(d)
            expect[o + j] = -math.sin(angle)
            expect[o + j + da // 2] = math.cos(angle)
            assert np.allclose(y, expect, atol=1e-15, rtol=0)


def test_rope_preserves_pair_norms():
    rng = np.random.default_rng(1)
    T, H, W, d = 3, 4, 5, 128
    x = rng.standard_normal((2, T * H * W, 3, d))
    y = oracle.rope_3d(x, T, H, W)
    d_t, d_h, d_w = oracle.rope_axis_sizes(d)
    o = 0
    for da in (d_t, d_h, d_w):
        half = da // 2
        n_x = x[..., o:o + half] ** 2 + x[..., o + half:o + da] ** 2
        n_y = y[..., o:o + half] ** 2 + y[..., o + half:o + da] ** 2
        assert np.allclose(n_x, n_y, rtol=1e-12, atol=1e-12)
        o += da


def test_rope_relative_position_property():
    # <R(q, P1), R(k, P2)> depends only on P1 - P2 (per axis).
    rng = np.random.default_rng(2)
    d = 128
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, 1, d))
    base_pairs = [((1, 2, 3), (4, 0, 6)), ((0, 9, 1), (2, 2, 2))]
    for p1, p2 in base_pairs:
        ref = None
        for shift in ((0, 0, 0), (5, 0, 0), (0, 7, 0), (0, 0, 11), (3, 4, 5)):
            a = [p1[i] + shift[i] for i in range(3)]
            b = [p2[i] + shift[i] for i in range(3)]
            rq = oracle.rope_3d_at(q, [a[0]], [a[1]], [a[2]])
            rk = oracle.rope_3d_at(k, [b[0]], [b[1]], [b[2]])
            dot = float((rq * rk).sum())
            if ref is None:
                ref = dot
            assert abs(dot - ref) < 1e-11
        # and it does change when only one position moves
        rq = oracle.rope_3d_at(q, [p1[0] + 1], [p1[1]], [p1[2]])
        rk = oracle.rope_3d_at(k, [p2[0]], [p2[1]], [p2[2]])
        assert abs(float((rq * rk).sum()) - ref) > 1e-6


def test_rope_1d_special_case_is_textbook_complex_rotation():
    # With T = H = 1 only the w chunk rotates, and it is 1-D RoPE along w: each
    # rotate-half pair (x1, x2) is the complex number x1 + i x2 multiplied by e^{i w theta_j}.
    rng = np.random.default_rng(3)
    W, d = 9, 64
    x = rng.standard_normal((1, W, 2, d))
    y = oracle.rope_3d(x, 1, 1, W)
    d_t, d_h, d_w = oracle.rope_axis_sizes(d)
    o = d_t + d_h
    half = d_w // 2
    z = x[..., o:o + half] + 1j * x[..., o + half:o + d_w]
    inv_freq = np.array([10000.0 ** (-(2.0 * j) / d_w) for j in range(half)])
    rot = np.exp(1j * np.arange(W)[:, None] * inv_freq[None, :])[None, :, None, :]
    zr = z * rot
    assert np.allclose(y[..., o:o + half], zr.real, atol=1e-13)
    assert np.allclose(y[..., o + half:o + d_w], zr.imag, atol=1e-13)
    assert np.array_equal(y[..., :o], x[..., :o])   # t and h chunks at position 0 are untouched


def _read_position_golden():
    grids = []
    with open(os.path.join(GOLDEN, "positions_hand_derived.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "grid":
                grids.append((int(parts[1]), int(parts[2]), int(parts[3]), []))
            else:
                grids[-1][3].append(tuple(int(p) for p in parts))
    return grids


POSITION_GOLDEN = _read_position_golden()


@pytest.mark.parametrize("T,H,W,rows", POSITION_GOLDEN)
def test_token_positions_match_hand_derived_golden(T, H, W, rows):
    # Frame-major flattening with T, H > 1: a dropped "mod H" on h, or h and w in
    # swapped roles, changes several of these hand-written rows.
    t, h, w = oracle.token_positions(T, H, W)
    assert [r[0] for r in rows] == list(range(T * H * W))
    assert t.tolist() == [r[1] for r in rows]
    assert h.tolist() == [r[2] for r in rows]
    assert w.tolist() == [r[3] for r in rows]


@pytest.mark.parametrize("d", [64, 128])
def test_rope_3d_worked_values_on_a_3d_grid(d):
    # Token 23 of the 2 x 3 x 4 grid sits at (t, h, w) = (1, 2, 3) (hand-derived golden).
    # A unit vector on slot j of an axis chunk of size d_a turns by pos * 10000^(-2j/d_a):
    # j = 0 gives the position itself, j = 1 the hand-evaluated powers of ten below.
    T, H, W, n = 2, 3, 4, 23
    assert POSITION_GOLDEN[0][3][n] == (23, 1, 2, 3)
    if d == 64:   # chunks 16 / 24 / 24
        chunks = {"t": (0, 16, 1, 10.0 ** -0.5), "h": (16, 24, 2, 10.0 ** (-1.0 / 3.0)),
                  "w": (40, 24, 3, 10.0 ** (-1.0 / 3.0))}
    else:         # chunks 32 / 48 / 48
        chunks = {"t": (0, 32, 1, 10.0 ** -0.25), "h": (32, 48, 2, 10.0 ** (-1.0 / 6.0)),
                  "w": (80, 48, 3, 10.0 ** (-1.0 / 6.0))}
    for axis, (o, da, pos, freq1) in chunks.items():
        for j, angle in ((0, float(pos)), (1, pos * freq1)):
            x = np.zeros((1, T * H * W, 1, d))
            x[0, n, 0, o + j] = 1.0
            y = oracle.rope_3d(x, T, H, W)[0, n, 0]
            expect = np.zeros(d)
            expect[o + j] = math.cos(angle)
            expect[o + j + da // 2] = math.sin(angle)
            assert np.allclose(y, expect, atol=1e-15, rtol=0), (axis, j)


@pytest.mark.parametrize("T,H,W,rows", POSITION_GOLDEN)
def test_rope_3d_is_per_axis_complex_rotation_at_golden_positions(T, H, W, rows):
    # On every token of the grid, each axis chunk is 1-D RoPE along that axis: the pair
    # (x1, x2) read as x1 + i x2 is multiplied by e^{i pos theta_j}, with the token's grid
    # position taken from the hand-derived golden rather than from the oracle.
    rng = np.random.default_rng(10)
    d = 64
    x = rng.standard_normal((2, T * H * W, 3, d))
    y = oracle.rope_3d(x, T, H, W)
    pos = np.array([[r[1], r[2], r[3]] for r in rows], dtype=np.float64)   # (N, 3)
    o = 0
    for a, da in enumerate((16, 24, 24)):
        half = da // 2
        z = x[..., o:o + half] + 1j * x[..., o + half:o + da]
        inv_freq = np.array([10000.0 ** (-(2.0 * j) / da) for j in range(half)])
        rot = np.exp(1j * pos[:, a][:, None] * inv_freq[None, :])[None, :, None, :]
        assert np.allclose(y[..., o:o + half], (z * rot).real, atol=1e-13)
        assert np.allclose(y[..., o + half:o + da], (z * rot).imag, atol=1e-13)
        o += da


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _sdpa_fp64(q, k, v):
    # torch's scaled_dot_product_attention (the call the Open-Sora Plan page makes),
    # on the CPU in float64; (batch, L, d) per head -> default scale 1/sqrt(d)
    with torch.no_grad():
        return torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 37, 64)) * 2.0
    k = rng.standard_normal((3, 53, 64)) * 2.0
    v = rng.standard_normal((3, 53, 64))
    assert np.allclose(oracle.attention(q, k, v), _sdpa_fp64(q, k, v), atol=1e-12, rtol=0)


def test_k1_is_dense_rope_attention_via_sdpa():
    # sparse_k = 1: the permutation is the identity, so Skiparse is dense full-3D
    # attention of the RoPE'd q and k ("Full 3D Attention", Open-Sora Plan docs).
    rng = np.random.default_rng(5)
    T, H, W, heads, d = 2, 3, 4, 2, 64
    N = T * H * W
    q, k, v = (rng.standard_normal((2, N, heads, d)) for _ in range(3))
    for mode in (oracle.SINGLE, oracle.GROUP):
        got = oracle.skiparse_attention(q, k, v, T, H, W, 1, mode)
        rq = oracle.rope_3d(q, T, H, W)
        rk = oracle.rope_3d(k, T, H, W)
        for b in range(2):
            for hh in range(heads):
                want = _sdpa_fp64(rq[b, :, hh][None], rk[b, :, hh][None], v[b, :, hh][None])[0]
                assert np.allclose(got[b, :, hh], want, atol=1e-12, rtol=0)


def _brute_force_skiparse(q, k, v, T, H, W, sparse_k, mode):
    """Plain Python loops, membership straight from the prose (no rearrange used)."""
    B, N, heads, d = q.shape
    rq = oracle.rope_3d(q, T, H, W)
    rk = oracle.rope_3d(k, T, H, W)
    out = np.zeros_like(rq)
    for n in range(N):
        if mode == oracle.SINGLE:
            members = [m for m in range(N) if m % sparse_k == n % sparse_k]
        else:
            members = [m for m in range(N) if (m // sparse_k) % sparse_k == (n // sparse_k) % sparse_k]
        for b in range(B):
            for hh in range(heads):
                scores = [sum(rq[b, n, hh, i] * rk[b, m, hh, i] for i in range(d)) / math.sqrt(d)
                          for m in members]
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                for i in range(d):
                    out[b, n, hh, i] = sum(w[j] * v[b, m, hh, i] for j, m in enumerate(members)) / tot
    return out


@pytest.mark.parametrize("mode,sparse_k", [(oracle.SINGLE, 2), (oracle.GROUP, 2), (oracle.SINGLE, 4), (oracle.GROUP, 4)])
def test_skiparse_matches_python_loop_brute_force(mode, sparse_k):
    rng = np.random.default_rng(6 + sparse_k + mode)
    T, H, W, heads, d = 2, 2, 8, 1, 16
    N = T * H * W
    q, k, v = (rng.standard_normal((1, N, heads, d)) for _ in range(3))
    got = oracle.skiparse_attention(q, k, v, T, H, W, sparse_k, mode)
    want = _brute_force_skiparse(q, k, v, T, H, W, sparse_k, mode)
    assert np.allclose(got, want, atol=1e-12, rtol=0)


def test_uniform_softmax_closed_form():
    # q = 0 makes every score 0 whatever RoPE does, so each output row is the plain
    # mean of v over the token's scope.
    rng = np.random.default_rng(7)
    T, H, W, heads, d, sk = 4, 8, 8, 2, 64, 2
    N = T * H * W
    q = np.zeros((1, N, heads, d))
    k = rng.standard_normal((1, N, heads, d))
    v = rng.integers(-4, 5, size=(1, N, heads, d)).astype(np.float64)
    for mode in (oracle.SINGLE, oracle.GROUP):
        got = oracle.skiparse_attention(q, k, v, T, H, W, sk, mode)
        for n in (0, 1, 2, 3, 77, N - 1):
            s = (n % sk) if mode == oracle.SINGLE else (n // sk) % sk
            if mode == oracle.SINGLE:
                mem = np.arange(s, N, sk)
            else:
                mem = np.array([m for m in range(N) if (m // sk) % sk == s])
            assert np.allclose(got[0, n], v[0, mem].mean(axis=0), atol=1e-13)


def test_rope_before_permute_differs_from_in_scope_positions():
    # The implementation note says RoPE must use the original grid positions.  The wrong
    # variant (RoPE by in-scope position) must give a clearly different answer.
    rng = np.random.default_rng(8)
    T, H, W, heads, d, sk = 4, 8, 8, 2, 64, 2
    N = T * H * W
    q, k, v = (rng.standard_normal((1, N, heads, d)) for _ in range(3))
    right = oracle.skiparse_attention(q, k, v, T, H, W, sk, oracle.SINGLE)
    # wrong order: rearrange first, then RoPE each scope as a sequence of L tokens on an
    # L = (T/2) x H x W grid
    rq = oracle.rope_rearrange(q, T, H, W, sk, oracle.SINGLE, apply_rope=False)
    rk = oracle.rope_rearrange(k, T, H, W, sk, oracle.SINGLE, apply_rope=False)
    rv = oracle.rope_rearrange(v, T, H, W, sk, oracle.SINGLE, apply_rope=False)
    rq = oracle.rope_3d(rq, T // 2, H, W)
    rk = oracle.rope_3d(rk, T // 2, H, W)
    o = oracle.attention(rq.transpose(0, 2, 1, 3), rk.transpose(0, 2, 1, 3), rv.transpose(0, 2, 1, 3))
    wrong = oracle.reverse_rows(o.transpose(0, 2, 1, 3), sk, oracle.SINGLE)
    assert np.abs(right - wrong).max() > 0.1


@pytest.mark.parametrize("mode,sparse_k,B", [(oracle.SINGLE, 2, 1), (oracle.GROUP, 2, 2), (oracle.SINGLE, 8, 2), (oracle.GROUP, 4, 1)])
def test_rows_function_matches_full_oracle(mode, sparse_k, B):
    rng = np.random.default_rng(9)
    T, H, W, heads, d = 4, 8, 8, 3, 64
    N = T * H * W
    q, k, v = (rng.standard_normal((B, N, heads, d)) for _ in range(3))
    full = oracle.skiparse_attention(q, k, v, T, H, W, sparse_k, mode)
    b_idx = rng.integers(0, B, size=40)
    t_idx = rng.integers(0, N, size=40)
    rows = oracle.skiparse_attention_rows(q, k, v, T, H, W, sparse_k, mode, b_idx, t_idx)
    assert np.allclose(rows, full[b_idx, t_idx], atol=1e-13, rtol=0)


def test_flops_formula():
    # Wan 2.1 report 4.3.1: beta = 4 forward -> 4 * b * s^2 * h per head-dim unit.
    assert oracle.skiparse_flops(1, 21120, 24, 128, 4) == 4.0 * 24 * 21120 * 5280 * 128
    assert oracle.skiparse_flops(1, 256, 2, 64, 1) == 4.0 * 2 * 256 * 256 * 64
