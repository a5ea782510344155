"""GPU tests of the pre-rotated path (skiparse_rope_qk + skiparse_attn_rotated through the C ABI).

Bars:
* rope_qk against the fp64 oracle's 3D RoPE: each element is the bf16 rounding of a float32
  rotation (float32 table, three float32 operations, the scale), so it lies within one bf16
  rounding (2^-8 relative) plus a few float32 ulps of the exact rotated value; elements whose
  bf16 rounding differs from that of the exact value must stay rare (near-ties only);
* attn_rotated(rope_qk(q, k), v) equals skiparse_attn(q, k, v) bit for bit: the same operands
  in the same contraction order, the same softmax;
* one case per mode against the fp64 oracle at the attention bars (max 2e-2, mean 2e-3);
* attn_rotated_lse equals attn_lse (output and log2-sum-exp) bit for bit, and
  attn_bwd_rotated on rope_qk's outputs equals attn_bwd on q, k bit for bit (the backward
  kernels stage the same operand bits either way); one backward case against the fp64
  oracle's chain rule at the bars of test_gpu_backward.py.
"""

import numpy as np
import pytest
import torch

import oracle
import skiparse_sparse_attention_amd as sk
from skiparse_sparse_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    sk.lib()
    yield


def _bf16_round(x64):
    return torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


@pytest.mark.parametrize("B,T,H,W,heads", [(1, 4, 8, 16, 2), (2, 3, 10, 12, 3), (1, 24, 22, 40, 4),
                                           (1, 3, 4, 8, 1), (1, 2, 4, 8, 64)])   # 1 head; 64 heads: 3 rounds of rows
def test_rope_qk_matches_the_oracle_rotation(B, T, H, W, heads):
    w = wl.Workload("rot", B, T, H, W, heads, 128, 1, oracle.SINGLE, "bf16")
    q, k, _ = wl.make_inputs(w, seed=1, device="cpu")
    print(f"rope_qk B={B} grid={T}x{H}x{W} heads={heads}", flush=True)
    qr, kr = sk.rope_qk(q.cuda(), k.cuda(), (T, H, W))
    torch.cuda.synchronize()
    scale = LOG2E / np.sqrt(128.0)
    for got_t, x, sc, name in ((qr, q, scale, "qr"), (kr, k, 1.0, "kr")):
        exact = oracle.rope_3d(x.float().numpy().astype(np.float64), T, H, W) * sc
        got = got_t.float().cpu().numpy().astype(np.float64)
        bound = 2.0 ** -8 * np.abs(exact) + 2.0 ** -20 * np.abs(x.float().numpy()).max() * sc
        err = np.abs(got - exact)
        flips = np.count_nonzero(got != _bf16_round(exact))
        print(f"{name}: max err/bound {(err / bound).max():.3f}, rounding flips {flips} of {got.size}", flush=True)
        assert (err <= bound).all(), name
        assert flips <= 1e-3 * got.size, name


CASES = [
    # B, T, H, W, heads, k, mode
    (1, 4, 8, 16, 2, 4, oracle.SINGLE),      # L = 128
    (1, 4, 10, 12, 3, 1, oracle.SINGLE),     # dense, ragged L = 480
    (2, 4, 10, 12, 2, 2, oracle.GROUP),      # B = 2, L = 240
    (1, 6, 10, 12, 2, 4, oracle.SINGLE),     # L = 180
    (1, 8, 12, 16, 2, 4, oracle.GROUP),      # L = 384
    (1, 4, 10, 16, 2, 8, oracle.SINGLE),     # L = 80
    (1, 4, 16, 16, 1, 8, oracle.GROUP),      # L = 128
    (1, 2, 4, 8, 2, 2, oracle.GROUP),        # L = 32: one partial tile
    (1, 4, 8, 16, 2, 16, oracle.SINGLE),     # k = 16, L = 32
    (2, 4, 8, 16, 3, 16, oracle.GROUP),      # k = 16, B = 2, L = 32
]


@pytest.mark.parametrize("B,T,H,W,heads,k,mode", CASES)
def test_rotated_attention_equals_fused(B, T, H, W, heads, k, mode):
    w = wl.Workload("rot", B, T, H, W, heads, 128, k, mode, "bf16")
    q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=2, device="cpu"))
    print(f"case B={B} grid={T}x{H}x{W} heads={heads} k={k} mode={mode}", flush=True)
    qr, kr = sk.rope_qk(q, kk, (T, H, W))
    got = sk.attn_rotated(qr, kr, v, (T, H, W), k, mode)
    ref = sk.attn(q, kk, v, (T, H, W), k, mode)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), (got.float() - ref.float()).abs().max().item()
    if k in (2, 4) and T * H * W <= 1536:
        want = oracle.skiparse_attention(*(x.float().cpu().numpy() for x in (q, kk, v)), T, H, W, k, mode)
        err = np.abs(got.float().cpu().numpy() - want)
        print(f"vs oracle: max {err.max():.3e} mean {err.mean():.3e}", flush=True)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3


@pytest.mark.parametrize("T,H,W,k,mode", [
    (1, 8, 8, 64, oracle.SINGLE),      # L = 1: every token attends only to itself
    (1, 4, 16, 32, oracle.SINGLE),     # L = 2
    (1, 1, 64, 8, oracle.GROUP),       # L = 8
    (2, 4, 8, 8, oracle.GROUP),        # L = 8 over a T x H x W grid with T, H > 1
])
def test_short_scopes_equal_fused(T, H, W, k, mode):
    w = wl.Workload("rot", 1, T, H, W, 2, 128, k, mode, "bf16")
    q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=23, device="cpu"))
    qr, kr = sk.rope_qk(q, kk, (T, H, W))
    got = sk.attn_rotated(qr, kr, v, (T, H, W), k, mode)
    ref = sk.attn(q, kk, v, (T, H, W), k, mode)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), (got.float() - ref.float()).abs().max().item()
    if T * H * W == k:
        assert torch.equal(got.view(torch.int16), v.view(torch.int16))
    want = oracle.skiparse_attention(*(x.float().cpu().numpy() for x in (q, kk, v)), T, H, W, k, mode)
    err = np.abs(got.float().cpu().numpy() - want)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())


def test_group_skip_with_one_scope_is_dense_attention():
    # k = 1: Single Skip and Group Skip both keep every token in one scope in token order
    T, H, W, heads = 2, 10, 12, 2
    w = wl.Workload("rot", 1, T, H, W, heads, 128, 1, oracle.SINGLE, "bf16")
    q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=41, device="cpu"))
    qr, kr = sk.rope_qk(q, kk, (T, H, W))
    outs = [f(mode) for mode in (oracle.SINGLE, oracle.GROUP)
            for f in (lambda m: sk.attn(q, kk, v, (T, H, W), 1, m),
                      lambda m: sk.attn_rotated(qr, kr, v, (T, H, W), 1, m))]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_peaked_scores_equal_fused():
    """q x 8: peaked softmax, the running reference moves between tiles."""
    T, H, W, heads, k, mode = 4, 8, 16, 2, 2, oracle.SINGLE
    w = wl.Workload("rot", 1, T, H, W, heads, 128, k, mode, "bf16")
    q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=4, device="cpu"))
    q = (q.float() * 8).to(torch.bfloat16)
    qr, kr = sk.rope_qk(q, kk, (T, H, W))
    got = sk.attn_rotated(qr, kr, v, (T, H, W), k, mode)
    ref = sk.attn(q, kk, v, (T, H, W), k, mode)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


@pytest.mark.parametrize("w", [wl.OSP_SINGLE, wl.OSP_GROUP, wl.HC_GROUP, wl.WAN_DENSE, wl.LONG_GROUP,
                               wl.LONG_SINGLE], ids=lambda w: w.name)
def test_full_size_equals_fused(w):
    """The bench workload (24x22x40, 24 heads, k = 4), in the bench's launch configuration, and
    the other full-size workloads (up to N = 46080, B = 2, 40 heads, k = 1 and 8): bit-exact
    against the fused kernel everywhere."""
    print(f"full size {w.name}", flush=True)
    q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=0, device="cpu"))
    qr, kr = sk.rope_qk(q, kk, w.grid)
    got = sk.attn_rotated(qr, kr, v, w.grid, w.sparse_k, w.mode)
    ref = sk.attn(q, kk, v, w.grid, w.sparse_k, w.mode)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


BWD_CASES = [
    # B, T, H, W, heads, k, mode
    (1, 4, 8, 16, 2, 4, oracle.SINGLE),      # L = 128
    (2, 4, 10, 12, 2, 2, oracle.GROUP),      # B = 2, ragged L = 240
    (1, 4, 10, 12, 3, 1, oracle.SINGLE),     # dense, ragged L = 480
    (1, 4, 10, 16, 2, 8, oracle.SINGLE),     # L = 80
    (1, 4, 16, 16, 1, 8, oracle.GROUP),      # L = 128
    (2, 4, 8, 16, 3, 16, oracle.GROUP),      # k = 16, B = 2, L = 32
    (1, 2, 6, 216, 2, 4, oracle.GROUP),      # T + H + W = 224, the table limit
]


@pytest.mark.parametrize("B,T,H,W,heads,k,mode", BWD_CASES)
def test_rotated_training_step_equals_fused(B, T, H, W, heads, k, mode):
    w = wl.Workload("rot", B, T, H, W, heads, 128, k, mode, "bf16")
    q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=5, device="cpu"))
    do = wl.make_output_grad(w, seed=6, device="cuda")
    print(f"training step B={B} grid={T}x{H}x{W} heads={heads} k={k} mode={mode}", flush=True)
    qr, kr = sk.rope_qk(q, kk, (T, H, W))
    out_r, lse_r = sk.attn_rotated_lse(qr, kr, v, (T, H, W), k, mode)
    out_f, lse_f = sk.attn_lse(q, kk, v, (T, H, W), k, mode)
    torch.cuda.synchronize()
    assert torch.equal(out_r, out_f)
    assert torch.equal(lse_r, lse_f)
    g_r = sk.attn_bwd_rotated(qr, kr, v, out_r, do, lse_r, (T, H, W), k, mode)
    g_f = sk.attn_bwd(q, kk, v, out_f, do, lse_f, (T, H, W), k, mode)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g_r, g_f):
        assert torch.equal(a, b), (name, (a.float() - b.float()).abs().max().item())


@pytest.mark.parametrize("T,H,W,k,mode", [
    (1, 8, 8, 64, oracle.SINGLE),      # L = 1
    (1, 4, 16, 32, oracle.SINGLE),     # L = 2
    (2, 4, 8, 8, oracle.GROUP),        # L = 8
])
def test_training_step_on_short_scopes(T, H, W, k, mode):
    """Scopes of 1, 2 and 8 tokens: the rotated training step equals the fused one bit for
    bit.  With L = 1 each weight is 1, so dZ = dP - D vanishes up to the rounding of two
    float32 dot products of 128 terms: dq and dk stay below 1e-3 and dv equals dO within bf16
    rounding.  Longer scopes against the oracle's chain rule."""
    w = wl.Workload("rot", 1, T, H, W, 2, 128, k, mode, "bf16")
    q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=31, device="cpu"))
    do = wl.make_output_grad(w, seed=32, device="cuda")
    qr, kr = sk.rope_qk(q, kk, (T, H, W))
    out_r, lse_r = sk.attn_rotated_lse(qr, kr, v, (T, H, W), k, mode)
    out_f, lse_f = sk.attn_lse(q, kk, v, (T, H, W), k, mode)
    g_r = sk.attn_bwd_rotated(qr, kr, v, out_r, do, lse_r, (T, H, W), k, mode)
    g_f = sk.attn_bwd(q, kk, v, out_f, do, lse_f, (T, H, W), k, mode)
    torch.cuda.synchronize()
    assert torch.equal(out_r, out_f) and torch.equal(lse_r, lse_f)
    for name, a, b in zip(("dq", "dk", "dv"), g_r, g_f):
        assert torch.equal(a, b), name
    if T * H * W == k:
        dq, dk, dv = (g.double().cpu().numpy() for g in g_r)
        assert np.abs(dq).max() <= 1e-3 and np.abs(dk).max() <= 1e-3
        don = do.double().cpu().numpy()
        assert np.abs(dv - don).max() <= 2.0 ** -8 * np.abs(don).max()
        return
    host = [x.double().cpu().numpy() for x in (q, kk, v, do)]
    want = oracle.skiparse_attention_backward(*host, T, H, W, k, mode)
    for name, g, r in zip(("dq", "dk", "dv"), g_r, want):
        got = g.double().cpu().numpy()
        rel = np.linalg.norm(got - r) / np.linalg.norm(r)
        mx = np.abs(got - r).max() / np.abs(r).max()
        print(f"{name} L={T * H * W // k}: relrms {rel:.3e} max/maxref {mx:.3e}", flush=True)
        assert rel <= 1e-2 and mx <= 2.5e-2, name


@pytest.mark.parametrize("T,H,W,heads,k,mode", [
    (3, 8, 12, 2, 3, oracle.SINGLE),    # L = 96: two query tiles
    (3, 12, 18, 2, 3, oracle.GROUP),    # L = 216: four query tiles, the last ragged
])
def test_rotated_backward_k_not_dividing_the_tile(T, H, W, heads, k, mode):
    """k = 3 (the backward's per-tile cursor path, whose query-tile loads are rebuilt every
    tile): the rotated backward on the fused forward's out and lse equals the plain backward
    bit for bit."""
    print(f"k = 3 backward grid={T}x{H}x{W} mode={mode}", flush=True)
    w = wl.Workload("rot", 1, T, H, W, heads, 128, k, mode, "bf16")
    q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=7, device="cpu"))
    do = wl.make_output_grad(w, seed=8, device="cuda")
    out, lse = sk.attn_lse(q, kk, v, (T, H, W), k, mode)
    qr, kr = sk.rope_qk(q, kk, (T, H, W))
    g_r = sk.attn_bwd_rotated(qr, kr, v, out, do, lse, (T, H, W), k, mode)
    g_f = sk.attn_bwd(q, kk, v, out, do, lse, (T, H, W), k, mode)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g_r, g_f):
        assert torch.equal(a, b), name


def test_rotated_backward_matches_the_oracle():
    T, H, W, heads, k, mode = 4, 8, 16, 2, 4, oracle.GROUP
    w = wl.Workload("rot", 1, T, H, W, heads, 128, k, mode, "bf16")
    q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=9, device="cpu"))
    do = wl.make_output_grad(w, seed=10, device="cuda")
    qr, kr = sk.rope_qk(q, kk, (T, H, W))
    out, lse = sk.attn_rotated_lse(qr, kr, v, (T, H, W), k, mode)
    grads = sk.attn_bwd_rotated(qr, kr, v, out, do, lse, (T, H, W), k, mode)
    torch.cuda.synchronize()
    host = [x.double().cpu().numpy() for x in (q, kk, v, do)]
    want = oracle.skiparse_attention_backward(*host, T, H, W, k, mode)
    for name, g, r in zip(("dq", "dk", "dv"), grads, want):
        got = g.double().cpu().numpy()
        rel = np.linalg.norm(got - r) / np.linalg.norm(r)
        mx = np.abs(got - r).max() / np.abs(r).max()
        print(f"{name}: relrms {rel:.3e} max/maxref {mx:.3e}", flush=True)
        assert rel <= 1e-2 and mx <= 2.5e-2, name


@pytest.mark.parametrize("w", [wl.OSP_SINGLE, wl.OSP_GROUP], ids=lambda w: w.name)
def test_full_size_training_step_equals_fused(w):
    print(f"full-size training step {w.name}", flush=True)
    q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=0, device="cpu"))
    do = wl.make_output_grad(w, seed=1, device="cuda")
    qr, kr = sk.rope_qk(q, kk, w.grid)
    out, lse = sk.attn_rotated_lse(qr, kr, v, w.grid, w.sparse_k, w.mode)
    out_f, lse_f = sk.attn_lse(q, kk, v, w.grid, w.sparse_k, w.mode)
    torch.cuda.synchronize()
    assert torch.equal(out, out_f) and torch.equal(lse, lse_f)
    g_r = sk.attn_bwd_rotated(qr, kr, v, out, do, lse, w.grid, w.sparse_k, w.mode)
    torch.cuda.synchronize()
    g_r = [g.clone() for g in g_r]
    g_f = sk.attn_bwd(q, kk, v, out, do, lse, w.grid, w.sparse_k, w.mode)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g_r, g_f):
        assert torch.equal(a, b), name


def test_rotated_training_step_graph_replays_bit_exactly():
    """The rotated training step (RoPE pass, forward with log2-sum-exp, backward: five
    launches, no allocation, no memset) captured in a HIP graph and replayed three times, with
    eager work on every output between the replays; each replay equals the eager results."""
    T, H, W, heads, k, mode = 4, 8, 16, 2, 4, oracle.GROUP
    w = wl.Workload("rot", 1, T, H, W, heads, 128, k, mode, "bf16")
    q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=11, device="cpu"))
    do = wl.make_output_grad(w, seed=12, device="cuda")
    qr, kr = torch.empty_like(q), torch.empty_like(kk)
    out = torch.empty_like(q)
    lse = torch.empty((1, heads, T * H * W), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    outputs = (qr, kr, out, lse, delta) + grads

    def step():
        sk.rope_qk(q, kk, (T, H, W), outs=(qr, kr))
        sk.attn_rotated_lse(qr, kr, v, (T, H, W), k, mode, out=out, lse=lse)
        sk.attn_bwd_rotated(qr, kr, v, out, do, lse, (T, H, W), k, mode, grads=grads, delta=delta)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outputs:
            t.fill_(float(rep + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, ref in zip(("qr", "kr", "out", "lse", "delta", "dq", "dk", "dv"), outputs, eager):
            assert torch.equal(t, ref), (rep, name)
