"""CPU tests of the C-ABI library: it loads, exports every declared symbol, and
its host-side logic (validation, index tables, FLOP count) is right.  No
compute call reaches a device here: every call below either runs host code
only or is rejected by validation before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import skiparse_sparse_attention_amd as sk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skiparse.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sk.LIB_PATH), reason="library not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(skiparse_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for want in ("skiparse_attn", "skiparse_rope_remap", "skiparse_rearrange", "skiparse_reverse",
                 "skiparse_validate", "skiparse_scope_table", "skiparse_attn_flops",
                 "skiparse_status_string", "skiparse_version", "skiparse_attn_lse",
                 "skiparse_attn_bwd", "skiparse_attn_bwd_flops", "skiparse_quant8", "skiparse_attn8",
                 "skiparse_q8_scope_pitch", "skiparse_attn_schedule", "skiparse_rope_qk",
                 "skiparse_attn_rotated", "skiparse_attn_rotated_lse", "skiparse_attn_bwd_rotated",
                 "skiparse_attn_schedule_rotated", "skiparse_attn_bwd_rotated_static"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(sk.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings():
    assert "gfx950" in sk.version()
    for st in range(0, 8):
        assert sk.status_string(st)
    assert sk.status_string(99) == "unknown status"


# fake, non-overlapping "device" addresses: validation only compares ranges
Q, K, V, OUT = 1 << 40, 2 << 40, 3 << 40, 4 << 40
GOOD = dict(B=1, T=4, H=8, W=8, heads=2, head_dim=64, sparse_k=2, mode=0, dtype=1)


def _validate(q=Q, k=K, v=V, out=OUT, **kw):
    a = dict(GOOD)
    a.update(kw)
    return sk.lib().skiparse_validate(q, k, v, a["B"], a["T"], a["H"], a["W"], a["heads"],
                                      a["head_dim"], a["sparse_k"], a["mode"], a["dtype"], out)


def test_validate_accepts_good_arguments():
    assert _validate() == sk.OK
    assert _validate(mode=1) == sk.OK  # 256 % 4 == 0
    assert _validate(head_dim=128, dtype=0, sparse_k=8, mode=0) == sk.OK


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), sk.E_NULL), (dict(k=None), sk.E_NULL), (dict(v=None), sk.E_NULL),
    (dict(out=None), sk.E_NULL),
    (dict(B=0), sk.E_SHAPE), (dict(T=-1), sk.E_SHAPE), (dict(heads=0), sk.E_SHAPE),
    (dict(sparse_k=0), sk.E_SHAPE),
    (dict(T=1 << 20, H=1 << 20, W=4), sk.E_SHAPE),          # T*H*W overflows int32
    (dict(head_dim=96), sk.E_UNSUPPORTED), (dict(mode=2), sk.E_UNSUPPORTED),
    (dict(dtype=5), sk.E_UNSUPPORTED),
    (dict(sparse_k=3), sk.E_DIVISIBILITY),                  # 256 % 3
    (dict(sparse_k=32, mode=1), sk.E_DIVISIBILITY),         # 256 % 1024
    (dict(sparse_k=512), sk.E_DIVISIBILITY),
    (dict(T=400, H=4, W=4, head_dim=128), sk.E_UNSUPPORTED),  # T + H + W > 192
    (dict(out=Q + 64), sk.E_ALIAS), (dict(out=V - 64), sk.E_ALIAS), (dict(out=K), sk.E_ALIAS),
])
def test_validate_rejects(kw, status):
    assert _validate(**kw) == status


def test_attn_rejects_slabs_beyond_32bit_offsets():
    # 1 batch x 131072 tokens x 64 heads x 128 x 2 bytes = 2 GiB > the 32-bit offset range
    L = sk.lib()
    assert L.skiparse_attn(Q, K, V, 1, 32, 64, 64, 64, 128, 1, 0, 0, OUT, None) == sk.E_UNSUPPORTED
    # a huge k pushes the tokens of out-of-scope rows (up to N + 256k + k^2) past the range
    assert L.skiparse_validate(Q, K, V, 1, 64, 32, 32, 8, 128, 65536, 0, 0, OUT) == sk.E_UNSUPPORTED
    assert L.skiparse_validate(Q, K, V, 1, 64, 32, 32, 8, 128, 256, 0, 0, OUT) == sk.OK


def test_attn_rejects_before_any_device_call():
    # invalid calls must return their code without touching the (absent) GPU
    L = sk.lib()
    assert L.skiparse_attn(Q, K, V, 1, 4, 8, 8, 2, 64, 3, 0, 1, OUT, None) == sk.E_DIVISIBILITY
    assert L.skiparse_attn(Q, K, V, 1, 4, 8, 8, 2, 64, 2, 0, 1, Q, None) == sk.E_ALIAS
    assert L.skiparse_rope_remap(Q, K, V, 1, 4, 8, 8, 2, 64, 2, 0, 1, OUT, OUT, OUT + (1 << 30), None) == sk.E_ALIAS
    assert L.skiparse_rearrange(None, 1, 4, 8, 8, 2, 64, 2, 0, 1, 0, OUT, None) == sk.E_NULL
    assert L.skiparse_reverse(Q, 1, 4, 8, 8, 2, 65, 2, 0, 1, OUT, None) == sk.E_UNSUPPORTED


@pytest.mark.parametrize("N,k", [(256, 1), (256, 2), (256, 4), (256, 8), (21120, 4), (36864, 4),
                                 (32760, 1), (32760, 2), (46080, 8), (27, 3), (36, 3), (480, 4)])
@pytest.mark.parametrize("mode", [oracle.SINGLE, oracle.GROUP])
def test_scope_table_matches_oracle_exactly(N, k, mode):
    if mode == oracle.GROUP and N % (k * k):
        with pytest.raises(sk.SkiparseError):
            sk.scope_table(N, k, mode)
        return
    got = sk.scope_table(N, k, mode)
    assert got.dtype == np.int64
    assert np.array_equal(got, oracle.scope_table(N, k, mode))


def test_attn_flops_matches_definition():
    assert sk.attn_flops(1, (24, 22, 40), 24, 128, 4) == oracle.skiparse_flops(1, 21120, 24, 128, 4)
    assert sk.attn_flops(2, (20, 48, 48), 24, 128, 8) == oracle.skiparse_flops(2, 46080, 24, 128, 8)
    assert sk.attn_flops(0, (1, 1, 1), 1, 64, 1) < 0


def test_attn_flops_backward_is_twice_the_forward():
    assert sk.attn_bwd_flops(1, (24, 22, 40), 24, 128, 4) == oracle.skiparse_backward_flops(1, 21120, 24, 128, 4)
    assert sk.attn_bwd_flops(2, (20, 48, 48), 24, 128, 8) == oracle.skiparse_backward_flops(2, 46080, 24, 128, 8)
    assert sk.attn_bwd_flops(1, (0, 1, 1), 1, 64, 1) < 0


LSE, DO, DQ, DK, DV, DELTA = 5 << 40, 6 << 40, 7 << 40, 8 << 40, 9 << 40, 10 << 40


def _bwd(**kw):
    a = dict(q=Q, k=K, v=V, out=OUT, dout=DO, lse=LSE, dq=DQ, dk=DK, dv=DV, delta=DELTA)
    a.update({x: kw.pop(x) for x in list(kw) if x in a})
    g = dict(GOOD)
    g.update(kw)
    return sk.lib().skiparse_attn_bwd(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], g["B"], g["T"],
                                      g["H"], g["W"], g["heads"], g["head_dim"], g["sparse_k"], g["mode"],
                                      g["dtype"], a["dq"], a["dk"], a["dv"], a["delta"], None)


def test_backward_and_lse_reject_before_any_device_call():
    L = sk.lib()
    assert L.skiparse_attn_lse(Q, K, V, 1, 4, 8, 8, 2, 64, 2, 0, 1, OUT, None, None) == sk.E_NULL
    assert L.skiparse_attn_lse(Q, K, V, 1, 4, 8, 8, 2, 64, 2, 0, 1, OUT, Q, None) == sk.E_ALIAS
    assert L.skiparse_attn_lse(Q, K, V, 1, 4, 8, 8, 2, 64, 3, 0, 1, OUT, LSE, None) == sk.E_DIVISIBILITY
    assert _bwd(delta=None) == sk.E_NULL
    assert _bwd(lse=None) == sk.E_NULL
    assert _bwd(dq=K) == sk.E_ALIAS            # a gradient over an input
    assert _bwd(dv=DK) == sk.E_ALIAS           # two gradients in one buffer
    assert _bwd(delta=DO) == sk.E_ALIAS        # the workspace over an input
    assert _bwd(delta=LSE) == sk.E_ALIAS       # the workspace over the log2-sum-exp
    assert _bwd(sparse_k=3) == sk.E_DIVISIBILITY
    assert _bwd(head_dim=96) == sk.E_UNSUPPORTED


def test_q8_scope_pitch():
    L = sk.lib()
    assert L.skiparse_q8_scope_pitch(24, 22, 40, 4) == 5312       # L = 5280 rounded up to 64
    assert L.skiparse_q8_scope_pitch(4, 8, 16, 4) == 128           # L = 128 already a multiple
    assert L.skiparse_q8_scope_pitch(1, 1, 3, 1) == 64
    assert L.skiparse_q8_scope_pitch(2, 2, 5, 3) < 0               # N not divisible by k


def _q8(**kw):
    a = dict(q=Q, k=K, v=V, q8=DQ, qa=DK, k8=DV, ka=DELTA, vt8=DO, va=LSE)
    a.update({x: kw.pop(x) for x in list(kw) if x in a})
    g = dict(B=1, T=4, H=8, W=16, heads=2, head_dim=128, sparse_k=4, mode=0, dtype=0)
    g.update(kw)
    return sk.lib().skiparse_quant8(a["q"], a["k"], a["v"], g["B"], g["T"], g["H"], g["W"], g["heads"],
                                    g["head_dim"], g["sparse_k"], g["mode"], g["dtype"], a["q8"], a["qa"],
                                    a["k8"], a["ka"], a["vt8"], a["va"], None)


def _a8(**kw):
    a = dict(q8=DQ, qa=DK, k8=DV, ka=DELTA, vt8=DO, va=LSE, out=OUT)
    a.update({x: kw.pop(x) for x in list(kw) if x in a})
    g = dict(B=1, T=4, H=8, W=16, heads=2, head_dim=128, sparse_k=4, mode=0, dtype=0)
    g.update(kw)
    return sk.lib().skiparse_attn8(a["q8"], a["qa"], a["k8"], a["ka"], a["vt8"], a["va"], g["B"], g["T"],
                                   g["H"], g["W"], g["heads"], g["head_dim"], g["sparse_k"], g["mode"],
                                   g["dtype"], a["out"], None)


def test_8bit_calls_reject_before_any_device_call():
    assert _q8(vt8=None) == sk.E_NULL
    assert _q8(head_dim=64) == sk.E_UNSUPPORTED       # the 8-bit path is head_dim 128 only
    assert _q8(T=3, H=8, W=8, sparse_k=3) == sk.E_UNSUPPORTED     # 3 does not divide 64
    assert _q8(sparse_k=3) == sk.E_DIVISIBILITY
    assert _q8(q8=Q) == sk.E_ALIAS                     # an output over an input
    assert _q8(ka=DELTA, va=DELTA) == sk.E_ALIAS       # two outputs in one buffer
    assert _q8(B=3000, heads=30) == sk.E_UNSUPPORTED   # B*heads beyond the statistics grid
    assert _a8(out=None) == sk.E_NULL
    assert _a8(head_dim=64) == sk.E_UNSUPPORTED
    assert _a8(out=DV) == sk.E_ALIAS                   # the output over an operand
    assert _a8(dtype=2) == sk.E_UNSUPPORTED


def test_schedule_rejects_before_any_device_call():
    L = sk.lib()
    good = sk.Layer(Q, K, V, OUT, 2, 0)
    bad_k = sk.Layer(Q, K, V, OUT, 3, 0)          # N = 256 is not divisible by 3
    alias = sk.Layer(Q, K, V, Q, 2, 0)            # out over q
    arr = (sk.Layer * 3)(good, bad_k, good)
    args = (1, 4, 8, 8, 2, 64, 1, None)           # B, T, H, W, heads, head_dim, dtype, stream
    assert L.skiparse_attn_schedule(arr, 3, *args) == sk.E_DIVISIBILITY
    assert L.skiparse_attn_schedule((sk.Layer * 2)(good, alias), 2, *args) == sk.E_ALIAS
    assert L.skiparse_attn_schedule(None, 1, *args) == sk.E_NULL
    assert L.skiparse_attn_schedule(arr, 0, *args) == sk.E_SHAPE
    assert L.skiparse_attn_schedule(arr, 5000, *args) == sk.E_SHAPE


def test_u_schedule_shape():
    assert sk.u_schedule(8, 8) == [(1, 0), (2, 1), (4, 0), (8, 1), (8, 0), (4, 1), (2, 0), (1, 1)]
    ks = [k for k, _ in sk.u_schedule(9, 4)]
    assert ks == ks[::-1] and ks[0] == 1 and max(ks) == 4


def test_rotated_path_rejects_before_any_device_call():
    L = sk.lib()
    # skiparse_rope_qk(q, k, B, T, H, W, heads, head_dim, dtype, qr, kr, stream)
    g = (1, 4, 8, 8, 2, 128, 0)
    assert L.skiparse_rope_qk(Q, K, *g, V, None, None) == sk.E_NULL
    assert L.skiparse_rope_qk(Q, K, 1, 4, 8, 8, 2, 64, 0, V, OUT, None) == sk.E_UNSUPPORTED   # head_dim 128 only
    assert L.skiparse_rope_qk(Q, K, 1, 4, 8, 8, 2, 128, 1, V, OUT, None) == sk.E_UNSUPPORTED  # bf16 only
    assert L.skiparse_rope_qk(Q, K, *g, Q, OUT, None) == sk.E_ALIAS      # qr over q
    assert L.skiparse_rope_qk(Q, K, *g, V, K, None) == sk.E_ALIAS        # kr over k
    assert L.skiparse_rope_qk(Q, K, *g, V, V, None) == sk.E_ALIAS        # qr and kr in one buffer
    assert L.skiparse_rope_qk(Q, K, 0, 4, 8, 8, 2, 128, 0, V, OUT, None) == sk.E_SHAPE
    # skiparse_attn_rotated(qr, kr, v, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, out, stream)
    assert L.skiparse_attn_rotated(Q, K, V, 1, 4, 8, 8, 2, 128, 2, 0, 0, None, None) == sk.E_NULL
    assert L.skiparse_attn_rotated(Q, K, V, 1, 4, 8, 8, 2, 64, 2, 0, 0, OUT, None) == sk.E_UNSUPPORTED
    assert L.skiparse_attn_rotated(Q, K, V, 1, 4, 8, 8, 2, 128, 2, 0, 1, OUT, None) == sk.E_UNSUPPORTED
    assert L.skiparse_attn_rotated(Q, K, V, 1, 3, 8, 8, 2, 128, 3, 0, 0, OUT, None) == sk.E_UNSUPPORTED  # 3 does not divide 64
    assert L.skiparse_attn_rotated(Q, K, V, 1, 4, 8, 8, 2, 128, 3, 0, 0, OUT, None) == sk.E_DIVISIBILITY
    assert L.skiparse_attn_rotated(Q, K, V, 1, 4, 8, 8, 2, 128, 2, 0, 0, K, None) == sk.E_ALIAS


def test_rotated_lse_and_backward_reject_before_any_device_call():
    L = sk.lib()
    # skiparse_attn_rotated_lse(qr, kr, v, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, out, lse, stream)
    assert L.skiparse_attn_rotated_lse(Q, K, V, 1, 4, 8, 8, 2, 128, 2, 0, 0, OUT, None, None) == sk.E_NULL
    assert L.skiparse_attn_rotated_lse(Q, K, V, 1, 4, 8, 8, 2, 128, 2, 0, 0, OUT, Q, None) == sk.E_ALIAS
    assert L.skiparse_attn_rotated_lse(Q, K, V, 1, 4, 8, 8, 2, 64, 2, 0, 0, OUT, DELTA, None) == sk.E_UNSUPPORTED
    # skiparse_attn_bwd_rotated(qr, kr, v, out, dout, lse, B, T, H, W, heads, head_dim, sparse_k, mode, dtype,
    #                           dq, dk, dv, delta, stream)
    base = [Q, K, V, OUT, DO, LSE, 1, 4, 8, 8, 2, 128, 2, 0, 0, DQ, DK, DV, DELTA, None]   # valid: never called as is
    bad = list(base); bad[11] = 64
    assert L.skiparse_attn_bwd_rotated(*bad) == sk.E_UNSUPPORTED      # head_dim 128 only
    bad = list(base); bad[14] = 1
    assert L.skiparse_attn_bwd_rotated(*bad) == sk.E_UNSUPPORTED      # bf16 only
    bad = list(base); bad[15] = Q
    assert L.skiparse_attn_bwd_rotated(*bad) == sk.E_ALIAS
    bad = list(base); bad[5] = None
    assert L.skiparse_attn_bwd_rotated(*bad) == sk.E_NULL


def test_static_workspace_backward_rejects_before_any_device_call():
    L = sk.lib()
    # skiparse_attn_bwd_rotated_static(qr, kr, v, out, dout, lse, B, T, H, W, heads, head_dim, sparse_k,
    #                                  mode, dtype, dq, dk, dv, stream): no delta argument
    base = [Q, K, V, OUT, DO, LSE, 1, 4, 8, 8, 2, 128, 2, 0, 0, DQ, DK, DV, None]   # valid: never called as is
    bad = list(base); bad[11] = 64
    assert L.skiparse_attn_bwd_rotated_static(*bad) == sk.E_UNSUPPORTED
    bad = list(base); bad[16] = V
    assert L.skiparse_attn_bwd_rotated_static(*bad) == sk.E_ALIAS
    bad = list(base); bad[17] = LSE
    assert L.skiparse_attn_bwd_rotated_static(*bad) == sk.E_ALIAS
    bad = list(base); bad[0] = None
    assert L.skiparse_attn_bwd_rotated_static(*bad) == sk.E_NULL
    # B*heads*N = 5 * 32 * 32768 > SKIPARSE_STATIC_DELTA_MAX: rejected before the workspace is
    # looked up (a valid size otherwise; the fake addresses are 1 TiB apart)
    big = [Q, K, V, OUT, DO, LSE, 5, 8, 64, 64, 32, 128, 1, 0, 0, DQ, DK, DV, None]
    assert 5 * 32 * 32768 > sk.STATIC_DELTA_MAX
    assert L.skiparse_attn_bwd_rotated_static(*big) == sk.E_WORKSPACE
    assert "static workspace" in sk.status_string(sk.E_WORKSPACE)


def test_rotated_schedule_rejects_before_any_device_call():
    L = sk.lib()
    good = sk.Layer(Q, K, V, OUT, 2, 0)
    arr = (sk.Layer * 2)(good, good)
    QR, KR = 11 << 40, 12 << 40
    # skiparse_attn_schedule_rotated(layers, n, B, T, H, W, heads, head_dim, dtype, qr, kr, stream)
    assert L.skiparse_attn_schedule_rotated(arr, 2, 1, 4, 8, 8, 2, 128, 0, None, KR, None) == sk.E_NULL
    assert L.skiparse_attn_schedule_rotated(arr, 2, 1, 4, 8, 8, 2, 128, 0, QR, QR, None) == sk.E_ALIAS     # one scratch
    assert L.skiparse_attn_schedule_rotated(arr, 2, 1, 4, 8, 8, 2, 128, 0, V, KR, None) == sk.E_ALIAS      # over a layer's v
    assert L.skiparse_attn_schedule_rotated(arr, 2, 1, 4, 8, 8, 2, 128, 0, QR, OUT, None) == sk.E_ALIAS    # over a layer's out
    assert L.skiparse_attn_schedule_rotated(arr, 2, 1, 4, 8, 8, 2, 64, 0, QR, KR, None) == sk.E_UNSUPPORTED
    assert L.skiparse_attn_schedule_rotated(arr, 2, 1, 4, 8, 8, 2, 128, 1, QR, KR, None) == sk.E_UNSUPPORTED
    k3 = (sk.Layer * 1)(sk.Layer(Q, K, V, OUT, 3, 0))
    assert L.skiparse_attn_schedule_rotated(k3, 1, 1, 3, 8, 8, 2, 128, 0, QR, KR, None) == sk.E_UNSUPPORTED  # 3 does not divide 64
    assert L.skiparse_attn_schedule_rotated(arr, 0, 1, 4, 8, 8, 2, 128, 0, QR, KR, None) == sk.E_SHAPE


def test_grid_limit_applies_only_to_the_table_kernels():
    # T + H + W = 229 > SKIPARSE_MAX_GRID_SUM.  Every call below also has an output that
    # overlaps an input: a call that applies the grid limit returns E_UNSUPPORTED first, a call
    # that takes any grid reaches its alias check and returns E_ALIAS (no device call either way).
    L = sk.lib()
    T, H, W = 2, 3, 224
    assert T + H + W > sk.MAX_GRID_SUM
    dims = (1, T, H, W, 2, 128)
    # table kernels: the fused forward (and its validation) and the 8-bit quantisation pass
    assert L.skiparse_validate(Q, K, V, *dims, 4, 1, 0, Q) == sk.E_UNSUPPORTED
    assert L.skiparse_attn(Q, K, V, *dims, 4, 1, 0, Q, None) == sk.E_UNSUPPORTED
    assert L.skiparse_quant8(Q, K, V, *dims, 4, 1, 0, Q, DO, DQ, DK, DV, DELTA, None) == sk.E_UNSUPPORTED
    # RoPE+remap outside bf16 / head_dim 128 keeps the table
    assert L.skiparse_rope_remap(Q, K, V, 1, T, H, W, 2, 64, 4, 1, 0, Q, DQ, DK, None) == sk.E_UNSUPPORTED
    # per-token RoPE pairs or no RoPE: any grid
    assert L.skiparse_rope_qk(Q, K, *dims, 0, Q, DK, None) == sk.E_ALIAS
    assert L.skiparse_attn_rotated(Q, K, V, *dims, 4, 1, 0, K, None) == sk.E_ALIAS
    assert L.skiparse_rope_remap(Q, K, V, *dims, 4, 1, 0, Q, DQ, DK, None) == sk.E_ALIAS
    assert L.skiparse_rearrange(Q, *dims, 4, 1, 0, 1, Q, None) == sk.E_ALIAS          # bf16, with RoPE
    assert L.skiparse_reverse(Q, *dims, 4, 1, 0, Q, None) == sk.E_ALIAS
