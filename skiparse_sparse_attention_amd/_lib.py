"""ctypes binding of ``libskiparse_amd.so`` (C ABI: include/skiparse.h).

Argument marshalling only: tensors are passed by device pointer, the stream is
torch's current HIP stream, and every step of the computation runs in the
library's kernels.  There is no fallback: if the library is not built the
calls raise.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libskiparse_amd.so")

SINGLE = 0
GROUP = 1
BF16 = 0
FP32 = 1

OK = 0
E_NULL = 1
E_SHAPE = 2
E_DIVISIBILITY = 3
E_UNSUPPORTED = 4
E_ALIAS = 5
E_DEVICE = 6

MAX_GRID_SUM = 192

_lib = None


class Layer(ctypes.Structure):
    """One entry of a schedule (the C struct skiparse_layer)."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("sparse_k", ctypes.c_int), ("mode", ctypes.c_int)]


class SkiparseError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def lib():
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m skiparse_sparse_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        dims = [i] * 6  # B, T, H, W, heads, head_dim
        L.skiparse_attn.argtypes = [vp, vp, vp] + dims + [i, i, i, vp, vp]
        L.skiparse_attn.restype = i
        L.skiparse_rope_remap.argtypes = [vp, vp, vp] + dims + [i, i, i, vp, vp, vp, vp]
        L.skiparse_rope_remap.restype = i
        L.skiparse_rearrange.argtypes = [vp] + dims + [i, i, i, i, vp, vp]
        L.skiparse_rearrange.restype = i
        L.skiparse_reverse.argtypes = [vp] + dims + [i, i, i, vp, vp]
        L.skiparse_reverse.restype = i
        L.skiparse_validate.argtypes = [vp, vp, vp] + dims + [i, i, i, vp]
        L.skiparse_validate.restype = i
        L.skiparse_scope_table.argtypes = [i64, i, i, ctypes.POINTER(ctypes.c_int64)]
        L.skiparse_scope_table.restype = i
        L.skiparse_attn_flops.argtypes = [i] * 7
        L.skiparse_attn_flops.restype = ctypes.c_double
        L.skiparse_attn_lse.argtypes = [vp, vp, vp] + dims + [i, i, i, vp, vp, vp]
        L.skiparse_attn_lse.restype = i
        L.skiparse_attn_bwd.argtypes = [vp] * 6 + dims + [i, i, i] + [vp] * 5
        L.skiparse_attn_bwd.restype = i
        L.skiparse_attn_bwd_flops.argtypes = [i] * 7
        L.skiparse_attn_bwd_flops.restype = ctypes.c_double
        L.skiparse_q8_scope_pitch.argtypes = [i] * 4
        L.skiparse_q8_scope_pitch.restype = i
        L.skiparse_quant8.argtypes = [vp, vp, vp] + dims + [i, i, i] + [vp] * 7
        L.skiparse_quant8.restype = i
        L.skiparse_attn8.argtypes = [vp] * 6 + dims + [i, i, i, vp, vp]
        L.skiparse_attn8.restype = i
        L.skiparse_attn_schedule.argtypes = [ctypes.POINTER(Layer), i] + dims + [i, vp]
        L.skiparse_attn_schedule.restype = i
        L.skiparse_rope_qk.argtypes = [vp, vp] + dims + [i, vp, vp, vp]
        L.skiparse_rope_qk.restype = i
        L.skiparse_attn_rotated.argtypes = [vp, vp, vp] + dims + [i, i, i, vp, vp]
        L.skiparse_attn_rotated.restype = i
        L.skiparse_attn_rotated_lse.argtypes = [vp, vp, vp] + dims + [i, i, i, vp, vp, vp]
        L.skiparse_attn_rotated_lse.restype = i
        L.skiparse_attn_bwd_rotated.argtypes = [vp] * 6 + dims + [i, i, i] + [vp] * 5
        L.skiparse_attn_bwd_rotated.restype = i
        L.skiparse_attn_schedule_rotated.argtypes = [ctypes.POINTER(Layer), i] + dims + [i, vp, vp, vp]
        L.skiparse_attn_schedule_rotated.restype = i
        L.skiparse_status_string.argtypes = [i]
        L.skiparse_status_string.restype = ctypes.c_char_p
        L.skiparse_version.argtypes = []
        L.skiparse_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().skiparse_status_string(int(status)).decode()


def version() -> str:
    return lib().skiparse_version().decode()


def _check(status: int, where: str):
    if status != OK:
        raise SkiparseError(status, where)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dims(x, grid):
    if x.dim() != 4:
        raise ValueError("expected a (B, N, heads, head_dim) tensor")
    if not x.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    T, H, W = (int(g) for g in grid)
    B, N, heads, d = x.shape
    if N != T * H * W:
        raise ValueError(f"N={N} does not match the grid {T}x{H}x{W}")
    return B, T, H, W, heads, d


def attn(q, k, v, grid, sparse_k, mode, out=None, stream=None):
    """Fused Skiparse attention: q, k, v (B, N, heads, d) on the GPU -> out, same shape/dtype."""
    import torch
    B, T, H, W, heads, d = _dims(q, grid)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k, v must share shape, dtype and be contiguous")
    if out is None:
        out = torch.empty_like(q)
    _check(lib().skiparse_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                               int(sparse_k), int(mode), _dtype_code(q), out.data_ptr(),
                               _stream_ptr(stream)), "skiparse_attn")
    return out


def rope_qk(q, k, grid, outs=None, stream=None):
    """3D RoPE of q and k once (bf16, head_dim 128): returns (qr, kr), qr with the softmax
    scale log2(e)/sqrt(d) folded in -- the operands of attn_rotated."""
    import torch
    B, T, H, W, heads, d = _dims(q, grid)
    if k.shape != q.shape or k.dtype != q.dtype or not k.is_contiguous():
        raise ValueError("q, k must share shape, dtype and be contiguous")
    qr, kr = outs if outs is not None else (torch.empty_like(q), torch.empty_like(k))
    for t in (qr, kr):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("qr, kr must match q's shape and dtype and be contiguous")
    _check(lib().skiparse_rope_qk(q.data_ptr(), k.data_ptr(), B, T, H, W, heads, d, _dtype_code(q),
                                  qr.data_ptr(), kr.data_ptr(), _stream_ptr(stream)), "skiparse_rope_qk")
    return qr, kr


def attn_rotated(qr, kr, v, grid, sparse_k, mode, out=None, stream=None):
    """Skiparse attention on rope_qk's outputs; equals attn(q, k, v, ...) bit for bit."""
    import torch
    B, T, H, W, heads, d = _dims(qr, grid)
    for t in (kr, v):
        if t.shape != qr.shape or t.dtype != qr.dtype or not t.is_contiguous():
            raise ValueError("qr, kr, v must share shape, dtype and be contiguous")
    if out is None:
        out = torch.empty_like(v)
    _check(lib().skiparse_attn_rotated(qr.data_ptr(), kr.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                                       int(sparse_k), int(mode), _dtype_code(qr), out.data_ptr(),
                                       _stream_ptr(stream)), "skiparse_attn_rotated")
    return out


def attn_rotated_lse(qr, kr, v, grid, sparse_k, mode, out=None, lse=None, stream=None):
    """attn_rotated that also returns each row's log2-sum-exp (B, heads, N) fp32; equals
    attn_lse(q, k, v, ...) bit for bit."""
    import torch
    B, T, H, W, heads, d = _dims(qr, grid)
    for t in (kr, v):
        if t.shape != qr.shape or t.dtype != qr.dtype or not t.is_contiguous():
            raise ValueError("qr, kr, v must share shape, dtype and be contiguous")
    if out is None:
        out = torch.empty_like(v)
    if lse is None:
        lse = torch.empty((B, heads, T * H * W), dtype=torch.float32, device=v.device)
    _check(lib().skiparse_attn_rotated_lse(qr.data_ptr(), kr.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                                           int(sparse_k), int(mode), _dtype_code(qr), out.data_ptr(),
                                           lse.data_ptr(), _stream_ptr(stream)), "skiparse_attn_rotated_lse")
    return out, lse


def attn_bwd_rotated(qr, kr, v, out, dout, lse, grid, sparse_k, mode, grads=None, delta=None, stream=None):
    """attn_bwd on rope_qk's outputs: (dq, dk, dv) with respect to the unrotated q, k and v;
    equals attn_bwd(q, k, v, ...) bit for bit."""
    import torch
    B, T, H, W, heads, d = _dims(qr, grid)
    for t in (kr, v, out, dout):
        if t.shape != qr.shape or t.dtype != qr.dtype or not t.is_contiguous():
            raise ValueError("qr, kr, v, out, dout must share shape, dtype and be contiguous")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, heads, T * H * W) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous (B, heads, N) float32 tensor")
    if grads is None:
        grads = tuple(torch.empty_like(v) for _ in range(3))
    if delta is None:
        delta = torch.empty((B, heads, T * H * W), dtype=torch.float32, device=v.device)
    dq, dk, dv = grads
    _check(lib().skiparse_attn_bwd_rotated(qr.data_ptr(), kr.data_ptr(), v.data_ptr(), out.data_ptr(),
                                           dout.data_ptr(), lse.data_ptr(), B, T, H, W, heads, d,
                                           int(sparse_k), int(mode), _dtype_code(qr), dq.data_ptr(),
                                           dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                                           _stream_ptr(stream)), "skiparse_attn_bwd_rotated")
    return dq, dk, dv


def u_schedule(n_layers, k_max, modes=(SINGLE, GROUP)):
    """A U-shaped per-layer (sparse_k, mode) list: dense (k = 1) at both ends, doubling towards
    the middle up to k_max, modes alternating -- one example of the knob, not numbers from
    the pages."""
    out = []
    for i in range(int(n_layers)):
        depth = min(i, n_layers - 1 - i)
        out.append((min(1 << depth, int(k_max)), modes[i % len(modes)]))
    return out


def attn_schedule(layers, grid, stream=None):
    """Run a schedule: `layers` is a list of (q, k, v, out, sparse_k, mode); all layers share
    shape and dtype.  One validation pass, then one launch per layer on one stream."""
    if not layers:
        raise ValueError("empty schedule")
    q0 = layers[0][0]
    B, T, H, W, heads, d = _dims(q0, grid)
    arr = (Layer * len(layers))()
    for i, (q, k, v, out, sk_, mode) in enumerate(layers):
        for t in (q, k, v, out):
            if t.shape != q0.shape or t.dtype != q0.dtype or not t.is_contiguous():
                raise ValueError("every layer's q, k, v, out must share shape, dtype and be contiguous")
        arr[i] = Layer(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), int(sk_), int(mode))
    _check(lib().skiparse_attn_schedule(arr, len(layers), B, T, H, W, heads, d, _dtype_code(q0),
                                        _stream_ptr(stream)), "skiparse_attn_schedule")
    return [layer[3] for layer in layers]


def attn_schedule_rotated(layers, grid, scratch=None, stream=None):
    """attn_schedule with every layer run as the RoPE pass into `scratch` (qr, kr: two tensors
    shaped like q, reused by all layers) and the attention on the rotated operands; equals
    attn_schedule bit for bit (head_dim 128, bf16, every sparse_k dividing 64)."""
    import torch
    if not layers:
        raise ValueError("empty schedule")
    q0 = layers[0][0]
    B, T, H, W, heads, d = _dims(q0, grid)
    arr = (Layer * len(layers))()
    for i, (q, k, v, out, sk_, mode) in enumerate(layers):
        for t in (q, k, v, out):
            if t.shape != q0.shape or t.dtype != q0.dtype or not t.is_contiguous():
                raise ValueError("every layer's q, k, v, out must share shape, dtype and be contiguous")
        arr[i] = Layer(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), int(sk_), int(mode))
    qr, kr = scratch if scratch is not None else (torch.empty_like(q0), torch.empty_like(q0))
    for t in (qr, kr):
        if t.shape != q0.shape or t.dtype != q0.dtype or not t.is_contiguous():
            raise ValueError("scratch tensors must match the layers' shape and dtype and be contiguous")
    _check(lib().skiparse_attn_schedule_rotated(arr, len(layers), B, T, H, W, heads, d, _dtype_code(q0),
                                                qr.data_ptr(), kr.data_ptr(), _stream_ptr(stream)),
           "skiparse_attn_schedule_rotated")
    return [layer[3] for layer in layers]


def attn_lse(q, k, v, grid, sparse_k, mode, out=None, lse=None, stream=None):
    """Fused Skiparse attention that also returns each row's log2-sum-exp (B, heads, N) fp32."""
    import torch
    B, T, H, W, heads, d = _dims(q, grid)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k, v must share shape, dtype and be contiguous")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, heads, T * H * W), dtype=torch.float32, device=q.device)
    _check(lib().skiparse_attn_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                                   int(sparse_k), int(mode), _dtype_code(q), out.data_ptr(),
                                   lse.data_ptr(), _stream_ptr(stream)), "skiparse_attn_lse")
    return out, lse


def attn_bwd(q, k, v, out, dout, lse, grid, sparse_k, mode, grads=None, delta=None, stream=None):
    """Gradients (dq, dk, dv) of a loss through Skiparse attention, given dout = dLoss/dout.

    ``out`` and ``lse`` come from :func:`attn_lse` on the same inputs; ``delta`` is an
    optional (B, heads, N) fp32 workspace.
    """
    import torch
    B, T, H, W, heads, d = _dims(q, grid)
    for t in (k, v, out, dout):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k, v, out, dout must share shape, dtype and be contiguous")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, heads, T * H * W) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous (B, heads, N) float32 tensor")
    if grads is None:
        grads = tuple(torch.empty_like(q) for _ in range(3))
    if delta is None:
        delta = torch.empty((B, heads, T * H * W), dtype=torch.float32, device=q.device)
    dq, dk, dv = grads
    _check(lib().skiparse_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   dout.data_ptr(), lse.data_ptr(), B, T, H, W, heads, d,
                                   int(sparse_k), int(mode), _dtype_code(q), dq.data_ptr(),
                                   dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                                   _stream_ptr(stream)), "skiparse_attn_bwd")
    return dq, dk, dv


def attn_bwd_flops(B, grid, heads, head_dim, sparse_k):
    T, H, W = (int(g) for g in grid)
    return float(lib().skiparse_attn_bwd_flops(int(B), T, H, W, int(heads), int(head_dim), int(sparse_k)))


Q8_KEYS = ("q8", "q_amax", "k8", "k_amax", "vt8", "v_amax")


def q8_scope_pitch(grid, sparse_k):
    """Lp: the channel-row pitch (keys) of vt8, L rounded up to a multiple of 64."""
    T, H, W = (int(g) for g in grid)
    lp = lib().skiparse_q8_scope_pitch(T, H, W, int(sparse_k))
    if lp < 0:
        raise SkiparseError(-lp, "skiparse_q8_scope_pitch")
    return lp


def quant8(q, k, v, grid, sparse_k, mode, outs=None, stream=None):
    """8-bit operands of q, k, v for :func:`attn8`: a dict with q8 (int8), q_amax, k8 (int8),
    k_amax, vt8 (uint8 E4M3 codes) and v_amax (float32), in the layouts of include/skiparse.h."""
    import torch
    B, T, H, W, heads, d = _dims(q, grid)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k, v must share shape, dtype and be contiguous")
    N = T * H * W
    if outs is None:
        lp = q8_scope_pitch(grid, sparse_k)
        dev = q.device
        outs = {"q8": torch.empty((B, N, heads, d), dtype=torch.int8, device=dev),
                "q_amax": torch.empty((B, N, heads), dtype=torch.float32, device=dev),
                "k8": torch.empty((B, N, heads, d), dtype=torch.int8, device=dev),
                "k_amax": torch.empty((B, heads), dtype=torch.float32, device=dev),
                "vt8": torch.empty((B, heads, int(sparse_k), d, lp), dtype=torch.uint8, device=dev),
                "v_amax": torch.empty((B, heads, d), dtype=torch.float32, device=dev)}
    _check(lib().skiparse_quant8(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                                 int(sparse_k), int(mode), _dtype_code(q),
                                 *(outs[key].data_ptr() for key in Q8_KEYS), _stream_ptr(stream)),
           "skiparse_quant8")
    return outs


def attn8(qz, grid, sparse_k, mode, out_dtype=None, out=None, stream=None):
    """8-bit Skiparse attention of :func:`quant8`'s operands -> (B, N, heads, d) bf16 (or fp32)."""
    import torch
    q8 = qz["q8"]
    B, T, H, W, heads, d = _dims(q8, grid)
    for key in Q8_KEYS:
        if not qz[key].is_contiguous():
            raise ValueError(f"{key} must be contiguous")
    if out is None:
        out = torch.empty(q8.shape, dtype=out_dtype or torch.bfloat16, device=q8.device)
    _check(lib().skiparse_attn8(*(qz[key].data_ptr() for key in Q8_KEYS), B, T, H, W, heads, d,
                                int(sparse_k), int(mode), _dtype_code(out), out.data_ptr(),
                                _stream_ptr(stream)), "skiparse_attn8")
    return out


def rope_remap(q, k, v, grid, sparse_k, mode, outs=None, stream=None):
    """RoPE(q), RoPE(k), v rearranged to (k*B, N/k, heads, d); returns (rq, rk, rv)."""
    import torch
    B, T, H, W, heads, d = _dims(q, grid)
    shape = (sparse_k * B, (T * H * W) // sparse_k, heads, d)
    if outs is None:
        outs = tuple(torch.empty(shape, dtype=q.dtype, device=q.device) for _ in range(3))
    rq, rk, rv = outs
    _check(lib().skiparse_rope_remap(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                                     int(sparse_k), int(mode), _dtype_code(q), rq.data_ptr(),
                                     rk.data_ptr(), rv.data_ptr(), _stream_ptr(stream)),
           "skiparse_rope_remap")
    return rq, rk, rv


def rearrange(x, grid, sparse_k, mode, apply_rope=False, out=None, stream=None):
    """One tensor (B, N, heads, d) -> (k*B, N/k, heads, d), optionally rotated by 3D RoPE."""
    import torch
    B, T, H, W, heads, d = _dims(x, grid)
    if out is None:
        out = torch.empty((sparse_k * B, (T * H * W) // sparse_k, heads, d), dtype=x.dtype, device=x.device)
    _check(lib().skiparse_rearrange(x.data_ptr(), B, T, H, W, heads, d, int(sparse_k), int(mode),
                                    _dtype_code(x), int(bool(apply_rope)), out.data_ptr(),
                                    _stream_ptr(stream)), "skiparse_rearrange")
    return out


def reverse(x, grid, sparse_k, mode, out=None, stream=None):
    """(k*B, N/k, heads, d) -> (B, N, heads, d), the inverse of :func:`rearrange`."""
    import torch
    T, H, W = (int(g) for g in grid)
    kB, L, heads, d = x.shape
    B = kB // sparse_k
    if out is None:
        out = torch.empty((B, T * H * W, heads, d), dtype=x.dtype, device=x.device)
    _check(lib().skiparse_reverse(x.data_ptr(), B, T, H, W, heads, d, int(sparse_k), int(mode),
                                  _dtype_code(x), out.data_ptr(), _stream_ptr(stream)),
           "skiparse_reverse")
    return out


def scope_table(N, sparse_k, mode):
    """Host-side (k, N/k) int64 table: token index of position p of scope s (numpy array)."""
    import numpy as np
    out = np.empty(int(N), dtype=np.int64)
    _check(lib().skiparse_scope_table(int(N), int(sparse_k), int(mode),
                                      out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
           "skiparse_scope_table")
    return out.reshape(int(sparse_k), int(N) // int(sparse_k))


def attn_flops(B, grid, heads, head_dim, sparse_k):
    T, H, W = (int(g) for g in grid)
    return lib().skiparse_attn_flops(int(B), T, H, W, int(heads), int(head_dim), int(sparse_k))
