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
# SKIPARSE_AMD_LIB names another build of the same library (the host-sanitizer build of the
# CPU tests); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("SKIPARSE_AMD_LIB") or os.path.join(HERE, "libskiparse_amd.so")

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
E_WORKSPACE = 7

# capacity of attn_bwd_rotated_static's workspace: B*heads*N fp32 values
STATIC_DELTA_MAX = 4194304

# largest T + H + W of the calls that keep the whole RoPE table in LDS (include/skiparse.h)
MAX_GRID_SUM = 224

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
        L.skiparse_attn_bwd_rotated_static.argtypes = [vp] * 6 + dims + [i, i, i] + [vp] * 4
        L.skiparse_attn_bwd_rotated_static.restype = i
        L.skiparse_attn_schedule_rotated.argtypes = [ctypes.POINTER(Layer), i] + dims + [i, vp, vp, vp]
        L.skiparse_attn_schedule_rotated.restype = i
        L.skiparse_probe_mfma.argtypes = [i, i, vp, vp]
        L.skiparse_probe_mfma.restype = i
        L.skiparse_probe_mfma_flops.argtypes = [i, i]
        L.skiparse_probe_mfma_flops.restype = ctypes.c_double
        L.skiparse_probe_stream.argtypes = [vp, vp, i64, i, vp]
        L.skiparse_probe_stream.restype = i
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


def _dtype_code(dtype):
    import torch
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float32:
        return FP32
    raise ValueError(f"unsupported dtype {dtype} (bfloat16 or float32)")


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _grid(grid):
    T, H, W = (int(g) for g in grid)
    return T, H, W


def _sparse_k(sparse_k):
    k = int(sparse_k)
    if k < 1:
        raise ValueError(f"sparse_k must be >= 1 (got {k})")
    return k


def _lead_dims(x, grid, name):
    """(B, T, H, W, heads, d) of the call's first (B, N, heads, head_dim) operand."""
    import torch
    if not isinstance(x, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if x.dim() != 4:
        raise ValueError(f"{name} must be a (B, N, heads, head_dim) tensor")
    T, H, W = _grid(grid)
    B, N, heads, d = (int(e) for e in x.shape)
    if N != T * H * W:
        raise ValueError(f"{name}: N={N} does not match the grid {T}x{H}x{W}")
    return B, T, H, W, heads, d


def _validate(specs):
    """Check every tensor a call hands to the library: (tensor, name, shape, dtype) each.

    The library takes raw device pointers and cannot check them, so anything else (a host
    tensor, a tensor on another GPU, a short, mistyped or strided buffer) is rejected here
    with ValueError before the library is called.  Shapes, dtypes and contiguity are checked
    for all tensors first, then that all of them live on the same GPU.
    """
    import torch
    for t, name, shape, dtype in specs:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch.Tensor")
        if tuple(t.shape) != tuple(int(e) for e in shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    device = specs[0][0].device
    for t, name, _, _ in specs:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (it is on {t.device})")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the call's first operand on {device}")


def _alloc(t, shape, dtype, like):
    import torch
    return t if t is not None else torch.empty(tuple(shape), dtype=dtype, device=like.device)


def attn(q, k, v, grid, sparse_k, mode, out=None, stream=None):
    """Fused Skiparse attention: q, k, v (B, N, heads, d) on the GPU -> out, same shape/dtype."""
    B, T, H, W, heads, d = _lead_dims(q, grid, "q")
    code = _dtype_code(q.dtype)
    out = _alloc(out, q.shape, q.dtype, q)
    _validate([(q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype), (v, "v", q.shape, q.dtype),
               (out, "out", q.shape, q.dtype)])
    _check(lib().skiparse_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                               int(sparse_k), int(mode), code, out.data_ptr(),
                               _stream_ptr(stream)), "skiparse_attn")
    return out


def rope_qk(q, k, grid, outs=None, stream=None):
    """3D RoPE of q and k once (bf16, head_dim 128): returns (qr, kr), qr with the softmax
    scale log2(e)/sqrt(d) folded in -- the operands of attn_rotated."""
    B, T, H, W, heads, d = _lead_dims(q, grid, "q")
    code = _dtype_code(q.dtype)
    qr, kr = outs if outs is not None else (None, None)
    qr, kr = _alloc(qr, q.shape, q.dtype, q), _alloc(kr, q.shape, q.dtype, q)
    _validate([(q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype),
               (qr, "qr", q.shape, q.dtype), (kr, "kr", q.shape, q.dtype)])
    _check(lib().skiparse_rope_qk(q.data_ptr(), k.data_ptr(), B, T, H, W, heads, d, code,
                                  qr.data_ptr(), kr.data_ptr(), _stream_ptr(stream)), "skiparse_rope_qk")
    return qr, kr


def attn_rotated(qr, kr, v, grid, sparse_k, mode, out=None, stream=None):
    """Skiparse attention on rope_qk's outputs; equals attn(q, k, v, ...) bit for bit."""
    B, T, H, W, heads, d = _lead_dims(qr, grid, "qr")
    code = _dtype_code(qr.dtype)
    out = _alloc(out, qr.shape, qr.dtype, qr)
    _validate([(qr, "qr", qr.shape, qr.dtype), (kr, "kr", qr.shape, qr.dtype),
               (v, "v", qr.shape, qr.dtype), (out, "out", qr.shape, qr.dtype)])
    _check(lib().skiparse_attn_rotated(qr.data_ptr(), kr.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                                       int(sparse_k), int(mode), code, out.data_ptr(),
                                       _stream_ptr(stream)), "skiparse_attn_rotated")
    return out


def _lse_shape(B, heads, T, H, W):
    return (B, heads, T * H * W)


def attn_rotated_lse(qr, kr, v, grid, sparse_k, mode, out=None, lse=None, stream=None):
    """attn_rotated that also returns each row's log2-sum-exp (B, heads, N) fp32; equals
    attn_lse(q, k, v, ...) bit for bit."""
    import torch
    B, T, H, W, heads, d = _lead_dims(qr, grid, "qr")
    code = _dtype_code(qr.dtype)
    ls = _lse_shape(B, heads, T, H, W)
    out = _alloc(out, qr.shape, qr.dtype, qr)
    lse = _alloc(lse, ls, torch.float32, qr)
    _validate([(qr, "qr", qr.shape, qr.dtype), (kr, "kr", qr.shape, qr.dtype),
               (v, "v", qr.shape, qr.dtype), (out, "out", qr.shape, qr.dtype),
               (lse, "lse", ls, torch.float32)])
    _check(lib().skiparse_attn_rotated_lse(qr.data_ptr(), kr.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                                           int(sparse_k), int(mode), code, out.data_ptr(),
                                           lse.data_ptr(), _stream_ptr(stream)), "skiparse_attn_rotated_lse")
    return out, lse


def _bwd_args(q, k, v, out, dout, lse, grid, grads, delta, names):
    import torch
    B, T, H, W, heads, d = _lead_dims(q, grid, names[0])
    code = _dtype_code(q.dtype)
    ls = _lse_shape(B, heads, T, H, W)
    if grads is None:
        grads = (None, None, None)
    if len(grads) != 3:
        raise ValueError("grads must be a (dq, dk, dv) triple")
    dq, dk, dv = (_alloc(g, q.shape, q.dtype, q) for g in grads)
    delta = _alloc(delta, ls, torch.float32, q)
    specs = [(t, n, q.shape, q.dtype) for t, n in zip((q, k, v, out, dout), names)]
    specs += [(lse, "lse", ls, torch.float32), (dq, "dq", q.shape, q.dtype),
              (dk, "dk", q.shape, q.dtype), (dv, "dv", q.shape, q.dtype),
              (delta, "delta", ls, torch.float32)]
    _validate(specs)
    return (B, T, H, W, heads, d), code, (dq, dk, dv), delta


def attn_bwd_rotated(qr, kr, v, out, dout, lse, grid, sparse_k, mode, grads=None, delta=None, stream=None):
    """attn_bwd on rope_qk's outputs: (dq, dk, dv) with respect to the unrotated q, k and v;
    equals attn_bwd(q, k, v, ...) bit for bit."""
    dims, code, (dq, dk, dv), delta = _bwd_args(qr, kr, v, out, dout, lse, grid, grads, delta,
                                                ("qr", "kr", "v", "out", "dout"))
    _check(lib().skiparse_attn_bwd_rotated(qr.data_ptr(), kr.data_ptr(), v.data_ptr(), out.data_ptr(),
                                           dout.data_ptr(), lse.data_ptr(), *dims,
                                           int(sparse_k), int(mode), code, dq.data_ptr(),
                                           dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                                           _stream_ptr(stream)), "skiparse_attn_bwd_rotated")
    return dq, dk, dv


def attn_bwd_rotated_static(qr, kr, v, out, dout, lse, grid, sparse_k, mode, grads=None, stream=None):
    """attn_bwd_rotated with its delta workspace in the library's static per-GPU array (the
    call allocates nothing when ``grads`` are given); equal to attn_bwd_rotated bit for bit.
    B*heads*N must not exceed STATIC_DELTA_MAX, and calls that overlap on one GPU race on
    the shared workspace."""
    dims, code, (dq, dk, dv), _ = _bwd_args(qr, kr, v, out, dout, lse, grid, grads, lse,
                                            ("qr", "kr", "v", "out", "dout"))
    _check(lib().skiparse_attn_bwd_rotated_static(qr.data_ptr(), kr.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                  dout.data_ptr(), lse.data_ptr(), *dims,
                                                  int(sparse_k), int(mode), code, dq.data_ptr(),
                                                  dk.data_ptr(), dv.data_ptr(), _stream_ptr(stream)),
           "skiparse_attn_bwd_rotated_static")
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


def _schedule_specs(layers, grid):
    if not layers:
        raise ValueError("empty schedule")
    q0 = layers[0][0]
    B, T, H, W, heads, d = _lead_dims(q0, grid, "layer 0 q")
    code = _dtype_code(q0.dtype)
    specs = []
    for i, layer in enumerate(layers):
        if len(layer) != 6:
            raise ValueError(f"layer {i} must be (q, k, v, out, sparse_k, mode)")
        for t, n in zip(layer[:4], ("q", "k", "v", "out")):
            specs.append((t, f"layer {i} {n}", q0.shape, q0.dtype))
    return specs, (B, T, H, W, heads, d), code, q0


def _schedule_array(layers):
    arr = (Layer * len(layers))()
    for i, (q, k, v, out, sk_, mode) in enumerate(layers):
        arr[i] = Layer(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), int(sk_), int(mode))
    return arr


def attn_schedule(layers, grid, stream=None):
    """Run a schedule: `layers` is a list of (q, k, v, out, sparse_k, mode); all layers share
    shape and dtype.  One validation pass, then one launch per layer on one stream."""
    specs, dims, code, _ = _schedule_specs(layers, grid)
    _validate(specs)
    _check(lib().skiparse_attn_schedule(_schedule_array(layers), len(layers), *dims, code,
                                        _stream_ptr(stream)), "skiparse_attn_schedule")
    return [layer[3] for layer in layers]


def attn_schedule_rotated(layers, grid, scratch=None, stream=None):
    """attn_schedule with every layer run as the RoPE pass into `scratch` (qr, kr: two tensors
    shaped like q, reused by all layers) and the attention on the rotated operands; equals
    attn_schedule bit for bit (head_dim 128, bf16, every sparse_k dividing 64)."""
    specs, dims, code, q0 = _schedule_specs(layers, grid)
    qr, kr = scratch if scratch is not None else (None, None)
    qr, kr = _alloc(qr, q0.shape, q0.dtype, q0), _alloc(kr, q0.shape, q0.dtype, q0)
    _validate(specs + [(qr, "scratch qr", q0.shape, q0.dtype), (kr, "scratch kr", q0.shape, q0.dtype)])
    _check(lib().skiparse_attn_schedule_rotated(_schedule_array(layers), len(layers), *dims, code,
                                                qr.data_ptr(), kr.data_ptr(), _stream_ptr(stream)),
           "skiparse_attn_schedule_rotated")
    return [layer[3] for layer in layers]


def attn_lse(q, k, v, grid, sparse_k, mode, out=None, lse=None, stream=None):
    """Fused Skiparse attention that also returns each row's log2-sum-exp (B, heads, N) fp32."""
    import torch
    B, T, H, W, heads, d = _lead_dims(q, grid, "q")
    code = _dtype_code(q.dtype)
    ls = _lse_shape(B, heads, T, H, W)
    out = _alloc(out, q.shape, q.dtype, q)
    lse = _alloc(lse, ls, torch.float32, q)
    _validate([(q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype), (v, "v", q.shape, q.dtype),
               (out, "out", q.shape, q.dtype), (lse, "lse", ls, torch.float32)])
    _check(lib().skiparse_attn_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                                   int(sparse_k), int(mode), code, out.data_ptr(),
                                   lse.data_ptr(), _stream_ptr(stream)), "skiparse_attn_lse")
    return out, lse


def attn_bwd(q, k, v, out, dout, lse, grid, sparse_k, mode, grads=None, delta=None, stream=None):
    """Gradients (dq, dk, dv) of a loss through Skiparse attention, given dout = dLoss/dout.

    ``out`` and ``lse`` come from :func:`attn_lse` on the same inputs; ``delta`` is an
    optional (B, heads, N) fp32 workspace.
    """
    dims, code, (dq, dk, dv), delta = _bwd_args(q, k, v, out, dout, lse, grid, grads, delta,
                                                ("q", "k", "v", "out", "dout"))
    _check(lib().skiparse_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   dout.data_ptr(), lse.data_ptr(), *dims,
                                   int(sparse_k), int(mode), code, dq.data_ptr(),
                                   dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                                   _stream_ptr(stream)), "skiparse_attn_bwd")
    return dq, dk, dv


def attn_bwd_flops(B, grid, heads, head_dim, sparse_k):
    T, H, W = _grid(grid)
    return float(lib().skiparse_attn_bwd_flops(int(B), T, H, W, int(heads), int(head_dim), int(sparse_k)))


Q8_KEYS = ("q8", "q_amax", "k8", "k_amax", "vt8", "v_amax")


def q8_scope_pitch(grid, sparse_k):
    """Lp: the channel-row pitch (keys) of vt8, L rounded up to a multiple of 64."""
    T, H, W = _grid(grid)
    lp = lib().skiparse_q8_scope_pitch(T, H, W, int(sparse_k))
    if lp < 0:
        raise SkiparseError(-lp, "skiparse_q8_scope_pitch")
    return lp


def _q8_specs(B, N, heads, d, grid, sparse_k):
    import torch
    lp = q8_scope_pitch(grid, sparse_k)
    return {"q8": ((B, N, heads, d), torch.int8), "q_amax": ((B, N, heads), torch.float32),
            "k8": ((B, N, heads, d), torch.int8), "k_amax": ((B, heads), torch.float32),
            "vt8": ((B, heads, _sparse_k(sparse_k), d, lp), torch.uint8),
            "v_amax": ((B, heads, d), torch.float32)}


def quant8(q, k, v, grid, sparse_k, mode, outs=None, stream=None):
    """8-bit operands of q, k, v for :func:`attn8`: a dict with q8 (int8), q_amax, k8 (int8),
    k_amax, vt8 (uint8 E4M3 codes) and v_amax (float32), in the layouts of include/skiparse.h."""
    B, T, H, W, heads, d = _lead_dims(q, grid, "q")
    code = _dtype_code(q.dtype)
    specs = _q8_specs(B, T * H * W, heads, d, grid, sparse_k)
    if outs is None:
        outs = {key: _alloc(None, shape, dt, q) for key, (shape, dt) in specs.items()}
    missing = [key for key in Q8_KEYS if key not in outs]
    if missing:
        raise ValueError(f"outs lacks {missing}")
    _validate([(q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype), (v, "v", q.shape, q.dtype)]
              + [(outs[key], key, *specs[key]) for key in Q8_KEYS])
    _check(lib().skiparse_quant8(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                                 int(sparse_k), int(mode), code,
                                 *(outs[key].data_ptr() for key in Q8_KEYS), _stream_ptr(stream)),
           "skiparse_quant8")
    return outs


def attn8(qz, grid, sparse_k, mode, out_dtype=None, out=None, stream=None):
    """8-bit Skiparse attention of :func:`quant8`'s operands -> (B, N, heads, d) bf16 (or fp32)."""
    import torch
    missing = [key for key in Q8_KEYS if key not in qz]
    if missing:
        raise ValueError(f"qz lacks {missing}")
    q8 = qz["q8"]
    B, T, H, W, heads, d = _lead_dims(q8, grid, "q8")
    specs = _q8_specs(B, T * H * W, heads, d, grid, sparse_k)
    if out is None:
        out = _alloc(None, q8.shape, out_dtype or torch.bfloat16, q8)
    code = _dtype_code(out.dtype)
    _validate([(qz[key], key, *specs[key]) for key in Q8_KEYS] + [(out, "out", q8.shape, out.dtype)])
    _check(lib().skiparse_attn8(*(qz[key].data_ptr() for key in Q8_KEYS), B, T, H, W, heads, d,
                                int(sparse_k), int(mode), code, out.data_ptr(),
                                _stream_ptr(stream)), "skiparse_attn8")
    return out


def _rearranged_shape(B, T, H, W, heads, d, sparse_k):
    k = _sparse_k(sparse_k)
    N = T * H * W
    if N % k:
        raise ValueError(f"N={N} is not divisible by sparse_k={k}")
    return (k * B, N // k, heads, d)


def rope_remap(q, k, v, grid, sparse_k, mode, outs=None, stream=None):
    """RoPE(q), RoPE(k), v rearranged to (k*B, N/k, heads, d); returns (rq, rk, rv)."""
    B, T, H, W, heads, d = _lead_dims(q, grid, "q")
    code = _dtype_code(q.dtype)
    shape = _rearranged_shape(B, T, H, W, heads, d, sparse_k)
    if outs is None:
        outs = (None, None, None)
    if len(outs) != 3:
        raise ValueError("outs must be an (rq, rk, rv) triple")
    rq, rk, rv = (_alloc(o, shape, q.dtype, q) for o in outs)
    _validate([(q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype), (v, "v", q.shape, q.dtype),
               (rq, "rq", shape, q.dtype), (rk, "rk", shape, q.dtype), (rv, "rv", shape, q.dtype)])
    _check(lib().skiparse_rope_remap(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, W, heads, d,
                                     int(sparse_k), int(mode), code, rq.data_ptr(),
                                     rk.data_ptr(), rv.data_ptr(), _stream_ptr(stream)),
           "skiparse_rope_remap")
    return rq, rk, rv


def rearrange(x, grid, sparse_k, mode, apply_rope=False, out=None, stream=None):
    """One tensor (B, N, heads, d) -> (k*B, N/k, heads, d), optionally rotated by 3D RoPE."""
    B, T, H, W, heads, d = _lead_dims(x, grid, "x")
    code = _dtype_code(x.dtype)
    shape = _rearranged_shape(B, T, H, W, heads, d, sparse_k)
    out = _alloc(out, shape, x.dtype, x)
    _validate([(x, "x", x.shape, x.dtype), (out, "out", shape, x.dtype)])
    _check(lib().skiparse_rearrange(x.data_ptr(), B, T, H, W, heads, d, int(sparse_k), int(mode),
                                    code, int(bool(apply_rope)), out.data_ptr(),
                                    _stream_ptr(stream)), "skiparse_rearrange")
    return out


def reverse(x, grid, sparse_k, mode, out=None, stream=None):
    """(k*B, N/k, heads, d) -> (B, N, heads, d), the inverse of :func:`rearrange`."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError("x must be a (k*B, N/k, heads, head_dim) tensor")
    T, H, W = _grid(grid)
    k = _sparse_k(sparse_k)
    kB, L, heads, d = (int(e) for e in x.shape)
    if kB % k or L * k != T * H * W:
        raise ValueError(f"x of shape {tuple(x.shape)} is not a sparse_k={k} rearrangement of the "
                         f"grid {T}x{H}x{W}")
    B = kB // k
    code = _dtype_code(x.dtype)
    out = _alloc(out, (B, T * H * W, heads, d), x.dtype, x)
    _validate([(x, "x", x.shape, x.dtype), (out, "out", (B, T * H * W, heads, d), x.dtype)])
    _check(lib().skiparse_reverse(x.data_ptr(), B, T, H, W, heads, d, k, int(mode),
                                  code, out.data_ptr(), _stream_ptr(stream)),
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


def probe_mfma(blocks, iters, out=None, stream=None):
    """Measurement probe: one launch of `blocks` x 256 threads issuing only bf16 matrix
    products; returns (out, FLOPs of the launch).  `out` holds blocks*256 fp32 checksums."""
    import torch
    if out is None:
        out = torch.empty(int(blocks) * 256, dtype=torch.float32, device="cuda")
    _validate([(out, "out", (int(blocks) * 256,), torch.float32)])
    _check(lib().skiparse_probe_mfma(int(blocks), int(iters), out.data_ptr(), _stream_ptr(stream)),
           "skiparse_probe_mfma")
    return out, float(lib().skiparse_probe_mfma_flops(int(blocks), int(iters)))


def probe_stream(src, dst, blocks, stream=None):
    """Measurement probe: copy src to dst (same size, contiguous, a multiple of 16 bytes) with
    16-byte nontemporal loads and stores over `blocks` workgroups."""
    nbytes = src.numel() * src.element_size()
    _validate([(src, "src", src.shape, src.dtype), (dst, "dst", src.shape, src.dtype)])
    _check(lib().skiparse_probe_stream(src.data_ptr(), dst.data_ptr(), nbytes, int(blocks), _stream_ptr(stream)),
           "skiparse_probe_stream")
    return dst
