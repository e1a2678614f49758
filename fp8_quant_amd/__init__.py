"""fp8_quant_amd: RMSNorm -> partial NeoX RoPE -> per-row FP8 e4m3fn on MI355X.

Python binding of ``librnq.so`` (C ABI declared in ``include/rnq.h``). The
functions named ``rnq_*`` mirror the C entry points one to one: they take
torch tensors that live on the GPU, check shapes and dtypes, and pass raw
pointers, sizes and torch's current stream through ctypes. Every step of the
computation runs in the HIP kernels; there is no CPU path. If the library has
not been built, the first call raises.

Convenience wrappers (``qk_norm_rope_fp8``, ``rmsnorm``, ``rmsnorm_bwd``,
``rmsnorm_rope``, ``rmsnorm_rope_bwd``, ``rmsnorm_rope_fp8_grouped``) allocate
the outputs with torch and call the same entry points; ``prepare_*`` functions
marshal once and return a launcher for tight loops or graph capture;
``fp8_quant_amd.autograd`` wraps RMSNorm and RMSNorm + RoPE as autograd
Functions. For example, the attention prologue of 4096 tokens with 32 query
and 8 key/value heads of width 128 (bf16 on the GPU, cos/sin fp32 [4096, 64])::

    import fp8_quant_amd as rnq
    q8, k8, q_scale, k_scale = rnq.qk_norm_rope_fp8(q, k, wq, wk, cos, sin)
    # q8: float8_e4m3fn [4096, 32, 128], q_scale: float32 [4096, 32]; same for k

and with q and k as views into a fused QKV projection output, each token's
cos/sin row looked up by position::

    q = qkv[:, :32 * 128].view(T, 32, 128); k = qkv[:, 32 * 128:40 * 128].view(T, 8, 128)
    q8, k8, q_scale, k_scale = rnq.qk_norm_rope_fp8(q, k, wq, wk, cos_table, sin_table,
                                                    positions=pos_int32)
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "RnqError",
    "library_path",
    "load_library",
    "rnq_status_string",
    "rnq_abi_version",
    "rnq_qk_norm_rope_fp8",
    "rnq_rmsnorm_rope",
    "rnq_rmsnorm_fwd",
    "rnq_rmsnorm_bwd",
    "rnq_rmsnorm_bwd_workspace_size",
    "rnq_rmsnorm_rope_fp8_grouped",
    "rnq_rmsnorm_rope_bwd",
    "rnq_rmsnorm_rope_bwd_noalloc",
    "RNQ_NOALLOC_SCRATCH_BYTES",
    "rnq_qk_norm_rope_fp8_ex",
    "rnq_rmsnorm_rope_ex",
    "prepare_qk_norm_rope_fp8",
    "prepare_qk_norm_rope_fp8_ex",
    "prepare_rmsnorm_rope_ex",
    "prepare_rmsnorm_rope_fp8_grouped",
    "prepare_rmsnorm_rope",
    "prepare_rmsnorm_fwd",
    "prepare_rmsnorm_bwd",
    "prepare_rmsnorm_rope_bwd",
    "prepare_rmsnorm_rope_bwd_noalloc",
    "qk_norm_rope_fp8",
    "rmsnorm",
    "rmsnorm_bwd",
    "rmsnorm_rope",
    "rmsnorm_rope_fp8_grouped",
    "rmsnorm_rope_bwd",
    "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
EXPORTED_SYMBOLS = (
    "rnq_status_string",
    "rnq_last_error",
    "rnq_abi_version",
    "rnq_rmsnorm_fwd",
    "rnq_rmsnorm_bwd_workspace_size",
    "rnq_rmsnorm_bwd",
    "rnq_rmsnorm_rope",
    "rnq_qk_norm_rope_fp8",
    "rnq_rmsnorm_rope_fp8_grouped",
    "rnq_rmsnorm_rope_bwd",
    "rnq_qk_norm_rope_fp8_ex",
    "rnq_rmsnorm_rope_ex",
    "rnq_baseline_norm_rope_quant_unfused",
    "rnq_baseline_qk_design",
    "rnq_baseline_stream",
    "rnq_rmsnorm_rope_bwd_noalloc",
    "rnq_baseline_stream_policy",
)

RNQ_BF16 = 0
RNQ_F16 = 1
RNQ_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # the library's static backward scratch (include/rnq.h)


class RnqError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}" if detail else name)
        self.status = status


_lib = None


def library_path() -> str:
    return os.environ.get("RNQ_LIBRARY", os.path.join(_HERE, "librnq.so"))


def load_library():
    """Load librnq.so once; raise if it is missing (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library not built: {path} is missing (run `python -m fp8_quant_amd.build`)"
        )
    lib = ctypes.CDLL(path)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.rnq_status_string.argtypes = [i32]
    lib.rnq_status_string.restype = ctypes.c_char_p
    lib.rnq_last_error.argtypes = []
    lib.rnq_last_error.restype = ctypes.c_char_p
    lib.rnq_abi_version.argtypes = []
    lib.rnq_abi_version.restype = i32
    lib.rnq_rmsnorm_fwd.argtypes = [vp, vp, vp, vp, i64, i64, f32, i32, vp]
    lib.rnq_rmsnorm_fwd.restype = i32
    lib.rnq_rmsnorm_bwd_workspace_size.argtypes = [i64, i64]
    lib.rnq_rmsnorm_bwd_workspace_size.restype = ctypes.c_size_t
    lib.rnq_rmsnorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, f32, i32, vp]
    lib.rnq_rmsnorm_bwd.restype = i32
    lib.rnq_rmsnorm_rope.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, vp]
    lib.rnq_rmsnorm_rope.restype = i32
    lib.rnq_qk_norm_rope_fp8.argtypes = [vp] * 12 + [i64] * 5 + [f32, f32, i32, vp]
    lib.rnq_qk_norm_rope_fp8.restype = i32
    lib.rnq_rmsnorm_rope_fp8_grouped.argtypes = [vp] * 7 + [i64] * 5 + [f32, f32, i32, vp]
    lib.rnq_rmsnorm_rope_fp8_grouped.restype = i32
    lib.rnq_rmsnorm_rope_bwd.argtypes = [vp] * 9 + [ctypes.c_size_t] + [i64] * 4 + [f32, i32, vp]
    lib.rnq_rmsnorm_rope_bwd.restype = i32
    lib.rnq_qk_norm_rope_fp8_ex.argtypes = [vp, i64, vp, i64] + [vp] * 5 + [i64] + [vp] * 6 + [i64] * 5 + [f32, f32,
                                                                                                       i32, vp]
    lib.rnq_qk_norm_rope_fp8_ex.restype = i32
    lib.rnq_rmsnorm_rope_ex.argtypes = [vp, i64] + [vp] * 4 + [i64, vp] + [i64] * 4 + [f32, i32, vp]
    lib.rnq_rmsnorm_rope_ex.restype = i32
    lib.rnq_baseline_norm_rope_quant_unfused.argtypes = [vp] * 8 + [i64] * 4 + [f32, f32, i32, vp]
    lib.rnq_baseline_norm_rope_quant_unfused.restype = i32
    lib.rnq_baseline_qk_design.argtypes = [vp] * 10 + [i64] * 6 + [f32, f32, i32, vp]
    lib.rnq_baseline_qk_design.restype = i32
    lib.rnq_baseline_stream.argtypes = [vp, i64, vp, vp]
    lib.rnq_baseline_stream.restype = i32
    lib.rnq_baseline_stream_policy.argtypes = [vp, i64, vp, i32, vp]
    lib.rnq_baseline_stream_policy.restype = i32
    lib.rnq_rmsnorm_rope_bwd_noalloc.argtypes = [vp] * 8 + [i64] * 4 + [f32, i32, vp]
    lib.rnq_rmsnorm_rope_bwd_noalloc.restype = i32
    _lib = lib
    return lib


# ------------------------------------------------------------------ marshalling


def _torch():
    import torch

    return torch


def _ptr(t):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"tensor on {t.device}: the rnq kernels need GPU tensors (no CPU path)")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _token_view(t, heads: int, width: int, what: str):
    """Pointer and token stride (elements) of a [T, heads, width] view whose rows of one
    token are contiguous (a slice of a fused projection output, say); stride 0 when the
    whole tensor is contiguous."""
    if t is None:
        return None, 0
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"tensor on {t.device}: the rnq kernels need GPU tensors (no CPU path)")
    if t.is_contiguous():
        return ctypes.c_void_p(t.data_ptr()), 0
    if t.dim() != 3 or t.stride(2) != 1 or (heads > 1 and t.stride(1) != width):
        raise ValueError(f"{what}: expected a [T, H, D] view with contiguous rows inside a token "
                         f"(strides (S, {width}, 1)), got strides {tuple(t.stride())}")
    return ctypes.c_void_p(t.data_ptr()), int(t.stride(0))


def _positions(positions, tokens: int):
    torch = _torch()
    if positions is None:
        return None
    if positions.dtype != torch.int32:
        raise TypeError(f"positions: dtype {positions.dtype}, expected torch.int32")
    if tuple(positions.shape) != (tokens,):
        raise ValueError(f"positions: shape {tuple(positions.shape)}, expected {(tokens,)}")
    return _ptr(positions)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return RNQ_BF16
    if t.dtype == torch.float16:
        return RNQ_F16
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp16)")


def _stream(t, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int):
    if status != 0:
        lib = load_library()
        name = lib.rnq_status_string(status).decode()
        detail = lib.rnq_last_error().decode()
        raise RnqError(status, name, detail)


def _expect(t, dtype, shape, what):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")


# ------------------------------------------------------------- C entry points


def rnq_status_string(status: int) -> str:
    return load_library().rnq_status_string(status).decode()


def rnq_abi_version() -> int:
    return load_library().rnq_abi_version()


def rnq_qk_norm_rope_fp8(q, k, wq, wk, cos, sin, q_fp8, k_fp8, q_scale, k_scale, q_y=None, k_y=None,
                         *, eps: float = 1e-6, fp8_max: float = 448.0, stream=None) -> None:
    """QK-norm + RoPE + FP8 into caller-provided outputs (see include/rnq.h)."""
    prepare_qk_norm_rope_fp8(q, k, wq, wk, cos, sin, q_fp8, k_fp8, q_scale, k_scale, q_y, k_y,
                             eps=eps, fp8_max=fp8_max, stream=stream)()


def _launcher(fn, args, *tensors):
    """A zero-argument callable that enqueues ``fn(*args)``. The marshalled
    arguments are raw device addresses, so the tensors they point into are kept
    referenced by the launcher for as long as it exists."""
    keep = tuple(t for t in tensors if t is not None)

    def launch():
        status = fn(*args)
        if status != 0:
            _check(status)
    launch.tensors = keep
    return launch


def prepare_qk_norm_rope_fp8(q, k, wq, wk, cos, sin, q_fp8, k_fp8, q_scale, k_scale, q_y=None, k_y=None,
                             *, eps: float = 1e-6, fp8_max: float = 448.0, stream=None):
    """Check and marshal the arguments once; returns a zero-argument callable that
    enqueues ``rnq_qk_norm_rope_fp8`` on the stream (for tight launch loops)."""
    torch = _torch()
    lib = load_library()
    T, Hq, D = q.shape
    Hk = 0 if k is None else k.shape[1]
    half = 0 if cos is None else cos.shape[-1]
    dt = q.dtype
    if k is not None:
        _expect(k, dt, (T, Hk, D), "k")
    _expect(wq, dt, (D,), "wq")
    _expect(wk, dt, (D,), "wk")
    if cos is not None:
        _expect(cos, torch.float32, (T, half), "cos")
        _expect(sin, torch.float32, (T, half), "sin")
    for o, H, nm in ((q_fp8, Hq, "q_fp8"), (k_fp8, Hk, "k_fp8")):
        if o is not None and o.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{nm}: expected uint8 or float8_e4m3fn")
        if o is not None and tuple(o.shape) != (T, H, D):
            raise ValueError(f"{nm}: shape {tuple(o.shape)}, expected {(T, H, D)}")
    _expect(q_scale, torch.float32, (T, Hq), "q_scale")
    _expect(k_scale, torch.float32, (T, Hk), "k_scale")
    _expect(q_y, dt, (T, Hq, D), "q_y")
    _expect(k_y, dt, (T, Hk, D), "k_y")
    args = (
        _ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(cos), _ptr(sin),
        _ptr(q_fp8), _ptr(k_fp8), _ptr(q_scale), _ptr(k_scale), _ptr(q_y), _ptr(k_y),
        T, Hq, Hk, D, 2 * half, eps, fp8_max, _dtype_code(q), _stream(q, stream),
    )
    return _launcher(lib.rnq_qk_norm_rope_fp8, args, q, k, wq, wk, cos, sin, q_fp8, k_fp8, q_scale, k_scale,
                     q_y, k_y)


def rnq_qk_norm_rope_fp8_ex(q, k, wq, wk, cos, sin, q_fp8, k_fp8, q_scale, k_scale, q_y=None, k_y=None, *,
                            positions=None, eps: float = 1e-6, fp8_max: float = 448.0, stream=None) -> None:
    """rnq_qk_norm_rope_fp8 with q / k as [T, H, D] views (token stride from the view) and
    cos/sin rows gathered through int32 ``positions`` [T] from a [table_rows, R/2] table."""
    prepare_qk_norm_rope_fp8_ex(q, k, wq, wk, cos, sin, q_fp8, k_fp8, q_scale, k_scale, q_y, k_y,
                                positions=positions, eps=eps, fp8_max=fp8_max, stream=stream)()


def prepare_qk_norm_rope_fp8_ex(q, k, wq, wk, cos, sin, q_fp8, k_fp8, q_scale, k_scale, q_y=None, k_y=None, *,
                                positions=None, eps: float = 1e-6, fp8_max: float = 448.0, stream=None):
    torch = _torch()
    lib = load_library()
    T, Hq, D = q.shape
    Hk = 0 if k is None else k.shape[1]
    half = 0 if cos is None else cos.shape[-1]
    dt = q.dtype
    if k is not None and (k.dtype != dt or tuple(k.shape) != (T, Hk, D)):
        raise ValueError(f"k: expected {dt} of shape {(T, Hk, D)}")
    _expect(wq, dt, (D,), "wq")
    _expect(wk, dt, (D,), "wk")
    table_rows = T if positions is None else (0 if cos is None else cos.shape[0])
    if cos is not None:
        _expect(cos, torch.float32, (table_rows, half), "cos")
        _expect(sin, torch.float32, (table_rows, half), "sin")
    for o, H, nm in ((q_fp8, Hq, "q_fp8"), (k_fp8, Hk, "k_fp8")):
        if o is not None and o.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{nm}: expected uint8 or float8_e4m3fn")
        if o is not None and tuple(o.shape) != (T, H, D):
            raise ValueError(f"{nm}: shape {tuple(o.shape)}, expected {(T, H, D)}")
    _expect(q_scale, torch.float32, (T, Hq), "q_scale")
    _expect(k_scale, torch.float32, (T, Hk), "k_scale")
    _expect(q_y, dt, (T, Hq, D), "q_y")
    _expect(k_y, dt, (T, Hk, D), "k_y")
    qp, qs_ = _token_view(q, Hq, D, "q")
    kp, ks_ = _token_view(k, Hk, D, "k")
    args = (
        qp, qs_, kp, ks_, _ptr(wq), _ptr(wk), _ptr(cos), _ptr(sin), _positions(positions, T), table_rows,
        _ptr(q_fp8), _ptr(k_fp8), _ptr(q_scale), _ptr(k_scale), _ptr(q_y), _ptr(k_y),
        T, Hq, Hk, D, 2 * half, eps, fp8_max, _dtype_code(q), _stream(q, stream),
    )
    return _launcher(lib.rnq_qk_norm_rope_fp8_ex, args, q, k, wq, wk, cos, sin, positions, q_fp8, k_fp8,
                     q_scale, k_scale, q_y, k_y)


def rnq_rmsnorm_rope_ex(x, w, cos, sin, y, *, positions=None, rows_per_token: int = 1, eps: float = 1e-6,
                        stream=None) -> None:
    """rnq_rmsnorm_rope with x as a [T, rows_per_token, N] view (or a [M, N] view when
    rows_per_token is 1) and cos/sin gathered through int32 ``positions`` [T]."""
    prepare_rmsnorm_rope_ex(x, w, cos, sin, y, positions=positions, rows_per_token=rows_per_token, eps=eps,
                            stream=stream)()


def prepare_rmsnorm_rope_ex(x, w, cos, sin, y, *, positions=None, rows_per_token: int = 1, eps: float = 1e-6,
                            stream=None):
    torch = _torch()
    lib = load_library()
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    r = max(rows_per_token, 1)
    T = M // r
    half = 0 if cos is None else cos.shape[-1]
    _expect(w, x.dtype, (N,), "w")
    if y is not None and (y.dtype != x.dtype or y.numel() != M * N or not y.is_contiguous()):
        raise ValueError(f"y: expected a contiguous {x.dtype} tensor of {M} x {N}")
    table_rows = T if positions is None else (0 if cos is None else cos.shape[0])
    if cos is not None:
        _expect(cos, torch.float32, (table_rows, half), "cos")
        _expect(sin, torch.float32, (table_rows, half), "sin")
    if x.dim() == 2 and r == 1 and not x.is_contiguous():
        xv = x.unsqueeze(1)
    else:
        xv = x if x.dim() == 3 else x.reshape(T, r, N) if x.is_contiguous() else x
    xp, xs = _token_view(xv, r, N, "x")
    args = (xp, xs, _ptr(w), _ptr(cos), _ptr(sin), _positions(positions, T), table_rows, _ptr(y), M, N, 2 * half,
            rows_per_token, eps, _dtype_code(x), _stream(x, stream))
    return _launcher(lib.rnq_rmsnorm_rope_ex, args, x, w, cos, sin, positions, y)


def rnq_rmsnorm_rope(x, w, cos, sin, y, *, rows_per_token: int = 1, eps: float = 1e-6, stream=None) -> None:
    prepare_rmsnorm_rope(x, w, cos, sin, y, rows_per_token=rows_per_token, eps=eps, stream=stream)()


def prepare_rmsnorm_rope(x, w, cos, sin, y, *, rows_per_token: int = 1, eps: float = 1e-6, stream=None):
    torch = _torch()
    lib = load_library()
    M, N = x.shape
    half = 0 if cos is None else cos.shape[-1]
    _expect(w, x.dtype, (N,), "w")
    _expect(y, x.dtype, (M, N), "y")
    if cos is not None:
        _expect(cos, torch.float32, (M // max(rows_per_token, 1), half), "cos")
        _expect(sin, torch.float32, (M // max(rows_per_token, 1), half), "sin")
    args = (_ptr(x), _ptr(w), _ptr(cos), _ptr(sin), _ptr(y), M, N, 2 * half,
            rows_per_token, eps, _dtype_code(x), _stream(x, stream))
    return _launcher(lib.rnq_rmsnorm_rope, args, x, w, cos, sin, y)


def rnq_rmsnorm_fwd(x, w, y, rstd=None, *, eps: float = 1e-6, stream=None) -> None:
    prepare_rmsnorm_fwd(x, w, y, rstd, eps=eps, stream=stream)()


def prepare_rmsnorm_fwd(x, w, y, rstd=None, *, eps: float = 1e-6, stream=None):
    torch = _torch()
    lib = load_library()
    M, N = x.shape
    _expect(w, x.dtype, (N,), "w")
    _expect(y, x.dtype, (M, N), "y")
    _expect(rstd, torch.float32, (M,), "rstd")
    args = (_ptr(x), _ptr(w), _ptr(y), _ptr(rstd), M, N, eps, _dtype_code(x), _stream(x, stream))
    return _launcher(lib.rnq_rmsnorm_fwd, args, x, w, y, rstd)


def rnq_rmsnorm_bwd_workspace_size(M: int, N: int) -> int:
    return int(load_library().rnq_rmsnorm_bwd_workspace_size(M, N))


def rnq_rmsnorm_bwd(x, w, grad_y, grad_x, grad_w, workspace, rstd=None, *, eps: float = 1e-6, stream=None) -> None:
    prepare_rmsnorm_bwd(x, w, grad_y, grad_x, grad_w, workspace, rstd, eps=eps, stream=stream)()


def prepare_rmsnorm_bwd(x, w, grad_y, grad_x, grad_w, workspace, rstd=None, *, eps: float = 1e-6, stream=None):
    torch = _torch()
    lib = load_library()
    M, N = x.shape
    _expect(w, x.dtype, (N,), "w")
    _expect(grad_y, x.dtype, (M, N), "grad_y")
    _expect(grad_x, x.dtype, (M, N), "grad_x")
    _expect(grad_w, torch.float32, (N,), "grad_w")
    _expect(rstd, torch.float32, (M,), "rstd")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(x), _ptr(w), _ptr(grad_y), _ptr(rstd), _ptr(grad_x), _ptr(grad_w),
            _ptr(workspace), ws_bytes, M, N, eps, _dtype_code(x), _stream(x, stream))
    return _launcher(lib.rnq_rmsnorm_bwd, args, x, w, grad_y, rstd, grad_x, grad_w, workspace)


def rnq_rmsnorm_rope_bwd(x, w, grad_y, cos, sin, grad_x, grad_w, workspace, rstd=None, *, rows_per_token: int = 1,
                         eps: float = 1e-6, stream=None) -> None:
    """Backward of rnq_rmsnorm_rope into caller-provided grad_x, grad_w (fp32) and workspace."""
    prepare_rmsnorm_rope_bwd(x, w, grad_y, cos, sin, grad_x, grad_w, workspace, rstd, rows_per_token=rows_per_token,
                             eps=eps, stream=stream)()


def prepare_rmsnorm_rope_bwd(x, w, grad_y, cos, sin, grad_x, grad_w, workspace, rstd=None, *,
                             rows_per_token: int = 1, eps: float = 1e-6, stream=None):
    torch = _torch()
    lib = load_library()
    M, N = x.shape
    half = 0 if cos is None else cos.shape[-1]
    _expect(w, x.dtype, (N,), "w")
    _expect(grad_y, x.dtype, (M, N), "grad_y")
    _expect(grad_x, x.dtype, (M, N), "grad_x")
    _expect(grad_w, torch.float32, (N,), "grad_w")
    _expect(rstd, torch.float32, (M,), "rstd")
    if cos is not None:
        _expect(cos, torch.float32, (M // max(rows_per_token, 1), half), "cos")
        _expect(sin, torch.float32, (M // max(rows_per_token, 1), half), "sin")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(x), _ptr(w), _ptr(grad_y), _ptr(cos), _ptr(sin), _ptr(rstd), _ptr(grad_x), _ptr(grad_w),
            _ptr(workspace), ws_bytes, M, N, 2 * half, rows_per_token, eps, _dtype_code(x), _stream(x, stream))
    return _launcher(lib.rnq_rmsnorm_rope_bwd, args, x, w, grad_y, cos, sin, rstd, grad_x, grad_w, workspace)


def rnq_rmsnorm_rope_bwd_noalloc(x, w, grad_y, cos, sin, grad_x, grad_w, rstd=None, *, rows_per_token: int = 1,
                                 eps: float = 1e-6, stream=None) -> None:
    """rnq_rmsnorm_rope_bwd with the grad_w partials in the library's static device
    scratch (no workspace, nothing allocated; calls that overlap on one GPU race)."""
    prepare_rmsnorm_rope_bwd_noalloc(x, w, grad_y, cos, sin, grad_x, grad_w, rstd, rows_per_token=rows_per_token,
                                     eps=eps, stream=stream)()


def prepare_rmsnorm_rope_bwd_noalloc(x, w, grad_y, cos, sin, grad_x, grad_w, rstd=None, *, rows_per_token: int = 1,
                                     eps: float = 1e-6, stream=None):
    torch = _torch()
    lib = load_library()
    M, N = x.shape
    half = 0 if cos is None else cos.shape[-1]
    _expect(w, x.dtype, (N,), "w")
    _expect(grad_y, x.dtype, (M, N), "grad_y")
    _expect(grad_x, x.dtype, (M, N), "grad_x")
    _expect(grad_w, torch.float32, (N,), "grad_w")
    _expect(rstd, torch.float32, (M,), "rstd")
    if cos is not None:
        _expect(cos, torch.float32, (M // max(rows_per_token, 1), half), "cos")
        _expect(sin, torch.float32, (M // max(rows_per_token, 1), half), "sin")
    args = (_ptr(x), _ptr(w), _ptr(grad_y), _ptr(cos), _ptr(sin), _ptr(rstd), _ptr(grad_x), _ptr(grad_w),
            M, N, 2 * half, rows_per_token, eps, _dtype_code(x), _stream(x, stream))
    return _launcher(lib.rnq_rmsnorm_rope_bwd_noalloc, args, x, w, grad_y, cos, sin, rstd, grad_x, grad_w)


def rnq_rmsnorm_rope_fp8_grouped(x, w, cos, sin, codes, scales, y=None, *, group_size: int = 128,
                                 rows_per_token: int = 1, eps: float = 1e-6, fp8_max: float = 448.0,
                                 stream=None) -> None:
    """RMSNorm + RoPE + FP8 with one scale per group into caller-provided outputs."""
    prepare_rmsnorm_rope_fp8_grouped(x, w, cos, sin, codes, scales, y, group_size=group_size,
                                     rows_per_token=rows_per_token, eps=eps, fp8_max=fp8_max, stream=stream)()


def prepare_rmsnorm_rope_fp8_grouped(x, w, cos, sin, codes, scales, y=None, *, group_size: int = 128,
                                     rows_per_token: int = 1, eps: float = 1e-6, fp8_max: float = 448.0,
                                     stream=None):
    torch = _torch()
    lib = load_library()
    M, N = x.shape
    half = 0 if cos is None else cos.shape[-1]
    _expect(w, x.dtype, (N,), "w")
    _expect(y, x.dtype, (M, N), "y")
    if cos is not None:
        _expect(cos, torch.float32, (M // max(rows_per_token, 1), half), "cos")
        _expect(sin, torch.float32, (M // max(rows_per_token, 1), half), "sin")
    if codes.dtype not in (torch.uint8, torch.float8_e4m3fn) or tuple(codes.shape) != (M, N):
        raise ValueError(f"codes: expected uint8 or float8_e4m3fn of shape {(M, N)}")
    _expect(scales, torch.float32, (M, N // group_size if group_size > 0 else 0), "scales")
    args = (_ptr(x), _ptr(w), _ptr(cos), _ptr(sin), _ptr(y), _ptr(codes), _ptr(scales), M, N, 2 * half,
            rows_per_token, group_size, eps, fp8_max, _dtype_code(x), _stream(x, stream))
    return _launcher(lib.rnq_rmsnorm_rope_fp8_grouped, args, x, w, cos, sin, y, codes, scales)


# ------------------------------------------------------- allocating wrappers


def qk_norm_rope_fp8(q, k, wq, wk, cos, sin, *, positions=None, eps=1e-6, fp8_max=448.0, return_y=False):
    """Returns (q8, k8, q_scale, k_scale[, q_y, k_y]); codes as torch.float8_e4m3fn.

    q / k may be [T, H, D] views with contiguous rows inside a token (slices of a
    fused QKV output); with int32 ``positions`` [T], cos/sin are a [table_rows, R/2]
    table indexed by position."""
    torch = _torch()
    T, Hq, D = q.shape
    Hk = 0 if k is None else k.shape[1]
    dev = q.device
    q8 = torch.empty((T, Hq, D), dtype=torch.uint8, device=dev)
    k8 = torch.empty((T, Hk, D), dtype=torch.uint8, device=dev)
    qs = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    ks = torch.empty((T, Hk), dtype=torch.float32, device=dev)
    qy = torch.empty((T, Hq, D), dtype=q.dtype, device=dev) if return_y else None
    ky = (torch.empty((T, Hk, D), dtype=q.dtype, device=dev) if k is not None else None) if return_y else None
    contiguous = q.is_contiguous() and (k is None or k.is_contiguous())
    if contiguous and positions is None:
        rnq_qk_norm_rope_fp8(q, k, wq, wk, cos, sin, q8, k8 if Hk else None, qs, ks if Hk else None, qy, ky,
                             eps=eps, fp8_max=fp8_max)
    else:
        rnq_qk_norm_rope_fp8_ex(q, k, wq, wk, cos, sin, q8, k8 if Hk else None, qs, ks if Hk else None, qy, ky,
                                positions=positions, eps=eps, fp8_max=fp8_max)
    out = (q8.view(torch.float8_e4m3fn), k8.view(torch.float8_e4m3fn), qs, ks)
    return out + (qy, ky) if return_y else out


def rmsnorm(x, w, *, eps=1e-6, return_rstd=False):
    torch = _torch()
    y = torch.empty_like(x)
    rstd = torch.empty((x.shape[0],), dtype=torch.float32, device=x.device) if return_rstd else None
    rnq_rmsnorm_fwd(x, w, y, rstd, eps=eps)
    return (y, rstd) if return_rstd else y


def rmsnorm_bwd(x, w, grad_y, rstd=None, *, eps=1e-6):
    """Returns (grad_x, grad_w fp32)."""
    torch = _torch()
    M, N = x.shape
    gx = torch.empty_like(x)
    gw = torch.empty((N,), dtype=torch.float32, device=x.device)
    ws = torch.empty((max(rnq_rmsnorm_bwd_workspace_size(M, N), 16) // 4,), dtype=torch.float32, device=x.device)
    rnq_rmsnorm_bwd(x, w, grad_y, gx, gw, ws, rstd, eps=eps)
    return gx, gw


def rmsnorm_rope_bwd(x, w, grad_y, cos, sin, rstd=None, *, rows_per_token=1, eps=1e-6):
    """Returns (grad_x, grad_w fp32) of rmsnorm_rope."""
    torch = _torch()
    M, N = x.shape
    gx = torch.empty_like(x)
    gw = torch.empty((N,), dtype=torch.float32, device=x.device)
    ws = torch.empty((max(rnq_rmsnorm_bwd_workspace_size(M, N), 16) // 4,), dtype=torch.float32, device=x.device)
    rnq_rmsnorm_rope_bwd(x, w, grad_y, cos, sin, gx, gw, ws, rstd, rows_per_token=rows_per_token, eps=eps)
    return gx, gw


def rmsnorm_rope(x, w, cos, sin, *, rows_per_token=1, positions=None, eps=1e-6):
    """y [M, N] (contiguous); x may be a strided view, cos/sin gathered through ``positions``."""
    torch = _torch()
    if x.is_contiguous() and x.dim() == 2 and positions is None:
        y = torch.empty_like(x)
        rnq_rmsnorm_rope(x, w, cos, sin, y, rows_per_token=rows_per_token, eps=eps)
        return y
    N = x.shape[-1]
    y = torch.empty((x.numel() // N, N), dtype=x.dtype, device=x.device)
    rnq_rmsnorm_rope_ex(x, w, cos, sin, y, positions=positions, rows_per_token=rows_per_token, eps=eps)
    return y


def rmsnorm_rope_fp8_grouped(x, w, cos, sin, *, group_size=128, rows_per_token=1, eps=1e-6, fp8_max=448.0,
                             return_y=False):
    """Returns (codes as torch.float8_e4m3fn [M, N], scales [M, N / group_size][, y])."""
    torch = _torch()
    M, N = x.shape
    codes = torch.empty((M, N), dtype=torch.uint8, device=x.device)
    scales = torch.empty((M, N // group_size), dtype=torch.float32, device=x.device)
    y = torch.empty_like(x) if return_y else None
    rnq_rmsnorm_rope_fp8_grouped(x, w, cos, sin, codes, scales, y, group_size=group_size,
                                 rows_per_token=rows_per_token, eps=eps, fp8_max=fp8_max)
    out = (codes.view(torch.float8_e4m3fn), scales)
    return out + (y,) if return_y else out
