"""Bindings of the measurement baselines (include/rnq_baselines.h): argument
marshalling only, as for the hot-path entry points."""

from __future__ import annotations

import ctypes

from . import _dtype_code, _expect, _launcher, _ptr, _stream, _torch, load_library

__all__ = [
    "prepare_norm_rope_quant_unfused",
    "prepare_qk_design",
    "norm_rope_quant_unfused",
    "qk_design",
    "prepare_stream",
]


def prepare_norm_rope_quant_unfused(x, w, cos, sin, normed, rotated, codes, scales, *, rows_per_token=1, eps=1e-6,
                                    fp8_max=448.0, stream=None):
    """RMSNorm -> RoPE -> per-row FP8 as three launches (intermediates in ``normed``, ``rotated``)."""
    torch = _torch()
    lib = load_library()
    M, N = x.shape
    half = 0 if cos is None else cos.shape[-1]
    _expect(w, x.dtype, (N,), "w")
    _expect(normed, x.dtype, (M, N), "normed")
    _expect(rotated, x.dtype, (M, N), "rotated")
    if cos is not None:
        _expect(cos, torch.float32, (M // max(rows_per_token, 1), half), "cos")
        _expect(sin, torch.float32, (M // max(rows_per_token, 1), half), "sin")
    if codes.dtype not in (torch.uint8, torch.float8_e4m3fn) or tuple(codes.shape) != (M, N):
        raise ValueError(f"codes: expected uint8 or float8_e4m3fn of shape {(M, N)}")
    _expect(scales, torch.float32, (M,), "scales")
    args = (_ptr(x), _ptr(w), _ptr(cos), _ptr(sin), _ptr(normed), _ptr(rotated), _ptr(codes), _ptr(scales), M, N,
            2 * half, rows_per_token, eps, fp8_max, _dtype_code(x), _stream(x, stream))
    return _launcher(lib.rnq_baseline_norm_rope_quant_unfused, args, x, w, cos, sin, normed, rotated, codes, scales)


def norm_rope_quant_unfused(x, w, cos, sin, *, rows_per_token=1, eps=1e-6, fp8_max=448.0):
    """Returns (codes as torch.float8_e4m3fn [M, N], scales [M])."""
    torch = _torch()
    M, N = x.shape
    normed, rotated = torch.empty_like(x), torch.empty_like(x)
    codes = torch.empty((M, N), dtype=torch.uint8, device=x.device)
    scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    prepare_norm_rope_quant_unfused(x, w, cos, sin, normed, rotated, codes, scales, rows_per_token=rows_per_token,
                                    eps=eps, fp8_max=fp8_max)()
    return codes.view(torch.float8_e4m3fn), scales


def prepare_qk_design(q, k, wq, wk, cos, sin, q_fp8, k_fp8, q_scale, k_scale, *, rows_per_block, eps=1e-6,
                      fp8_max=448.0, stream=None):
    """The chapter 28 design with ``rows_per_block`` rows per workgroup (A: 1, B: 8, C: all heads)."""
    torch = _torch()
    lib = load_library()
    T, Hq, D = q.shape
    Hk = 0 if k is None else k.shape[1]
    half = 0 if cos is None else cos.shape[-1]
    if k is not None:
        _expect(k, q.dtype, (T, Hk, D), "k")
    _expect(wq, q.dtype, (D,), "wq")
    _expect(wk, q.dtype, (D,), "wk")
    if cos is not None:
        _expect(cos, torch.float32, (T, half), "cos")
        _expect(sin, torch.float32, (T, half), "sin")
    _expect(q_scale, torch.float32, (T, Hq), "q_scale")
    _expect(k_scale, torch.float32, (T, Hk), "k_scale")
    args = (_ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(cos), _ptr(sin), _ptr(q_fp8), _ptr(k_fp8), _ptr(q_scale),
            _ptr(k_scale), T, Hq, Hk, D, 2 * half, rows_per_block, eps, fp8_max, _dtype_code(q), _stream(q, stream))
    return _launcher(lib.rnq_baseline_qk_design, args, q, k, wq, wk, cos, sin, q_fp8, k_fp8, q_scale, k_scale)


def qk_design(q, k, wq, wk, cos, sin, *, rows_per_block, eps=1e-6, fp8_max=448.0):
    """Returns (q8, k8, q_scale, k_scale) as qk_norm_rope_fp8 does."""
    torch = _torch()
    T, Hq, D = q.shape
    Hk = 0 if k is None else k.shape[1]
    dev = q.device
    q8 = torch.empty((T, Hq, D), dtype=torch.uint8, device=dev)
    k8 = torch.empty((T, Hk, D), dtype=torch.uint8, device=dev)
    qs = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    ks = torch.empty((T, Hk), dtype=torch.float32, device=dev)
    prepare_qk_design(q, k, wq, wk, cos, sin, q8, k8 if Hk else None, qs, ks if Hk else None,
                      rows_per_block=rows_per_block, eps=eps, fp8_max=fp8_max)()
    return q8.view(torch.float8_e4m3fn), k8.view(torch.float8_e4m3fn), qs, ks


def prepare_stream(src, dst=None, *, store_policy=0, stream=None):
    """The memory floor: reads all of ``src`` (its size a multiple of 2048 bytes) and
    writes half as many bytes to ``dst``, stored nontemporal (``store_policy`` 0) or
    with device scope (1); ``src=None`` gives a launch of one empty workgroup (the
    cost of a launch). Returns a zero-argument launcher."""
    lib = load_library()
    if src is None:
        s = stream if stream is not None else _torch().cuda.current_stream()
        return _launcher(lib.rnq_baseline_stream, (None, 0, None, ctypes.c_void_p(s.cuda_stream)))
    nbytes = src.numel() * src.element_size()
    if dst is None or dst.numel() * dst.element_size() < nbytes // 2:
        raise ValueError("dst must hold at least half of src's bytes")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous")
    return _launcher(lib.rnq_baseline_stream_policy,
                     (_ptr(src), nbytes, _ptr(dst), int(store_policy), _stream(src, stream)), src, dst)

