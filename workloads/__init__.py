"""Seeded synthetic inputs for the RMSNorm -> partial NeoX RoPE -> FP8 prologue.

This module is shared by the HIP path (tests, bench) and by the CPU oracle. It
holds no arithmetic of the method itself: it only draws random numbers, rounds
them to the input dtype, and builds the cos/sin table that the method takes as
an input. Everything is generated on the host with ``torch.Generator("cpu")``
so that both sides see identical bytes.

Workloads (sizes follow the tutorial pages' problem statement: rows ``[M, N]``
where M = tokens x heads, weight ``[N]``, cos/sin ``[tokens, rope_dim/2]``):

* ``qk_small``   - 256 rows x 128, rope 64, bf16, one cos/sin row per row (pos = row)
* ``rmsnorm_4k`` - 4096 x 4096 bf16, RMSNorm forward and backward
* ``norm_rope_fp16`` - 16384 rows x 128, rope 64, fp16 x = 2*N(0,1), random positions
* ``qk_4k``      - 4096 tokens x (32 q + 8 kv) heads x 128, full rope, 1% outliers x20
* ``qk_64k``     - 65536 tokens x (64 q + 8 kv) heads x 128, full rope, theta = 1e6
* ``grouped_small`` - 256 rows x 4096, rope 128, fp16, one scale per 128 elements
  (the shape of the fusion page's own check of its per-group kernel)
* ``grouped_4k`` - 4096 rows x 4096, rope 128, bf16, one scale per 128 elements, y written
* ``qk_4k_fused`` - ``qk_4k``'s shapes read from a fused QKV projection output
  [4096, (32 + 2*8) * 128] (q and k are strided views), cos/sin gathered through
  positions (8 packed sequences, positions restart at 0 in each) from a
  [4096, 64] table
* ``norm_rope_pos`` - ``norm_rope_fp16``'s shapes with cos/sin gathered through
  the random positions from a [8192, 32] table instead of one table row per row
* ``nrq_4k`` - the chapter 13 ledger page's norm+rope+quant plan size: 4096 x 4096
  bf16, rope 128, one FP8 scale per row (fused, or as three kernels)
* ``norm_rope_4k`` - RMSNorm + partial RoPE (no quant) on rows wider than a head:
  4096 x 4096 bf16, rope 128, one cos/sin row per row (pos = row)
"""

from __future__ import annotations

import dataclasses
import hashlib

import numpy as np
import torch

__all__ = [
    "WORKLOADS",
    "Workload",
    "generate",
    "rope_table",
    "bits",
    "sha256",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "qk" (norm+rope+fp8), "norm_rope", "rmsnorm", "grouped" (norm+rope+per-group fp8)
    seed: int
    tokens: int = 0
    q_heads: int = 0
    kv_heads: int = 0
    head_dim: int = 0
    rope_dim: int = 0
    rows: int = 0  # for rmsnorm / norm_rope: M
    width: int = 0  # for rmsnorm / norm_rope: N
    dtype: str = "bf16"
    theta: float = 10000.0
    eps: float = 1e-6
    fp8_max: float = 448.0
    outlier_p: float = 0.0
    outlier_mul: float = 20.0
    write_y: bool = False
    x_std: float = 1.0
    positions: str = "index"  # "index" (pos = token/row index) or "random:<hi>"
    group_size: int = 0  # grouped: elements per scale
    cache_rows: int = 0  # > 0: cos/sin are a [cache_rows, R/2] table indexed through positions
    fused_qkv: bool = False  # qk: q and k are views into one [T, (Hq + 2 Hk) * D] buffer
    description: str = ""


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(
            "qk_small", "qk", seed=1001, tokens=256, q_heads=1, kv_heads=0, head_dim=128,
            rope_dim=64, write_y=True,
            description="fused RMSNorm + partial RoPE + FP8, 256 rows x 128, rope 64, bf16, y written",
        ),
        Workload(
            "rmsnorm_4k", "rmsnorm", seed=1002, rows=4096, width=4096,
            description="RMSNorm forward + backward, 4096 x 4096 bf16",
        ),
        Workload(
            "norm_rope_fp16", "norm_rope", seed=1003, rows=16384, width=128, rope_dim=64,
            dtype="fp16", x_std=2.0, positions="random:8192",
            description="RMSNorm + partial RoPE (no quant), 16384 x 128, rope 64, fp16",
        ),
        Workload(
            "qk_4k", "qk", seed=1004, tokens=4096, q_heads=32, kv_heads=8, head_dim=128,
            rope_dim=128, outlier_p=0.01,
            description="QK-norm + RoPE + FP8, 4096 tokens x (32+8) heads x 128, bf16",
        ),
        Workload(
            "qk_64k", "qk", seed=1005, tokens=65536, q_heads=64, kv_heads=8, head_dim=128,
            rope_dim=128, theta=1e6,
            description="QK-norm + RoPE + FP8, 65536 tokens x (64+8) heads x 128, bf16, theta 1e6",
        ),
        Workload(
            "grouped_small", "grouped", seed=1006, rows=256, width=4096, rope_dim=128, dtype="fp16",
            group_size=128, write_y=True,
            description="RMSNorm + RoPE + per-group FP8, 256 x 4096, rope 128, fp16, groups of 128",
        ),
        Workload(
            "grouped_4k", "grouped", seed=1007, rows=4096, width=4096, rope_dim=128, group_size=128,
            write_y=True,
            description="RMSNorm + RoPE + per-group FP8, 4096 x 4096, rope 128, bf16, groups of 128, y written",
        ),
        Workload(
            "qk_4k_fused", "qk", seed=1008, tokens=4096, q_heads=32, kv_heads=8, head_dim=128,
            rope_dim=128, outlier_p=0.01, positions="segments:8", cache_rows=4096, fused_qkv=True,
            description="QK-norm + RoPE + FP8 on q/k views of a fused QKV output, 4096 tokens x (32+8) heads "
                        "x 128, positions of 8 packed sequences into a 4096-row cos/sin table",
        ),
        Workload(
            "nrq_4k", "grouped", seed=1010, rows=4096, width=4096, rope_dim=128, group_size=4096,
            description="RMSNorm + RoPE + per-row FP8 on 4096 x 4096 bf16 rows, rope 128 (the ledger page's plan)",
        ),
        Workload(
            "norm_rope_4k", "norm_rope", seed=1011, rows=4096, width=4096, rope_dim=128,
            description="RMSNorm + partial RoPE (no quant), 4096 x 4096 bf16 rows, rope 128",
        ),
        Workload(
            "norm_rope_pos", "norm_rope", seed=1009, rows=16384, width=128, rope_dim=64,
            dtype="fp16", x_std=2.0, positions="random:8192", cache_rows=8192,
            description="RMSNorm + partial RoPE, 16384 x 128, rope 64, fp16, cos/sin gathered by position "
                        "from an 8192-row table",
        ),
    ]
}

_TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def rope_table(positions: np.ndarray, rope_dim: int, theta: float) -> tuple[np.ndarray, np.ndarray]:
    """cos/sin tables ``[len(positions), rope_dim/2]`` fp32.

    The pages take cos/sin as inputs and do not say how they are made; the
    usual NeoX convention is used: frequency i is theta^(-2i/rope_dim), the
    angle is position x frequency. Angles and cos/sin are evaluated in fp64
    and rounded to fp32 once.
    """
    half = rope_dim // 2
    pos = np.asarray(positions, dtype=np.float64)
    if half == 0:
        z = np.zeros((pos.shape[0], 0), dtype=np.float32)
        return z, z.copy()
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / rope_dim)
    ang = pos[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _positions(spec: str, n: int, g: torch.Generator) -> np.ndarray:
    if spec == "index":
        return np.arange(n, dtype=np.int64)
    kind, arg = spec.split(":")
    if kind == "random":
        return torch.randint(0, int(arg), (n,), generator=g).numpy().astype(np.int64)
    assert kind == "segments"
    # int(arg) packed sequences of random lengths; positions restart at 0 in each
    cuts = np.sort(torch.randperm(max(n - 1, 1), generator=g)[: int(arg) - 1].numpy() + 1) if n > 1 else []
    starts = np.concatenate([[0], cuts]).astype(np.int64)
    idx = np.arange(n, dtype=np.int64)
    return idx - starts[np.searchsorted(starts, idx, side="right") - 1]


def _tables(wl: "Workload", pos: np.ndarray, out: dict) -> None:
    """cos/sin per token, or a position-indexed table plus the int32 positions."""
    if wl.cache_rows:
        cos, sin = rope_table(np.arange(wl.cache_rows), wl.rope_dim, wl.theta)
        out["positions"] = torch.from_numpy(pos.astype(np.int32))
    else:
        cos, sin = rope_table(pos, wl.rope_dim, wl.theta)
    out["cos"], out["sin"] = torch.from_numpy(cos), torch.from_numpy(sin)


def _normal(shape, g, std=1.0):
    return torch.randn(*shape, generator=g, dtype=torch.float32) * std


def _with_outliers(x: torch.Tensor, g: torch.Generator, p: float, mul: float) -> torch.Tensor:
    if p <= 0:
        return x
    mask = torch.rand(x.shape, generator=g) < p
    return torch.where(mask, x * mul, x)


def generate(name_or_wl, *, tokens: int | None = None, seed: int | None = None) -> dict:
    """Build the inputs of a workload on the host.

    ``tokens`` (qk) or rows (others) may be overridden to build a smaller
    instance of the same recipe. Returned tensors are CPU tensors in the
    workload dtype; cos/sin are fp32 numpy arrays wrapped as tensors.
    """
    wl = WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    g = torch.Generator("cpu").manual_seed(wl.seed if seed is None else seed)
    dt = _TORCH_DT[wl.dtype]
    out: dict = {"workload": wl}
    if wl.kind == "qk":
        T = wl.tokens if tokens is None else tokens
        D, Hq, Hk = wl.head_dim, wl.q_heads, wl.kv_heads
        q = _with_outliers(_normal((T, Hq, D), g, wl.x_std), g, wl.outlier_p, wl.outlier_mul)
        k = _with_outliers(_normal((T, Hk, D), g, wl.x_std), g, wl.outlier_p, wl.outlier_mul)
        wq = 1.0 + 0.1 * _normal((D,), g)
        wk = 1.0 + 0.1 * _normal((D,), g)
        pos = _positions(wl.positions, T, g)
        _tables(wl, pos, out)
        out.update(
            q=q.to(dt), k=k.to(dt), wq=wq.to(dt), wk=wk.to(dt),
            tokens=T, q_heads=Hq, kv_heads=Hk, head_dim=D, rope_dim=wl.rope_dim,
        )
        if wl.fused_qkv:
            # [T, (Hq + 2 Hk) * D]: q heads, k heads, then v heads (v is not read)
            v = _normal((T, Hk, D), g)
            out["qkv"] = torch.cat([out["q"].reshape(T, -1), out["k"].reshape(T, -1), v.to(dt).reshape(T, -1)], 1)
    elif wl.kind in ("norm_rope", "grouped"):
        M = wl.rows if tokens is None else tokens
        N = wl.width
        x = _normal((M, N), g, wl.x_std)
        w = 1.0 + 0.1 * _normal((N,), g)
        pos = _positions(wl.positions, M, g)
        _tables(wl, pos, out)
        out.update(
            x=x.to(dt), w=w.to(dt),
            rows=M, width=N, rope_dim=wl.rope_dim, rows_per_token=1, group_size=wl.group_size,
        )
    elif wl.kind == "rmsnorm":
        M = wl.rows if tokens is None else tokens
        N = wl.width
        x = _normal((M, N), g, wl.x_std)
        w = _normal((N,), g)
        gy = _normal((M, N), g)
        out.update(x=x.to(dt), w=w.to(dt), grad_y=gy.to(dt), rows=M, width=N)
    else:  # pragma: no cover
        raise ValueError(wl.kind)
    return out


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a 16-bit float tensor as uint16 (a reinterpretation, no rounding)."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def sha256(t) -> str:
    a = t if isinstance(t, np.ndarray) else bits(t)
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
