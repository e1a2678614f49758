"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare."""

from __future__ import annotations

import numpy as np
import torch

import fp8_quant_amd as rnq
import oracle
import workloads
from oracle import codecs

DT_NAME = {torch.bfloat16: "bf16", torch.float16: "fp16"}


def gpu(t):
    return None if t is None else t.contiguous().cuda()


def run_qk_gpu(d, *, eps=1e-6, fp8_max=448.0, with_y=False):
    """Run rnq_qk_norm_rope_fp8 on workload dict ``d`` (CPU tensors); returns numpy results."""
    q, k = gpu(d["q"]), gpu(d["k"]) if d["k"] is not None and d["k"].shape[1] else None
    T, Hq, D = d["q"].shape
    Hk = 0 if k is None else k.shape[1]
    dev = q.device
    q8 = torch.full((T, Hq, D), 0xAB, dtype=torch.uint8, device=dev)
    k8 = torch.full((T, Hk, D), 0xAB, dtype=torch.uint8, device=dev) if Hk else None
    qs = torch.full((T, Hq), float("nan"), dtype=torch.float32, device=dev)
    ks = torch.full((T, Hk), float("nan"), dtype=torch.float32, device=dev) if Hk else None
    qy = torch.empty_like(q) if with_y else None
    ky = torch.empty_like(k) if (with_y and k is not None) else None
    cos = gpu(d["cos"]) if d["cos"].shape[-1] else None
    sin = gpu(d["sin"]) if d["sin"].shape[-1] else None
    rnq.rnq_qk_norm_rope_fp8(q, k, gpu(d["wq"]), gpu(d["wk"]) if Hk else None, cos, sin,
                             q8, k8, qs, ks, qy, ky, eps=eps, fp8_max=fp8_max)
    torch.cuda.synchronize()
    out = {
        "q_codes": q8.cpu().numpy(), "q_scale": qs.cpu().numpy(),
        "k_codes": None if k8 is None else k8.cpu().numpy(),
        "k_scale": None if ks is None else ks.cpu().numpy(),
        "q_y": None if qy is None else workloads.bits(qy),
        "k_y": None if ky is None else workloads.bits(ky),
    }
    return out


def oracle_qk(d, *, eps=1e-6, fp8_max=448.0, tokens=None):
    dt = DT_NAME[d["q"].dtype]
    k = d["k"] if d["k"] is not None and d["k"].shape[1] else None
    return oracle.qk_norm_rope_fp8(
        workloads.bits(d["q"]), None if k is None else workloads.bits(k),
        workloads.bits(d["wq"]), None if k is None else workloads.bits(d["wk"]),
        d["cos"].numpy(), d["sin"].numpy(), eps=eps, fp8_max=fp8_max, dtype=dt, tokens=tokens,
    )


def unproven_rows(x_bits: np.ndarray, dtype: str) -> np.ndarray:
    """Rows whose fp64 sum of squares is not proven exact (there the kernel's own
    fp64 summation order could round differently; tolerances apply)."""
    x32 = codecs.dtype_to_f32(x_bits.reshape(-1, x_bits.shape[-1]), dtype)
    _, exact = oracle.sum_squares_exact_mask(x32)
    return ~exact


def ulp_distance_16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in representable steps between two arrays of bf16/fp16 bit patterns."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a) - ordered(b))


def code_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x80, -(x & 0x7F), x)
    return np.abs(ordered(a) - ordered(b))


def assert_rows_match(name, got_y, got_codes, got_scale, ref_y, ref_codes, ref_scale, loose_rows):
    """Bit-exact on every row the oracle proves exact; on the others the stated
    tolerances (|dy| <= 1 ulp, codes within 1 step, scale rel err <= 1e-6)."""
    D = (got_codes if got_codes is not None else got_y).shape[-1]
    loose = np.asarray(loose_rows).reshape(-1)
    strict = ~loose
    msgs = []
    if got_y is not None:
        gy, ry = got_y.reshape(-1, D), ref_y.reshape(-1, D)
        bad = (gy != ry).any(axis=1)
        if np.any(bad & strict):
            i = int(np.flatnonzero(bad & strict)[0])
            j = int(np.flatnonzero(gy[i] != ry[i])[0])
            msgs.append(f"{name}: y differs on {int((bad & strict).sum())} proven rows; first row {i} col {j}: "
                        f"gpu {gy[i, j]:#06x} oracle {ry[i, j]:#06x}")
        if np.any(loose):
            assert ulp_distance_16(gy[loose], ry[loose]).max(initial=0) <= 1, f"{name}: y beyond 1 ulp"
    if got_codes is not None:
        gc, rc = got_codes.reshape(-1, D), ref_codes.reshape(-1, D)
        gs, rs = got_scale.reshape(-1), ref_scale.reshape(-1)
        badc = (gc != rc).any(axis=1)
        if np.any(badc & strict):
            i = int(np.flatnonzero(badc & strict)[0])
            j = int(np.flatnonzero(gc[i] != rc[i])[0])
            msgs.append(f"{name}: codes differ on {int((badc & strict).sum())} proven rows; first row {i} col {j}: "
                        f"gpu {gc[i, j]:#04x} oracle {rc[i, j]:#04x} (scale gpu {gs[i]!r} oracle {rs[i]!r})")
        bads = gs.view(np.uint32) != rs.view(np.uint32)
        if np.any(bads & strict):
            i = int(np.flatnonzero(bads & strict)[0])
            msgs.append(f"{name}: scale differs on {int((bads & strict).sum())} proven rows; first row {i}: "
                        f"gpu {gs[i]!r} oracle {rs[i]!r}")
        if np.any(loose):
            assert code_distance(gc[loose], rc[loose]).max(initial=0) <= 1, f"{name}: code beyond 1 step"
            assert (code_distance(gc[loose], rc[loose]) > 0).mean() <= 1e-4, f"{name}: too many 1-step codes"
            np.testing.assert_allclose(gs[loose], rs[loose], rtol=1e-6, atol=0)
    assert not msgs, "\n".join(msgs)


def compare_qk(name, d, got, ref, dtype="bf16"):
    for part in ("q", "k"):
        if ref[part + "_codes"] is None:
            assert got[part + "_codes"] is None or got[part + "_codes"].size == 0
            continue
        x = workloads.bits(d[part])
        loose = unproven_rows(x, dtype)
        assert_rows_match(f"{name}/{part}", got[part + "_y"], got[part + "_codes"], got[part + "_scale"],
                          ref[part + "_y"] if got[part + "_y"] is not None else None,
                          ref[part + "_codes"], ref[part + "_scale"], loose)
