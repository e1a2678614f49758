"""The allocation-free backward (rnq_rmsnorm_rope_bwd_noalloc, through the C ABI)
against the workspace entry point it is a variant of (rnq_rmsnorm_rope_bwd):
the same kernels over the same row partition, so grad_x and grad_w must be
equal bit for bit. Each case makes two calls in a row, the second on a smaller
input: the static scratch keeps the first call's partial rows, and none of
them may reach the second call's grad_w. The smaller call is also checked
against the CPU oracle at the backward's tolerance.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_quant_amd as rnq
import oracle
import workloads
from oracle import codecs

pytestmark = pytest.mark.gpu

DT = {torch.bfloat16: "bf16", torch.float16: "fp16"}


def _inputs(M, N, R, seed, dtype, rows_per_token):
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(M, N, generator=g).to(dtype)
    w = (1 + 0.1 * torch.randn(N, generator=g)).to(dtype)
    gy = torch.randn(M, N, generator=g).to(dtype)
    cos, sin = workloads.rope_table(np.arange(M // rows_per_token) * 5 % 4096, R, 10000.0)
    return x, w, gy, torch.from_numpy(cos), torch.from_numpy(sin)


def _call_both(label, M, N, R, seed, dtype, rows_per_token=1, saved_rstd=False):
    print(f"[noalloc] {label}: M {M} N {N} rope {R} rows_per_token {rows_per_token} {dtype}", flush=True)
    x, w, gy, cos, sin = _inputs(M, N, R, seed, dtype, rows_per_token)
    dev = torch.device("cuda:0")
    xd, wd, gyd = x.to(dev), w.to(dev), gy.to(dev)
    cd, sd = (cos.to(dev), sin.to(dev)) if R else (None, None)
    rstd = None
    if saved_rstd:
        _, rstd = rnq.rmsnorm(xd, wd, return_rstd=True)
    ref_gx, ref_gw = rnq.rmsnorm_rope_bwd(xd, wd, gyd, cd, sd, rstd, rows_per_token=rows_per_token)
    gx = torch.empty_like(xd)
    gw = torch.full((N,), float("nan"), dtype=torch.float32, device=dev)
    rnq.rnq_rmsnorm_rope_bwd_noalloc(xd, wd, gyd, cd, sd, gx, gw, rstd, rows_per_token=rows_per_token)
    torch.cuda.synchronize()
    assert torch.equal(gx.view(torch.int16), ref_gx.view(torch.int16)), f"{label}: grad_x differs"
    assert torch.equal(gw.view(torch.int32), ref_gw.view(torch.int32)), f"{label}: grad_w differs"
    return x, w, gy, cos, sin, gx, gw


def _against_oracle(label, x, w, gy, cos, sin, gx, gw, rows_per_token):
    R = 2 * cos.shape[-1]
    ref_dx, ref_dw, _ = oracle.rmsnorm_rope_bwd(workloads.bits(x), workloads.bits(w), workloads.bits(gy),
                                                cos.numpy()[:, : R // 2], sin.numpy()[:, : R // 2], 1e-6,
                                                DT[x.dtype], rows_per_token)
    dx = codecs.dtype_to_f32(workloads.bits(gx), DT[x.dtype]).astype(np.float64)
    dw = gw.cpu().numpy().astype(np.float64)
    row_rms = np.sqrt((ref_dx**2).mean(axis=1, keepdims=True))
    err = (np.abs(dx - ref_dx) / (np.abs(ref_dx) + row_rms)).max()
    errw = (np.abs(dw - ref_dw) / (np.abs(ref_dw) + np.sqrt((ref_dw**2).mean()))).max()
    print(f"[noalloc] {label}: vs oracle dx {err:.3g} dw {errw:.3g}", flush=True)
    assert err <= 2e-2 and errw <= 2e-2


CASES = [
    # (first call), (second, smaller call)
    ("wide rows", (4096, 4096, 0, torch.bfloat16, 1, False), (1000, 2048, 0, torch.bfloat16, 1, False)),
    ("rope tail", (16384, 128, 64, torch.float16, 1, False), (520, 128, 64, torch.float16, 4, True)),
    # the RoPE backward's 512 blocks x 16384 fp32 partials: every byte of the static scratch
    ("full scratch", (8192, 16384, 128, torch.bfloat16, 1, True), (3, 64, 0, torch.bfloat16, 1, False)),
]


@pytest.mark.parametrize("label,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_the_workspace_entry_on_two_calls(label, first, second):
    M, N, R, dt, rpt, saved = first
    assert rnq.rnq_rmsnorm_bwd_workspace_size(M, N) <= rnq.RNQ_NOALLOC_SCRATCH_BYTES
    _call_both(label + " (first)", M, N, R, 31, dt, rpt, saved)
    M, N, R, dt, rpt, saved = second
    out = _call_both(label + " (second, smaller)", M, N, R, 32, dt, rpt, saved)
    _against_oracle(label + " (second, smaller)", *out, rows_per_token=rpt)


def test_noalloc_rejects_what_the_workspace_entry_rejects():
    dev = torch.device("cuda:0")
    x = torch.zeros(8, 16392, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(16392, dtype=torch.bfloat16, device=dev)
    gw = torch.zeros(16392, dtype=torch.float32, device=dev)
    with pytest.raises(rnq.RnqError) as e:
        rnq.rnq_rmsnorm_rope_bwd_noalloc(x, w, x, None, None, torch.empty_like(x), gw)
    assert e.value.status == 3  # wider than any row the backward takes
