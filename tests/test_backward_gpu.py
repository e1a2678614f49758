"""GPU parity of the backward paths against the CPU oracle: the narrow-row
RMSNorm backward, the RoPE backward (rnq_rmsnorm_rope_bwd), and the autograd
Functions built on them.

Bar (the backward's tolerance): |a - b| <= 2e-2 * (|b| + rms of b's row) for
grad_x, the same with the rms over all columns for grad_w; grad_w is
bitwise reproducible from call to call.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_quant_amd as rnq
import oracle
import workloads
from fp8_quant_amd import autograd as rag
from oracle import codecs

from _parity import gpu

pytestmark = pytest.mark.gpu

DT = {torch.bfloat16: "bf16", torch.float16: "fp16"}


def _close(name, x_dt, gx, gw, ref_dx, ref_dw):
    dx = codecs.dtype_to_f32(workloads.bits(gx), DT[x_dt]).astype(np.float64)
    dw = gw.detach().float().cpu().numpy().astype(np.float64)
    row_rms = np.sqrt((ref_dx**2).mean(axis=1, keepdims=True))
    err = np.abs(dx - ref_dx) / (np.abs(ref_dx) + row_rms)
    errw = np.abs(dw - ref_dw) / (np.abs(ref_dw) + np.sqrt((ref_dw**2).mean()))
    print(f"[bwd] {name}: max rel err dx {err.max():.3g} dw {errw.max():.3g}", flush=True)
    assert err.max() <= 2e-2, f"{name}: dx rel err {err.max():.3g}"
    assert errw.max() <= 2e-2, f"{name}: dw rel err {errw.max():.3g}"


def _case(M, N, R, seed, dtype=torch.bfloat16, rows_per_token=1, std=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    x = (std * torch.randn(M, N, generator=g)).to(dtype)
    w = (1 + 0.1 * torch.randn(N, generator=g)).to(dtype)
    gy = torch.randn(M, N, generator=g).to(dtype)
    cos, sin = workloads.rope_table(np.arange(M // rows_per_token) * 7 % 8192, R, 10000.0)
    return x, w, gy, torch.from_numpy(cos), torch.from_numpy(sin)


def _rope_bwd(name, x, w, gy, cos, sin, rows_per_token=1, rstd=None):
    print(f"[bwd] {name}: x{tuple(x.shape)} rope {2 * cos.shape[-1]} rows_per_token {rows_per_token}", flush=True)
    gx, gw = rnq.rmsnorm_rope_bwd(gpu(x), gpu(w), gpu(gy), gpu(cos), gpu(sin), None if rstd is None else gpu(rstd),
                                  rows_per_token=rows_per_token)
    torch.cuda.synchronize()
    ref_dx, ref_dw, _ = oracle.rmsnorm_rope_bwd(workloads.bits(x), workloads.bits(w), workloads.bits(gy),
                                                cos.numpy(), sin.numpy(), 1e-6, DT[x.dtype], rows_per_token)
    _close(name, x.dtype, gx, gw, ref_dx, ref_dw)
    return gx, gw


# ---------------------------------------------------------- rnq_rmsnorm_rope_bwd


@pytest.mark.parametrize("M,N,R,dtype", [
    (1, 64, 16, torch.bfloat16), (7, 64, 64, torch.bfloat16), (100, 128, 64, torch.bfloat16),
    (1000, 128, 128, torch.float16), (333, 256, 96, torch.bfloat16), (65, 512, 512, torch.bfloat16),
    (64, 512, 128, torch.float16), (300, 128, 0, torch.bfloat16),
])
def test_rope_bwd_shapes(M, N, R, dtype):
    x, w, gy, cos, sin = _case(M, N, R, seed=M * 13 + N + R, dtype=dtype)
    _rope_bwd(f"M{M} N{N} R{R} {DT[dtype]}", x, w, gy, cos, sin)


def test_rope_bwd_norm_rope_fp16_size_and_determinism():
    """The 16384 x 128 fp16 RMSNorm+RoPE workload's shape (rope 64, one table row per row)."""
    d = workloads.generate("norm_rope_fp16")
    g = torch.Generator("cpu").manual_seed(91)
    gy = torch.randn(d["x"].shape, generator=g).to(d["x"].dtype)
    gx, gw = _rope_bwd("norm_rope_fp16 bwd", d["x"], d["w"], gy, d["cos"], d["sin"], d["rows_per_token"])
    gx2, gw2 = rnq.rmsnorm_rope_bwd(gpu(d["x"]), gpu(d["w"]), gpu(gy), gpu(d["cos"]), gpu(d["sin"]),
                                    rows_per_token=d["rows_per_token"])
    torch.cuda.synchronize()
    assert torch.equal(gx2.cpu(), gx.cpu()) and torch.equal(gw2.view(torch.int32).cpu(), gw.view(torch.int32).cpu())


def test_rope_bwd_shared_table_rows_and_saved_rstd():
    T, H, N, R = 96, 8, 128, 128
    x, w, gy, cos, sin = _case(T * H, N, R, seed=92, rows_per_token=H)
    gx, gw = _rope_bwd("rows_per_token 8", x, w, gy, cos, sin, rows_per_token=H)
    _, rstd = rnq.rmsnorm(gpu(x), gpu(w), return_rstd=True)
    gx2, gw2 = rnq.rmsnorm_rope_bwd(gpu(x), gpu(w), gpu(gy), gpu(cos), gpu(sin), rstd, rows_per_token=H)
    torch.cuda.synchronize()
    # the saved rstd equals the recomputed one, so the results are identical
    assert torch.equal(gx2.cpu(), gx.cpu()) and torch.equal(gw2.view(torch.int32).cpu(), gw.view(torch.int32).cpu())


def test_rope_bwd_zero_rope_equals_rmsnorm_bwd():
    x, w, gy, cos, sin = _case(500, 256, 0, seed=93)
    a = rnq.rmsnorm_rope_bwd(gpu(x), gpu(w), gpu(gy), None, None)
    b = rnq.rmsnorm_bwd(gpu(x), gpu(w), gpu(gy))
    torch.cuda.synchronize()
    assert torch.equal(a[0].cpu(), b[0].cpu()) and torch.equal(a[1].view(torch.int32).cpu(), b[1].view(torch.int32).cpu())


def test_rope_bwd_identity_table_equals_rmsnorm_bwd():
    x, w, gy, cos, sin = _case(200, 128, 64, seed=94)
    one, zero = torch.ones_like(cos), torch.zeros_like(sin)
    a = rnq.rmsnorm_rope_bwd(gpu(x), gpu(w), gpu(gy), gpu(one), gpu(zero))
    b = rnq.rmsnorm_bwd(gpu(x), gpu(w), gpu(gy))
    torch.cuda.synchronize()
    assert torch.equal(a[0].cpu(), b[0].cpu()) and torch.equal(a[1].view(torch.int32).cpu(), b[1].view(torch.int32).cpu())


@pytest.mark.parametrize("M,N", [(16384, 128), (3, 64), (4099, 256), (20000, 512)])
def test_narrow_rmsnorm_bwd(M, N):
    x, w, gy, _, _ = _case(M, N, 0, seed=M + N, dtype=torch.float16 if N == 128 else torch.bfloat16)
    print(f"[bwd] narrow rmsnorm bwd M{M} N{N}", flush=True)
    gx, gw = rnq.rmsnorm_bwd(gpu(x), gpu(w), gpu(gy))
    torch.cuda.synchronize()
    ref_dx, ref_dw, _ = oracle.rmsnorm_bwd(workloads.bits(x), workloads.bits(w), workloads.bits(gy), 1e-6, DT[x.dtype])
    _close(f"narrow M{M} N{N}", x.dtype, gx, gw, ref_dx, ref_dw)


def test_rope_bwd_invalid_arguments_raise():
    x, w, gy, cos, sin = _case(8, 4096, 2048, seed=95)
    print("[bwd] invalid arguments", flush=True)
    with pytest.raises(rnq.RnqError, match="UNSUPPORTED"):  # tails above 1024 columns only on rows of 64..512
        rnq.rmsnorm_rope_bwd(gpu(x), gpu(w), gpu(gy), gpu(cos), gpu(sin))
    x, w, gy, cos, sin = _case(8, 128, 64, seed=96, rows_per_token=4)
    with pytest.raises(rnq.RnqError, match="SHAPE"):  # 6 rows over a 2-row table at 4 rows per token
        rnq.rmsnorm_rope_bwd(gpu(x[:6]), gpu(w), gpu(gy[:6]), gpu(cos[:1]), gpu(sin[:1]), rows_per_token=4)


# ------------------------------------------------------------------ autograd


def test_autograd_rmsnorm_matches_oracle_and_forward():
    g = torch.Generator("cpu").manual_seed(97)
    x = torch.randn(4, 256, 1024, generator=g).to(torch.bfloat16)
    w = (1 + 0.1 * torch.randn(1024, generator=g)).to(torch.bfloat16)
    gy = torch.randn(4, 256, 1024, generator=g).to(torch.bfloat16)
    print("[bwd] autograd rmsnorm [4, 256, 1024]", flush=True)
    xg = gpu(x).requires_grad_(True)
    wg = gpu(w).requires_grad_(True)
    y = rag.rmsnorm(xg, wg)
    y.backward(gpu(gy))
    torch.cuda.synchronize()
    assert y.shape == x.shape and xg.grad.shape == x.shape and wg.grad.dtype == torch.bfloat16
    assert torch.equal(y.detach().cpu(), rnq.rmsnorm(gpu(x.view(-1, 1024)), gpu(w)).view(x.shape).cpu())
    ref_dx, ref_dw, _ = oracle.rmsnorm_bwd(workloads.bits(x.view(-1, 1024)), workloads.bits(w),
                                           workloads.bits(gy.view(-1, 1024)), 1e-6)
    # grad_w is cast to the weight dtype (bf16): one more rounding, inside the tolerance
    _close("autograd rmsnorm", torch.bfloat16, xg.grad.view(-1, 1024), wg.grad, ref_dx, ref_dw)


def test_autograd_rmsnorm_rope_qk_layout():
    """x [T, H, D] with a per-token table: rows_per_token = H by default."""
    T, H, D, R = 64, 8, 128, 128
    x, w, gy, cos, sin = _case(T * H, D, R, seed=98, rows_per_token=H)
    print("[bwd] autograd rmsnorm_rope [64, 8, 128]", flush=True)
    xg = gpu(x.view(T, H, D)).requires_grad_(True)
    wg = gpu(w).requires_grad_(True)
    y = rag.rmsnorm_rope(xg, wg, gpu(cos), gpu(sin))
    (y.float() * gpu(gy.view(T, H, D)).float()).sum().backward()
    torch.cuda.synchronize()
    y_ref = rnq.rmsnorm_rope(gpu(x), gpu(w), gpu(cos), gpu(sin), rows_per_token=H)
    assert torch.equal(y.detach().view(T * H, D).cpu(), y_ref.cpu())
    ref_dx, ref_dw, _ = oracle.rmsnorm_rope_bwd(workloads.bits(x), workloads.bits(w), workloads.bits(gy),
                                                cos.numpy(), sin.numpy(), 1e-6, "bf16", H)
    _close("autograd rmsnorm_rope", torch.bfloat16, xg.grad.view(T * H, D), wg.grad, ref_dx, ref_dw)


def test_autograd_only_weight_grad():
    x, w, gy, cos, sin = _case(32, 64, 32, seed=99)
    wg = gpu(w).requires_grad_(True)
    y = rag.rmsnorm_rope(gpu(x), wg, gpu(cos), gpu(sin))
    y.backward(gpu(gy))
    torch.cuda.synchronize()
    _, ref_dw, _ = oracle.rmsnorm_rope_bwd(workloads.bits(x), workloads.bits(w), workloads.bits(gy),
                                           cos.numpy(), sin.numpy(), 1e-6, "bf16", 1)
    dw = wg.grad.float().cpu().numpy()
    assert np.abs(dw - ref_dw).max() <= 2e-2 * (np.abs(ref_dw).max() + 1e-30)


# ------------------------------- rows of 1024, 2048 and 4096: one wave per row

ROW = [
    # M, N, R, dtype, rows_per_token, saved rstd
    (1, 1024, 0, torch.bfloat16, 1, False),    # one row: one wave of one block
    (9, 1024, 16, torch.float16, 1, True),     # the narrowest tail
    (300, 2048, 64, torch.bfloat16, 3, False),
    (1000, 2048, 0, torch.float16, 1, True),   # 4 rows per block: waves 4..7 without a row
    (777, 4096, 256, torch.float16, 1, False),
    (2100, 4096, 512, torch.bfloat16, 7, True),  # the widest tail these rows take (every lane of the last slot)
    (4096, 1024, 128, torch.bfloat16, 8, False),
]


@pytest.mark.parametrize("M,N,R,dtype,rpt,saved", ROW, ids=[f"{m}x{n}r{r}" for m, n, r, _, _, _ in ROW])
def test_row_bwd_shapes(M, N, R, dtype, rpt, saved):
    """Rows of 1024, 2048 and 4096 elements with tails up to 512 columns go
    through the wave-per-row backward: ragged row counts leave the waves of a
    block with no row, one row or several; saved and recomputed rstd."""
    x, w, gy, cos, sin = _case(M, N, R, seed=5 * M + N + R, dtype=dtype, rows_per_token=rpt)
    rstd = rnq.rmsnorm(gpu(x), gpu(w), return_rstd=True)[1] if saved else None
    _rope_bwd(f"row bwd M{M} N{N} R{R} {DT[dtype]} saved {saved}", x, w, gy, cos, sin, rpt, rstd)


# ------------------------------------------- grad_w: every row counted exactly once

EDGE = [
    # M, N, R, dtype, rows_per_token
    (4096, 4096, 0, torch.bfloat16, 1),     # wide rows: 256 blocks of 16 rows
    (4100, 2048, 0, torch.bfloat16, 1),     # ragged: 242 blocks of 17 rows, the last one of 3
    (16384, 128, 0, torch.float16, 1),      # narrow rows: 256 blocks of 64
    (16384, 128, 64, torch.float16, 1),     # narrow rows through the RoPE backward: 256 blocks of 64
    (2048, 4096, 128, torch.bfloat16, 2),   # wide rows through the RoPE backward: 256 blocks of 8
    (3000, 4096, 512, torch.bfloat16, 3),   # 250 blocks of 12: waves 0..3 take two rows, 4..7 one
    (2000, 8192, 128, torch.bfloat16, 1),   # workgroup-per-row RoPE backward: 500 blocks of 4
    (20000, 256, 0, torch.bfloat16, 1),     # 254 blocks of 79, the last one of 13
]


@pytest.mark.parametrize("M,N,R,dtype,rpt", EDGE, ids=[f"{m}x{n}r{r}" for m, n, r, _, _ in EDGE])
def test_grad_w_counts_block_edge_rows_once(M, N, R, dtype, rpt):
    """grad_y is nonzero only on the first and last rows of a few of the fixed
    row blocks (the first, one in the middle, the last) and on row M - 1: a row
    dropped from, or counted twice in, the block partition or the fixed-order
    reduction moves a column of grad_w by a whole row's gy * xn, which the
    per-column bound 1e-4 * sum over rows of |gy * xn| catches (the 2e-2 rule
    of the full-size tests cannot see one row out of thousands)."""
    # the partition: about 256 blocks, or 512 for the RoPE backward up to 8192
    # rows when it runs a workgroup per row (rows other than 64..512, 1024,
    # 2048 and 4096 wide, or tails above 512 columns)
    wave_per_row = N in (1024, 2048, 4096) and R <= 512
    target = 512 if (R and M <= 8192 and not wave_per_row) else 256
    rpb = -(-M // target)
    blocks = -(-M // rpb)
    picks = sorted({r for b in (0, blocks // 2, blocks - 1) for r in (b * rpb, min(b * rpb + rpb, M) - 1)} | {M - 1})
    print(f"[bwd] grad_w edge rows M{M} N{N} R{R}: {blocks} blocks of {rpb}, rows {picks}", flush=True)
    x, w, gy, cos, sin = _case(M, N, R, seed=M + N + R, dtype=dtype, rows_per_token=rpt)
    mask = torch.zeros(M, 1, dtype=torch.bool)
    mask[picks] = True
    gy = torch.where(mask, gy, torch.zeros_like(gy))
    if R:
        _, gw = rnq.rmsnorm_rope_bwd(gpu(x), gpu(w), gpu(gy), gpu(cos), gpu(sin), rows_per_token=rpt)
    else:
        _, gw = rnq.rmsnorm_bwd(gpu(x), gpu(w), gpu(gy))
    torch.cuda.synchronize()
    xb, wb, gb = workloads.bits(x), workloads.bits(w), workloads.bits(gy)
    dt = DT[dtype]
    ref_dx, ref_dw, rstd = oracle.rmsnorm_rope_bwd(xb, wb, gb, cos.numpy(), sin.numpy(), 1e-6, dt, rpt)
    # sum over rows of |gn * xn| per column (gn: grad_y through the transposed rotation)
    xn = codecs.dtype_to_f32(xb, dt).astype(np.float64) * rstd[:, None]
    t = np.arange(M) // rpt
    gn = oracle.rope_bwd_rotate(codecs.dtype_to_f32(gb, dt).astype(np.float64), cos.numpy()[t], sin.numpy()[t])
    mag = np.abs(gn * xn).sum(axis=0)
    err = np.abs(gw.cpu().numpy().astype(np.float64) - ref_dw)
    worst = (err / np.maximum(mag, 1e-30)).max()
    print(f"[bwd] grad_w edge rows: worst |dw - ref| / sum|gy xn| = {worst:.3g}", flush=True)
    assert np.all(err <= 1e-4 * mag + 1e-30)
