"""Path R (RMSNorm + partial NeoX RoPE, no quantisation: the chapter 13 fusion
page's rms_norm_rope_fused) and its backward on rows other than 64..512 wide
(up to 16384 elements, tails up to 1024 columns), against the CPU oracle.

Bars: y bit-exact on rows whose sum of squares the oracle proves exact (every
bf16 row here; most fp16 rows of 4096 are not provably exact in fp64, and the
stated tolerance applies to those); grad_x / grad_w within |a - b| <= 2e-2 (|b| + rms of b's row, or
of all of grad_w), and grad_w bitwise reproducible from call to call.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_quant_amd as rnq
import oracle
import workloads
from oracle import codecs

from _parity import assert_rows_match, gpu, unproven_rows

pytestmark = pytest.mark.gpu

DT = {torch.bfloat16: "bf16", torch.float16: "fp16"}


def _inputs(M, N, R, dtype, rows_per_token, seed, random_angles=False):
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(M, N, generator=g).to(dtype)
    w = (1 + 0.1 * torch.randn(N, generator=g)).to(dtype)
    T = M // rows_per_token
    if random_angles:
        # the fusion page's own check: one random angle per (row, pair)
        ang = np.random.default_rng(seed).uniform(-np.pi, np.pi, (T, R // 2))
        cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    else:
        cos, sin = workloads.rope_table(np.arange(T) * 7 % 8192, R, 10000.0)
    return x, w, torch.from_numpy(cos), torch.from_numpy(sin)


FWD = [
    # M, N, R, dtype, rows_per_token
    (256, 4096, 128, torch.float16, 1),    # the fusion page's check shape
    (4096, 4096, 128, torch.bfloat16, 1),  # the ledger page's plan size
    (300, 1000, 64, torch.bfloat16, 1),    # a width that is no power of two
    (96, 8192, 1024, torch.float16, 4),    # the widest tail, 4 rows per table row
    (17, 16384, 512, torch.bfloat16, 1),   # the widest rows
    (64, 24, 16, torch.bfloat16, 2),       # narrower than a head
    (33, 2048, 0, torch.bfloat16, 1),      # no tail: RMSNorm alone through the same kernel
]


@pytest.mark.parametrize("M,N,R,dtype,rpt", FWD, ids=[f"{m}x{n}r{r}" for m, n, r, _, _ in FWD])
def test_wide_rmsnorm_rope_matches_the_oracle(M, N, R, dtype, rpt):
    x, w, cos, sin = _inputs(M, N, R, dtype, rpt, M + N + R, random_angles=(M, N) == (256, 4096))
    print(f"[wide] rmsnorm_rope M{M} N{N} R{R} {DT[dtype]} rows_per_token {rpt}", flush=True)
    y = rnq.rmsnorm_rope(gpu(x), gpu(w), gpu(cos) if R else None, gpu(sin) if R else None, rows_per_token=rpt)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_rope(workloads.bits(x), workloads.bits(w), cos.numpy(), sin.numpy(), 1e-6, DT[dtype], rpt)
    loose = unproven_rows(workloads.bits(x), DT[dtype])
    assert_rows_match(f"wide rmsnorm_rope {M}x{N}", workloads.bits(y), None, None, ref, None, None, loose)


def test_norm_rope_4k_full_size():
    """The norm_rope_4k workload (4096 x 4096 bf16, rope 128), every row."""
    d = workloads.generate("norm_rope_4k")
    print(f"[wide] norm_rope_4k: x{tuple(d['x'].shape)}", flush=True)
    y = rnq.rmsnorm_rope(gpu(d["x"]), gpu(d["w"]), gpu(d["cos"]), gpu(d["sin"]))
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_rope(workloads.bits(d["x"]), workloads.bits(d["w"]), d["cos"].numpy(), d["sin"].numpy())
    loose = unproven_rows(workloads.bits(d["x"]), "bf16")
    assert_rows_match("norm_rope_4k", workloads.bits(y), None, None, ref, None, None, loose)


def test_wide_rmsnorm_rope_without_tail_equals_rmsnorm_fwd():
    """R = 0 through the wide path R kernel equals the library's RMSNorm forward bit for bit."""
    x, w, _, _ = _inputs(128, 3072, 0, torch.bfloat16, 1, 5)
    y0 = rnq.rmsnorm_rope(gpu(x), gpu(w), None, None)
    y1 = rnq.rmsnorm(gpu(x), gpu(w))
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("M,N,R,rpt,pad,with_pos", [
    (64, 2048, 256, 2, 8, True),     # [T, 2, N] view with a padded token stride, positions
    (40, 4096, 128, 1, 24, False),   # row-strided x, one table row per row
    (24, 1536, 1024, 3, 0, True),
])
def test_wide_rmsnorm_rope_ex_views_and_positions(M, N, R, rpt, pad, with_pos):
    T = M // rpt
    g = torch.Generator("cpu").manual_seed(M + N + R + pad)
    x = torch.randn(M, N, generator=g).to(torch.bfloat16)
    w = (1 + 0.1 * torch.randn(N, generator=g)).to(torch.bfloat16)
    buf = torch.randn(T, rpt * N + pad, generator=g).to(torch.bfloat16)
    buf[:, : rpt * N] = x.view(T, rpt * N)
    table_rows = 2 * T if with_pos else T
    cos, sin = workloads.rope_table(np.arange(table_rows) * 3, R, 10000.0)
    # positions include ones past the table (they read its last row)
    pos = (torch.randint(0, table_rows + 3, (T,), generator=g, dtype=torch.int32) if with_pos else None)
    print(f"[wide] rmsnorm_rope_ex M{M} N{N} R{R} rpt{rpt} pad{pad} positions {with_pos}", flush=True)
    bg = gpu(buf)
    xv = bg[:, : rpt * N].view(T, rpt, N) if rpt > 1 else bg[:, :N]
    y = rnq.rmsnorm_rope(xv, gpu(w), gpu(torch.from_numpy(cos)), gpu(torch.from_numpy(sin)), rows_per_token=rpt,
                         positions=None if pos is None else gpu(pos))
    torch.cuda.synchronize()
    rows = np.arange(T) if pos is None else np.minimum(pos.numpy().astype(np.int64), table_rows - 1)
    ref = oracle.rmsnorm_rope(workloads.bits(x), workloads.bits(w), cos[rows], sin[rows], 1e-6, "bf16", rpt)
    loose = unproven_rows(workloads.bits(x), "bf16")
    assert_rows_match(f"wide rmsnorm_rope_ex M{M} N{N}", workloads.bits(y), None, None, ref, None, None, loose)


# ---------------------------------------------------------------- the backward


def _close(name, dtype, gx, gw, ref_dx, ref_dw):
    dx = codecs.dtype_to_f32(workloads.bits(gx), DT[dtype]).astype(np.float64)
    dw = gw.cpu().numpy().astype(np.float64)
    row_rms = np.sqrt((ref_dx**2).mean(axis=1, keepdims=True))
    err = (np.abs(dx - ref_dx) / (np.abs(ref_dx) + row_rms)).max()
    errw = (np.abs(dw - ref_dw) / (np.abs(ref_dw) + np.sqrt((ref_dw**2).mean()))).max()
    print(f"[wide] {name}: max rel err dx {err:.3g} dw {errw:.3g}", flush=True)
    assert err <= 2e-2, f"{name}: dx rel err {err:.3g}"
    assert errw <= 2e-2, f"{name}: dw rel err {errw:.3g}"


BWD = [
    # M, N, R, dtype, rows_per_token, saved rstd
    (4096, 4096, 128, torch.bfloat16, 1, False),
    (256, 4096, 128, torch.float16, 1, True),
    (300, 1000, 64, torch.bfloat16, 3, False),
    (100, 2048, 1024, torch.float16, 2, True),   # 256-thread workgroups, widest tail
    (64, 16384, 1024, torch.bfloat16, 1, False),  # four chunks per lane
    (96, 8192, 512, torch.bfloat16, 4, True),
]


@pytest.mark.parametrize("M,N,R,dtype,rpt,saved", BWD, ids=[f"{m}x{n}r{r}" for m, n, r, _, _, _ in BWD])
def test_wide_rmsnorm_rope_bwd_matches_the_oracle(M, N, R, dtype, rpt, saved):
    x, w, cos, sin = _inputs(M, N, R, dtype, rpt, 3 * M + N + R)
    gy = torch.randn(M, N, generator=torch.Generator("cpu").manual_seed(M + 1)).to(dtype)
    print(f"[wide] rope bwd M{M} N{N} R{R} {DT[dtype]} rows_per_token {rpt} saved {saved}", flush=True)
    xd, wd = gpu(x), gpu(w)
    rstd = rnq.rmsnorm(xd, wd, return_rstd=True)[1] if saved else None
    gx, gw = rnq.rmsnorm_rope_bwd(xd, wd, gpu(gy), gpu(cos), gpu(sin), rstd, rows_per_token=rpt)
    gx2, gw2 = rnq.rmsnorm_rope_bwd(xd, wd, gpu(gy), gpu(cos), gpu(sin), rstd, rows_per_token=rpt)
    torch.cuda.synchronize()
    assert torch.equal(gw.view(torch.int32), gw2.view(torch.int32)) and torch.equal(gx, gx2)
    ref_dx, ref_dw, _ = oracle.rmsnorm_rope_bwd(workloads.bits(x), workloads.bits(w), workloads.bits(gy),
                                                cos.numpy(), sin.numpy(), 1e-6, DT[dtype], rpt)
    _close(f"rope bwd {M}x{N} R{R}", dtype, gx, gw, ref_dx, ref_dw)


def test_wide_rope_bwd_identity_rotation_equals_rmsnorm_bwd():
    """cos = 1, sin = 0 makes the transposed rotation the identity: the wide RoPE
    backward then gives the plain RMSNorm backward's bits. (256 rows: both
    backwards' row partitions are then one row per block, so grad_w is summed in
    the same order.)"""
    M, N, R = 256, 4096, 256
    x, w, _, _ = _inputs(M, N, R, torch.bfloat16, 1, 77)
    gy = torch.randn(M, N, generator=torch.Generator("cpu").manual_seed(78)).to(torch.bfloat16)
    ones = torch.ones(M, R // 2)
    zeros = torch.zeros(M, R // 2)
    gx, gw = rnq.rmsnorm_rope_bwd(gpu(x), gpu(w), gpu(gy), gpu(ones), gpu(zeros))
    gx0, gw0 = rnq.rmsnorm_bwd(gpu(x), gpu(w), gpu(gy))
    torch.cuda.synchronize()
    assert torch.equal(gx.view(torch.int16), gx0.view(torch.int16))
    assert torch.equal(gw.view(torch.int32), gw0.view(torch.int32))
