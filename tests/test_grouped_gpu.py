"""GPU parity of the per-group FP8 entry point (rnq_rmsnorm_rope_fp8_grouped)
against the CPU oracle, element by element.

Bar: bit-exact y, codes and per-group scales on every row whose sum of
squares the oracle proves exact in fp64; on other rows |dy| <= 1 ulp, codes
within one step on <= 0.01 % of elements and scale relative error <= 1e-6.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_quant_amd as rnq
import oracle
import workloads

import _ties
from _parity import code_distance, gpu, ulp_distance_16, unproven_rows

pytestmark = pytest.mark.gpu

DT = {torch.bfloat16: "bf16", torch.float16: "fp16"}


def _run(x, w, cos, sin, group_size, *, rows_per_token=1, eps=1e-6, fp8_max=448.0, with_y=True):
    M, N = x.shape
    xg = gpu(x)
    codes = torch.full((M, N), 0xAB, dtype=torch.uint8, device=xg.device)
    scales = torch.full((M, N // group_size), float("nan"), dtype=torch.float32, device=xg.device)
    y = torch.empty_like(xg) if with_y else None
    rnq.rnq_rmsnorm_rope_fp8_grouped(xg, gpu(w), gpu(cos) if cos is not None else None,
                                     gpu(sin) if sin is not None else None, codes, scales, y,
                                     group_size=group_size, rows_per_token=rows_per_token, eps=eps,
                                     fp8_max=fp8_max)
    torch.cuda.synchronize()
    return (None if y is None else workloads.bits(y)), codes.cpu().numpy(), scales.cpu().numpy()


def _oracle(x, w, cos, sin, group_size, *, rows_per_token=1, eps=1e-6, fp8_max=448.0, rows=None):
    xb = workloads.bits(x) if rows is None else workloads.bits(x)[rows]
    return oracle.rmsnorm_rope_fp8_grouped(xb, workloads.bits(w), cos.numpy(), sin.numpy(), group_size, eps,
                                           fp8_max, DT[x.dtype], rows_per_token, rows)


def _compare(name, x_bits, dt, got, ref):
    gy, gc, gs = got
    ry, rc, rs = ref
    loose = unproven_rows(x_bits, dt)
    strict = ~loose
    msgs = []
    if gy is not None:
        bad = (gy != ry).any(axis=1) & strict
        if bad.any():
            i = int(np.flatnonzero(bad)[0]); j = int(np.flatnonzero(gy[i] != ry[i])[0])
            msgs.append(f"{name}: y differs on {int(bad.sum())} rows; row {i} col {j}: {gy[i, j]:#06x} vs {ry[i, j]:#06x}")
        if loose.any():
            assert ulp_distance_16(gy[loose], ry[loose]).max(initial=0) <= 1
    bad = (gc != rc).any(axis=1) & strict
    if bad.any():
        i = int(np.flatnonzero(bad)[0]); j = int(np.flatnonzero(gc[i] != rc[i])[0])
        msgs.append(f"{name}: codes differ on {int(bad.sum())} rows; row {i} col {j}: {gc[i, j]:#04x} vs {rc[i, j]:#04x}")
    bad = (gs.view(np.uint32) != rs.view(np.uint32)).any(axis=1) & strict
    if bad.any():
        i = int(np.flatnonzero(bad)[0]); g = int(np.flatnonzero(gs[i] != rs[i])[0])
        msgs.append(f"{name}: scales differ on {int(bad.sum())} rows; row {i} group {g}: {gs[i, g]!r} vs {rs[i, g]!r}")
    if loose.any():
        assert code_distance(gc[loose], rc[loose]).max(initial=0) <= 1
        assert (code_distance(gc[loose], rc[loose]) > 0).mean() <= 1e-4
        np.testing.assert_allclose(gs[loose], rs[loose], rtol=1e-6, atol=0)
    assert not msgs, "\n".join(msgs)


def _case(M, N, R, seed, dtype=torch.bfloat16, std=1.0, rows_per_token=1, theta=10000.0):
    g = torch.Generator("cpu").manual_seed(seed)
    x = (torch.randn(M, N, generator=g) * std).to(dtype)
    w = (1 + 0.1 * torch.randn(N, generator=g)).to(dtype)
    cos, sin = workloads.rope_table(np.arange(M // rows_per_token), R, theta)
    return x, w, torch.from_numpy(cos), torch.from_numpy(sin)


def _check(name, x, w, cos, sin, group_size, **kw):
    print(f"[grouped] {name}: x{tuple(x.shape)} rope {2 * cos.shape[-1]} group {group_size} {kw}", flush=True)
    with_y = kw.pop("with_y", True)
    got = _run(x, w, cos, sin, group_size, with_y=with_y, **kw)
    ref = _oracle(x, w, cos, sin, group_size, **kw)
    _compare(name, workloads.bits(x), DT[x.dtype], got, (ref[0] if with_y else None, ref[1], ref[2]))
    return got, ref


# ------------------------------------------------------------------ named workloads


def test_grouped_small_full():
    d = workloads.generate("grouped_small")
    _check("grouped_small", d["x"], d["w"], d["cos"], d["sin"], d["group_size"])


def test_grouped_4k_sampled_rows():
    d = workloads.generate("grouped_4k")
    M = d["rows"]
    print(f"[grouped] grouped_4k sampled: x{tuple(d['x'].shape)}", flush=True)
    got = _run(d["x"], d["w"], d["cos"], d["sin"], d["group_size"])
    rng = np.random.default_rng(7)
    rows = np.unique(np.r_[np.arange(64), np.arange(M - 64, M), rng.choice(M, 256, replace=False)])
    ref = _oracle(d["x"], d["w"], d["cos"], d["sin"], d["group_size"], rows=rows)
    _compare("grouped_4k", workloads.bits(d["x"])[rows], "bf16",
             (got[0][rows], got[1][rows], got[2][rows]), ref)


# ------------------------------------------------------------------ shapes and parameters


@pytest.mark.parametrize("M,N,R,group", [
    (3, 64, 16, 8), (17, 128, 64, 16), (33, 1000, 0, 8), (5, 1024, 128, 32), (9, 2048, 256, 64),
    (7, 4096, 1024, 512), (4, 4104, 64, 8), (2, 8192, 128, 256), (3, 16384, 512, 128),
])
def test_grouped_shapes(M, N, R, group):
    x, w, cos, sin = _case(M, N, R, M * 31 + N)
    _check(f"M{M} N{N} R{R} g{group}", x, w, cos, sin, group)


@pytest.mark.parametrize("fp8_max", [448.0, 240.0])
def test_grouped_quotients_on_e4m3_midpoints(fp8_max):
    """Rows with mean square 1 (RMSNorm with eps = 0 and w = 1 is then the
    identity) whose y / scale land exactly on e4m3 rounding midpoints: 32 of
    them side by side as 4096-wide rows with groups of 128 (each group one tie
    row), and one per row with a single scale (group_size = N = 128). The
    quotient must be the correctly rounded one for the codes to match."""
    bits = _ties.normalised_tie_rows(fp8_max)
    bits = bits[_ties.lowest_square_bit(bits) > 12 - 53]  # exact float64 sums at the 4096-wide total 2^12
    n = (len(bits) // 32) * 32
    wide = np.ascontiguousarray(bits[:n].reshape(n // 32, 4096))
    assert len(wide) >= 2 and not unproven_rows(wide, "bf16").any()
    for name, xb in (("4096-wide, groups of 128", wide), ("128-wide, one group", bits)):
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16)
        w = torch.ones(x.shape[1], dtype=torch.bfloat16)
        z = torch.zeros(x.shape[0], 0)
        _check(f"ties {name} fp8_max {fp8_max}", x, w, z, z, 128, eps=0.0, fp8_max=fp8_max)


def test_grouped_fp16_rows_per_token_and_no_y():
    x, w, cos, sin = _case(24, 512, 64, 5, dtype=torch.float16, std=2.0, rows_per_token=4)
    _check("fp16 rpt4", x, w, cos, sin, 64, rows_per_token=4)
    _check("fp16 rpt4 no y", x, w, cos, sin, 64, rows_per_token=4, with_y=False)


@pytest.mark.parametrize("fp8_max", [240.0, 57.5, 58.0, 0.5])
def test_grouped_fp8_max(fp8_max):
    x, w, cos, sin = _case(16, 1024, 128, 11)
    _check(f"fp8_max {fp8_max}", x, w, cos, sin, 128, fp8_max=fp8_max)


def test_grouped_degenerate_rows():
    x, w, cos, sin = _case(8, 512, 64, 12)
    x[0] = 0  # zero row: every group at the 1e-4 floor
    x[1, :128] = 0  # one zero group inside a normal row
    x[2] = (x[2].float() * 1e-30).to(x.dtype)  # tiny row
    _check("degenerate", x, w, cos, sin, 128)


def test_one_group_per_row_equals_the_row_kernel():
    # cross-entry: group_size == N gives the per-row scale of rnq_qk_norm_rope_fp8 (one head per token)
    x, w, cos, sin = _case(64, 128, 64, 13)
    print("[grouped] cross-entry 64x128 g128 vs qk_norm_rope_fp8", flush=True)
    gy, gc, gs = _run(x, w, cos, sin, 128)
    q8, _, qs, _, qy, _ = rnq.qk_norm_rope_fp8(gpu(x.view(64, 1, 128)), None, gpu(w), None, gpu(cos), gpu(sin),
                                                return_y=True)
    torch.cuda.synchronize()
    strict = ~unproven_rows(workloads.bits(x), "bf16")
    assert strict.sum() > 32
    assert np.array_equal(gy[strict], workloads.bits(qy).reshape(64, 128)[strict])
    assert np.array_equal(gc[strict], q8.view(torch.uint8).cpu().numpy().reshape(64, 128)[strict])
    assert np.array_equal(gs[strict, 0].view(np.uint32), qs.cpu().numpy().reshape(64)[strict].view(np.uint32))


def test_grouped_invalid_arguments_raise():
    x, w, cos, sin = _case(4, 384, 64, 14)
    xg, wg, cg, sg = gpu(x), gpu(w), gpu(cos), gpu(sin)
    codes = torch.empty((4, 384), dtype=torch.uint8, device=xg.device)
    print("[grouped] invalid arguments", flush=True)
    with pytest.raises(rnq.RnqError, match="UNSUPPORTED"):  # 48 divides 384 but is no power of two
        rnq.rnq_rmsnorm_rope_fp8_grouped(xg, wg, cg, sg, codes, torch.empty((4, 8), device=xg.device), group_size=48)
    with pytest.raises(rnq.RnqError, match="SHAPE"):  # 256 does not divide 384
        rnq.rnq_rmsnorm_rope_fp8_grouped(xg, wg, cg, sg, codes, torch.empty((4, 1), device=xg.device), group_size=256)
    # M = 0: nothing launched, no error
    rnq.rnq_rmsnorm_rope_fp8_grouped(xg[:0], wg, cg[:0], sg[:0], codes[:0],
                                     torch.empty((0, 3), device=xg.device), group_size=128)
