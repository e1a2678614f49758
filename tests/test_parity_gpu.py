"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Bar: bit-exact y, codes and scales on every row whose sum of squares the
oracle proves exact in fp64 (all rows of these workloads in practice); on any
other row |dy| <= 1 ulp, codes within one step on <= 0.01 % of elements and
scale relative error <= 1e-6. Backward: |a - b| <= 2e-2 * (|b| + rms of the
reference row / column).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_quant_amd as rnq
import oracle
import workloads
from oracle import codecs

import _ties
from _parity import (
    assert_rows_match,
    compare_qk,
    gpu,
    oracle_qk,
    run_qk_gpu,
    unproven_rows,
)

pytestmark = pytest.mark.gpu


def _qk_case(T, Hq, Hk, D, R, seed, dtype=torch.bfloat16, std=1.0, outliers=0.0, theta=10000.0):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(T, Hq, D, generator=g) * std
    k = torch.randn(T, Hk, D, generator=g) * std
    if outliers:
        q = torch.where(torch.rand(q.shape, generator=g) < outliers, q * 20, q)
        k = torch.where(torch.rand(k.shape, generator=g) < outliers, k * 20, k)
    wq = 1 + 0.1 * torch.randn(D, generator=g)
    wk = 1 + 0.1 * torch.randn(D, generator=g)
    cos, sin = workloads.rope_table(np.arange(T), R, theta)
    return {"q": q.to(dtype), "k": k.to(dtype), "wq": wq.to(dtype), "wk": wk.to(dtype),
            "cos": torch.from_numpy(cos), "sin": torch.from_numpy(sin)}


def _check_qk(name, d, *, eps=1e-6, fp8_max=448.0, with_y=True):
    dt = "bf16" if d["q"].dtype == torch.bfloat16 else "fp16"
    print(f"[parity] {name}: q{tuple(d['q'].shape)} k{tuple(d['k'].shape)} rope {2 * d['cos'].shape[-1]}", flush=True)
    got = run_qk_gpu(d, eps=eps, fp8_max=fp8_max, with_y=with_y)
    ref = oracle_qk(d, eps=eps, fp8_max=fp8_max)
    compare_qk(name, d, got, ref, dt)
    return got, ref


# ------------------------------------------------------------------ named workloads


def test_qk_small_fused_partial_rope_with_y():
    d = workloads.generate("qk_small")
    got, ref = _check_qk("qk_small", d, with_y=True)
    assert got["q_y"] is not None


def test_qk_4k_full_size():
    """4096 tokens x (32 + 8) heads x 128, every row, in the launch shape the bench times (no y)."""
    d = workloads.generate("qk_4k")
    got, ref = _check_qk("qk_4k", d, with_y=False)
    # and again with y written, which exposes the rounded rows themselves
    got_y = run_qk_gpu(d, with_y=True)
    compare_qk("qk_4k+y", d, got_y, ref)
    assert np.array_equal(got_y["q_codes"], got["q_codes"])


@pytest.fixture(scope="module")
def qk_64k_run():
    """The 65536-token workload (64 + 8 heads x 128, 1.2 GB of input) through the GPU once."""
    d = workloads.generate("qk_64k")
    print("[parity] qk_64k generated", flush=True)
    got = run_qk_gpu(d, with_y=False)
    print("[parity] qk_64k ran on the GPU", flush=True)
    return d, got


def _oracle_chunk(d, got, part, lo, hi):
    """Compare tokens [lo, hi) of one tensor with the oracle, row by row."""
    T, H, D = d[part].shape
    xb = workloads.bits(d[part])[lo:hi]
    wb = workloads.bits(d["w" + part])
    toks = np.repeat(np.arange(lo, hi), H)
    c, s = d["cos"].numpy()[toks], d["sin"].numpy()[toks]
    rows = xb.reshape(-1, D)
    y, codes, scale = oracle.norm_rope_quant_rows(rows, wb, c, s, 1e-6, 448.0)
    assert_rows_match(f"qk_64k/{part} tokens {lo}..{hi}", None, got[part + "_codes"][lo:hi].reshape(-1, D),
                      got[part + "_scale"][lo:hi].reshape(-1), None, codes, scale, unproven_rows(rows, "bf16"))
    return rows.shape[0]


@pytest.mark.parametrize("quarter", [0, 1, 2, 3])
def test_qk_64k_every_row(qk_64k_run, quarter):
    """65536 tokens x (64 + 8) heads x 128, every row of a quarter of the tokens
    (the four cases cover the whole workload), against the oracle in 1024-token
    chunks (about 10 s of oracle time per quarter)."""
    d, got = qk_64k_run
    T = d["q"].shape[0]
    lo, hi = quarter * T // 4, (quarter + 1) * T // 4
    done = sum(_oracle_chunk(d, got, part, a, min(a + 1024, hi)) for part in ("q", "k") for a in range(lo, hi, 1024))
    print(f"[parity] qk_64k tokens {lo}..{hi}: {done} rows checked", flush=True)
    assert done == (hi - lo) * (d["q"].shape[1] + d["k"].shape[1])


def test_norm_rope_fp16_full_size():
    d = workloads.generate("norm_rope_fp16")
    x, w = gpu(d["x"]), gpu(d["w"])
    y = rnq.rmsnorm_rope(x, w, gpu(d["cos"]), gpu(d["sin"]), rows_per_token=1)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_rope(workloads.bits(d["x"]), workloads.bits(d["w"]), d["cos"].numpy(),
                              d["sin"].numpy(), dtype="fp16")
    xb = workloads.bits(d["x"])
    assert_rows_match("norm_rope_fp16", workloads.bits(y), None, None, ref, None, None, unproven_rows(xb, "fp16"))


def test_rmsnorm_4k_forward_and_rstd():
    d = workloads.generate("rmsnorm_4k")
    x, w = gpu(d["x"]), gpu(d["w"])
    y, rstd = rnq.rmsnorm(x, w, return_rstd=True)
    torch.cuda.synchronize()
    ref_y, ref_rstd = oracle.rmsnorm_fwd(workloads.bits(d["x"]), workloads.bits(d["w"]), 1e-6)
    loose = unproven_rows(workloads.bits(d["x"]), "bf16")
    assert_rows_match("rmsnorm_4k", workloads.bits(y), None, None, ref_y, None, None, loose)
    r = rstd.cpu().numpy()
    assert np.array_equal(r.view(np.uint32)[~loose], ref_rstd.view(np.uint32)[~loose])


def _bwd_check(name, x, w, gy, gx, gw, rstd_given=None):
    ref_dx, ref_dw, _ = oracle.rmsnorm_bwd(workloads.bits(x), workloads.bits(w), workloads.bits(gy), 1e-6,
                                           "bf16" if x.dtype == torch.bfloat16 else "fp16", rstd=rstd_given)
    dt = "bf16" if x.dtype == torch.bfloat16 else "fp16"
    dx = codecs.dtype_to_f32(workloads.bits(gx), dt).astype(np.float64)
    dw = gw.cpu().numpy().astype(np.float64)
    row_rms = np.sqrt((ref_dx**2).mean(axis=1, keepdims=True))
    err = np.abs(dx - ref_dx) / (np.abs(ref_dx) + row_rms)
    assert err.max() <= 2e-2, f"{name}: dx rel err {err.max():.3g}"
    col_rms = np.sqrt((ref_dw**2).mean())
    errw = np.abs(dw - ref_dw) / (np.abs(ref_dw) + col_rms)
    assert errw.max() <= 2e-2, f"{name}: dw rel err {errw.max():.3g}"
    print(f"[parity] {name}: max rel err dx {err.max():.3g} dw {errw.max():.3g}", flush=True)


def test_rmsnorm_4k_backward_and_determinism():
    d = workloads.generate("rmsnorm_4k")
    x, w, gy = gpu(d["x"]), gpu(d["w"]), gpu(d["grad_y"])
    gx, gw = rnq.rmsnorm_bwd(x, w, gy)
    gx2, gw2 = rnq.rmsnorm_bwd(x, w, gy)
    torch.cuda.synchronize()
    _bwd_check("rmsnorm_4k bwd", d["x"], d["w"], d["grad_y"], gx, gw)
    assert torch.equal(gx, gx2) and torch.equal(gw.view(torch.int32), gw2.view(torch.int32))
    # with the rstd saved by the forward
    _, rstd = rnq.rmsnorm(x, w, return_rstd=True)
    gx3, gw3 = rnq.rmsnorm_bwd(x, w, gy, rstd)
    torch.cuda.synchronize()
    assert torch.equal(gx3, gx) and torch.equal(gw3.view(torch.int32), gw.view(torch.int32))


# ------------------------------------------------------------------ shapes and edges


@pytest.mark.parametrize(
    "T,Hq,Hk,D,R",
    [
        (37, 3, 2, 128, 64),   # rows not a multiple of a pass; passes mix q and k rows
        (5, 1, 0, 128, 128),   # a single partial pass
        (1, 1, 1, 128, 128),
        (64, 4, 4, 64, 16),
        (33, 2, 1, 256, 128),
        (17, 2, 2, 512, 256),
        (50, 8, 8, 128, 0),    # no rope: plain RMSNorm + FP8
        (40, 0, 3, 128, 64),   # k heads only
        (300, 32, 8, 128, 128),
    ],
)
def test_qk_shapes(T, Hq, Hk, D, R):
    d = _qk_case(T, Hq, Hk, D, R, seed=T * 1000 + Hq * 10 + Hk + D + R)
    _check_qk(f"qk T{T} Hq{Hq} Hk{Hk} D{D} R{R}", d)


@pytest.mark.parametrize(
    "T,Hq,Hk,D,R,with_y",
    [
        # head counts multiples of the rows per pass (64 / (D / 16)): every pass
        # lies inside one token and one tensor. The tail widths cover the
        # table loads at 4, 8 and 16 bytes per lane (D <= 128, 256, 512), rope
        # tails that fill the row, tails whose code chunks are swapped between
        # lane pairs (plain part and tail multiples of 32 columns), and tails
        # that keep two 8-byte code stores per lane (R = 16, 48).
        (9, 16, 16, 64, 64, False),
        (9, 16, 0, 64, 32, True),
        (11, 8, 8, 128, 64, False),
        (11, 8, 8, 128, 48, True),
        (11, 8, 16, 128, 16, False),
        (13, 4, 4, 256, 256, True),
        (13, 4, 8, 256, 96, False),
        (7, 2, 2, 512, 512, False),
        (7, 2, 4, 512, 160, True),
        (7, 6, 2, 512, 64, False),
    ],
)
def test_qk_aligned_passes(T, Hq, Hk, D, R, with_y):
    d = _qk_case(T, Hq, Hk, D, R, seed=T * 977 + Hq * 31 + Hk * 7 + D + R, outliers=0.01)
    _check_qk(f"qk aligned T{T} Hq{Hq} Hk{Hk} D{D} R{R}", d, with_y=with_y)


@pytest.mark.parametrize("fp8_max", [58.0, 232.0, 0.5])
def test_qk_aligned_passes_with_a_binding_clamp_or_small_fp8_max(fp8_max):
    """Head-aligned passes through the per-pass-branch variant of the loop: fp8_max on
    an e4m3 rounding midpoint (the clamp binds on about half of the rows) or below 1
    (the scale by IEEE division)."""
    for T, Hq, Hk, D, R in ((11, 8, 8, 128, 128), (9, 16, 16, 64, 32), (7, 2, 4, 512, 160)):
        d = _qk_case(T, Hq, Hk, D, R, seed=T * 131 + D + int(fp8_max), outliers=0.02)
        _check_qk(f"qk aligned T{T} H{Hq}+{Hk} D{D} R{R} fp8_max {fp8_max}", d, fp8_max=fp8_max)


def test_qk_code_outputs_8_byte_aligned():
    """Code outputs that are 8- but not 16-byte aligned (allowed by the entry point)
    take the two 8-byte stores per lane instead of the whole 16-byte chunks."""
    for T, Hq, Hk, D, R in ((11, 8, 8, 128, 128), (9, 16, 16, 64, 32), (13, 4, 8, 256, 96)):
        d = _qk_case(T, Hq, Hk, D, R, seed=T * 17 + D + R, outliers=0.01)
        print(f"[parity] qk codes at +8 bytes: T{T} H{Hq}+{Hk} D{D} R{R}", flush=True)
        dev = torch.device("cuda:0")
        qb = torch.empty(T * Hq * D + 16, dtype=torch.uint8, device=dev)
        kb = torch.empty(T * Hk * D + 16, dtype=torch.uint8, device=dev)
        q8, k8 = qb[8:8 + T * Hq * D].view(T, Hq, D), kb[8:8 + T * Hk * D].view(T, Hk, D)
        assert q8.data_ptr() % 16 == 8 and k8.data_ptr() % 16 == 8
        qs = torch.empty(T, Hq, device=dev)
        ks = torch.empty(T, Hk, device=dev)
        rnq.prepare_qk_norm_rope_fp8(gpu(d["q"]), gpu(d["k"]), gpu(d["wq"]), gpu(d["wk"]), gpu(d["cos"]),
                                     gpu(d["sin"]), q8, k8, qs, ks)()
        torch.cuda.synchronize()
        ref = oracle_qk(d)
        assert np.array_equal(q8.cpu().numpy(), ref["q_codes"]) and np.array_equal(k8.cpu().numpy(), ref["k_codes"])
        assert np.array_equal(qs.cpu().numpy().view(np.uint32), ref["q_scale"].view(np.uint32))
        assert np.array_equal(ks.cpu().numpy().view(np.uint32), ref["k_scale"].view(np.uint32))


def _tie_case(bits, T, Hq, Hk):
    x = torch.from_numpy(bits[: T * (Hq + Hk)].view(np.int16)).view(torch.bfloat16).reshape(T, Hq + Hk, 128)
    one = torch.ones(128, dtype=torch.bfloat16)
    return {"q": x[:, :Hq].contiguous(), "k": x[:, Hq:].contiguous(), "wq": one, "wk": one,
            "cos": torch.zeros(T, 0), "sin": torch.zeros(T, 0)}


@pytest.mark.parametrize("fp8_max", [448.0, 240.0])
def test_qk_quotients_on_e4m3_midpoints(fp8_max):
    """Rows that normalise exactly (mean square a power of 4, eps = 0, w = 1) and
    put y / scale exactly on e4m3 rounding midpoints, where a code flips with
    one rounding more or less: the kernel's quotient must be the correctly
    rounded one. Head-aligned passes (8 q + 8 k heads) and per-lane rows (1 head)."""
    bits = _ties.normalised_tie_rows(fp8_max)
    n = len(bits)
    for name, T, Hq, Hk in (("aligned", n // 16, 8, 8), ("per-lane rows", n, 1, 0)):
        d = _tie_case(bits, T, Hq, Hk)
        _check_qk(f"qk ties {name} fp8_max {fp8_max}", d, eps=0.0, fp8_max=fp8_max)


def test_qk_fp16_inputs_and_smaller_fp8_max():
    d = _qk_case(64, 4, 2, 128, 64, seed=77, dtype=torch.float16, std=3.0)
    _check_qk("qk fp16", d, fp8_max=448.0)
    d = _qk_case(64, 4, 2, 128, 128, seed=78, outliers=0.05)
    _check_qk("qk fp8_max 240", d, fp8_max=240.0)
    _check_qk("qk fp8_max 57.5", d, fp8_max=57.5)
    # 58 lies on an e4m3 rounding boundary (between 56 and 60): the clamp binds
    _check_qk("qk fp8_max 58 (clamped)", d, fp8_max=58.0)
    # below 1 the scale takes the IEEE division path
    _check_qk("qk fp8_max 0.5", d, fp8_max=0.5)


def test_qk_degenerate_rows():
    """Zero rows (codes keep the sign of w), constant rows, tiny and huge values, eps = 0."""
    d = _qk_case(16, 4, 2, 128, 64, seed=79)
    q = d["q"].float()
    q[0] = 0.0
    q[1] = 1.0
    q[2] = -3.0
    q[3, :, :64] = 0.0
    q[4] *= 1e-30
    q[5] *= 1e30
    q[6, 0, 5] = 1e4
    d["q"] = q.to(torch.bfloat16)
    wq = d["wq"].float()
    wq[::3] *= -1
    d["wq"] = wq.to(torch.bfloat16)
    _check_qk("qk degenerate", d)
    # eps = 0 on rows whose sum of squares stays a normal fp32 number
    d2 = _qk_case(16, 4, 2, 128, 64, seed=84)
    q2 = d2["q"].float()
    q2[0] = 0.25
    q2[1, :, 7] = -2.0
    q2[2] *= 1e-20  # mean(x^2) far below 2^-100: the IEEE rstd path
    d2["q"] = q2.to(torch.bfloat16)
    _check_qk("qk eps 0", d2, eps=0.0)


def test_qk_zero_tokens_is_a_no_op():
    d = _qk_case(0, 4, 2, 128, 64, seed=80)
    got = run_qk_gpu(d)
    assert got["q_codes"].size == 0


def test_qk_repeatable_bitwise():
    d = _qk_case(256, 32, 8, 128, 128, seed=81, outliers=0.01)
    a = run_qk_gpu(d)
    b = run_qk_gpu(d)
    for key in ("q_codes", "k_codes"):
        assert np.array_equal(a[key], b[key])
    for key in ("q_scale", "k_scale"):
        assert np.array_equal(a[key].view(np.uint32), b[key].view(np.uint32))


@pytest.mark.parametrize("N", [64, 128, 256, 512, 72, 1000, 2048, 4104, 16384])
def test_rmsnorm_widths(N):
    M = 33
    g = torch.Generator("cpu").manual_seed(N)
    x = (torch.randn(M, N, generator=g) * 2).to(torch.bfloat16)
    w = torch.randn(N, generator=g).to(torch.bfloat16)
    x[3] = 0
    print(f"[parity] rmsnorm M{M} N{N}", flush=True)
    y, rstd = rnq.rmsnorm(gpu(x), gpu(w), return_rstd=True)
    torch.cuda.synchronize()
    ref_y, ref_rstd = oracle.rmsnorm_fwd(workloads.bits(x), workloads.bits(w), 1e-6)
    loose = unproven_rows(workloads.bits(x), "bf16")
    assert_rows_match(f"rmsnorm N{N}", workloads.bits(y), None, None, ref_y, None, None, loose)
    assert np.array_equal(rstd.cpu().numpy().view(np.uint32)[~loose], ref_rstd.view(np.uint32)[~loose])


@pytest.mark.parametrize("M,N", [(1, 128), (3, 4104), (257, 1024), (1000, 512), (64, 16384)])
def test_rmsnorm_bwd_shapes(M, N):
    g = torch.Generator("cpu").manual_seed(M * 7 + N)
    x = torch.randn(M, N, generator=g).to(torch.bfloat16)
    w = torch.randn(N, generator=g).to(torch.bfloat16)
    gy = torch.randn(M, N, generator=g).to(torch.bfloat16)
    gx, gw = rnq.rmsnorm_bwd(gpu(x), gpu(w), gpu(gy))
    torch.cuda.synchronize()
    _bwd_check(f"bwd M{M} N{N}", x, w, gy, gx, gw)


def test_rmsnorm_rope_grouped_table_rows():
    """rows_per_token > 1: every head of a token reads that token's table row."""
    T, H, N, R = 50, 6, 128, 64
    g = torch.Generator("cpu").manual_seed(82)
    x = torch.randn(T * H, N, generator=g).to(torch.bfloat16)
    w = (1 + 0.1 * torch.randn(N, generator=g)).to(torch.bfloat16)
    cos, sin = workloads.rope_table(np.arange(T) * 3, R, 10000.0)
    y = rnq.rmsnorm_rope(gpu(x), gpu(w), gpu(torch.from_numpy(cos)), gpu(torch.from_numpy(sin)), rows_per_token=H)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_rope(workloads.bits(x), workloads.bits(w), cos, sin, rows_per_token=H)
    assert_rows_match("rmsnorm_rope grouped", workloads.bits(y), None, None, ref, None, None,
                      unproven_rows(workloads.bits(x), "bf16"))


def test_cross_entry_rope_zero_equals_rmsnorm():
    g = torch.Generator("cpu").manual_seed(83)
    x = torch.randn(100, 256, generator=g).to(torch.bfloat16)
    w = torch.randn(256, generator=g).to(torch.bfloat16)
    a = rnq.rmsnorm(gpu(x), gpu(w))
    b = rnq.rmsnorm_rope(gpu(x), gpu(w), None, None)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


FP16_SPECIALS = [
    # N, R, rows_per_token, positions
    (64, 64, 1, False),
    (128, 64, 1, False),    # passes of whole tokens
    (128, 64, 4, False),
    (128, 128, 8, True),    # position-indexed table rows
    (256, 128, 2, False),
    (512, 16, 1, False),
    (128, 0, 1, False),     # no tail
]


@pytest.mark.parametrize("N,R,rpt,with_pos", FP16_SPECIALS, ids=[f"N{n}R{r}h{h}{'p' if p else ''}"
                                                                 for n, r, h, p in FP16_SPECIALS])
def test_rmsnorm_rope_fp16_signed_zeros_and_subnormals(N, R, rpt, with_pos):
    """fp16 path R bit for bit where the outputs are -0 / +0 (zero rows of either
    sign, zero weights of either sign, zero and unit table entries), fp16
    subnormals (tiny weights, a row dominated by one element, tiny table
    entries) and products that underflow fp32."""
    T = 48
    M = T * rpt
    g = torch.Generator("cpu").manual_seed(N * 7 + R + rpt)
    x = torch.randn(M, N, generator=g)
    x[0] = 0.0
    x[1] = -0.0
    x[2, ::2] = -0.0
    x[2, 1::2] = 0.0
    x[2, 3] = 1.5
    x[3] = 1e-3 * torch.randn(N, generator=g)
    x[3, 5] = 60000.0
    x[4, : N // 2] = -0.0
    w = 1 + 0.1 * torch.randn(N, generator=g)
    w[::5] *= -1
    w[1::7] = 0.0
    w[2::7] = -0.0
    w[3::11] = 1e-5
    w[4::13] = -3e-7
    x, w = x.to(torch.float16), w.to(torch.float16)
    rows = 2 * T if with_pos else T
    cos, sin = workloads.rope_table(np.arange(rows) * 5, R, 10000.0)
    cos, sin = cos.copy(), sin.copy()
    if R:
        cos[::3, ::4] = 0.0
        sin[::3, ::4] = 1.0
        cos[1::3, 1::4] = -0.0
        sin[1::3, 1::4] = -1.0
        cos[2::3, 2::4] = 1e-30
        sin[2::3, 3::4] = -1e-38
    pos = torch.randint(0, rows, (T,), generator=g, dtype=torch.int32) if with_pos else None
    print(f"[fp16 specials] N{N} R{R} rows_per_token {rpt} positions {with_pos}", flush=True)
    y = rnq.rmsnorm_rope(gpu(x), gpu(w), gpu(torch.from_numpy(cos)) if R else None,
                         gpu(torch.from_numpy(sin)) if R else None, rows_per_token=rpt,
                         positions=None if pos is None else gpu(pos))
    torch.cuda.synchronize()
    t = np.arange(T) if pos is None else pos.numpy().astype(np.int64)
    ref = oracle.rmsnorm_rope(workloads.bits(x), workloads.bits(w), cos[t], sin[t], 1e-6, "fp16", rpt)
    got = workloads.bits(y)
    assert (got == 0x8000).any() and (got == 0).any()  # both zeros occur
    assert_rows_match(f"fp16 specials N{N} R{R}", got, None, None, ref, None, None,
                      unproven_rows(workloads.bits(x), "fp16"))
    if R == 0:
        y0 = rnq.rmsnorm(gpu(x), gpu(w))
        torch.cuda.synchronize()
        assert np.array_equal(workloads.bits(y0), got)


def test_invalid_arguments_raise_before_launch():
    x = torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rnq.RnqError) as e:
        rnq.rnq_rmsnorm_rope(x, w, None, None, torch.empty_like(x), rows_per_token=3)
    assert e.value.status == 2
    with pytest.raises(rnq.RnqError) as e:
        rnq.qk_norm_rope_fp8(x.view(4, 1, 128), None, w, None,
                             torch.zeros(4, 64, device="cuda"), torch.zeros(4, 64, device="cuda"), fp8_max=500.0)
    assert e.value.status == 4
    with pytest.raises(ValueError):
        rnq.rmsnorm(x.cpu(), w.cpu())  # no CPU path
