"""Seeded random-shape sweeps of the entry points against the CPU oracle (on
top of the hand-picked shapes of the other GPU tests). Every case prints its
parameters before it runs; the shapes are small enough for the oracle to
check every element."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_quant_amd as rnq
import oracle
import workloads

from _parity import assert_rows_match, compare_qk, gpu, run_qk_gpu, oracle_qk, unproven_rows

pytestmark = pytest.mark.gpu

DT = {torch.bfloat16: "bf16", torch.float16: "fp16"}
SEEDS = list(range(12))


def _rand_qk_case(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128, 256, 512]))
    R = int(rng.choice([r for r in (0, 16, 32, 64, D, D) if r <= D]))
    T = int(rng.integers(1, 90))
    Hq = int(rng.integers(0, 12))
    Hk = int(rng.integers(0 if Hq else 1, 6))
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float16
    std = float(rng.choice([0.01, 1.0, 30.0]))
    fp8_max = float(rng.choice([448.0, 448.0, 240.0, 57.0]))
    g = torch.Generator("cpu").manual_seed(seed)
    q = (torch.randn(T, Hq, D, generator=g) * std).to(dtype)
    k = (torch.randn(T, Hk, D, generator=g) * std).to(dtype)
    wq = (1 + 0.2 * torch.randn(D, generator=g)).to(dtype)
    wk = (1 + 0.2 * torch.randn(D, generator=g)).to(dtype)
    cos, sin = workloads.rope_table(rng.integers(0, 100000, T), R, float(rng.choice([1e4, 1e6])))
    return {"q": q, "k": k, "wq": wq, "wk": wk, "cos": torch.from_numpy(cos), "sin": torch.from_numpy(sin)}, fp8_max


@pytest.mark.parametrize("seed", SEEDS)
def test_qk_random_shapes(seed):
    d, fp8_max = _rand_qk_case(seed)
    print(f"[sweep] qk seed {seed}: q{tuple(d['q'].shape)} k{tuple(d['k'].shape)} rope {2 * d['cos'].shape[-1]} "
          f"{DT[d['q'].dtype]} fp8_max {fp8_max}", flush=True)
    got = run_qk_gpu(d, fp8_max=fp8_max, with_y=bool(seed % 2))
    ref = oracle_qk(d, fp8_max=fp8_max)
    compare_qk(f"qk seed {seed}", d, got, ref, DT[d["q"].dtype])


@pytest.mark.parametrize("seed", SEEDS)
def test_grouped_random_shapes(seed):
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.choice([8, 16, 32, 64, 128, 256, 512]))
    N = G * int(rng.integers(1, max(2, 16384 // G // 4)))
    N = min(N, 16384)
    R = int(rng.choice([r for r in (0, 16, 64, 128, 256, 1024) if r <= N]))
    rpt = int(rng.choice([1, 2, 4]))
    M = rpt * int(rng.integers(1, 12))
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float16
    g = torch.Generator("cpu").manual_seed(seed)
    x = (torch.randn(M, N, generator=g) * float(rng.choice([0.05, 1.0, 8.0]))).to(dtype)
    w = (1 + 0.2 * torch.randn(N, generator=g)).to(dtype)
    cos, sin = workloads.rope_table(rng.integers(0, 5000, M // rpt), R, 10000.0)
    print(f"[sweep] grouped seed {seed}: x({M}, {N}) group {G} rope {R} rows/token {rpt} {DT[dtype]}", flush=True)
    codes, scales, y = rnq.rmsnorm_rope_fp8_grouped(gpu(x), gpu(w), gpu(torch.from_numpy(cos)),
                                                    gpu(torch.from_numpy(sin)), group_size=G, rows_per_token=rpt,
                                                    return_y=True)
    torch.cuda.synchronize()
    ry, rc, rs = oracle.rmsnorm_rope_fp8_grouped(workloads.bits(x), workloads.bits(w), cos, sin, G, 1e-6, 448.0,
                                                 DT[dtype], rpt)
    strict = ~unproven_rows(workloads.bits(x), DT[dtype])
    gy, gc, gs = workloads.bits(y), codes.view(torch.uint8).cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(gy[strict], ry[strict])
    assert np.array_equal(gc[strict], rc[strict])
    assert np.array_equal(gs[strict].view(np.uint32), rs[strict].view(np.uint32))


@pytest.mark.parametrize("seed", SEEDS[:8])
def test_rope_bwd_random_shapes(seed):
    rng = np.random.default_rng(3000 + seed)
    N = int(rng.choice([64, 128, 256, 512]))
    R = int(rng.choice([r for r in (0, 16, 32, 64, 128, 256, 512) if r <= N]))
    rpt = int(rng.choice([1, 3, 8]))
    M = rpt * int(rng.integers(1, 400))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float16
    g = torch.Generator("cpu").manual_seed(seed)
    x = (torch.randn(M, N, generator=g) * float(rng.choice([0.1, 1.0, 4.0]))).to(dtype)
    w = (1 + 0.2 * torch.randn(N, generator=g)).to(dtype)
    gy = torch.randn(M, N, generator=g).to(dtype)
    cos, sin = workloads.rope_table(rng.integers(0, 5000, M // rpt), R, 10000.0)
    print(f"[sweep] rope bwd seed {seed}: x({M}, {N}) rope {R} rows/token {rpt} {DT[dtype]}", flush=True)
    gx, gw = rnq.rmsnorm_rope_bwd(gpu(x), gpu(w), gpu(gy), gpu(torch.from_numpy(cos)), gpu(torch.from_numpy(sin)),
                                  rows_per_token=rpt)
    torch.cuda.synchronize()
    ref_dx, ref_dw, _ = oracle.rmsnorm_rope_bwd(workloads.bits(x), workloads.bits(w), workloads.bits(gy), cos, sin,
                                                1e-6, DT[dtype], rpt)
    from oracle import codecs
    dx = codecs.dtype_to_f32(workloads.bits(gx), DT[dtype]).astype(np.float64)
    err = np.abs(dx - ref_dx) / (np.abs(ref_dx) + np.sqrt((ref_dx**2).mean(axis=1, keepdims=True)))
    errw = np.abs(gw.cpu().numpy() - ref_dw) / (np.abs(ref_dw) + np.sqrt((ref_dw**2).mean()))
    assert err.max() <= 2e-2 and errw.max() <= 2e-2, (err.max(), errw.max())


@pytest.mark.parametrize("seed", SEEDS[:8])
def test_wide_bwd_random_shapes(seed):
    """Rows wider than a head: 1024, 2048 and 4096 go through the wave-per-row
    backward when the tail is at most 512 columns, other widths and wider tails
    through the workgroup-per-row one; saved or recomputed rstd."""
    rng = np.random.default_rng(4000 + seed)
    N = int(rng.choice([1024, 2048, 4096, 4096, 1536, 3000, 8192]))
    R = int(rng.choice([r for r in (0, 16, 64, 128, 512, 1024) if r <= N]))
    rpt = int(rng.choice([1, 2, 5]))
    M = rpt * int(rng.integers(1, max(2, 600 // rpt)))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float16
    saved = bool(rng.random() < 0.4)
    g = torch.Generator("cpu").manual_seed(100 + seed)
    x = (torch.randn(M, N, generator=g) * float(rng.choice([0.1, 1.0, 4.0]))).to(dtype)
    w = (1 + 0.2 * torch.randn(N, generator=g)).to(dtype)
    gy = torch.randn(M, N, generator=g).to(dtype)
    cos, sin = workloads.rope_table(rng.integers(0, 5000, M // rpt), R, 10000.0)
    print(f"[sweep] wide bwd seed {seed}: x({M}, {N}) rope {R} rows/token {rpt} {DT[dtype]} saved {saved}",
          flush=True)
    xd, wd = gpu(x), gpu(w)
    rstd = rnq.rmsnorm(xd, wd, return_rstd=True)[1] if saved else None
    gx, gw = rnq.rmsnorm_rope_bwd(xd, wd, gpu(gy), gpu(torch.from_numpy(cos)), gpu(torch.from_numpy(sin)), rstd,
                                  rows_per_token=rpt)
    torch.cuda.synchronize()
    ref_dx, ref_dw, _ = oracle.rmsnorm_rope_bwd(workloads.bits(x), workloads.bits(w), workloads.bits(gy), cos, sin,
                                                1e-6, DT[dtype], rpt)
    from oracle import codecs
    dx = codecs.dtype_to_f32(workloads.bits(gx), DT[dtype]).astype(np.float64)
    err = np.abs(dx - ref_dx) / (np.abs(ref_dx) + np.sqrt((ref_dx**2).mean(axis=1, keepdims=True)))
    errw = np.abs(gw.cpu().numpy() - ref_dw) / (np.abs(ref_dw) + np.sqrt((ref_dw**2).mean()))
    assert err.max() <= 2e-2 and errw.max() <= 2e-2, (err.max(), errw.max())


@pytest.mark.parametrize("seed", SEEDS)
def test_whole_token_positions_random(seed):
    """Path R and one-tensor prologues whose passes hold whole tokens (the heads per
    token divide the rows per pass), cos/sin gathered through positions that run
    below zero and past the table (clamped to its last row), in padded token-strided
    views."""
    rng = np.random.default_rng(5000 + seed)
    D = int(rng.choice([64, 128, 256, 512]))
    G = 1024 // D  # rows per pass
    heads = int(rng.choice([h for h in (1, 2, 4, 8) if h < G]))
    T = (G // heads) * int(rng.integers(1, 12))
    R = int(rng.choice([r for r in (16, 32, 64, D) if r <= D]))
    dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float16
    pad = int(rng.choice([0, 8, 24]))
    table_rows = int(rng.integers(1, 3 * T + 1))
    quant = bool(rng.random() < 0.5)
    g = torch.Generator("cpu").manual_seed(500 + seed)
    x = (torch.randn(T, heads, D, generator=g) * float(rng.choice([0.05, 1.0, 20.0]))).to(dtype)
    w = (1 + 0.2 * torch.randn(D, generator=g)).to(dtype)
    buf = torch.zeros(T, heads * D + pad, dtype=dtype)
    buf[:, : heads * D] = x.reshape(T, -1)
    pos = torch.from_numpy(rng.integers(-3, table_rows + 4, T).astype(np.int32))
    cos, sin = workloads.rope_table(rng.integers(0, 100000, table_rows), R, float(rng.choice([1e4, 1e6])))
    p = pos.numpy().astype(np.int64)
    rows = np.where((p < 0) | (p >= table_rows), table_rows - 1, p)
    print(f"[sweep] whole tokens seed {seed}: T{T} heads{heads} D{D} R{R} {DT[dtype]} pad{pad} "
          f"table {table_rows} {'qk' if quant else 'path R'}", flush=True)
    xv = gpu(buf)[:, : heads * D].view(T, heads, D)
    cg, sg = gpu(torch.from_numpy(cos)), gpu(torch.from_numpy(sin))
    if quant:
        dev = xv.device
        q8 = torch.full((T, heads, D), 0xAB, dtype=torch.uint8, device=dev)
        qs = torch.full((T, heads), float("nan"), device=dev)
        qy = torch.empty((T, heads, D), dtype=dtype, device=dev) if seed % 2 else None
        rnq.rnq_qk_norm_rope_fp8_ex(xv, None, gpu(w), None, cg, sg, q8, None, qs, None, qy, None, positions=gpu(pos))
        torch.cuda.synchronize()
        got = {"q_codes": q8.cpu().numpy(), "q_scale": qs.cpu().numpy(), "k_codes": None, "k_scale": None,
               "q_y": None if qy is None else workloads.bits(qy), "k_y": None}
        ref = oracle.qk_norm_rope_fp8(workloads.bits(x), None, workloads.bits(w), None, cos, sin, dtype=DT[dtype],
                                      tokens=rows)
        compare_qk(f"whole tokens seed {seed}", {"q": x, "k": None}, got, ref, DT[dtype])
    else:
        y = rnq.rmsnorm_rope(xv if heads > 1 else xv[:, 0], gpu(w), cg, sg, rows_per_token=heads, positions=gpu(pos))
        torch.cuda.synchronize()
        ref = oracle.rmsnorm_rope(workloads.bits(x.reshape(-1, D)), workloads.bits(w), cos[rows], sin[rows], 1e-6,
                                  DT[dtype], heads)
        loose = unproven_rows(workloads.bits(x.reshape(-1, D)), DT[dtype])
        assert_rows_match(f"whole tokens seed {seed}", workloads.bits(y), None, None, ref, None, None, loose)
