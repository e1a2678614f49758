"""GPU checks of NEXT-4: one FP8 scale per row on wide rows (the fused path the
unfused plan is compared with) against the oracle, the unfused three-kernel
plan bit-identical to the fused kernel, and the chapter 28 designs A/B/C
bit-identical to the row kernel."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_quant_amd as rnq
import oracle
import workloads
from fp8_quant_amd import baselines

from _parity import gpu, run_qk_gpu, unproven_rows

pytestmark = pytest.mark.gpu

DT = {torch.bfloat16: "bf16", torch.float16: "fp16"}


def _rows(M, N, R, seed, dtype=torch.bfloat16, rpt=1):
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(M, N, generator=g).to(dtype)
    w = (1 + 0.1 * torch.randn(N, generator=g)).to(dtype)
    cos, sin = workloads.rope_table(np.arange(M // rpt), R, 10000.0)
    return x, w, torch.from_numpy(cos), torch.from_numpy(sin)


def _check_per_row(name, x, w, cos, sin, codes, scales, rpt=1, rows=None):
    xb = workloads.bits(x) if rows is None else workloads.bits(x)[rows]
    _, rc, rs = oracle.rmsnorm_rope_fp8_grouped(xb, workloads.bits(w), cos.numpy(), sin.numpy(), x.shape[1], 1e-6,
                                                448.0, DT[x.dtype], rpt, rows)
    gc = codes.view(torch.uint8).cpu().numpy()
    gs = scales.cpu().numpy().reshape(-1)
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    strict = ~unproven_rows(xb, DT[x.dtype])
    assert np.array_equal(gc[strict], rc[strict]), f"{name}: codes differ"
    assert np.array_equal(gs[strict].view(np.uint32), rs.reshape(-1)[strict].view(np.uint32)), f"{name}: scales differ"


@pytest.mark.parametrize("M,N,R,dtype", [
    (64, 4096, 128, torch.bfloat16), (5, 16384, 1024, torch.bfloat16), (33, 1000, 0, torch.float16),
    (17, 72, 16, torch.bfloat16), (40, 128, 64, torch.float16), (9, 2056, 64, torch.bfloat16),
])
def test_one_scale_per_row(M, N, R, dtype):
    x, w, cos, sin = _rows(M, N, R, seed=M + N + R, dtype=dtype)
    print(f"[baselines] per-row grouped M{M} N{N} R{R} {DT[dtype]}", flush=True)
    codes, scales = rnq.rmsnorm_rope_fp8_grouped(gpu(x), gpu(w), gpu(cos), gpu(sin), group_size=N)
    torch.cuda.synchronize()
    _check_per_row(f"M{M} N{N}", x, w, cos, sin, codes, scales)


@pytest.mark.parametrize("M,N,R,rpt", [(256, 4096, 128, 1), (96, 1024, 64, 4), (50, 136, 16, 1)])
def test_unfused_plan_equals_fused(M, N, R, rpt):
    x, w, cos, sin = _rows(M, N, R, seed=7 * M + N, rpt=rpt)
    print(f"[baselines] unfused M{M} N{N} R{R} rpt{rpt}", flush=True)
    xg, wg, cg, sg = gpu(x), gpu(w), gpu(cos), gpu(sin)
    uc, us = baselines.norm_rope_quant_unfused(xg, wg, cg, sg, rows_per_token=rpt)
    fc, fs = rnq.rmsnorm_rope_fp8_grouped(xg, wg, cg, sg, group_size=N, rows_per_token=rpt)
    torch.cuda.synchronize()
    assert torch.equal(uc.view(torch.uint8).cpu(), fc.view(torch.uint8).cpu())
    assert torch.equal(us.view(torch.int32).cpu(), fs.view(-1).view(torch.int32).cpu())
    _check_per_row(f"unfused M{M}", x, w, cos, sin, uc, us, rpt)


def test_nrq_4k_fused_and_unfused_sampled():
    d = workloads.generate("nrq_4k")
    print("[baselines] nrq_4k", flush=True)
    xg, wg, cg, sg = gpu(d["x"]), gpu(d["w"]), gpu(d["cos"]), gpu(d["sin"])
    fc, fs = rnq.rmsnorm_rope_fp8_grouped(xg, wg, cg, sg, group_size=d["width"])
    uc, us = baselines.norm_rope_quant_unfused(xg, wg, cg, sg)
    torch.cuda.synchronize()
    assert torch.equal(uc.view(torch.uint8).cpu(), fc.view(torch.uint8).cpu())
    assert torch.equal(us.view(torch.int32).cpu(), fs.view(-1).view(torch.int32).cpu())
    rng = np.random.default_rng(5)
    rows = np.unique(np.r_[0, d["rows"] - 1, rng.choice(d["rows"], 128, replace=False)])
    _check_per_row("nrq_4k", d["x"], d["w"], d["cos"], d["sin"], fc, fs, 1, rows)


def _design_equals_rows_kernel(name, d, rpbs):
    ref = run_qk_gpu(d)
    q, k = gpu(d["q"]), gpu(d["k"])
    for rpb in rpbs:
        print(f"[baselines] {name} design rows_per_block {rpb}", flush=True)
        q8, k8, qs, ks = baselines.qk_design(q, k, gpu(d["wq"]), gpu(d["wk"]), gpu(d["cos"]), gpu(d["sin"]),
                                             rows_per_block=rpb)
        torch.cuda.synchronize()
        assert np.array_equal(q8.view(torch.uint8).cpu().numpy(), ref["q_codes"]), f"{name} rpb {rpb}: q codes"
        assert np.array_equal(k8.view(torch.uint8).cpu().numpy(), ref["k_codes"]), f"{name} rpb {rpb}: k codes"
        assert np.array_equal(qs.cpu().numpy().view(np.uint32), ref["q_scale"].view(np.uint32))
        assert np.array_equal(ks.cpu().numpy().view(np.uint32), ref["k_scale"].view(np.uint32))


def test_designs_abc_equal_row_kernel_qk_4k():
    d = workloads.generate("qk_4k")
    _design_equals_rows_kernel("qk_4k", d, [1, 8, 40])


@pytest.mark.parametrize("D,R,Hq,Hk,rpbs", [(64, 32, 6, 2, [1, 2, 8]), (256, 128, 4, 4, [1, 4, 8]),
                                            (512, 512, 2, 2, [1, 2])])
def test_designs_other_widths(D, R, Hq, Hk, rpbs):
    g = torch.Generator("cpu").manual_seed(D + R)
    T = 37
    cos, sin = workloads.rope_table(np.arange(T), R, 10000.0)
    d = {"q": torch.randn(T, Hq, D, generator=g).to(torch.bfloat16),
         "k": torch.randn(T, Hk, D, generator=g).to(torch.bfloat16),
         "wq": (1 + 0.1 * torch.randn(D, generator=g)).to(torch.bfloat16),
         "wk": (1 + 0.1 * torch.randn(D, generator=g)).to(torch.bfloat16),
         "cos": torch.from_numpy(cos), "sin": torch.from_numpy(sin)}
    _design_equals_rows_kernel(f"D{D}", d, rpbs)


def test_stream_floor_kernel():
    """The memory-floor kernel writes, for every 2 KB block of src, the XOR of its two halves."""
    g = torch.Generator("cpu").manual_seed(5)
    src = torch.randint(0, 256, (7 * 2048,), dtype=torch.uint8, generator=g)
    dst = torch.full((7 * 1024 + 64,), 0xAB, dtype=torch.uint8)
    sg, dg = gpu(src), gpu(dst)
    baselines.prepare_stream(sg, dg)()
    baselines.prepare_stream(None)()  # one empty workgroup
    torch.cuda.synchronize()
    blocks = src.numpy().reshape(7, 2, 1024)
    want = np.bitwise_xor(blocks[:, 0], blocks[:, 1]).reshape(-1)
    got = dg.cpu().numpy()
    assert np.array_equal(got[: 7 * 1024], want) and np.all(got[7 * 1024:] == 0xAB)

