"""GPU parity of the strided / position-indexed entry points
(rnq_qk_norm_rope_fp8_ex, rnq_rmsnorm_rope_ex) against the CPU oracle.

The oracle computes on values, so the inputs are handed to it contiguous and
with the cos/sin rows already gathered (table row positions[t], clamped into
the table, for token t). Bar: bit-exact on rows whose sum of squares the
oracle proves exact, the stated tolerances elsewhere (as for the contiguous
entry points).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_quant_amd as rnq
import oracle
import workloads

from _parity import assert_rows_match, compare_qk, gpu, unproven_rows

pytestmark = pytest.mark.gpu

DT = {torch.bfloat16: "bf16", torch.float16: "fp16"}


def _fused(T, Hq, Hk, D, seed, dtype=torch.bfloat16, extra=0):
    """q, k (contiguous copies) and a [T, (Hq + 2 Hk) * D + extra] buffer holding them."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(T, Hq, D, generator=g).to(dtype)
    k = torch.randn(T, Hk, D, generator=g).to(dtype)
    v = torch.randn(T, Hk * D + extra, generator=g).to(dtype)
    qkv = torch.cat([q.reshape(T, -1), k.reshape(T, -1), v], 1)
    wq = (1 + 0.1 * torch.randn(D, generator=g)).to(dtype)
    wk = (1 + 0.1 * torch.randn(D, generator=g)).to(dtype)
    return q, k, qkv, wq, wk


def _views(qkv_gpu, T, Hq, Hk, D):
    q = qkv_gpu[:, : Hq * D].view(T, Hq, D)
    k = qkv_gpu[:, Hq * D : (Hq + Hk) * D].view(T, Hk, D) if Hk else None
    return q, k


def _run_ex(qv, kv, wq, wk, cos, sin, positions, with_y):
    T, Hq, D = qv.shape
    Hk = 0 if kv is None else kv.shape[1]
    dev = qv.device
    q8 = torch.full((T, Hq, D), 0xAB, dtype=torch.uint8, device=dev)
    k8 = torch.full((T, Hk, D), 0xAB, dtype=torch.uint8, device=dev) if Hk else None
    qs = torch.full((T, Hq), float("nan"), device=dev)
    ks = torch.full((T, Hk), float("nan"), device=dev) if Hk else None
    qy = torch.empty((T, Hq, D), dtype=qv.dtype, device=dev) if with_y else None
    ky = torch.empty((T, Hk, D), dtype=qv.dtype, device=dev) if with_y and Hk else None
    rnq.rnq_qk_norm_rope_fp8_ex(qv, kv, wq, wk if Hk else None, cos, sin, q8, k8, qs, ks, qy, ky,
                                positions=positions)
    torch.cuda.synchronize()
    return {"q_codes": q8.cpu().numpy(), "q_scale": qs.cpu().numpy(),
            "k_codes": None if k8 is None else k8.cpu().numpy(), "k_scale": None if ks is None else ks.cpu().numpy(),
            "q_y": None if qy is None else workloads.bits(qy), "k_y": None if ky is None else workloads.bits(ky)}


def _oracle(q, k, wq, wk, cos, sin, rows):
    """cos/sin rows ``rows`` (one per token) of the table."""
    Hk = 0 if k is None else k.shape[1]
    return oracle.qk_norm_rope_fp8(workloads.bits(q), workloads.bits(k) if Hk else None, workloads.bits(wq),
                                   workloads.bits(wk) if Hk else None, cos.numpy(), sin.numpy(),
                                   dtype=DT[q.dtype], tokens=np.asarray(rows))


@pytest.mark.parametrize("T,Hq,Hk,D,R,extra,with_pos", [
    (64, 32, 8, 128, 128, 0, True),     # aligned passes (heads multiples of 8), fused QKV, positions
    (50, 3, 2, 128, 64, 8, True),       # per-lane rows (odd head counts), padded token stride
    (33, 4, 4, 64, 16, 0, False),       # strides only, per-token table
    (17, 2, 1, 256, 128, 24, True),
    (9, 1, 1, 512, 512, 0, True),
    (40, 0, 3, 128, 64, 0, True),       # k heads only
])
def test_qk_fused_views_and_positions(T, Hq, Hk, D, R, extra, with_pos):
    q, k, qkv, wq, wk = _fused(T, Hq, Hk, D, seed=T * 7 + Hq + D + extra, extra=extra)
    g = torch.Generator("cpu").manual_seed(T + R)
    table_rows = 3 * T if with_pos else T
    cos, sin = workloads.rope_table(np.arange(table_rows) * 5 % 10007, R, 10000.0)
    cos, sin = torch.from_numpy(cos), torch.from_numpy(sin)
    pos = torch.randint(0, table_rows, (T,), generator=g, dtype=torch.int32) if with_pos else None
    print(f"[strided] T{T} Hq{Hq} Hk{Hk} D{D} R{R} extra {extra} positions {with_pos}", flush=True)
    qkv_g = gpu(qkv)
    qv, kv = _views(qkv_g, T, Hq, Hk, D)
    if Hq == 0:  # k heads only: k goes in the first slot as for the contiguous entry
        qv = qkv_g[:, :0].view(T, 0, D)
    got = _run_ex(qv, kv, gpu(wq), gpu(wk), gpu(cos), gpu(sin), None if pos is None else gpu(pos), with_y=True)
    rows = np.arange(T) if pos is None else pos.numpy()
    ref = _oracle(q, k, wq, wk, cos, sin, rows)
    compare_qk(f"strided T{T} Hq{Hq} Hk{Hk} D{D}", {"q": q, "k": k}, got, ref)


def test_qk_positions_out_of_range_read_the_last_row():
    T, Hq, Hk, D, R = 32, 8, 8, 128, 128
    q, k, qkv, wq, wk = _fused(T, Hq, Hk, D, seed=501)
    table_rows = 20
    cos, sin = workloads.rope_table(np.arange(table_rows) + 3, R, 10000.0)
    cos, sin = torch.from_numpy(cos), torch.from_numpy(sin)
    pos = torch.arange(T, dtype=torch.int32) - 6  # -6 .. 25: negative and past-the-end positions
    print("[strided] clamped positions", flush=True)
    qv, kv = _views(gpu(qkv), T, Hq, Hk, D)
    got = _run_ex(qv, kv, gpu(wq), gpu(wk), gpu(cos), gpu(sin), gpu(pos), with_y=False)
    p = pos.numpy().astype(np.int64)
    rows = np.where((p < 0) | (p >= table_rows), table_rows - 1, p)
    ref = _oracle(q, k, wq, wk, cos, sin, rows)
    compare_qk("clamped positions", {"q": q, "k": k}, got, ref)


@pytest.mark.parametrize("T,H,D,R,extra,with_y,dtype", [
    (24, 4, 128, 128, 8, True, torch.bfloat16),   # 2 tokens per pass of 8 rows, padded token stride
    (40, 1, 128, 64, 0, True, torch.bfloat16),    # one row per token: 8 tokens per pass
    (36, 2, 256, 128, 16, True, torch.bfloat16),  # 2 tokens per pass of 4 rows
    (20, 1, 512, 256, 0, True, torch.bfloat16),   # 2 tokens per pass of 2 rows
    (32, 8, 64, 32, 8, True, torch.bfloat16),     # 2 tokens per pass of 16 rows
    (24, 4, 128, 128, 0, False, torch.bfloat16),  # codes and scales only
    (40, 2, 128, 32, 8, False, torch.float16),    # fp16, rope on the last quarter
    (48, 1, 64, 64, 0, True, torch.float16),      # fp16, one row per token: 16 tokens per pass
])
def test_qk_one_tensor_whole_tokens_per_pass_with_positions(T, H, D, R, extra, with_y, dtype):
    """One tensor whose passes hold whole tokens (its heads divide the rows per
    pass): each rope lane gathers its own token's table row; positions below zero
    or past the table's end read its last row."""
    q, _, qkv, wq, _ = _fused(T, H, 0, D, seed=T * 11 + H + D, dtype=dtype, extra=extra)
    table_rows = T // 2 + 3
    cos, sin = workloads.rope_table(np.arange(table_rows) * 7 % 8191, R, 10000.0)
    cos, sin = torch.from_numpy(cos), torch.from_numpy(sin)
    g = torch.Generator("cpu").manual_seed(T + D)
    pos = torch.randint(-3, table_rows + 4, (T,), generator=g, dtype=torch.int32)
    print(f"[strided] one tensor, whole tokens per pass: T{T} H{H} D{D} R{R} extra {extra}", flush=True)
    qv, _ = _views(gpu(qkv), T, H, 0, D)
    got = _run_ex(qv, None, gpu(wq), None, gpu(cos), gpu(sin), gpu(pos), with_y=with_y)
    p = pos.numpy().astype(np.int64)
    rows = np.where((p < 0) | (p >= table_rows), table_rows - 1, p)
    ref = _oracle(q, None, wq, None, cos, sin, rows)
    compare_qk(f"one tensor T{T} H{H} D{D}", {"q": q, "k": None}, got, ref, dtype=DT[dtype])


def test_qk_4k_fused_full_size_matches_contiguous_entry():
    """The fused-QKV workload at full size: bit-identical to the contiguous entry on
    gathered tables (the same arithmetic), and to the oracle on sampled tokens."""
    d = workloads.generate("qk_4k_fused")
    T, Hq, Hk, D = d["tokens"], d["q_heads"], d["kv_heads"], d["head_dim"]
    print(f"[strided] qk_4k_fused: qkv{tuple(d['qkv'].shape)} table{tuple(d['cos'].shape)}", flush=True)
    qv, kv = _views(gpu(d["qkv"]), T, Hq, Hk, D)
    got = _run_ex(qv, kv, gpu(d["wq"]), gpu(d["wk"]), gpu(d["cos"]), gpu(d["sin"]), gpu(d["positions"]),
                  with_y=False)
    pos = d["positions"].numpy().astype(np.int64)
    gathered = {"q": d["q"], "k": d["k"], "wq": d["wq"], "wk": d["wk"],
                "cos": d["cos"][pos].contiguous(), "sin": d["sin"][pos].contiguous()}
    from _parity import run_qk_gpu
    ref_gpu = run_qk_gpu(gathered)
    for key in ("q_codes", "k_codes", "q_scale", "k_scale"):
        assert np.array_equal(got[key].view(np.uint8), ref_gpu[key].view(np.uint8)), key
    rng = np.random.default_rng(3)
    toks = np.unique(np.r_[0, T - 1, rng.choice(T, 96, replace=False)])
    ref = _oracle(d["q"][toks], d["k"][toks], d["wq"], d["wk"], d["cos"], d["sin"], pos[toks])
    sub = {key: (None if v is None else v[toks]) for key, v in got.items()}
    compare_qk("qk_4k_fused sampled", {"q": d["q"][toks], "k": d["k"][toks]}, sub, ref)


def test_qk_allocating_wrapper_takes_views_and_positions():
    T, Hq, Hk, D, R = 24, 8, 8, 128, 64
    q, k, qkv, wq, wk = _fused(T, Hq, Hk, D, seed=502)
    cos, sin = workloads.rope_table(np.arange(100), R, 10000.0)
    pos = torch.arange(T, dtype=torch.int32) * 3
    qv, kv = _views(gpu(qkv), T, Hq, Hk, D)
    q8, k8, qs, ks = rnq.qk_norm_rope_fp8(qv, kv, gpu(wq), gpu(wk), gpu(torch.from_numpy(cos)),
                                          gpu(torch.from_numpy(sin)), positions=gpu(pos))
    torch.cuda.synchronize()
    ref = _oracle(q, k, wq, wk, torch.from_numpy(cos), torch.from_numpy(sin), pos.numpy())
    got = {"q_codes": q8.view(torch.uint8).cpu().numpy(), "k_codes": k8.view(torch.uint8).cpu().numpy(),
           "q_scale": qs.cpu().numpy(), "k_scale": ks.cpu().numpy(), "q_y": None, "k_y": None}
    compare_qk("wrapper", {"q": q, "k": k}, got, ref)


# ------------------------------------------------------------------ rnq_rmsnorm_rope_ex


def test_norm_rope_pos_full_size():
    d = workloads.generate("norm_rope_pos")
    print(f"[strided] norm_rope_pos: x{tuple(d['x'].shape)} table{tuple(d['cos'].shape)}", flush=True)
    y = rnq.rmsnorm_rope(gpu(d["x"]), gpu(d["w"]), gpu(d["cos"]), gpu(d["sin"]), positions=gpu(d["positions"]))
    torch.cuda.synchronize()
    pos = d["positions"].numpy().astype(np.int64)
    ref = oracle.rmsnorm_rope(workloads.bits(d["x"]), workloads.bits(d["w"]), d["cos"].numpy()[pos],
                              d["sin"].numpy()[pos], 1e-6, "fp16")
    loose = unproven_rows(workloads.bits(d["x"]), "fp16")
    assert_rows_match("norm_rope_pos", workloads.bits(y), None, None, ref, None, None, loose)


@pytest.mark.parametrize("M,N,R,rpt,pad,with_pos", [
    (300, 128, 64, 1, 8, True),     # row-strided x, one table row per row
    (96, 64, 32, 4, 16, True),      # [T, 4, N] view with padded token stride
    (80, 256, 128, 8, 0, False),    # contiguous x, per-token table
    (40, 512, 256, 2, 24, True),
    (256, 128, 64, 1, 8, False),    # row-strided x, whole tokens per pass (8 rows of 8 tokens)
    (96, 64, 32, 4, 16, False),     # [T, 4, N] view with padded stride, 4 tokens per pass
])
def test_rmsnorm_rope_ex_views(M, N, R, rpt, pad, with_pos):
    T = M // rpt
    g = torch.Generator("cpu").manual_seed(M + N + R)
    x = torch.randn(M, N, generator=g).to(torch.bfloat16)
    w = (1 + 0.1 * torch.randn(N, generator=g)).to(torch.bfloat16)
    buf = torch.randn(T, rpt * N + pad, generator=g).to(torch.bfloat16)
    buf[:, : rpt * N] = x.view(T, rpt * N)
    table_rows = 2 * T if with_pos else T
    cos, sin = workloads.rope_table(np.arange(table_rows) * 3, R, 10000.0)
    pos = torch.randint(0, table_rows, (T,), generator=g, dtype=torch.int32) if with_pos else None
    print(f"[strided] rmsnorm_rope_ex M{M} N{N} R{R} rpt{rpt} pad{pad} positions {with_pos}", flush=True)
    bg = gpu(buf)
    xv = bg[:, : rpt * N].view(T, rpt, N) if rpt > 1 else bg[:, :N]
    y = rnq.rmsnorm_rope(xv, gpu(w), gpu(torch.from_numpy(cos)), gpu(torch.from_numpy(sin)), rows_per_token=rpt,
                         positions=None if pos is None else gpu(pos))
    torch.cuda.synchronize()
    rows = np.arange(T) if pos is None else pos.numpy().astype(np.int64)
    ref = oracle.rmsnorm_rope(workloads.bits(x), workloads.bits(w), cos[rows], sin[rows], 1e-6, "bf16", rpt)
    loose = unproven_rows(workloads.bits(x), "bf16")
    assert_rows_match(f"rmsnorm_rope_ex M{M} N{N}", workloads.bits(y), None, None, ref, None, None, loose)


@pytest.mark.parametrize("M,N,R,rpt,pad", [
    (256, 128, 64, 1, 0),   # 8 tokens per pass
    (128, 64, 32, 4, 8),    # 4 tokens per pass of 16 rows, padded token stride
    (96, 256, 128, 2, 16),  # 2 tokens per pass of 4 rows
])
def test_rmsnorm_rope_whole_tokens_per_pass_positions_out_of_range(M, N, R, rpt, pad):
    """Path R with positions on passes of whole tokens: every lane gathers its
    token's table row; out-of-range positions read the table's last row."""
    T = M // rpt
    g = torch.Generator("cpu").manual_seed(M * 3 + N + R)
    x = torch.randn(M, N, generator=g).to(torch.float16)
    w = (1 + 0.1 * torch.randn(N, generator=g)).to(torch.float16)
    buf = torch.randn(T, rpt * N + pad, generator=g).to(torch.float16)
    buf[:, : rpt * N] = x.view(T, rpt * N)
    table_rows = T // 3 + 2
    cos, sin = workloads.rope_table(np.arange(table_rows) * 5, R, 10000.0)
    pos = torch.randint(-4, table_rows + 5, (T,), generator=g, dtype=torch.int32)
    print(f"[strided] rmsnorm_rope whole tokens per pass M{M} N{N} R{R} rpt{rpt} pad{pad}", flush=True)
    bg = gpu(buf)
    xv = bg[:, : rpt * N].view(T, rpt, N) if rpt > 1 else bg[:, :N]
    y = rnq.rmsnorm_rope(xv, gpu(w), gpu(torch.from_numpy(cos)), gpu(torch.from_numpy(sin)), rows_per_token=rpt,
                         positions=gpu(pos))
    torch.cuda.synchronize()
    p = pos.numpy().astype(np.int64)
    rows = np.where((p < 0) | (p >= table_rows), table_rows - 1, p)
    ref = oracle.rmsnorm_rope(workloads.bits(x), workloads.bits(w), cos[rows], sin[rows], 1e-6, "fp16", rpt)
    loose = unproven_rows(workloads.bits(x), "fp16")
    assert_rows_match(f"rmsnorm_rope whole tokens M{M} N{N}", workloads.bits(y), None, None, ref, None, None, loose)


@pytest.mark.parametrize("past", [False, True])
def test_rmsnorm_rope_positions_table_near_2gib(past):
    """Whole-token passes gather table rows at 32-bit byte offsets: a table just below
    2 GiB per half takes that path with rows near its end, one just past it the
    per-lane layout (64-bit addressing). Only the rows the positions name are written."""
    M, N, R, rpt = 64, 128, 64, 1
    half = R // 2
    limit = (1 << 31) // (4 * half)  # table rows at which one table reaches 2 GiB
    table_rows = limit + 8 if past else limit - 1
    g = torch.Generator("cpu").manual_seed(991 + past)
    x = torch.randn(M, N, generator=g).to(torch.float16)
    w = (1 + 0.1 * torch.randn(N, generator=g)).to(torch.float16)
    last = table_rows - 1
    pos = torch.tensor([last, last - 1, 0, 5, last - 77, table_rows, -1, last - 3] * (M // 8), dtype=torch.int32)
    rows = np.where((pos.numpy() < 0) | (pos.numpy() >= table_rows), last, pos.numpy()).astype(np.int64)
    used = np.unique(rows)
    cu, su = workloads.rope_table(used % 8191 + 1, R, 10000.0)
    print(f"[strided] table of {table_rows} rows ({'past' if past else 'below'} 2 GiB per half)", flush=True)
    cos_g = torch.empty((table_rows, half), dtype=torch.float32, device="cuda")
    sin_g = torch.empty((table_rows, half), dtype=torch.float32, device="cuda")
    idx = torch.from_numpy(used).cuda()
    cos_g[idx] = torch.from_numpy(cu).cuda()
    sin_g[idx] = torch.from_numpy(su).cuda()
    y = rnq.rmsnorm_rope(gpu(x), gpu(w), cos_g, sin_g, rows_per_token=rpt, positions=gpu(pos))
    torch.cuda.synchronize()
    where = {r: i for i, r in enumerate(used)}
    sel = np.array([where[r] for r in rows])
    ref = oracle.rmsnorm_rope(workloads.bits(x), workloads.bits(w), cu[sel], su[sel], 1e-6, "fp16", rpt)
    del cos_g, sin_g
    torch.cuda.empty_cache()
    loose = unproven_rows(workloads.bits(x), "fp16")
    assert_rows_match(f"rmsnorm_rope table near 2 GiB past={past}", workloads.bits(y), None, None, ref, None, None,
                      loose)


def test_strided_invalid_arguments_raise():
    T, Hq, Hk, D = 8, 2, 2, 128
    q, k, qkv, wq, wk = _fused(T, Hq, Hk, D, seed=503)
    cos, sin = (torch.from_numpy(a) for a in workloads.rope_table(np.arange(T), 64, 10000.0))
    dev = torch.device("cuda")
    q8 = torch.empty((T, Hq, D), dtype=torch.uint8, device=dev)
    qs = torch.empty((T, Hq), device=dev)
    print("[strided] invalid arguments", flush=True)
    big = gpu(torch.zeros(T, Hq * D + 4, dtype=torch.bfloat16))
    with pytest.raises(rnq.RnqError, match="UNSUPPORTED"):  # token stride not a multiple of 8 elements
        rnq.rnq_qk_norm_rope_fp8_ex(big[:, : Hq * D].view(T, Hq, D), None, gpu(wq), None, gpu(cos), gpu(sin), q8,
                                    None, qs, None)
    with pytest.raises(TypeError):  # positions must be int32
        rnq.rnq_qk_norm_rope_fp8_ex(gpu(q), None, gpu(wq), None, gpu(cos), gpu(sin), q8, None, qs, None,
                                    positions=gpu(torch.arange(T)))


@pytest.mark.parametrize("Hq,Hk", [(8, 8), (3, 1)])  # aligned passes, per-lane rows
def test_token_stride_beyond_32_bits(Hq, Hk):
    """Two tokens 2^31 + 8 elements apart (an 8.6 GB buffer): the input offsets are 64-bit."""
    T, D, R = 2, 128, 128
    stride = (1 << 31) + 8
    q, k, _, wq, wk = _fused(T, Hq, Hk, D, seed=504 + Hq)
    cos, sin = (torch.from_numpy(a) for a in workloads.rope_table(np.arange(T), R, 10000.0))
    print(f"[strided] token stride 2^31 + 8, Hq{Hq} Hk{Hk}", flush=True)
    buf = torch.empty(T * stride, dtype=torch.bfloat16, device="cuda")
    view = buf.as_strided((T, Hq + Hk, D), (stride, D, 1))
    view.copy_(gpu(torch.cat([q, k], 1)))
    qv = buf.as_strided((T, Hq, D), (stride, D, 1))
    kv = buf.as_strided((T, Hk, D), (stride, D, 1), Hq * D)
    got = _run_ex(qv, kv, gpu(wq), gpu(wk), gpu(cos), gpu(sin), None, with_y=True)
    del buf, view, qv, kv
    torch.cuda.empty_cache()
    ref = _oracle(q, k, wq, wk, cos, sin, np.arange(T))
    compare_qk("stride 2^31+8", {"q": q, "k": k}, got, ref)
