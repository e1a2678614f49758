"""The C ABI used from plain C: tests/csrc/c_client.c includes only
include/rnq.h and the HIP runtime's C API, and links librnq.so.

CPU: the client compiles as strict C99 (-Wall -Wextra -Werror) against the
header, and the argument-validation statuses it checks come back as the
header documents them (no launch, no GPU needed).
GPU: the client runs rnq_qk_norm_rope_fp8 on a seeded problem read from a
file; its codes and scales match the oracle bit for bit on the rows whose
fp64 sum of squares is proven exact (the others within the parity tolerances).
"""

from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import _c_client
import fp8_quant_amd as rnq
import workloads
from _parity import assert_rows_match, oracle_qk, unproven_rows

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "fp8_quant_amd", "librnq.so")


def _need_build_tools():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(LIB):
        pytest.skip("librnq.so not built (python -m fp8_quant_amd.build)")


def test_c_client_compiles_as_c99_and_gets_the_documented_statuses(tmp_path):
    _need_build_tools()
    exe = _c_client.build(str(tmp_path / "c_client"))
    pr = subprocess.run([exe, "errors"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=60)
    assert pr.returncode == 0, pr.stdout
    lines = pr.stdout.strip().splitlines()
    assert lines == [
        "head_dim 96: RNQ_ERR_UNSUPPORTED: width or alignment not supported",
        "odd rope_dim: RNQ_ERR_SHAPE: invalid shape",
        "missing q: RNQ_ERR_NULL: a required pointer is NULL",
        "fp8_max 500: RNQ_ERR_ARG: invalid scalar argument",
        "zero rows: RNQ_OK",
    ], pr.stdout


@pytest.mark.gpu
def test_c_client_runs_the_prologue_bit_exact(tmp_path):
    if not os.path.exists(_c_client.EXE):
        pytest.fail("tests/bin/c_client is not built: run __graft_entry__.build() before the GPU tests")
    T, Hq, Hk, D, R = 37, 4, 2, 128, 64
    g = torch.Generator("cpu").manual_seed(2024)
    d = {"q": torch.randn(T, Hq, D, generator=g).to(torch.bfloat16),
         "k": torch.randn(T, Hk, D, generator=g).to(torch.bfloat16),
         "wq": (1 + 0.1 * torch.randn(D, generator=g)).to(torch.bfloat16),
         "wk": (1 + 0.1 * torch.randn(D, generator=g)).to(torch.bfloat16)}
    cos, sin = workloads.rope_table(np.arange(T) * 3, R, 10000.0)
    d["cos"], d["sin"] = torch.from_numpy(cos), torch.from_numpy(sin)
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        f.write(np.array([T, Hq, Hk, D, R, rnq.RNQ_BF16], dtype="<i8").tobytes())
        for part in ("q", "k", "wq", "wk"):
            f.write(workloads.bits(d[part]).astype("<u2").tobytes())
        f.write(cos.astype("<f4").tobytes())
        f.write(sin.astype("<f4").tobytes())
    out = tmp_path / "out.bin"
    print(f"[c_client] qk T{T} Hq{Hq} Hk{Hk} D{D} R{R} bf16", flush=True)
    pr = subprocess.run([_c_client.EXE, "qk", str(src), str(out)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                        text=True, timeout=120)
    assert pr.returncode == 0, pr.stdout
    raw = out.read_bytes()
    nq, nk = T * Hq * D, T * Hk * D
    assert len(raw) == nq + nk + 4 * T * (Hq + Hk)
    got = {"q_codes": np.frombuffer(raw, np.uint8, nq).reshape(T, Hq, D),
           "k_codes": np.frombuffer(raw, np.uint8, nk, nq).reshape(T, Hk, D),
           "q_scale": np.frombuffer(raw, "<f4", T * Hq, nq + nk).reshape(T, Hq),
           "k_scale": np.frombuffer(raw, "<f4", T * Hk, nq + nk + 4 * T * Hq).reshape(T, Hk)}
    ref = oracle_qk(d)
    for part in ("q", "k"):
        loose = unproven_rows(workloads.bits(d[part]), "bf16")
        print(f"[c_client] {part}: {int((~loose).sum())} of {loose.size} rows proven exact", flush=True)
        assert (~loose).sum() >= loose.size // 2
        assert_rows_match(f"c_client/{part}", None, got[part + "_codes"], got[part + "_scale"], None,
                          ref[part + "_codes"], ref[part + "_scale"], loose)
