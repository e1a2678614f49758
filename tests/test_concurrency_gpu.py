"""Calls from several host threads on several streams at once: the library keeps
no shared mutable state, so concurrent calls on different streams give the
same bytes as the same calls made one after another.
"""

from __future__ import annotations

import threading

import pytest
import torch

import fp8_quant_amd as rnq
import workloads

from _parity import gpu

pytestmark = pytest.mark.gpu


def _inputs(seed, T=96, Hq=16, Hk=8, D=128):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(T, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(T, Hk, D, generator=g).to(torch.bfloat16)
    wq = (1 + 0.1 * torch.randn(D, generator=g)).to(torch.bfloat16)
    wk = (1 + 0.1 * torch.randn(D, generator=g)).to(torch.bfloat16)
    cos, sin = workloads.rope_table(torch.arange(T).numpy() * (seed % 7 + 1), D, 10000.0)
    return [gpu(t) for t in (q, k, wq, wk, torch.from_numpy(cos), torch.from_numpy(sin))]


def _bytes(out):
    return [t.view(torch.uint8).cpu() if t.dtype == torch.float8_e4m3fn else t.view(torch.int32).cpu() for t in out]


def test_concurrent_streams_match_serial_calls():
    n_threads, reps = 4, 8
    args = [_inputs(1000 + i) for i in range(n_threads)]
    print("[concurrency] serial reference", flush=True)
    ref = [_bytes(rnq.qk_norm_rope_fp8(*a)) for a in args]
    torch.cuda.synchronize()

    results = [None] * n_threads
    errors = []
    gate = threading.Barrier(n_threads)

    def worker(i):
        try:
            s = torch.cuda.Stream()  # default priority
            with torch.cuda.stream(s):
                gate.wait()
                outs = [rnq.qk_norm_rope_fp8(*args[i]) for _ in range(reps)]
            s.synchronize()
            results[i] = [_bytes(o) for o in outs]
        except Exception as e:  # reported below, with the thread that raised it
            errors.append((i, repr(e)))

    print(f"[concurrency] {n_threads} threads x {reps} calls on their own streams", flush=True)
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(n_threads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(n_threads):
        for rep in results[i]:
            for got, want in zip(rep, ref[i]):
                assert torch.equal(got, want), f"thread {i} differs from the serial call"
