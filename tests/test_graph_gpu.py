"""The entry points under HIP graph capture: a graph holding the QK prologue,
the grouped quantiser and the RMSNorm backward (two kernels, with its
workspace) is replayed several times, with new inputs written by eager work
and a synchronisation between replays; every replay must give the bytes the
eager calls give on the same inputs. (No call records a memset: outputs and
workspace are written by the kernels themselves.)
"""

from __future__ import annotations

import pytest
import torch

import fp8_quant_amd as rnq
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _fill(bufs, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    for t in bufs:
        t.copy_(torch.randn(t.shape, generator=g).to(t.dtype))


def test_graph_replays_match_eager_calls():
    T, Hq, Hk, D = 64, 8, 8, 128
    M, N = 96, 1024
    q = torch.empty(T, Hq, D, dtype=torch.bfloat16, device=DEV)
    k = torch.empty(T, Hk, D, dtype=torch.bfloat16, device=DEV)
    x = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    gy = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    wq = torch.ones(D, dtype=torch.bfloat16, device=DEV)
    wk = (1.5 * torch.ones(D)).to(torch.bfloat16).to(DEV)
    w = torch.linspace(0.5, 1.5, N).to(torch.bfloat16).to(DEV)
    cos, sin = (torch.from_numpy(a).to(DEV) for a in workloads.rope_table(torch.arange(T).numpy(), D, 10000.0))
    gcos, gsin = (torch.from_numpy(a).to(DEV) for a in workloads.rope_table(torch.arange(M).numpy(), 128, 10000.0))

    # outputs and workspace, allocated once, before capture
    q8 = torch.empty(T, Hq, D, dtype=torch.uint8, device=DEV)
    k8 = torch.empty(T, Hk, D, dtype=torch.uint8, device=DEV)
    qs = torch.empty(T, Hq, device=DEV)
    ks = torch.empty(T, Hk, device=DEV)
    codes = torch.empty(M, N, dtype=torch.uint8, device=DEV)
    scales = torch.empty(M, N // 128, device=DEV)
    gx = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    gw = torch.empty(N, device=DEV)
    ws = torch.empty(rnq.rnq_rmsnorm_bwd_workspace_size(M, N), dtype=torch.uint8, device=DEV)
    outs = (q8, k8, qs, ks, codes, scales, gx, gw)

    side = torch.cuda.Stream()  # default priority
    calls = [
        rnq.prepare_qk_norm_rope_fp8(q, k, wq, wk, cos, sin, q8, k8, qs, ks, stream=side),
        rnq.prepare_rmsnorm_rope_fp8_grouped(x, w, gcos, gsin, codes, scales, group_size=128, stream=side),
        rnq.prepare_rmsnorm_bwd(x, w, gy, gx, gw, ws, stream=side),
    ]

    def eager(seed):
        _fill((q, k, x, gy), seed)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for c in calls:
                c()
        side.synchronize()
        return [o.clone() for o in outs]

    expect = {seed: eager(seed) for seed in (1, 2, 3)}

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for c in calls:
            c()
    torch.cuda.synchronize()

    for rep, seed in enumerate((1, 2, 3, 2, 1, 3)):
        print(f"[graph] replay {rep} on inputs {seed}", flush=True)
        for o in outs:
            o.fill_(0)  # eager work between replays (a fill kernel, not a memset node)
        _fill((q, k, x, gy), seed)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("q8", "k8", "qs", "ks", "codes", "scales", "gx", "gw"), outs, expect[seed]):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {rep}: {name} differs"
