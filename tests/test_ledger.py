"""The ledger reproduces the pages' byte/FLOP models exactly, and the library's own counts."""

import json
import os

import pytest

from fp8_quant_amd import ledger

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ledger_pages.json")))


def test_p3_case_study_defaults():
    g = GOLD["p3_case_study"]
    s = ledger.QKShape()
    assert s.rows == g["rows"] and s.elems == g["elems"]
    assert ledger.p3_flops(s) == g["flops"]
    ideal = ledger.p3_ideal_bytes(s)
    assert ideal["payload"] == g["payload"]
    assert ideal["lookup"] == g["ideal_lookup"]
    assert ideal["total"] == g["ideal_total"]
    assert round(ledger.p3_flops(s) / ideal["total"], 3) == g["ai_3dp"]
    bw = 4502.4e9
    assert round(ideal["total"] / bw * 1e6, 3) == g["roof_us_at_4502_4"]
    for d, gd in zip(ledger.p3_designs(s, 8), g["designs"]):
        for key in ("rows_per_block", "grid", "waves", "on_chip", "lookup", "total"):
            assert d[key] == gd[key], (gd["name"], key)
        assert d["fits"]
        assert round(d["total"] / ideal["total"], 2) == gd["vs_ideal_2dp"]
        assert round(100 * d["lookup"] / d["total"], 1) == gd["lookup_share_pct_1dp"]
        assert round(d["total"] / bw * 1e6, 3) == gd["floor_us_3dp"]


def test_p3_on_chip_budget_flags_oversized_design():
    s = ledger.QKShape(on_chip_budget=16 * 1024)
    fits = [d["fits"] for d in ledger.p3_designs(s, 8)]
    assert fits == [True, True, False]


def test_p4_plan_pairs():
    g = GOLD["p4_ledger"]
    ais = []
    for (unf, fus), gp in zip(ledger.p4_plans(), g["pairs"]):
        assert unf["moved"] == gp["unfused_moved"] and fus["moved"] == gp["fused_moved"]
        assert unf["flops"] == gp["unfused_flops"] and fus["flops"] == gp["fused_flops"]
        assert round(unf["moved"] / 1e6, 4) == gp["unfused_mb"]
        assert round(fus["moved"] / 1e6, 4) == gp["fused_mb"]
        assert round(unf["moved"] / fus["moved"], 4) == gp["bytes_ratio"]
        assert round(unf["ai"], 6) == gp["unfused_ai"] and round(fus["ai"], 6) == gp["fused_ai"]
        assert fus["moved"] < unf["moved"]  # fusion always moves fewer bytes
        assert fus["kernels"] == 1 and unf["kernels"] > 1
        ais += [unf["ai"], fus["ai"]]
    assert [round(min(ais), 3), round(max(ais), 3)] == g["ai_range_3dp"]


def test_ledger_element_validation():
    with pytest.raises(ValueError):
        ledger.nbytes(4, "int3")
    with pytest.raises(ValueError):
        ledger.nbytes(-1, "float32")
    assert ledger.nbytes(3, "bfloat16") == 6 and ledger.nbytes(3, "float8_e4m3fn") == 3


def test_boundary_bytes_per_workload():
    g = GOLD["boundary_bytes"]
    b = ledger.qk_bytes(256, 1, 0, 128, 64, write_y=True)
    assert (b["reads"], b["writes"], b["total"]) == (g["qk_small"]["reads"], g["qk_small"]["writes"], g["qk_small"]["total"])
    assert ledger.qk_flops(256, 1, 0, 128, 64) == g["qk_small"]["flops"]
    assert ledger.rmsnorm_fwd_bytes(4096, 4096)["total"] == g["rmsnorm_4k_fwd"]["total"]
    assert ledger.rmsnorm_bwd_bytes(4096, 4096)["total"] == g["rmsnorm_4k_bwd"]["total"]
    b = ledger.norm_rope_bytes(16384, 128, 64)
    assert (b["reads"], b["writes"], b["total"]) == tuple(g["norm_rope_fp16"][k] for k in ("reads", "writes", "total"))
    for name, args in (("qk_4k", (4096, 32, 8, 128, 128)), ("qk_64k", (65536, 64, 8, 128, 128))):
        b = ledger.qk_bytes(*args)
        assert (b["reads"], b["writes"], b["total"]) == tuple(g[name][k] for k in ("reads", "writes", "total"))
        assert ledger.qk_flops(*args) == g[name]["flops"]
    # at full rope the chapter-28 FLOP rule and this library's agree
    assert ledger.qk_flops(4096, 32, 8, 128, 128) == ledger.p3_flops(ledger.QKShape())
