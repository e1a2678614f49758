"""Byte and FLOP ledger of the prologue (host-side bookkeeping, no device work).

Two models from the tilelang-tutorial pages are restated here so that the
measurements can be put next to them, plus the algorithmic byte count that
this library's GB/s figures use as their numerator.

* Chapter 13 ledger page (``ledger.py``): one kernel reads each input once
  and writes each output once; an intermediate tensor counts as a write of
  one kernel and a read of the next; add/sub/mul/div/max and each
  transcendental count one FLOP. Five unfused/fused plan pairs are modelled.
* Chapter 28 case-study page (``case_norm_rope_quant.py``): the QK-norm +
  RoPE + fp8 operator, its FLOP rule, its payload bytes, and the lookup
  bytes (norm weights and the cos/sin table) under three block designs:
  A = one row per block, B = a few rows per block, C = one token per block.

The chapter-28 model counts the table as 2 * tokens * head_dim * 4 bytes
(cos and sin at full head width); this library's boundary takes half-width
tables ``[tokens, rope_dim/2]`` so its own count (``qk_bytes``) is smaller.
"""

from __future__ import annotations

import dataclasses
import math

__all__ = [
    "BYTES_PER_ELEM",
    "nbytes",
    "plan_cost",
    "p4_plans",
    "QKShape",
    "p3_design",
    "p3_designs",
    "p3_ideal_bytes",
    "p3_flops",
    "qk_bytes",
    "norm_rope_bytes",
    "rmsnorm_fwd_bytes",
    "rmsnorm_bwd_bytes",
    "qk_flops",
]

BYTES_PER_ELEM = {"float32": 4, "float16": 2, "bfloat16": 2, "float8_e4m3fn": 1}


# ----------------------------------------------------------- chapter 13 ledger model
#
# The page's counting rules: every kernel launch reads each of its inputs once
# and writes each of its outputs once (so an intermediate costs a write in one
# launch and a read in the next), and add / sub / mul / div / max and each
# transcendental count one FLOP. Here a plan is a table with one row per launch
# -- (bytes read, bytes written, FLOPs) -- written straight from those rules.


def nbytes(count: int, dtype: str) -> int:
    """Bytes of ``count`` elements of ``dtype``."""
    if dtype not in BYTES_PER_ELEM:
        raise ValueError(f"no element width for dtype {dtype!r}")
    if count < 0:
        raise ValueError(f"element count must be >= 0 (got {count})")
    return count * BYTES_PER_ELEM[dtype]


def plan_cost(label: str, launches) -> dict:
    """Totals of a plan given as rows (bytes read, bytes written, FLOPs), one per launch."""
    moved = sum(r + w for r, w, _ in launches)
    flops = sum(f for _, _, f in launches)
    return {"label": label, "kernels": len(launches), "moved": moved, "flops": flops,
            "ai": flops / moved if moved else math.inf}


def _scale_add(n: int, dt: str):
    v = nbytes(n, dt)  # one vector
    # y = x * a + b: t = x * a, then y = t + b; fused, one launch
    return (plan_cost("scale+add, 2 kernels", [(v, v, n), (2 * v, v, n)]),
            plan_cost("scale+add, fused", [(2 * v, v, 2 * n)]))


def _rmsnorm(m: int, n: int, dt: str):
    big, row, wgt = nbytes(m * n, dt), nbytes(m, "float32"), nbytes(n, dt)
    eager = [
        (big, big, m * n),              # x * x
        (big, row, m * n),              # row sums of the squares
        (row, row, m),                  # + eps
        (row, row, m),                  # rsqrt
        (big + row, big, m * n),        # x * rstd
        (big + wgt, big, m * n),        # * w
    ]
    return (plan_cost("RMSNorm, 6 eager steps", eager),
            plan_cost("RMSNorm, fused", [(big + wgt, big, 4 * m * n + 2 * m)]))


def _layernorm(m: int, n: int, dt: str):
    big, row, vec = nbytes(m * n, dt), nbytes(m, "float32"), nbytes(n, dt)
    passes = [
        (big, big, m * n),              # x * x
        (big, row, m * n),              # row sums of x
        (big, row, m * n),              # row sums of x * x
        (big, big, m * n),              # x - mean
        (big, big, m * n),              # * rstd
        (big + 2 * vec, big, 2 * m * n),  # * g + b
    ]
    return (plan_cost("LayerNorm, multi-pass", passes),
            plan_cost("LayerNorm, fused", [(big + 2 * vec, big, 6 * m * n + 2 * m)]))


def _rope(tokens: int, heads: int, rope_dim: int, dt: str):
    values = tokens * heads * rope_dim
    big, tab = nbytes(values, dt), nbytes(values // 2, dt)
    steps = [
        (big, big, 0),                  # rotate_half(x)
        (2 * big, big, values),         # x * cos (broadcast to every value)
        (2 * big, big, values),         # rotated * sin
        (2 * big, big, values),         # sum
    ]
    return (plan_cost("RoPE, 4 steps", steps),
            plan_cost("RoPE, fused", [(big + 2 * tab, big, 3 * values)]))


def _norm_rope_quant(m: int, n: int, rope_dim: int, dt: str):
    big, wgt = nbytes(m * n, dt), nbytes(n, dt)
    tab = 2 * nbytes(m * rope_dim // 2, dt)  # cos and sin
    codes, amax = nbytes(m * n, "float8_e4m3fn"), nbytes(m, "float32")
    f_norm, f_rope, f_quant = 4 * m * n + 2 * m, 3 * m * rope_dim, 3 * m * n + m
    three = [
        (big + wgt, big, f_norm),           # RMSNorm writes the normalised rows
        (big + tab, big, f_rope),           # RoPE reads them back, writes the rotated rows
        (big, codes + amax, f_quant),       # the quantiser reads those
    ]
    one = [(big + wgt + tab, codes + amax, f_norm + f_rope + f_quant)]
    return plan_cost("norm+rope+quant, 3 kernels", three), plan_cost("norm+rope+quant, fused", one)


def p4_plans():
    """The chapter-13 ledger's five (unfused, fused) plan pairs at that page's default sizes."""
    return [
        _scale_add(1 << 20, "float32"),
        _rmsnorm(4096, 4096, "float16"),
        _layernorm(4096, 4096, "bfloat16"),
        _rope(4096, 32, 128, "float16"),
        _norm_rope_quant(4096, 4096, 128, "bfloat16"),
    ]


# ----------------------------------------------------------- chapter 28 design model


@dataclasses.dataclass(frozen=True)
class QKShape:
    tokens: int = 4096
    q_heads: int = 32
    kv_heads: int = 8
    head_dim: int = 128
    in_bytes: int = 2
    out_bytes: int = 1
    table_bytes: int = 4
    on_chip_budget: int = 192 * 1024
    sm_count: int = 132
    blocks_per_sm: int = 8

    @property
    def rows(self) -> int:
        return self.tokens * (self.q_heads + self.kv_heads)

    @property
    def elems(self) -> int:
        return self.rows * self.head_dim


def p3_flops(s: QKShape) -> int:
    """Chapter-28 FLOP rule: norm 2D + 3 + 2D per row, RoPE 6 per pair, absmax D, quant 2D."""
    d = s.head_dim
    return s.rows * (2 * d + 3 + 2 * d + 6 * (d // 2) + d + 2 * d)


def _p3_payload(s: QKShape) -> int:
    return s.elems * (s.in_bytes + s.out_bytes) + s.rows * 4


def _p3_weight_bytes(s: QKShape) -> int:
    return 2 * s.head_dim * s.in_bytes  # q weight and k weight


def _p3_table_bytes_per_token(s: QKShape) -> int:
    return 2 * s.head_dim * s.table_bytes  # cos and sin as the page counts them


def p3_ideal_bytes(s: QKShape) -> dict:
    payload = _p3_payload(s)
    lookup = _p3_weight_bytes(s) + s.tokens * _p3_table_bytes_per_token(s)
    return {"payload": payload, "lookup": lookup, "total": payload + lookup}


def p3_design(s: QKShape, name: str, rows_per_block: int, table_reads_per_token: float) -> dict:
    grid = math.ceil(s.rows / rows_per_block)
    lookup = grid * _p3_weight_bytes(s) + table_reads_per_token * s.tokens * _p3_table_bytes_per_token(s)
    payload = _p3_payload(s)
    d = s.head_dim
    on_chip = rows_per_block * (d * s.in_bytes + d * s.out_bytes + d * 4 + 4) + 2 * d * s.table_bytes
    resident = max(s.sm_count * s.blocks_per_sm, 1)
    return {
        "name": name,
        "rows_per_block": rows_per_block,
        "grid": grid,
        "waves": math.ceil(grid / resident),
        "on_chip": on_chip,
        "payload": payload,
        "lookup": lookup,
        "total": payload + lookup,
        "fits": on_chip <= s.on_chip_budget,
    }


def p3_designs(s: QKShape, rows_per_block_b: int = 8) -> list:
    per_token = s.q_heads + s.kv_heads
    return [
        p3_design(s, "A: one row per block", 1, float(per_token)),
        p3_design(s, f"B: {rows_per_block_b} rows per block", rows_per_block_b,
                  float(math.ceil(per_token / rows_per_block_b))),
        p3_design(s, "C: one whole token per block", per_token, 1.0),
    ]


# ----------------------------------------------- this library's algorithmic bytes


def qk_bytes(tokens, q_heads, kv_heads, head_dim, rope_dim, in_bytes=2, write_y=False) -> dict:
    """Bytes at the boundary of ``rnq_qk_norm_rope_fp8``: inputs read once, outputs written once,
    weights once per call and the token's cos/sin row (fp32, rope_dim/2 wide) once per token."""
    rows = tokens * (q_heads + kv_heads)
    reads = rows * head_dim * in_bytes + 2 * tokens * (rope_dim // 2) * 4
    reads += head_dim * in_bytes * ((q_heads > 0) + (kv_heads > 0))
    writes = rows * head_dim + rows * 4 + (rows * head_dim * in_bytes if write_y else 0)
    return {"rows": rows, "reads": reads, "writes": writes, "total": reads + writes}


def gathered_table_adjust(led: dict, tokens: int, rope_dim: int, unique_rows: int) -> dict:
    """Bytes of a call whose cos/sin rows are gathered through an int32 positions index:
    the per-token table term of ``led`` replaced by the distinct table rows touched (each
    read once) plus the 4-byte positions."""
    per_token = 2 * tokens * (rope_dim // 2) * 4
    reads = led["reads"] - per_token + 2 * unique_rows * (rope_dim // 2) * 4 + 4 * tokens
    out = dict(led, reads=reads)
    out["total"] = reads + led["writes"]
    return out


def qk_flops(tokens, q_heads, kv_heads, head_dim, rope_dim) -> int:
    """Chapter-28 rule with the RoPE term over rope_dim/2 pairs."""
    rows = tokens * (q_heads + kv_heads)
    d = head_dim
    return rows * (2 * d + 3 + 2 * d + 6 * (rope_dim // 2) + d + 2 * d)


def norm_rope_bytes(rows, width, rope_dim, rows_per_token=1, in_bytes=2) -> dict:
    tables = rows // rows_per_token
    reads = rows * width * in_bytes + width * in_bytes + 2 * tables * (rope_dim // 2) * 4
    writes = rows * width * in_bytes
    return {"rows": rows, "reads": reads, "writes": writes, "total": reads + writes}


def grouped_bytes(rows, width, rope_dim, group_size, rows_per_token=1, in_bytes=2, write_y=False) -> dict:
    """Bytes at the boundary of ``rnq_rmsnorm_rope_fp8_grouped``: x, the weight row and one
    cos/sin row per token read once; one code per element, one fp32 scale per group and
    (optionally) y written once."""
    tables = rows // rows_per_token
    reads = rows * width * in_bytes + width * in_bytes + 2 * tables * (rope_dim // 2) * 4
    writes = rows * width + rows * (width // group_size) * 4 + (rows * width * in_bytes if write_y else 0)
    return {"rows": rows, "reads": reads, "writes": writes, "total": reads + writes}


def rmsnorm_fwd_bytes(rows, width, in_bytes=2, write_rstd=False) -> dict:
    reads = rows * width * in_bytes + width * in_bytes
    writes = rows * width * in_bytes + (rows * 4 if write_rstd else 0)
    return {"rows": rows, "reads": reads, "writes": writes, "total": reads + writes}


def norm_rope_quant_bytes(rows, width, rope_dim, rows_per_token=1, group_size=None, in_bytes=2,
                          unfused=False) -> dict:
    """RMSNorm + RoPE + FP8 on [rows, width] rows with one scale per group (default: per row).
    Fused: x, the weight row and one cos/sin row per token read, codes and scales written.
    Unfused (three kernels, the ledger page's plan): the normalised and rotated rows are
    also written and read back once each."""
    g = width if group_size is None else group_size
    tables = rows // rows_per_token
    reads = rows * width * in_bytes + width * in_bytes + 2 * tables * (rope_dim // 2) * 4
    writes = rows * width + rows * (width // g) * 4
    if unfused:
        reads += 2 * rows * width * in_bytes
        writes += 2 * rows * width * in_bytes
    return {"rows": rows, "reads": reads, "writes": writes, "total": reads + writes}


def rope_bwd_bytes(rows, width, rope_dim, rows_per_token=1, in_bytes=2) -> dict:
    """Bytes at the boundary of ``rnq_rmsnorm_rope_bwd`` (rstd recomputed): x and grad_y
    read, the weight row and one cos/sin row per token read once, grad_x and fp32 grad_w
    written (the workspace, the method's own overhead, is reported apart)."""
    tables = rows // rows_per_token
    reads = 2 * rows * width * in_bytes + width * in_bytes + 2 * tables * (rope_dim // 2) * 4
    writes = rows * width * in_bytes + width * 4
    return {"rows": rows, "reads": reads, "writes": writes, "total": reads + writes}


def rmsnorm_bwd_bytes(rows, width, in_bytes=2, read_rstd=False) -> dict:
    reads = 2 * rows * width * in_bytes + width * in_bytes + (rows * 4 if read_rstd else 0)
    writes = rows * width * in_bytes + width * 4
    return {"rows": rows, "reads": reads, "writes": writes, "total": reads + writes}
