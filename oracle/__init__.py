"""CPU oracle for the RMSNorm -> partial NeoX RoPE -> per-row FP8 prologue.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package. It shares no code with the HIP library (no kernels, headers, helpers
or tables) and never imports it; the only module both sides use is the seeded
input generator in ``workloads``.

Everything here is plain numpy on the host, written from the definitions on the
tilelang-tutorial pages:

* chapter 13 fusion page ``rmsnorm_rope_quant.py`` - the PyTorch reference
  ``torch_reference_fused`` and its NeoX helper ``_torch_rope_neox``;
* chapter 17 page ``rmsnorm_tl.py`` - ``RMSNormTileLang.backward``;
* chapter 28 page ``case_norm_rope_quant.py`` - the QK-norm prologue (per
  (token, head) row, one cos/sin row per token, one fp32 scale per row).

Precision follows the pages: the reference upcasts to fp32, rounds the
normalised row and the rotated row back to the input dtype, divides by the
scale in fp32 and casts to float8_e4m3fn. The one step whose fp32 value
depends on an order the pages leave open, the sum of squares, is taken as the
exact sum rounded once to fp32 (see ``exact``). A float64 "truth" mode exists
for the pins that hold in real arithmetic, and the backward is evaluated in
float64.
"""

from .codecs import (
    bf16_round,
    bf16_to_f32,
    f16_round,
    f16_to_f32,
    e4m3_encode,
    e4m3_decode,
    E4M3_TABLE,
    dtype_round,
    dtype_to_f32,
)
from .exact import sum_squares_f32, sum_squares_exact_mask
from .prologue import (
    rmsnorm_fwd,
    rope_tail,
    quantize_rows,
    norm_rope_quant_rows,
    qk_norm_rope_fp8,
    rmsnorm_rope,
    quantize_groups,
    rmsnorm_rope_fp8_grouped,
    truth_norm_rope,
)
from .backward import rmsnorm_bwd, rope_bwd_rotate, rmsnorm_rope_bwd

__all__ = [
    "bf16_round", "bf16_to_f32", "f16_round", "f16_to_f32", "e4m3_encode", "e4m3_decode",
    "E4M3_TABLE", "dtype_round", "dtype_to_f32", "sum_squares_f32", "sum_squares_exact_mask",
    "rmsnorm_fwd", "rope_tail", "quantize_rows", "norm_rope_quant_rows", "qk_norm_rope_fp8",
    "rmsnorm_rope", "truth_norm_rope", "rmsnorm_bwd",
    "quantize_groups", "rmsnorm_rope_fp8_grouped", "rope_bwd_rotate", "rmsnorm_rope_bwd",
]
