"""Planted mistakes in the CPU oracle: each plausible slip (a dropped term, a
wrong sign, a wrong pairing or index, an inverted operand, a skipped floor,
clamp or rounding rule) is patched into the oracle in turn, and at least one
of the pins named with it must then fail. This shows the pins constrain every
step of the oracle, not only that the oracle agrees with itself. CPU only;
pytest's monkeypatch restores the oracle after each case.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import test_oracle_codecs as cpins
import test_oracle_pins as pins
from oracle import backward, codecs, exact, prologue

F32 = np.float32
_real = {
    "rope_tail": prologue.rope_tail,
    "rmsnorm_fwd": prologue.rmsnorm_fwd,
    "quantize_rows": prologue.quantize_rows,
    "quantize_groups": prologue.quantize_groups,
    "truth_norm_rope": prologue.truth_norm_rope,
    "qk_norm_rope_fp8": prologue.qk_norm_rope_fp8,
    "rmsnorm_rope": prologue.rmsnorm_rope,
    "rope_bwd_rotate": backward.rope_bwd_rotate,
    "_bwd_f64": backward._bwd_f64,
    "e4m3_encode": codecs.e4m3_encode,
}


# ------------------------------------------------------------------ the mistakes


def rope_other_direction(n_bits, cos, sin, dtype="bf16"):
    return _real["rope_tail"](n_bits, cos, -np.asarray(sin), dtype)


def rope_interleaved_pairs(n_bits, cos, sin, dtype="bf16"):
    """Pairs (2i, 2i + 1) of the tail instead of (p, p + R/2)."""
    half = cos.shape[-1]
    N = n_bits.shape[-1]
    R = 2 * half
    y = np.array(n_bits, copy=True)
    n = codecs.dtype_to_f32(n_bits, dtype)
    lo, hi = n[:, N - R::2], n[:, N - R + 1::2]
    c, s = np.asarray(cos, F32), np.asarray(sin, F32)
    y[:, N - R::2] = codecs.dtype_round((lo * c) - (hi * s), dtype)
    y[:, N - R + 1::2] = codecs.dtype_round((hi * c) + (lo * s), dtype)
    return y


def rope_leading_columns(n_bits, cos, sin, dtype="bf16"):
    """Rotates the first R columns instead of the last R."""
    R = 2 * cos.shape[-1]
    y = np.array(n_bits, copy=True)
    y[:, :R] = _real["rope_tail"](np.ascontiguousarray(n_bits[:, :R]), cos, sin, dtype)
    return y


def truth_other_direction(x_bits, w_bits, cos_rows, sin_rows, eps, dtype="bf16", round_intermediates=False):
    return _real["truth_norm_rope"](x_bits, w_bits, cos_rows, -np.asarray(sin_rows), eps, dtype, round_intermediates)


def _rstd_mutant(kind):
    def rstd(x32, eps):
        n = x32.shape[-1]
        s = exact.sum_squares_f32(x32)
        if kind == "no_eps":
            with np.errstate(divide="ignore"):
                return F32(1.0) / np.sqrt(s / F32(n))
        if kind == "n_minus_1":
            return F32(1.0) / np.sqrt(s / F32(n - 1) + F32(eps))
        if kind == "no_reciprocal":
            return np.sqrt(s / F32(n) + F32(eps))
        raise AssertionError(kind)
    return rstd


def rmsnorm_without_weight(x_bits, w_bits, eps, dtype="bf16"):
    x = codecs.dtype_to_f32(x_bits, dtype)
    rstd = prologue._rstd(x, eps)
    return codecs.dtype_round(x * rstd[:, None], dtype), rstd


def _quant_mutant(kind):
    def quantize_rows(y_bits, fp8_max, dtype="bf16"):
        y = codecs.dtype_to_f32(y_bits, dtype)
        amax = np.abs(y).max(axis=-1)
        scale = (amax if kind == "no_floor" else np.maximum(amax, F32(1e-4))) / F32(fp8_max)
        if kind == "inverted":
            scale = F32(fp8_max) / np.maximum(amax, F32(1e-4))
        with np.errstate(divide="ignore", invalid="ignore"):
            q = y * (F32(1.0) / scale)[:, None] if kind == "reciprocal" else y / scale[:, None]
        if kind != "no_clamp":
            q = np.minimum(np.maximum(q, -F32(fp8_max)), F32(fp8_max))
        q = np.nan_to_num(q, nan=0.0, posinf=448.0, neginf=-448.0).astype(F32)
        q = np.clip(q, -464.0, 464.0).astype(F32)
        return codecs.e4m3_encode(q), scale.astype(F32)
    return quantize_rows


def groups_share_the_row_scale(y_bits, group_size, fp8_max, dtype="bf16"):
    codes, scale = _real["quantize_rows"](y_bits, fp8_max, dtype)
    return codes, np.repeat(scale[:, None], y_bits.shape[1] // group_size, axis=1)


def qk_table_row_per_row(q_bits, k_bits, wq_bits, wk_bits, cos, sin, eps=1e-6, fp8_max=448.0, dtype="bf16",
                         tokens=None):
    """Row r (flattened over heads) takes table row r instead of its token's row."""
    out = {}
    for name, xb, wb in (("q", q_bits, wq_bits), ("k", k_bits, wk_bits)):
        T, H, D = xb.shape
        rows = xb.reshape(T * H, D)
        idx = np.arange(T * H) % len(cos)
        y, codes, scale = prologue.norm_rope_quant_rows(rows, wb, np.asarray(cos)[idx], np.asarray(sin)[idx],
                                                        eps, fp8_max, dtype)
        out[name + "_y"], out[name + "_codes"] = y.reshape(T, H, D), codes.reshape(T, H, D)
        out[name + "_scale"] = scale.reshape(T, H)
    return out


def rmsnorm_rope_table_row_per_row(x_bits, w_bits, cos, sin, eps=1e-6, dtype="bf16", rows_per_token=1, rows=None):
    """Row r takes table row r (wrapped into the table) instead of r // rows_per_token."""
    r = np.arange(x_bits.shape[0]) if rows is None else np.asarray(rows)
    t = r % len(cos)
    y, _, _ = prologue.norm_rope_quant_rows(x_bits, w_bits, np.asarray(cos)[t], np.asarray(sin)[t], eps, 448.0,
                                            dtype, quant=False)
    return y


def rmsnorm_rope_subset_ignores_rows(x_bits, w_bits, cos, sin, eps=1e-6, dtype="bf16", rows_per_token=1, rows=None):
    """The sampled rows' global indices are ignored (a sample takes table rows 0, 1, ...)."""
    return _real["rmsnorm_rope"](x_bits, w_bits, cos, sin, eps, dtype, rows_per_token, None)


def sum_squares_in_fp32_order(x32):
    x = np.asarray(x32, F32)
    acc = np.zeros(x.shape[:-1], F32)
    for j in range(x.shape[-1]):
        acc = acc + x[..., j] * x[..., j]
    return acc


def e4m3_ties_away_from_zero(x):
    x = np.asarray(x, dtype=F32)
    nudged = np.nextafter(np.abs(x), np.float32(np.inf)) * np.sign(x)
    return _real["e4m3_encode"](np.where(x == 0, x, nudged).astype(F32))


def _bwd_mutant(kind):
    def bwd(x, w, gy, eps, rstd):
        grad_x, grad_w, r = _real["_bwd_f64"](x, w, gy, eps, rstd)
        if kind == "no_mean_term":
            grad_x = r[:, None] * (gy * w[None, :])
        if kind == "dw_unnormalised":
            grad_w = (gy * x).sum(axis=0)
        return grad_x, grad_w, r
    return bwd


def rope_bwd_forward_rotation(gy, cos_rows, sin_rows):
    return _real["rope_bwd_rotate"](gy, cos_rows, -np.asarray(sin_rows))


# ---------------------------------------------------------------- cases and pins


def _set(monkeypatch, module, name, fn):
    monkeypatch.setattr(module, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


CASES = [
    ("rope turns the other way", [(prologue, "rope_tail", rope_other_direction)],
     [pins.test_rope_pairs_p_with_p_plus_half_of_the_tail, pins.test_m32_within_one_bf16_ulp_of_float64]),
    ("rope pairs neighbours", [(prologue, "rope_tail", rope_interleaved_pairs)],
     [pins.test_rope_pairs_p_with_p_plus_half_of_the_tail, pins.test_m32_within_one_bf16_ulp_of_float64]),
    ("rope on the leading columns", [(prologue, "rope_tail", rope_leading_columns)],
     [pins.test_rope_pairs_p_with_p_plus_half_of_the_tail, pins.test_m32_within_one_bf16_ulp_of_float64]),
    ("float64 truth turns the other way", [(prologue, "truth_norm_rope", truth_other_direction)],
     [pins.test_rope_is_the_complex_product, pins.test_m32_within_one_bf16_ulp_of_float64]),
    ("eps dropped", [(prologue, "_rstd", _rstd_mutant("no_eps"))], [pins.test_zero_row]),
    ("mean over N - 1", [(prologue, "_rstd", _rstd_mutant("n_minus_1"))],
     [lambda: pins.test_constant_row_normalises_to_plus_minus_w(3.0)]),
    ("sqrt without the reciprocal", [(prologue, "_rstd", _rstd_mutant("no_reciprocal"))],
     [lambda: pins.test_constant_row_normalises_to_plus_minus_w(3.0)]),
    ("weight dropped", [(prologue, "rmsnorm_fwd", rmsnorm_without_weight)],
     [lambda: pins.test_constant_row_normalises_to_plus_minus_w(3.0)]),
    ("no 1e-4 floor on amax", [(prologue, "quantize_rows", _quant_mutant("no_floor"))],
     [pins.test_zero_row, pins.test_scale_is_correctly_rounded_amax_over_fp8_max]),
    ("scale inverted", [(prologue, "quantize_rows", _quant_mutant("inverted"))],
     [pins.test_scale_is_correctly_rounded_amax_over_fp8_max, pins.test_max_code_is_448_for_rows_above_the_floor]),
    ("reciprocal multiply instead of division", [(prologue, "quantize_rows", _quant_mutant("reciprocal"))],
     [lambda: pins.test_codes_are_the_e4m3_of_the_correctly_rounded_quotient(448.0)]),
    ("no clamp before the cast", [(prologue, "quantize_rows", _quant_mutant("no_clamp"))],
     [pins.test_clamp_binds_when_fp8_max_is_an_e4m3_midpoint]),
    ("groups share the row's scale", [(prologue, "quantize_groups", groups_share_the_row_scale)],
     [lambda: pins.test_each_group_scale_is_its_own_absmax_over_fp8_max(64), pins.test_groups_are_independent]),
    ("table row per row, not per token", [(prologue, "qk_norm_rope_fp8", qk_table_row_per_row)],
     [pins.test_qk_shares_the_token_row_across_heads]),
    ("path R: table row per row, not per token", [(prologue, "rmsnorm_rope", rmsnorm_rope_table_row_per_row)],
     [lambda: pins.test_rmsnorm_rope_rows_of_a_token_share_its_table_row(4, 16, "bf16"),
      pins.test_grouped_rows_of_a_token_share_its_table_row]),
    ("path R: sampled rows read the sample's own table rows", [(prologue, "rmsnorm_rope",
                                                                rmsnorm_rope_subset_ignores_rows)],
     [lambda: pins.test_rmsnorm_rope_row_subset_equals_the_full_call(4)]),
    ("sum of squares accumulated in fp32", [(exact, "sum_squares_f32", sum_squares_in_fp32_order),
                                            (prologue, "sum_squares_f32", sum_squares_in_fp32_order),
                                            (pins, "sum_squares_f32", sum_squares_in_fp32_order)],
     [pins.test_sum_squares_equals_exact_rational_rounding]),
    ("e4m3 ties away from zero", [(codecs, "e4m3_encode", e4m3_ties_away_from_zero)],
     [cpins.test_e4m3_encode_matches_torch]),
    ("backward drops the mean term", [(backward, "_bwd_f64", _bwd_mutant("no_mean_term"))],
     [pins.test_backward_matches_central_differences]),
    ("grad_w from x instead of the normalised x", [(backward, "_bwd_f64", _bwd_mutant("dw_unnormalised"))],
     [pins.test_backward_matches_central_differences, pins.test_backward_single_row_dw]),
    ("rope backward uses the forward rotation", [(backward, "rope_bwd_rotate", rope_bwd_forward_rotation)],
     [pins.test_rope_backward_matches_central_differences,
      pins.test_rope_backward_rotation_is_orthogonal_and_inverts_the_forward]),
]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # (some mistakes produce inf / nan on the way)
@pytest.mark.parametrize("name,patches,pin_list", CASES, ids=[c[0] for c in CASES])
def test_a_planted_mistake_fails_a_pin(monkeypatch, name, patches, pin_list):
    # the unpatched oracle passes these pins
    for pin in pin_list:
        pin()
    for module, attr, fn in patches:
        _set(monkeypatch, module, attr, fn)
    caught = []
    for pin in pin_list:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(getattr(pin, "__name__", "pin"))
    assert caught, f"planted mistake '{name}' passed every pin named for it"
