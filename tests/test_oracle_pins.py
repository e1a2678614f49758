"""Pins of the CPU oracle against facts the pages and the mathematics fix.

Each test ties one part of the oracle to something other than the oracle's
own formula: a closed form, an identity of the rotation, a brute-force exact
computation, a special case, or finite differences.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import _ties
import oracle
from oracle import codecs
from oracle.exact import fraction_to_f32, sum_squares_exact_mask, sum_squares_f32

F32 = np.float32


def _bf16(x):
    return codecs.bf16_round(np.asarray(x, np.float32))


def _rows(M, N, seed, std=1.0):
    rng = np.random.default_rng(seed)
    return _bf16(rng.standard_normal((M, N)).astype(np.float32) * std)


def _table(M, half, seed):
    rng = np.random.default_rng(seed)
    ang = rng.uniform(-np.pi, np.pi, (M, half))
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


# ----------------------------------------------------------------- exact sum of squares


def _brute_sumsq(row):
    return fraction_to_f32(sum((Fraction(float(v)) ** 2 for v in row), Fraction(0)))


def test_sum_squares_equals_exact_rational_rounding():
    rng = np.random.default_rng(11)
    rows = []
    for _ in range(200):
        n = int(rng.integers(1, 40))
        v = rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n))  # wide dynamic range
        rows.append(codecs.bf16_to_f32(_bf16(v.astype(np.float32))))
    for r in rows:
        got = sum_squares_f32(r[None, :])[0]
        assert got.tobytes() == _brute_sumsq(r).tobytes()


def test_sum_squares_proof_flag_is_sound():
    """Rows flagged exact really are: the float64 sum equals the rational sum."""
    x = codecs.bf16_to_f32(_rows(300, 64, 12))
    x[:100, 0] *= np.float32(2.0**-40)  # force some rows out of the proven range
    s64, exact = sum_squares_exact_mask(x)
    assert exact.sum() > 150 and (~exact).sum() > 0
    for i in np.flatnonzero(exact)[:80]:
        tot = sum((Fraction(float(v)) ** 2 for v in x[i]), Fraction(0))
        assert Fraction(float(s64[i])) == tot


def test_fraction_to_f32_matches_float_rounding():
    rng = np.random.default_rng(13)
    for _ in range(2000):
        v = float(rng.standard_normal() * 2.0 ** rng.integers(-150, 120))
        got = fraction_to_f32(Fraction(abs(v)))
        assert got.tobytes() == np.float32(abs(v)).tobytes()  # a double is one exact rational
    # ties to even at the fp32 grid: 1 + 2^-24 lies halfway between 1 and 1 + 2^-23
    assert fraction_to_f32(Fraction(1) + Fraction(1, 1 << 24)) == np.float32(1.0)
    assert fraction_to_f32(Fraction(1) + Fraction(3, 1 << 24)) == np.float32(1.0 + 2.0**-22)


# ------------------------------------------------------------------------- RoPE pins


def test_rope_identity_when_cos_one_sin_zero():
    """cos = 1, sin = 0 leaves every nonzero value bit-identical.

    Zeros keep their value but IEEE addition decides their sign: -0 - (hi * 0)
    is +0 when hi < 0, so only the magnitude of a zero is pinned.
    """
    n = _rows(64, 128, 21)
    n[0, 100] = 0x8000
    n[1, 70] = 0x0000
    for half in (8, 32, 64):
        c = np.ones((64, half), F32)
        s = np.zeros((64, half), F32)
        y = oracle.rope_tail(n, c, s)
        nz = (n & 0x7FFF) != 0
        assert np.array_equal(y[nz], n[nz])
        assert np.all((y[~nz] & 0x7FFF) == 0)


def test_rope_preserves_pair_norm_in_exact_arithmetic():
    x = _rows(32, 128, 22)
    w = _bf16(1 + 0.1 * np.random.default_rng(23).standard_normal(128))
    c, s = _table(32, 32, 24)
    y = oracle.truth_norm_rope(x, w, c, s, 1e-6)
    n = oracle.truth_norm_rope(x, w, np.zeros((32, 0)), np.zeros((32, 0)), 1e-6)
    lo, hi = n[:, 64:96], n[:, 96:]
    ylo, yhi = y[:, 64:96], y[:, 96:]
    lhs = ylo**2 + yhi**2
    rhs = (lo**2 + hi**2) * (c.astype(np.float64) ** 2 + s.astype(np.float64) ** 2)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=0)
    assert np.array_equal(y[:, :64], n[:, :64])  # columns outside the rope tail pass through


def test_rope_is_the_complex_product():
    x = _rows(16, 64, 25)
    w = _bf16(np.ones(64))
    c, s = _table(16, 32, 26)
    y = oracle.truth_norm_rope(x, w, c, s, 1e-6)
    n = oracle.truth_norm_rope(x, w, np.zeros((16, 0)), np.zeros((16, 0)), 1e-6)
    z = (n[:, :32] + 1j * n[:, 32:]) * (c.astype(np.float64) + 1j * s.astype(np.float64))
    np.testing.assert_allclose(y[:, :32], z.real, rtol=0, atol=1e-14)
    np.testing.assert_allclose(y[:, 32:], z.imag, rtol=0, atol=1e-14)


def test_rope_pairs_p_with_p_plus_half_of_the_tail():
    """NeoX half split on the last R columns: a unit at tail column p rotates into p + R/2."""
    N, R = 32, 16
    n = np.zeros((1, N), np.uint16)
    n[0, N - R + 3] = _bf16(1.0)
    c = np.zeros((1, R // 2), F32)
    s = np.ones((1, R // 2), F32)  # rotation by +90 degrees
    y = codecs.bf16_to_f32(oracle.rope_tail(n, c, s))
    expect = np.zeros(N, F32)
    expect[N - R // 2 + 3] = 1.0
    assert np.array_equal(y[0], expect)


# ---------------------------------------------------------------------- RMSNorm pins


@pytest.mark.parametrize("a", [1.0, -1.0, 0.5, -0.5, 3.0, -3.0])
def test_constant_row_normalises_to_plus_minus_w(a):
    rng = np.random.default_rng(31)
    w = _bf16(rng.standard_normal(256))
    x = _bf16(np.full((4, 256), a, np.float32))
    y, _ = oracle.rmsnorm_fwd(x, w, 1e-6)
    expect = _bf16(np.sign(a) * codecs.bf16_to_f32(w))
    assert np.array_equal(y, np.broadcast_to(expect, y.shape))


def test_m32_within_one_bf16_ulp_of_float64():
    x = _rows(256, 128, 32)
    w = _bf16(1 + 0.1 * np.random.default_rng(33).standard_normal(128))
    c, s = _table(256, 32, 34)
    y32, _, _ = oracle.norm_rope_quant_rows(x, w, c, s, 1e-6, 448.0)
    y64 = oracle.truth_norm_rope(x, w, c, s, 1e-6, round_intermediates=True)
    # distance in bf16 steps between the oracle's y and the float64 composition
    y64b = codecs.bf16_round(y64.astype(np.float32))
    d = np.abs(y32.astype(np.int32) - y64b.astype(np.int32))
    same_sign = (y32 & 0x8000) == (y64b & 0x8000)
    assert np.all(d[same_sign] <= 1)
    assert np.mean(d == 0) > 0.999


def test_zero_row():
    w = _bf16(np.array([1.0, -2.0] * 64, np.float32))
    x = np.zeros((3, 128), np.uint16)
    c, s = _table(3, 32, 35)
    y, codes, scale = oracle.norm_rope_quant_rows(x, w, c, s, 1e-6, 448.0)
    assert np.all(codecs.bf16_to_f32(y) == 0)
    # sign of zero: +0 * w keeps w's sign outside the tail
    assert np.array_equal(codes[:, :64] & 0x80, np.where(codecs.bf16_to_f32(w[:64]) < 0, 0x80, 0)[None, :].repeat(3, 0))
    assert np.all((codes & 0x7F) == 0)
    assert np.all(scale == fraction_to_f32(Fraction(float(np.float32(1e-4))) / 448))


# ----------------------------------------------------------------- quantisation pins


def _exact_div_f32(a, b):
    return fraction_to_f32(Fraction(float(a)) / Fraction(float(b)))


def test_scale_is_correctly_rounded_amax_over_fp8_max():
    x = _rows(200, 128, 41)
    x[:5] = _bf16(codecs.bf16_to_f32(x[:5]) * 1e-7)  # rows below the 1e-4 floor
    w = _bf16(1 + 0.1 * np.random.default_rng(42).standard_normal(128))
    c, s = _table(200, 32, 43)
    for fp8_max in (448.0, 240.0, 57.0):
        y, codes, scale = oracle.norm_rope_quant_rows(x, w, c, s, 1e-6, fp8_max)
        amax = np.abs(codecs.bf16_to_f32(y)).max(axis=1)
        for i in range(200):
            a = max(float(amax[i]), float(np.float32(1e-4)))
            assert scale[i].tobytes() == _exact_div_f32(a, fp8_max).tobytes()


def test_max_code_is_448_for_rows_above_the_floor():
    d_in = _rows(500, 128, 44)
    w = _bf16(1 + 0.1 * np.random.default_rng(45).standard_normal(128))
    c, s = _table(500, 32, 46)
    y, codes, scale = oracle.norm_rope_quant_rows(d_in, w, c, s, 1e-6, 448.0)
    mag = codes & 0x7F
    assert np.all(mag.max(axis=1) == 0x7E)
    assert not np.any(mag == 0x7F)  # NaN never produced


def test_codes_decode_back_within_e4m3_rounding():
    x = _rows(300, 128, 47)
    w = _bf16(1 + 0.1 * np.random.default_rng(48).standard_normal(128))
    c, s = _table(300, 64, 49)
    y, codes, scale = oracle.norm_rope_quant_rows(x, w, c, s, 1e-6, 448.0)
    yv = codecs.bf16_to_f32(y).astype(np.float64)
    dec = codecs.e4m3_decode(codes).astype(np.float64) * scale[:, None].astype(np.float64)
    err = np.abs(dec - yv)
    q = np.abs(yv) / scale[:, None]
    normal = q >= 2.0**-6
    slack = 1e-6 * np.abs(yv) + 1e-30
    assert np.all(err[normal] <= 2.0**-4 * np.abs(yv[normal]) + slack[normal])
    sub_bound = 2.0**-10 * scale[:, None].astype(np.float64) * (1 + 1e-6)
    assert np.all(err[~normal] <= np.broadcast_to(sub_bound, err.shape)[~normal])


def test_clamp_applies_for_smaller_fp8_max():
    x = _rows(64, 128, 50)
    w = _bf16(np.ones(128))
    c, s = _table(64, 64, 51)
    _, codes, _ = oracle.norm_rope_quant_rows(x, w, c, s, 1e-6, 240.0)
    lim = int(codecs.e4m3_encode(np.float32(240.0)))
    assert (codes & 0x7F).max() == lim


@pytest.mark.parametrize("fp8_max", [448.0, 240.0])
def test_codes_are_the_e4m3_of_the_correctly_rounded_quotient(fp8_max):
    """On rows built to put y / scale on e4m3 rounding midpoints (where one
    rounding more or less flips the code), every code equals the e4m3 encoding
    of the exact rational y / scale rounded once to fp32 and clamped."""
    y = _ties.tie_rows(fp8_max)
    codes, scale = oracle.quantize_rows(y, fp8_max)
    yv = codecs.bf16_to_f32(y)
    n_ties = 0
    for i in range(y.shape[0]):
        sc = Fraction(float(scale[i]))
        assert scale[i].tobytes() == _exact_div_f32(float(np.abs(yv[i]).max()), fp8_max).tobytes()
        for j in range(y.shape[1]):
            r = Fraction(float(yv[i, j])) / sc
            q = fraction_to_f32(abs(r)) * np.float32(-1.0 if r < 0 else 1.0)
            q = np.float32(min(max(float(q), -fp8_max), fp8_max))
            assert codes[i, j] == codecs.e4m3_encode(q), (i, j, float(yv[i, j]))
            n_ties += float(q) != 0.0
    assert n_ties > 200


@pytest.mark.parametrize("fp8_max", [448.0, 240.0])
def test_exact_rmsnorm_rows_carry_the_ties_to_the_quantiser(fp8_max):
    """Rows whose mean square is a power of 4 normalise exactly (eps = 0, w = 1:
    y = x * 2^-k), so the tie structure reaches the quantiser intact; the
    codes then equal the exact-rational ones."""
    x = _ties.normalised_tie_rows(fp8_max)
    w = _bf16(np.ones(128))
    y, codes, scale = oracle.norm_rope_quant_rows(x, w, np.zeros((len(x), 0), F32), np.zeros((len(x), 0), F32),
                                                  0.0, fp8_max)
    xv, yv = codecs.bf16_to_f32(x), codecs.bf16_to_f32(y)
    ratio = yv[:, 0] / xv[:, 0]
    assert np.all(yv == xv * ratio[:, None])  # one power of two per row
    assert np.all(np.log2(ratio) == np.round(np.log2(ratio)))
    for i in range(len(x)):
        sc = Fraction(float(scale[i]))
        for j in range(128):
            r = Fraction(float(yv[i, j])) / sc
            q = fraction_to_f32(abs(r)) * np.float32(-1.0 if r < 0 else 1.0)
            q = np.float32(min(max(float(q), -fp8_max), fp8_max))
            assert codes[i, j] == codecs.e4m3_encode(q), (i, j)


def test_clamp_binds_when_fp8_max_is_an_e4m3_midpoint():
    """fp8_max = 232 lies halfway between the e4m3 values 224 and 240. Where
    RN(amax / 232) rounds down, amax / scale exceeds 232 and the clamp brings
    it back to 232, which encodes (ties to even) as 224; without the clamp it
    would encode as 240."""
    x = _rows(400, 128, 54)
    w = _bf16(1 + 0.1 * np.random.default_rng(55).standard_normal(128))
    c, s = _table(400, 64, 56)
    y, codes, scale = oracle.norm_rope_quant_rows(x, w, c, s, 1e-6, 232.0)
    amax = np.abs(codecs.bf16_to_f32(y)).max(axis=1)
    over = [Fraction(float(a)) / Fraction(float(sc)) > 232 for a, sc in zip(amax, scale)]
    assert 50 < sum(over) < 350  # the clamp binds on a good share of the rows
    assert np.all((codes & 0x7F).max(axis=1) == codecs.e4m3_encode(np.float32(224.0)))


def test_qk_shares_the_token_row_across_heads():
    """Every head of a token is rotated by that token's table row."""
    T, Hq, Hk, D = 5, 3, 2, 64
    rng = np.random.default_rng(52)
    q = _bf16(rng.standard_normal((T, Hq, D)))
    k = _bf16(rng.standard_normal((T, Hk, D)))
    wq = _bf16(1 + 0.1 * rng.standard_normal(D))
    wk = _bf16(1 + 0.1 * rng.standard_normal(D))
    c, s = _table(T, D // 2, 53)
    out = oracle.qk_norm_rope_fp8(q, k, wq, wk, c, s)
    for t in range(T):
        for h in range(Hk):
            y, codes, scale = oracle.norm_rope_quant_rows(k[t, h][None], wk, c[t][None], s[t][None], 1e-6, 448.0)
            assert np.array_equal(out["k_codes"][t, h], codes[0])
            assert out["k_scale"][t, h] == scale[0]


def _shared_table_case(T, H, D, half, seed, dtype="bf16"):
    rng = np.random.default_rng(seed)
    if dtype == "fp16":
        x = codecs.f16_round((2.0 * rng.standard_normal((T * H, D))).astype(F32))
        w = codecs.f16_round((1 + 0.1 * rng.standard_normal(D)).astype(F32))
    else:
        x = _bf16(rng.standard_normal((T * H, D)))
        w = _bf16(1 + 0.1 * rng.standard_normal(D))
    c, s = _table(T, half, seed + 1)
    return x, w, c, s


@pytest.mark.parametrize("H,half,dtype", [(4, 16, "bf16"), (5, 32, "fp16"), (3, 8, "bf16")])
def test_rmsnorm_rope_rows_of_a_token_share_its_table_row(H, half, dtype):
    """Path R with rows_per_token = H: row r takes table row r // H, i.e. every
    head of a token reads the token's one cos/sin row (chapter 28 page, module
    docstring). Equal to the same call on a table with each row written out H
    times, and to the QK entry's y (whose token sharing is pinned above)."""
    T, D = 6, 64
    x, w, c, s = _shared_table_case(T, H, D, half, 81, dtype)
    shared = oracle.rmsnorm_rope(x, w, c, s, 1e-6, dtype, rows_per_token=H)
    expanded = oracle.rmsnorm_rope(x, w, np.repeat(c, H, axis=0), np.repeat(s, H, axis=0), 1e-6, dtype)
    assert np.array_equal(shared, expanded)
    q = oracle.qk_norm_rope_fp8(x.reshape(T, H, D), None, w, None, c, s, dtype=dtype)
    assert np.array_equal(shared, q["q_y"].reshape(T * H, D))
    # a rotation by a different table row changes the result (the pin can see the map)
    other = oracle.rmsnorm_rope(x, w, np.roll(c, 1, axis=0), np.roll(s, 1, axis=0), 1e-6, dtype, rows_per_token=H)
    assert not np.array_equal(shared, other)


@pytest.mark.parametrize("H", [1, 4])
def test_rmsnorm_rope_row_subset_equals_the_full_call(H):
    """``rows=`` (global row indices of a sample) gives exactly the sampled rows of the full call."""
    T, D, half = 7, 64, 16
    x, w, c, s = _shared_table_case(T, H, D, half, 83)
    full = oracle.rmsnorm_rope(x, w, c, s, 1e-6, rows_per_token=H)
    rows = np.array([T * H - 1, 0, 5, 2 * H + 1, 3]) % (T * H)
    part = oracle.rmsnorm_rope(x[rows], w, c, s, 1e-6, rows_per_token=H, rows=rows)
    assert np.array_equal(part, full[rows])


def test_grouped_rows_of_a_token_share_its_table_row():
    """The per-group quantiser inherits the same row -> table-row map."""
    T, H, D, half = 4, 3, 128, 32
    x, w, c, s = _shared_table_case(T, H, D, half, 85)
    a = oracle.rmsnorm_rope_fp8_grouped(x, w, c, s, 32, rows_per_token=H)
    b = oracle.rmsnorm_rope_fp8_grouped(x, w, np.repeat(c, H, axis=0), np.repeat(s, H, axis=0), 32)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


# -------------------------------------------------------------------- backward pins


def _loss_exact(x, w, gy, eps):
    ms = (x * x).mean(axis=-1)
    rstd = 1.0 / np.sqrt(ms + eps)
    return float((gy * x * rstd[:, None] * w[None, :]).sum())


def test_backward_matches_central_differences():
    rng = np.random.default_rng(61)
    M, N = 3, 12
    eps = float(np.float32(1e-6))
    xb = _bf16(rng.standard_normal((M, N)))
    wb = _bf16(rng.standard_normal(N))
    gb = _bf16(rng.standard_normal((M, N)))
    dx, dw, _ = oracle.rmsnorm_bwd(xb, wb, gb, 1e-6)
    x = codecs.bf16_to_f32(xb).astype(np.float64)
    w = codecs.bf16_to_f32(wb).astype(np.float64)
    g = codecs.bf16_to_f32(gb).astype(np.float64)
    h = 1e-6
    fd_x = np.zeros_like(x)
    for i in range(M):
        for j in range(N):
            xp = x.copy(); xp[i, j] += h
            xm = x.copy(); xm[i, j] -= h
            fd_x[i, j] = (_loss_exact(xp, w, g, eps) - _loss_exact(xm, w, g, eps)) / (2 * h)
    fd_w = np.zeros_like(w)
    for j in range(N):
        wp = w.copy(); wp[j] += h
        wm = w.copy(); wm[j] -= h
        fd_w[j] = (_loss_exact(x, wp, g, eps) - _loss_exact(x, wm, g, eps)) / (2 * h)
    np.testing.assert_allclose(dx, fd_x, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dw, fd_w, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_backward_scale_invariance_identity(eps):
    """sum_j x_j dx_j = N * C * eps * rstd^2 per row (zero when eps = 0)."""
    rng = np.random.default_rng(62)
    M, N = 8, 96
    xb = _bf16(rng.standard_normal((M, N)))
    wb = _bf16(rng.standard_normal(N))
    gb = _bf16(rng.standard_normal((M, N)))
    dx, _, rstd = oracle.rmsnorm_bwd(xb, wb, gb, eps)
    x = codecs.bf16_to_f32(xb).astype(np.float64)
    w = codecs.bf16_to_f32(wb).astype(np.float64)
    g = codecs.bf16_to_f32(gb).astype(np.float64) * w
    xn = x * rstd[:, None]
    C = (g * xn).mean(axis=1)
    lhs = (x * dx).sum(axis=1)
    rhs = N * C * float(np.float32(eps)) * rstd**2
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-11 * np.abs(x * dx).sum(axis=1).max())


def test_backward_single_row_dw():
    rng = np.random.default_rng(63)
    xb = _bf16(rng.standard_normal((1, 40)))
    wb = _bf16(rng.standard_normal(40))
    gb = _bf16(rng.standard_normal((1, 40)))
    _, dw, rstd = oracle.rmsnorm_bwd(xb, wb, gb, 1e-6)
    x = codecs.bf16_to_f32(xb[0]).astype(np.float64)
    g = codecs.bf16_to_f32(gb[0]).astype(np.float64)
    np.testing.assert_allclose(dw, g * x * rstd[0], rtol=1e-15)


# ------------------------------------------------------- RoPE backward pins


def _loss_norm_rope_complex(x, w, gy, c, s, eps):
    """sum(gy * y) for y = RoPE(RMSNorm(x)) in real arithmetic; the tail pairs
    rotated as complex numbers (lo + i hi) * (c + i s)."""
    N, half = x.shape[-1], c.shape[-1]
    rstd = 1.0 / np.sqrt((x * x).mean(axis=-1) + eps)
    n = x * rstd[:, None] * w[None, :]
    z = (n[:, N - 2 * half : N - half] + 1j * n[:, N - half :]) * (c + 1j * s)
    y = np.concatenate([n[:, : N - 2 * half], z.real, z.imag], axis=1)
    return float((gy * y).sum())


def _rope_bwd_case(M=3, N=16, R=8, seed=71, rows_per_token=1):
    rng = np.random.default_rng(seed)
    xb = _bf16(rng.standard_normal((M, N)))
    wb = _bf16(1 + 0.3 * rng.standard_normal(N))
    gb = _bf16(rng.standard_normal((M, N)))
    c, s = _table(M // rows_per_token, R // 2, seed + 1)
    return xb, wb, gb, c, s


def test_rope_backward_matches_central_differences():
    M, N, R = 3, 16, 8
    xb, wb, gb, c, s = _rope_bwd_case(M, N, R)
    eps = float(np.float32(1e-6))
    dx, dw, _ = oracle.rmsnorm_rope_bwd(xb, wb, gb, c, s, 1e-6)
    x = codecs.bf16_to_f32(xb).astype(np.float64)
    w = codecs.bf16_to_f32(wb).astype(np.float64)
    g = codecs.bf16_to_f32(gb).astype(np.float64)
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    h = 1e-6

    def loss(xx, ww):
        return _loss_norm_rope_complex(xx, ww, g, c64, s64, eps)

    fd_x = np.zeros_like(x)
    for i in range(M):
        for j in range(N):
            xp = x.copy(); xp[i, j] += h
            xm = x.copy(); xm[i, j] -= h
            fd_x[i, j] = (loss(xp, w) - loss(xm, w)) / (2 * h)
    fd_w = np.zeros_like(w)
    for j in range(N):
        wp = w.copy(); wp[j] += h
        wm = w.copy(); wm[j] -= h
        fd_w[j] = (loss(x, wp) - loss(x, wm)) / (2 * h)
    np.testing.assert_allclose(dx, fd_x, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dw, fd_w, rtol=1e-6, atol=1e-8)


def test_rope_backward_matches_torch_autograd_float64():
    """Library routine: torch's reverse-mode AD of the same map, complex rotation, float64."""
    M, N, R = 6, 64, 32
    xb, wb, gb, c, s = _rope_bwd_case(M, N, R, seed=72)
    dx, dw, _ = oracle.rmsnorm_rope_bwd(xb, wb, gb, c, s, 1e-6)
    x = torch.tensor(codecs.bf16_to_f32(xb), dtype=torch.float64, requires_grad=True)
    w = torch.tensor(codecs.bf16_to_f32(wb), dtype=torch.float64, requires_grad=True)
    g = torch.tensor(codecs.bf16_to_f32(gb), dtype=torch.float64)
    rot = torch.complex(torch.tensor(c, dtype=torch.float64), torch.tensor(s, dtype=torch.float64))
    n = x * torch.rsqrt((x * x).mean(-1, keepdim=True) + float(np.float32(1e-6))) * w
    z = torch.complex(n[:, N - R : N - R // 2], n[:, N - R // 2 :]) * rot
    y = torch.cat([n[:, : N - R], z.real, z.imag], dim=1)
    (y * g).sum().backward()
    np.testing.assert_allclose(dx, x.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dw, w.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_rope_backward_special_cases_reduce_to_rmsnorm_backward():
    xb, wb, gb, c, s = _rope_bwd_case(5, 32, 16, seed=73)
    ref = oracle.rmsnorm_bwd(xb, wb, gb, 1e-6)
    # no rope tail
    z = np.zeros((5, 0), F32)
    out = oracle.rmsnorm_rope_bwd(xb, wb, gb, z, z, 1e-6)
    assert all(np.array_equal(a, b) for a, b in zip(out, ref))
    # identity rotation (cos 1, sin 0)
    out = oracle.rmsnorm_rope_bwd(xb, wb, gb, np.ones_like(c), np.zeros_like(s), 1e-6)
    assert all(np.array_equal(a, b) for a, b in zip(out, ref))


def test_rope_backward_rotation_is_orthogonal_and_inverts_the_forward():
    rng = np.random.default_rng(74)
    M, N, half = 4, 24, 8
    g = rng.standard_normal((M, N))
    c, s = _table(M, half, 75)
    gn = oracle.rope_bwd_rotate(g, c, s)
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    k = c64 * c64 + s64 * s64  # 1 up to the fp32 rounding of the table
    lo, hi = g[:, N - 2 * half : N - half], g[:, N - half :]
    glo, ghi = gn[:, N - 2 * half : N - half], gn[:, N - half :]
    np.testing.assert_allclose(glo**2 + ghi**2, (lo**2 + hi**2) * k, rtol=1e-12)
    # rotating back by the forward map gives k * g
    np.testing.assert_allclose(glo * c64 - ghi * s64, k * lo, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(ghi * c64 + glo * s64, k * hi, rtol=1e-12, atol=1e-15)
    assert np.array_equal(gn[:, : N - 2 * half], g[:, : N - 2 * half])


def test_rope_backward_rows_per_token_shares_the_table_row():
    xb, wb, gb, c, s = _rope_bwd_case(8, 32, 16, seed=76, rows_per_token=4)
    a = oracle.rmsnorm_rope_bwd(xb, wb, gb, c, s, 1e-6, rows_per_token=4)
    b = oracle.rmsnorm_rope_bwd(xb, wb, gb, np.repeat(c, 4, axis=0), np.repeat(s, 4, axis=0), 1e-6)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


# ----------------------------------------------------- consistency with the pages' torch code


def test_agrees_with_torch_reference_up_to_summation_order():
    """The pages' torch reference sums squares in torch's own order; results agree to 1 ulp.

    Not a pin (it shares the formula); it shows what the exact-sum reading changes.
    """
    rng = np.random.default_rng(71)
    M, N, half = 2048, 128, 32
    x = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((1 + 0.1 * rng.standard_normal(N)).astype(np.float32)).to(torch.bfloat16)
    c, s = _table(M, half, 72)
    cos, sin = torch.from_numpy(c), torch.from_numpy(s)
    rstd = torch.rsqrt(x.float().pow(2).mean(-1, keepdim=True) + 1e-6)
    normed = (x.float() * rstd * w.float().unsqueeze(0)).to(x.dtype)
    R = 2 * half
    lo, hi = normed[:, -R:].float()[:, :half], normed[:, -R:].float()[:, half:]
    y = torch.cat([normed[:, :-R], torch.cat([lo * cos - hi * sin, hi * cos + lo * sin], -1).to(x.dtype)], -1)
    yb = y.view(torch.int16).numpy().view(np.uint16)
    ours, _, _ = oracle.norm_rope_quant_rows(x.view(torch.int16).numpy().view(np.uint16),
                                             w.view(torch.int16).numpy().view(np.uint16), c, s, 1e-6, 448.0)
    d = np.abs(ours.astype(np.int32) - yb.astype(np.int32))
    assert np.all(d <= 1)
    assert np.mean(d == 0) > 0.9995


# ----------------------------------------------------------------- per-group scales


def test_one_group_per_row_equals_the_per_row_scale():
    y = _rows(64, 256, 70)
    codes_g, scale_g = oracle.quantize_groups(y, 256, 448.0)
    codes_r, scale_r = oracle.quantize_rows(y, 448.0)
    assert np.array_equal(codes_g, codes_r)
    assert np.array_equal(scale_g[:, 0].view(np.uint32), scale_r.view(np.uint32))


@pytest.mark.parametrize("group_size", [16, 64, 128])
def test_each_group_scale_is_its_own_absmax_over_fp8_max(group_size):
    rng = np.random.default_rng(71 + group_size)
    M, N = 8, 512
    G = N // group_size
    # every group gets its own magnitude, so a group read along the wrong axis shows
    mags = 2.0 ** rng.integers(-20, 6, size=(M, G))
    vals = rng.standard_normal((M, N)) * np.repeat(mags, group_size, axis=1)
    vals[0, :group_size] = 0.0  # one group entirely zero: the 1e-4 floor
    y = _bf16(vals.astype(np.float32))
    codes, scale = oracle.quantize_groups(y, group_size, 448.0)
    yv = codecs.bf16_to_f32(y)
    for i in range(M):
        for g in range(G):
            elems = [abs(float(v)) for v in yv[i, g * group_size:(g + 1) * group_size]]
            a = max(max(elems), float(np.float32(1e-4)))
            assert scale[i, g].tobytes() == _exact_div_f32(a, 448.0).tobytes()
            mag = codes[i, g * group_size:(g + 1) * group_size] & 0x7F
            if max(elems) >= 1e-4:
                assert mag.max() == 0x7E
            else:  # below the floor: the largest code is that of amax / scale, no longer 448
                q = _exact_div_f32(max(elems), float(scale[i, g]))
                assert mag.max() == (codecs.e4m3_encode(np.float32(q)) & 0x7F)
    assert np.all(codes[0, :group_size] & 0x7F == 0)


def test_groups_are_independent():
    y = _rows(16, 512, 72)
    codes, scale = oracle.quantize_groups(y, 128, 448.0)
    y2 = y.copy()
    y2[:, 128:256] = _bf16(codecs.bf16_to_f32(y[:, 128:256]) * 37.0)
    codes2, scale2 = oracle.quantize_groups(y2, 128, 448.0)
    keep = np.r_[0:128, 256:512]
    assert np.array_equal(codes[:, keep], codes2[:, keep])
    assert np.array_equal(scale[:, [0, 2, 3]], scale2[:, [0, 2, 3]])
    assert not np.array_equal(scale[:, 1], scale2[:, 1])


def test_grouped_pipeline_decodes_within_e4m3_rounding():
    x = _rows(32, 1024, 73)
    w = _bf16(1 + 0.1 * np.random.default_rng(74).standard_normal(1024))
    c, s = _table(32, 64, 75)
    y, codes, scale = oracle.rmsnorm_rope_fp8_grouped(x, w, c, s, 128)
    assert np.array_equal(y, oracle.rmsnorm_rope(x, w, c, s))
    yv = codecs.bf16_to_f32(y).astype(np.float64)
    sc = np.repeat(scale.astype(np.float64), 128, axis=1)
    dec = codecs.e4m3_decode(codes).astype(np.float64) * sc
    err = np.abs(dec - yv)
    normal = np.abs(yv) / sc >= 2.0**-6
    assert np.all(err[normal] <= 2.0**-4 * np.abs(yv[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= 2.0**-10 * sc[~normal] * (1 + 1e-6))
