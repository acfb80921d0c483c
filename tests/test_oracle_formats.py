"""Pins of the oracle's number formats (CPU only).

Each check compares oracle/formats.py with something other than itself: torch's
CPU casts (an independent library implementation), the OCP format tables under
tests/golden/, the tie rule of to_e2m1_rne ("Module compress", Functions), and
the exact Fraction-based implementation in tests/brute.py.
"""
import math
import os

import numpy as np
import pytest
import torch

import brute
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                parts = line.split()
                rows.append((int(parts[0], 16), float(parts[1])))
    return rows


# ---------------------------------------------------------------- bf16
def _sample_f32_patterns(per_exponent=64, seed=0):
    rng = np.random.default_rng(seed)
    exps = np.repeat(np.arange(0, 255, dtype=np.uint32), per_exponent)
    mant = rng.integers(0, 1 << 23, size=exps.size, dtype=np.uint32)
    sign = rng.integers(0, 2, size=exps.size, dtype=np.uint32)
    bits = (sign << 31) | (exps << 23) | mant
    # every exponent also gets exact ties with an even and an odd kept bit,
    # and the patterns just either side of a tie
    ties = []
    for e in range(0, 255):
        for low in (0x8000, 0x7FFF, 0x8001):
            for keep in (0x000000, 0x010000, 0x7E0000, 0x7F0000):
                ties.append((e << 23) | keep | low)
    ties = np.array(ties, dtype=np.uint32)
    bits = np.concatenate([bits, ties, ties | np.uint32(0x80000000)])
    return bits.view(np.float32)


def test_bf16_matches_torch_cast_over_all_exponents():
    x = _sample_f32_patterns()
    ours = F.bf16_round(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_bf16_special_values():
    x = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.4e38, -3.4e38], dtype=np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()
    assert np.array_equal(F.bf16_round(x).view(np.uint32), ref.view(np.uint32))
    assert np.isnan(F.bf16_round(np.array([np.nan], dtype=np.float32))[0])


def test_bf16_from_float64_rounds_once():
    # brute.bf16 rounds a binary64 with Python's half-to-even round(): the
    # oracle must agree, including values whose nearest f32 is a bf16 tie
    rng = np.random.default_rng(1)
    vals = rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, 4000))
    tie = np.float64(1.0 + 2.0 ** -8)  # exact bf16 midpoint between 1 and 1+2^-7
    vals = np.concatenate([vals, [tie + 2.0 ** -40, tie - 2.0 ** -40, tie, -tie - 2.0 ** -40]])
    ours = F.bf16_round(vals)
    ref = np.array([brute.bf16(float(v)) for v in vals], dtype=np.float64)
    assert np.array_equal(ours.astype(np.float64), ref)
    assert ours[-4] == np.float32(1.0 + 2.0 ** -7)   # above the tie rounds up
    assert ours[-3] == np.float32(1.0)               # below it rounds down
    assert ours[-2] == np.float32(1.0)               # the tie goes to even


def test_bf16_bits_roundtrip():
    x = np.array([1.0, -2.5, 1e-3], dtype=np.float32)
    assert np.array_equal(F.bf16_from_bits(F.bf16_bits(x)), F.bf16_round(x))


# ---------------------------------------------------------------- e4m3fn
def test_e4m3fn_table_matches_ocp_points():
    for code, value in _read_table("ocp_e4m3fn_points.txt"):
        assert F.E4M3FN_VALUES[code] == value
        assert F.e4m3fn_encode(np.array([value]))[0] == code
    assert F.E4M3FN_MAX == 448.0
    assert F.E4M3FN_VALUES.size == 127
    assert np.all(np.diff(F.E4M3FN_VALUES) > 0)


def test_e4m3fn_every_code_is_a_fixed_point():
    codes = np.arange(0x7F, dtype=np.uint8)
    assert np.array_equal(F.e4m3fn_encode(F.e4m3fn_decode(codes)), codes)


def test_e4m3fn_matches_torch_on_every_latent_scale_quotient():
    # every positive finite bf16 amax, raised to at least 6 * 2^-9, divided by 6 in f32:
    # exactly the quotients fp4_quant_e4m3 can hand to the scale rounding
    pats = np.arange(0x0001, 0x7F80, dtype=np.uint32) << 16
    amax = pats.view(np.float32)
    amax = np.maximum(amax, np.float32(F.AMAX_FLOOR))
    q = (amax / np.float32(6.0)).astype(np.float32)
    q = q[q <= 448.0]
    ours = F.e4m3fn_encode(q)
    ref = torch.from_numpy(q.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    assert q.size > 17000


def test_e4m3fn_midpoints_go_to_even_code_and_saturate():
    v = F.E4M3FN_VALUES
    mids = (v[:-1] + v[1:]) / 2
    codes = F.e4m3fn_encode(mids)
    lower = np.arange(126)
    expected = np.where(lower % 2 == 0, lower, lower + 1)
    assert np.array_equal(codes, expected)
    assert F.e4m3fn_encode(np.array([449.0, 1e6]))[0] == 0x7E
    with pytest.raises(ValueError):
        F.e4m3fn_encode(np.array([-1.0]))


def test_e4m3fn_matches_brute_fraction_search():
    rng = np.random.default_rng(2)
    q = np.exp2(rng.uniform(-10, 8.8, 300))
    ours = F.e4m3fn_encode(q)
    ref = [brute.e4m3fn(float(v))[0] for v in q]
    assert list(ours) == ref


# ---------------------------------------------------------------- e2m1
def test_e2m1_table_matches_ocp():
    table = _read_table("ocp_e2m1.txt")
    for code, value in table:
        dec = F.e2m1_decode(np.array([code], dtype=np.uint8))[0]
        assert dec == value and math.copysign(1, dec) == math.copysign(1, value)
    assert list(F.E2M1_VALUES) == [v for c, v in table[:8]]


def test_e2m1_ties_go_to_even_code():
    g = F.E2M1_VALUES
    mids = (g[:-1] + g[1:]) / 2            # 0.25 0.75 1.25 1.75 2.5 3.5 5
    got = F.e2m1_encode(mids)
    assert list(got) == [0, 2, 2, 4, 4, 6, 6]
    assert list(F.e2m1_decode(got)) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    eps = 1e-9
    assert list(F.e2m1_encode(mids + eps)) == [1, 2, 3, 4, 5, 6, 7]
    assert list(F.e2m1_encode(mids - eps)) == [0, 1, 2, 3, 4, 5, 6]
    assert list(F.e2m1_encode(-mids)) == [8, 10, 10, 12, 12, 14, 14]


def test_e2m1_saturates_and_keeps_sign_of_zero():
    assert list(F.e2m1_encode(np.array([6.0, 7.0, 100.0, -9.0]))) == [7, 7, 7, 15]
    assert list(F.e2m1_encode(np.array([0.0, -0.0, -0.1, 0.1]))) == [0, 8, 8, 0]


def test_e2m1_matches_threshold_method_over_all_bf16_and_scales():
    # independent method: count the midpoints m*s that |y| passes, with a tie
    # counted upward only where the upper code is even; exact in float64
    y = F.bf16_from_bits(np.arange(0, 0x7F80, 37, dtype=np.uint16)).astype(np.float64)
    y = np.concatenate([y, -y])
    scales = F.E4M3FN_VALUES[1:]
    mids = (F.E2M1_VALUES[:-1] + F.E2M1_VALUES[1:]) / 2
    for s in scales[::3]:
        codes = F.e2m1_encode(y / s).astype(np.int64)
        a = np.abs(y)
        mag = np.zeros(y.shape, dtype=np.int64)
        for k, m in enumerate(mids):
            upper_even = (k + 1) % 2 == 0
            mag += (a > m * s) | (upper_even & (a == m * s))
        ref = mag | (np.signbit(y).astype(np.int64) << 3)
        assert np.array_equal(codes, ref), s


# ---------------------------------------------------------------- fp4 round trip
def test_fp4_zero_block():
    codes, scales, deq = F.fp4_quant_e4m3(np.zeros((2, 32), dtype=np.float32))
    assert np.all(codes == 0) and np.all(scales == 0x01) and np.all(deq == 0)


def test_fp4_exact_grid_points_round_trip_exactly():
    # a block holding grid values times a scale that is already an e4m3 value
    # with amax = 6 * scale: the scale is found exactly and every value returns
    rng = np.random.default_rng(3)
    for s_code in (0x08, 0x20, 0x38, 0x3B, 0x50):
        s = F.E4M3FN_VALUES[s_code]
        mags = rng.choice(F.E2M1_VALUES, size=16)
        mags[5] = 6.0
        signs = rng.choice([-1.0, 1.0], size=16)
        y = F.bf16_round((mags * signs * s).astype(np.float32))[None, :]
        codes, scales, deq = F.fp4_quant_e4m3(y)
        assert scales[0, 0] == s_code
        assert np.array_equal(deq, y)


def test_fp4_packing_low_nibble_first():
    y = np.zeros((1, 16), dtype=np.float32)
    y[0, 0], y[0, 1], y[0, 15] = 6.0, -3.0, 0.5
    codes, scales, _ = F.fp4_quant_e4m3(y)
    assert scales[0, 0] == 0x38          # 6 / 6 = 1.0
    assert codes[0, 0] == (0x7 | (0xD << 4))
    assert codes[0, 7] == (0x0 | (0x1 << 4))
    assert np.array_equal(F.fp4_unpack(codes)[0, :2], [0x7, 0xD])


def test_fp4_error_bound_and_scale_rule():
    rng = np.random.default_rng(4)
    y = F.bf16_round((rng.standard_normal((64, 512)) * np.exp2(rng.integers(-8, 5, (64, 1)))).astype(np.float32))
    codes, scales, deq = F.fp4_quant_e4m3(y)
    s = F.e4m3fn_decode(scales).repeat(16, axis=1)
    amax = np.maximum(np.abs(y.reshape(64, 32, 16)).max(axis=2), F.AMAX_FLOOR).repeat(16, axis=1)
    err = np.abs(deq.astype(np.float64) - y)
    # half the widest grid gap (4 -> 6) is one scale unit; beyond 6 * scale
    # the value saturates to 6 * scale
    bound = np.maximum(s, amax - 6 * s) + 1e-12
    assert np.all(err <= bound)
    # the scale is within half an e4m3 step of amax / 6: 2^-4 relative for
    # normal values, half the subnormal spacing 2^-9 below 2^-6
    q = amax / 6
    half_step = np.where(q >= 2.0 ** -6, q * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(s - q) <= half_step * (1 + 1e-9))


def test_fp4_matches_brute_fraction_implementation():
    rng = np.random.default_rng(5)
    y = F.bf16_round((rng.standard_normal((6, 64)) * np.exp2(rng.integers(-12, 6, (6, 1)))).astype(np.float32))
    y[0, :16] = 0.0
    y[1, 16:32] = -0.0
    codes, scales, deq = F.fp4_quant_e4m3(y)
    unpacked = F.fp4_unpack(codes)
    for r in range(6):
        for b in range(4):
            blk = [float(v) for v in y[r, 16 * b:16 * b + 16]]
            bc, bs, bd = brute.fp4_block(blk)
            assert list(unpacked[r, 16 * b:16 * b + 16]) == bc
            assert scales[r, b] == bs
            assert [float(v) for v in deq[r, 16 * b:16 * b + 16]] == bd


def test_fp4_dequant_is_exact_in_bf16():
    # grid value * e4m3 scale has at most 6 significant bits, so the final
    # bf16 rounding of the round trip never changes it
    g = F.E2M1_VALUES[:, None]
    s = F.E4M3FN_VALUES[None, 1:]
    prod = (g * s).astype(np.float32)
    assert np.array_equal(F.bf16_round(prod), prod)


# ---------------------------------------------------------------- e8m0 fp4 round trip
def test_pow2_ceil_exponent_matches_brute():
    rng = np.random.default_rng(6)
    q = np.concatenate([np.exp2(rng.uniform(-126, 126, 500)),
                        np.exp2(np.arange(-126, 127, dtype=np.float64)),
                        np.nextafter(np.exp2(np.arange(-100, 100, 7, dtype=np.float64)), np.inf),
                        np.nextafter(np.exp2(np.arange(-100, 100, 7, dtype=np.float64)), 0)])
    ours = F.pow2_ceil_exponent(q)
    ref = [brute.pow2_ceil(float(v)) for v in q]
    assert list(ours) == ref
    with pytest.raises(ValueError):
        F.pow2_ceil_exponent(np.array([0.0]))


def test_fp4_e8m0_special_cases():
    # zero block: scale 2^-126 (byte 1), codes 0
    codes, scales, deq = F.fp4_quant_e8m0(np.zeros((1, 64), dtype=np.float32))
    assert np.all(scales == 1) and np.all(codes == 0) and np.all(deq == 0)
    # amax exactly 6 * 2^k: scale 2^k, grid values come back exactly
    rng = np.random.default_rng(7)
    for k in (-20, -3, 0, 5, 40):
        mags = rng.choice(F.E2M1_VALUES, size=32)
        mags[7] = 6.0
        y = (mags * rng.choice([-1.0, 1.0], 32) * 2.0 ** k).astype(np.float32)[None]
        codes, scales, deq = F.fp4_quant_e8m0(y)
        assert scales[0, 0] == k + 127
        assert np.array_equal(deq, y)
    # amax just above 6 * 2^k: the next power of two
    y = np.zeros((1, 32), dtype=np.float32)
    y[0, 0] = F.bf16_round(np.array([6.0 * 1.0078125], dtype=np.float32))[0]
    _, scales, _ = F.fp4_quant_e8m0(y)
    assert scales[0, 0] == 1 + 127


def test_fp4_e8m0_bounds():
    rng = np.random.default_rng(8)
    y = F.bf16_round((rng.standard_normal((64, 128)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32))
    codes, scales, deq = F.fp4_quant_e8m0(y)
    s = np.exp2(scales.astype(np.float64) - 127).repeat(32, axis=1)
    amax = np.maximum(np.abs(y.reshape(64, 4, 32)).max(axis=2), F.E8M0_AMAX_FLOOR).repeat(32, axis=1)
    # the power-of-two ceiling: amax / 6 <= scale < amax / 3
    assert np.all(s >= amax / 6) and np.all(s < amax / 3)
    # no saturation: |y / scale| <= 6, so the error is at most half the
    # widest grid gap (4 -> 6), one scale unit
    assert np.all(np.abs(deq.astype(np.float64) - y) <= s)


def test_fp4_e8m0_matches_brute_fraction_implementation():
    rng = np.random.default_rng(9)
    y = F.bf16_round((rng.standard_normal((6, 64)) * np.exp2(rng.integers(-40, 20, (6, 1)))).astype(np.float32))
    y[2, :32] = 0.0
    y[3, 32:] = -0.0
    codes, scales, deq = F.fp4_quant_e8m0(y)
    unpacked = F.fp4_unpack(codes)
    for r in range(6):
        for b in range(2):
            blk = [float(v) for v in y[r, 32 * b:32 * b + 32]]
            bc, bs, bd = brute.fp4_block_e8m0(blk)
            assert list(unpacked[r, 32 * b:32 * b + 32]) == bc
            assert scales[r, b] == bs
            assert [float(v) for v in deq[r, 32 * b:32 * b + 32]] == bd


def test_fp4_e8m0_top_of_the_bf16_range():
    # the largest finite bf16 value: amax / 6 lies in (2^125, 2^126], scale
    # 2^126 (byte 253); |y| / 2^126 ~ 3.98 takes code 4, whose value 2^128 is
    # past the bf16 range, so the dequantised value is inf; 2.98e38 (code 3,
    # value 3 * 2^126) still comes back finite
    top = np.float32(F.bf16_from_bits(np.array([0x7F7F], dtype=np.uint16))[0])
    y = np.zeros((1, 32), dtype=np.float32)
    y[0, 0], y[0, 1], y[0, 2] = top, -top, F.bf16_round(np.array([2.9e38], dtype=np.float32))[0]
    codes, scales, deq = F.fp4_quant_e8m0(y)
    assert scales[0, 0] == 253
    assert deq[0, 0] == np.inf and deq[0, 1] == -np.inf
    assert deq[0, 2] == np.float32(3.0 * 2.0 ** 126)
    bc, bs, bd = brute.fp4_block_e8m0([float(v) for v in y[0]])
    assert list(F.fp4_unpack(codes)[0]) == bc and bs == 253
    assert [float(v) for v in deq[0]] == bd
