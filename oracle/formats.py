"""Number formats of the compressor oracle: bf16, OCP e4m3fn, OCP e2m1, and the
latent's fp4 round trip.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module.

Every rounding here is written as its plain definition: list the representable
values of the target format, take the nearest one to the exact input, and break
an exact tie towards the even code. Nothing is derived from bit tricks, so a
reader can check each function against the format's definition by eye.

Sources:
  * "Module compress" (DeepSeek-V4.1 reference docs), Precision paragraph: the
    number types along the compressor. Arithmetic is f32 through pooling, a
    bf16 rounding sits in front of the RMSNorm, and the cached latent is kept
    in an fp4 form (e2m1 elements, one e4m3 scale per 16 values).
  * "Module compress", Functions, fp4_quant_e4m3_inplace: the latent's fp4
    round trip. Per block the scale comes from the block's largest magnitude
    (bounded below by 6 * 2^-9) over 6, rounded to e4m3; each value over the
    scale becomes an e2m1 code; code times scale, as bf16, overwrites the
    input.
  * "Module compress", Functions, to_e2m1_rne: the e2m1 rounding (nearest grid
    point, exact ties to the even code, the sign carried over).
  * "Module compress", Constants, LATENT_BLOCK: 16 values per e4m3 scale.
  * Format definitions (not on the pages): bf16 = the upper half of an IEEE
    binary32; e4m3fn and e2m1 = the OCP 8-bit floating point and OCP
    Microscaling (MX) v1.0 element formats.

Pins (tests/test_oracle_formats.py): bf16 against torch's CPU cast over sampled
bit patterns of every exponent; e4m3fn against torch's CPU float8_e4m3fn cast,
exhaustively over every quotient a/6 the latent can produce; e2m1 against the
OCP value table and every tie of the grid; the fp4 round trip against its
special cases (zero block, exact grid points, saturation, the error bound).
"""
from __future__ import annotations

import numpy as np

# Values per e4m3 scale in the latent's fp4 round trip ("Module compress",
# Constants, LATENT_BLOCK).
LATENT_BLOCK = 16

# Block length of the indexer's fp4 form, which shares one power-of-two
# scale among 32 values ("Module compress", Constants, FP4_BLOCK, and the
# Precision paragraph).
FP4_BLOCK = 32

# The amax floor of fp4_quant_e8m0_inplace: 6 * 2^-126, so that amax / 6 is
# at least the smallest normal power of two.
E8M0_AMAX_FLOOR = 6.0 * 2.0 ** -126

# The amax floor of fp4_quant_e4m3_inplace: 6 * 2^-9, so that amax / 6 is at
# least the smallest e4m3fn subnormal and the scale never flushes to zero.
AMAX_FLOOR = 6.0 * 2.0 ** -9


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------
def _bf16_magnitude_value(pattern: np.ndarray) -> np.ndarray:
    """float64 value of non-negative bf16 patterns given as the upper 16 bits
    of a binary32 (uint64 array); the pattern just past the largest finite one
    stands for 2^128, the value IEEE rounding compares against for overflow."""
    as32 = (np.minimum(pattern, 0x7F7F) << 16).astype(np.uint32).view(np.float32)
    return np.where(pattern >= 0x7F80, 2.0 ** 128, as32.astype(np.float64))


def bf16_round(x) -> np.ndarray:
    """Round float32 or float64 values to the nearest bf16 value, ties to even,
    with a single rounding from the input's exact value.

    bf16 keeps the sign, the 8 exponent bits and the top 7 mantissa bits of a
    binary32. For each input magnitude the candidates are three consecutive
    bf16 patterns around it (the upper half of its nearest f32 and the patterns
    on either side). The nearest candidate wins; on an exact tie the one whose
    last mantissa bit is 0 wins. A magnitude at or past the midpoint between
    the largest finite bf16 and 2^128 overflows to infinity. The sign is copied
    from the input. Returns float32 arrays holding the rounded values.
    """
    x = np.asarray(x)
    xd = x.astype(np.float64)
    mag = np.abs(xd)
    with np.errstate(over="ignore"):
        f = mag.astype(np.float32)
    top = (np.ascontiguousarray(f).view(np.uint32) >> 16).astype(np.int64)
    cands = np.stack([np.maximum(top - 1, 0), top, top + 1], axis=0).astype(np.uint64)
    vals = _bf16_magnitude_value(cands)
    dist = np.abs(vals - mag[None])
    best = dist.min(axis=0, keepdims=True)
    is_best = dist == best
    even = (cands & 1) == 0
    pick_even = (is_best & even).any(axis=0)
    choice = np.where(pick_even, np.argmax(is_best & even, axis=0), np.argmax(is_best, axis=0))
    pattern = np.take_along_axis(cands, choice[None], axis=0)[0]
    pattern = np.minimum(pattern, 0x7F80)  # 2^128 -> infinity
    out = (pattern << 16).astype(np.uint32).view(np.float32)
    out = np.copysign(out, xd).astype(np.float32)
    special = ~np.isfinite(xd)
    out[special] = xd[special].astype(np.float32)  # inf stays inf, NaN stays NaN
    return out


def bf16_bits(x) -> np.ndarray:
    """The 16-bit patterns of bf16_round(x)."""
    return (bf16_round(x).view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b) -> np.ndarray:
    """float32 values of 16-bit bf16 patterns."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


# --------------------------------------------------------------------------
# nearest-value search shared by the two small formats
# --------------------------------------------------------------------------
def _nearest_code(mag: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the table value nearest to each non-negative `mag`.

    `table` lists a format's non-negative values in code order (ascending). On
    an exact tie between two codes the even code wins. Values past the end of
    the table take its last code (saturation).
    """
    mag = np.asarray(mag, dtype=np.float64).reshape(-1)
    # saturation first: far past the table, float64 distances would all round
    # to the same value and stop telling the codes apart
    mag = np.minimum(mag, table[-1])
    out = np.empty(mag.size, dtype=np.uint8)
    codes = np.arange(table.size)
    chunk = 1 << 16  # bounds the [chunk, table] distance matrix
    for start in range(0, mag.size, chunk):
        part = mag[start:start + chunk]
        dist = np.abs(part[:, None] - table[None, :])
        best = dist.min(axis=1, keepdims=True)
        is_best = dist == best
        # prefer an even code among the nearest ones, else the first nearest one
        even_best = is_best & (codes[None, :] % 2 == 0)
        pick_even = even_best.any(axis=1)
        first_even = np.argmax(even_best, axis=1)
        first_any = np.argmax(is_best, axis=1)
        out[start:start + chunk] = np.where(pick_even, first_even, first_any)
    return out


# --------------------------------------------------------------------------
# OCP e4m3fn (the scale format)
# --------------------------------------------------------------------------
def _e4m3fn_table() -> np.ndarray:
    """Values of the codes 0x00..0x7e: 4 exponent bits with bias 7, 3 mantissa
    bits, subnormals at exponent field 0, no infinities, 0x7f is NaN."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m / 8.0 * 2.0 ** -6)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3FN_VALUES = _e4m3fn_table()
E4M3FN_MAX = float(E4M3FN_VALUES[-1])  # 448


def e4m3fn_encode(x) -> np.ndarray:
    """Round non-negative values to e4m3fn codes (nearest, ties to even code,
    saturating at 448). Negative inputs are rejected: scales are amax / 6."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~(x >= 0)):
        raise ValueError("e4m3fn_encode takes non-negative, non-NaN values")
    return _nearest_code(x, E4M3FN_VALUES).reshape(x.shape)


def e4m3fn_decode(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8)
    if np.any((code & 0x7F) == 0x7F):
        raise ValueError("NaN code")
    mag = E4M3FN_VALUES[code & 0x7F]
    return np.where(code & 0x80, -mag, mag)


# --------------------------------------------------------------------------
# OCP e2m1 (the fp4 element format)
# --------------------------------------------------------------------------
def _e2m1_table() -> np.ndarray:
    """Values of the magnitude codes 0..7: 2 exponent bits with bias 1 and one
    mantissa bit, subnormal at exponent field 0."""
    vals = []
    for code in range(8):
        e, m = code >> 1, code & 1
        if e == 0:
            vals.append(m * 0.5)
        else:
            vals.append((1.0 + m / 2.0) * 2.0 ** (e - 1))
    return np.array(vals, dtype=np.float64)


E2M1_VALUES = _e2m1_table()  # 0, 0.5, 1, 1.5, 2, 3, 4, 6


def e2m1_encode(v) -> np.ndarray:
    """to_e2m1_rne: the nearest e2m1 value, ties to the even code, magnitudes
    above 6 saturating to 6; the sign bit (0x8) is the sign bit of the input,
    so a negative value that rounds to zero keeps it."""
    v = np.asarray(v, dtype=np.float64)
    mag_code = _nearest_code(np.abs(v), E2M1_VALUES).reshape(v.shape)
    sign = np.signbit(v).astype(np.uint8) << 3
    return (mag_code | sign).astype(np.uint8)


def e2m1_decode(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8)
    mag = E2M1_VALUES[code & 7]
    return np.where(code & 8, -mag, mag)


# --------------------------------------------------------------------------
# the latent's fp4 round trip
# --------------------------------------------------------------------------
def fp4_quant_e4m3(y, block: int = LATENT_BLOCK):
    """fp4_quant_e4m3_inplace on rows of bf16 values.

    `y` is [rows, width] float32 holding bf16 values (width a multiple of
    `block`). Per block of `block` consecutive values of a row:
      a     = max(max |y|, 6 * 2^-9)
      scale = e4m3fn(round_f32(a / 6))       (a / 6 as one IEEE f32 division)
      code  = e2m1(y / scale)                 (the exact quotient's rounding)
      deq   = bf16(e2m1_value(code) * scale)
    Returns (codes [rows, width/2] u8, two codes per byte with the lower-index
    element in the low nibble; scales [rows, width/block] u8 e4m3fn bit
    patterns; deq [rows, width] float32 holding bf16 values).
    """
    y = np.asarray(y, dtype=np.float32)
    if y.ndim != 2 or y.shape[1] % block:
        raise ValueError("y must be [rows, width] with width a multiple of the block")
    rows, width = y.shape
    blocks = y.reshape(rows, width // block, block).astype(np.float64)
    amax = np.abs(blocks).max(axis=2)
    amax = np.maximum(amax, AMAX_FLOOR)
    quotient = (amax.astype(np.float32) / np.float32(6.0)).astype(np.float32)
    scale_code = e4m3fn_encode(quotient)
    scale = e4m3fn_decode(scale_code)  # exact, > 0
    # The quotient y / scale is exact or lies at least 2^-9 (relative) away
    # from every midpoint of the e2m1 grid (y has 8 significant bits, scale 4),
    # so its float64 value decides the same code as the exact quotient.
    v = blocks / scale[:, :, None]
    codes = e2m1_encode(v)
    # A block whose largest magnitude lies above 3.5 * 2^126 takes scale 2^126
    # and code 4: the decoded 2^128 lies past the f32 and bf16 range and becomes
    # inf, as round-to-nearest does on overflow.
    with np.errstate(over="ignore"):
        deq = bf16_round((e2m1_decode(codes) * scale[:, :, None]).astype(np.float32))
    codes = codes.reshape(rows, width)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale_code.astype(np.uint8), deq.reshape(rows, width)


def fp4_unpack(packed: np.ndarray) -> np.ndarray:
    """Inverse of the nibble packing: [rows, width/2] bytes -> [rows, width] codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# --------------------------------------------------------------------------
# the indexer's fp4 round trip (power-of-two scales)
# --------------------------------------------------------------------------
def pow2_ceil_exponent(q) -> np.ndarray:
    """The smallest integer e with 2^e >= q, for finite q > 0 (exact: from
    the float64 value's frexp, q = m * 2^x with 0.5 <= m < 1)."""
    q = np.asarray(q, dtype=np.float64)
    if np.any(~(q > 0)) or np.any(~np.isfinite(q)):
        raise ValueError("pow2_ceil_exponent takes finite positive values")
    m, x = np.frexp(q)
    return np.where(m == 0.5, x - 1, x).astype(np.int64)


def fp4_quant_e8m0(y, block: int = FP4_BLOCK):
    """fp4_quant_e8m0_inplace on rows of bf16 values.

    Per block of `block` consecutive values of a row:
      a     = max(max |y|, 6 * 2^-126)
      scale = 2^e, e the power-of-two ceiling exponent of round_f32(a / 6)
      code  = e2m1(y / scale)
      deq   = bf16(e2m1_value(code) * scale)
    The scale byte is the e8m0 pattern e + 127. Returns (codes [rows,
    width/2] u8, low nibble first; scales [rows, width/block] u8; deq [rows,
    width] float32 holding bf16 values).
    """
    y = np.asarray(y, dtype=np.float32)
    if y.ndim != 2 or y.shape[1] % block:
        raise ValueError("y must be [rows, width] with width a multiple of the block")
    rows, width = y.shape
    blocks = y.reshape(rows, width // block, block).astype(np.float64)
    amax = np.maximum(np.abs(blocks).max(axis=2), E8M0_AMAX_FLOOR)
    quotient = (amax.astype(np.float32) / np.float32(6.0)).astype(np.float32)
    e = pow2_ceil_exponent(quotient)
    scale = np.exp2(e.astype(np.float64))
    codes = e2m1_encode(blocks / scale[:, :, None])  # exact quotients
    # A block whose largest magnitude lies above 3.5 * 2^126 takes scale 2^126
    # and code 4: the decoded 2^128 lies past the f32 and bf16 range and becomes
    # inf, as round-to-nearest does on overflow.
    with np.errstate(over="ignore"):
        deq = bf16_round((e2m1_decode(codes) * scale[:, :, None]).astype(np.float32))
    codes = codes.reshape(rows, width)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8), deq.reshape(rows, width)
