"""RoPE of the compressed entries: CPU oracle (test infrastructure only).

Only tests/, the smoke check and the CPU-baseline leg of the benchmark may
import this module; the product path never does.

What the pages fix ("Compressed Sparse Attention . ratio m = 4", Full
compression path, "Normalize + RoPE + cache"; Released Flash configuration,
RoPE sub-dimension 64; "Module compress", Functions, yarn_freqs_cis): after the
RMSNorm the entry's rotary slice is rotated by its position's angles, then the
entry is cached; the angles come from a YaRN-corrected table of (cos, sin)
pairs, [positions][rope_dim / 2], built from compress_rope_theta. The
compressor itself returns the unrotated latent ("DeepSeek V4.1 . Pool token
pairs", Compressor listing, docstring: the indexer needs the unrotated form).

Readings (the pages leave these open):
  - the rotary slice is the last rope_dim features of the entry;
  - a rotary pair is two neighbouring features (2i, 2i+1) of the slice, and
    pair i turns by the angle of table column i: (a, b) -> (a c - b s, a s + b c);
  - the table has one row per compressed entry (the caller decides which token
    position entry j stands for when it builds row j);
  - the rotation is computed from the bf16 latent and rounded once to bf16;
  - theta, the YaRN scaling factor, the original context length and the ramp
    bounds are arguments: the pages give none of them.

yarn_inv_freq follows the "NTK-by-parts" interpolation of the YaRN paper (Peng
et al., 2023, section 3.2): dimension i has base frequency theta^(-2i/d) and
wavelength 2 pi / theta_i; with r = L / wavelength rotations over the original
context L, a dimension with r above beta_fast keeps its frequency, one with r
below beta_slow is divided by the scaling factor, and between the two the
frequency is blended linearly in r. (The paper's attention temperature scales
the attention logits, not this table, and is not part of it.)
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_round


def yarn_inv_freq(rope_dim: int, theta: float, factor: float = 1.0, original_max_pos: float | None = None,
                  beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """Per-pair angular frequencies [rope_dim / 2], float64."""
    if rope_dim <= 0 or rope_dim % 2:
        raise ValueError("rope_dim must be a positive even number")
    i = np.arange(rope_dim // 2, dtype=np.float64)
    base = float(theta) ** (-2.0 * i / rope_dim)
    if factor == 1.0 or original_max_pos is None:
        return base
    if not beta_fast > beta_slow:
        raise ValueError("beta_fast must exceed beta_slow")
    rotations = float(original_max_pos) * base / (2.0 * np.pi)
    keep = np.clip((rotations - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    return (1.0 - keep) * base / factor + keep * base


def rope_table(positions, inv_freq: np.ndarray) -> np.ndarray:
    """(cos, sin) of position * frequency, [len(positions)][rope_dim / 2][2],
    computed in float64 and rounded once to f32."""
    ang = np.outer(np.asarray(positions, dtype=np.float64), np.asarray(inv_freq, dtype=np.float64))
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def apply_rope(latent: np.ndarray, rows: np.ndarray, rope_dim: int) -> np.ndarray:
    """Rotate the last rope_dim features of each entry of `latent` [..., hd]
    (bf16 values) by its table row (`rows` [..., rope_dim / 2, 2] f32, one row
    per entry): pair i = features (hd - rope_dim + 2i, +1) turns by column i.
    Each new value is the exact a c - b s (or a s + b c) rounded once to bf16;
    the other features pass unchanged."""
    lat = np.asarray(latent, dtype=np.float32)
    hd = lat.shape[-1]
    if rope_dim <= 0 or rope_dim % 2 or rope_dim > hd:
        raise ValueError("rope_dim must be even and within the entry")
    rows = np.asarray(rows, dtype=np.float32)
    if rows.shape != lat.shape[:-1] + (rope_dim // 2, 2):
        raise ValueError("one (cos, sin) row per entry")
    out = lat.copy()
    pairs = lat[..., hd - rope_dim:].astype(np.float64).reshape(lat.shape[:-1] + (rope_dim // 2, 2))
    a, b = pairs[..., 0], pairs[..., 1]
    c, s = rows[..., 0].astype(np.float64), rows[..., 1].astype(np.float64)
    first = _round_sum_bf16(a * c, -(b * s))
    second = _round_sum_bf16(a * s, b * c)
    out[..., hd - rope_dim:] = np.stack([first, second], axis=-1).reshape(lat.shape[:-1] + (rope_dim,))
    return out


def _round_sum_bf16(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """bf16 nearest (ties to even) to the exact sum p + q of two float64
    values. The products of a bf16 and an f32 value are exact in float64; the
    sum is rounded once to float64 (hi) with the exact error lo (TwoSum). Only
    when hi falls exactly on a bf16 midpoint can lo change the bf16 result: hi
    is then moved one float64 step towards lo, which puts it on the exact
    sum's side of the midpoint without crossing another bf16 boundary."""
    hi = p + q
    z = hi - p
    lo = (p - (hi - z)) + (q - z)
    on_mid = _is_bf16_midpoint(hi)
    nudged = np.where(on_mid & (lo != 0), np.nextafter(hi, np.where(lo > 0, np.inf, -np.inf)), hi)
    return bf16_round(nudged)


def _is_bf16_midpoint(x: np.ndarray) -> np.ndarray:
    """x (float64) lies exactly halfway between two neighbouring bf16 values:
    it is an f32 value whose low 16 bits are 0x8000."""
    f = x.astype(np.float32)
    exact = f.astype(np.float64) == x
    return exact & ((np.ascontiguousarray(f).view(np.uint32) & 0xFFFF) == 0x8000)
