"""A second, independent implementation of the compressor for tiny inputs.

Pure Python: float (binary64) arithmetic, math.exp, Python's round() (which
rounds half to even), and fractions.Fraction where a rounding decision has to
be exact. It shares no code with oracle/ and is only used to pin the oracle on
inputs small enough for loops.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def f32(v: float) -> float:
    """Round a Python float to the nearest binary32 (struct packs with RNE)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def bf16(v: float) -> float:
    """Nearest bf16 (8 significant bits), ties to even, from a binary64 value."""
    if v == 0.0 or math.isinf(v) or math.isnan(v):
        return v
    m, e = math.frexp(v)          # v = m * 2^e, 0.5 <= |m| < 1
    q = round(m * 256.0)          # 8 significant bits, half to even
    r = math.ldexp(q, e - 8)
    if abs(r) >= 2.0 ** 128:      # past the largest finite bf16: overflow
        return math.copysign(math.inf, v)
    return r


def dot(a, b) -> float:
    """Exactly rounded dot product (Fractions), as a binary64."""
    return float(sum(Fraction(x) * Fraction(y) for x, y in zip(a, b)))


def e4m3fn(v: float) -> tuple[int, float]:
    """Nearest e4m3fn value to v >= 0 (ties to the even code, saturating at 448).
    Built from the format's parameters: values m/8 * 2^-6 below 2^-6, then
    (1 + m/8) * 2^(e-7) for e = 1..15 without the all-ones pattern."""
    best = None
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        val = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        d = abs(Fraction(v) - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code, val)
    return best[1], float(best[2])


# e2m1 midpoints between consecutive magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 and
# the code an exact midpoint goes to (the even one of the two).
_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e2m1(y: float, s: float) -> int:
    """e2m1 code of y / s by exact comparisons against the midpoints."""
    q = abs(Fraction(y) / Fraction(s))
    code = 0
    for k in range(7):
        mid = (Fraction(_E2M1[k]) + Fraction(_E2M1[k + 1])) / 2
        if q > mid or (q == mid and (k + 1) % 2 == 0):
            code = k + 1
    if math.copysign(1.0, y) < 0:
        code |= 8
    return code


def fp4_block(y: list[float]):
    """fp4 round trip of one block of 16 bf16 values: (codes, scale byte, deq)."""
    a = max(max(abs(v) for v in y), 6.0 * 2.0 ** -9)
    scale_code, s = e4m3fn(f32(a / 6.0))
    codes = [e2m1(v, s) for v in y]
    deq = [bf16(math.copysign(_E2M1[c & 7] * s, -1.0 if c & 8 else 1.0)) for c in codes]
    return codes, scale_code, deq


def softmax_pool(kv: list[list[float]], sc: list[list[float]], hd: int) -> list[float]:
    """sum_i softmax_i(sc) * kv_i per feature, in binary64, rounded to f32."""
    out = []
    for f in range(hd):
        logits = [row[f] for row in sc]
        m = max(logits)
        e = [0.0 if s == -math.inf else math.exp(s - m) for s in logits]
        den = sum(e)
        out.append(f32(sum(ei / den * row[f] for ei, row in zip(e, kv))))
    return out


def rmsnorm(p: list[float], eps: float) -> list[float]:
    u = [bf16(v) for v in p]
    ms = math.fsum(v * v for v in u) / len(u)
    r = 1.0 / math.sqrt(ms + eps)
    return [bf16(v * r) for v in u]


class BruteCompressor:
    """Streaming compressor over lists, one batch row, pages' readings:
    ratio 4 overlaps (branch A = first hd columns, branch B = last hd)."""

    def __init__(self, ratio, hd, wkv, wgate, ape, eps=1e-6):
        self.r, self.hd, self.eps = ratio, hd, eps
        self.wkv, self.wgate, self.ape = wkv, wgate, ape
        self.ov = ratio == 4
        width = 2 * hd if self.ov else hd
        rows = 2 * ratio if self.ov else ratio
        self.kv = [[0.0] * width for _ in range(rows)]
        self.sc = [[-math.inf] * width for _ in range(rows)]

    def _project(self, x, t):
        kv = [f32(dot(x, w)) for w in self.wkv]
        sc = [f32(dot(x, w)) for w in self.wgate]
        if self.ape is not None:
            sc = [f32(s + b) for s, b in zip(sc, self.ape[t % self.r])]
        return kv, sc

    def _emit(self, kv_rows, sc_rows):
        p = softmax_pool(kv_rows, sc_rows, self.hd)
        return p, rmsnorm(p, self.eps)

    def _window(self, prev_kv, prev_sc, cur_kv, cur_sc):
        hd = self.hd
        return ([row[hd:] for row in prev_kv] + [row[:hd] for row in cur_kv],
                [row[hd:] for row in prev_sc] + [row[:hd] for row in cur_sc])

    def prefill(self, xs):
        """xs: list of token vectors. Returns list of (pooled, latent)."""
        r, hd = self.r, self.hd
        proj = [self._project(x, t) for t, x in enumerate(xs)]
        n = len(xs) // r
        out = []
        for j in range(n):
            cur = proj[r * j:r * j + r]
            if self.ov:
                if j == 0:
                    prev_kv = [[0.0] * (2 * hd)] * r
                    prev_sc = [[-math.inf] * (2 * hd)] * r
                else:
                    prev_kv = [p[0] for p in proj[r * (j - 1):r * j]]
                    prev_sc = [p[1] for p in proj[r * (j - 1):r * j]]
                kv_rows, sc_rows = self._window(prev_kv, prev_sc, [c[0] for c in cur], [c[1] for c in cur])
            else:
                kv_rows, sc_rows = [c[0] for c in cur], [c[1] for c in cur]
            out.append(self._emit(kv_rows, sc_rows))
        rem = len(xs) - n * r
        base = r if self.ov else 0
        for i in range(rem):
            self.kv[base + i] = list(proj[n * r + i][0])
            self.sc[base + i] = list(proj[n * r + i][1])
        if self.ov:
            for i in range(r):
                if n > 0:
                    self.kv[i] = list(proj[(n - 1) * r + i][0])
                    self.sc[i] = list(proj[(n - 1) * r + i][1])
                else:
                    self.kv[i] = [0.0] * (2 * hd)
                    self.sc[i] = [-math.inf] * (2 * hd)
        return out

    def decode(self, x, pos):
        """One token at position pos > 0; returns (pooled, latent) or None."""
        r = self.r
        kv, sc = self._project(x, pos)
        slot = pos % r
        row = r + slot if self.ov else slot
        self.kv[row], self.sc[row] = kv, sc
        if (pos + 1) % r:
            return None
        if self.ov:
            kv_rows, sc_rows = self._window(self.kv[:r], self.sc[:r], self.kv[r:], self.sc[r:])
            res = self._emit(kv_rows, sc_rows)
            self.kv[:r] = [list(v) for v in self.kv[r:]]
            self.sc[:r] = [list(v) for v in self.sc[r:]]
            return res
        return self._emit(self.kv, self.sc)


def pow2_ceil(q: float) -> int:
    """Smallest integer e with 2^e >= q (exact, Fraction comparisons)."""
    fq = Fraction(q)
    e = 0
    while Fraction(2) ** e < fq:
        e += 1
    while Fraction(2) ** (e - 1) >= fq:
        e -= 1
    return e


def fp4_block_e8m0(y: list[float]):
    """Power-of-two-scaled fp4 round trip of one block (any length):
    (codes, scale byte, deq)."""
    a = max(max(abs(v) for v in y), 6.0 * 2.0 ** -126)
    e = pow2_ceil(f32(a / 6.0))
    s = 2.0 ** e
    codes = [e2m1(v, s) for v in y]
    deq = [bf16(math.copysign(_E2M1[c & 7] * s, -1.0 if c & 8 else 1.0)) for c in codes]
    return codes, e + 127, deq


def plain_projection(xs, wkv, eps=1e-6):
    """Ratio-1 compressor over a list of token vectors (bf16 values): for each
    token, (f32 projection, latent) with an exactly rounded dot product."""
    out = []
    for x in xs:
        p = [f32(dot(x, w)) for w in wkv]
        out.append((p, rmsnorm(p, eps)))
    return out


def bf16_of_fraction(v: Fraction) -> float:
    """Nearest bf16 to an exact rational, ties to even (normal range)."""
    if v == 0:
        return 0.0
    mag = abs(v)
    e = math.frexp(float(mag))[1] - 1          # 2^e <= mag < 2^(e+1), up to float's own rounding
    while Fraction(2) ** e > mag:
        e -= 1
    while Fraction(2) ** (e + 1) <= mag:
        e += 1
    q = round(mag / Fraction(2) ** (e - 7))    # 8 significant bits, half to even
    r = math.ldexp(q, e - 7)
    return r if v > 0 else -r


def rope(latent: list[float], rows: list[tuple[float, float]], rope_dim: int) -> list[float]:
    """Rotate the last rope_dim features of one entry as pairs (2i, 2i+1) by
    (cos, sin) row i, exactly, one rounding to bf16."""
    out = list(latent)
    start = len(latent) - rope_dim
    for i, (c, s) in enumerate(rows):
        a, b = Fraction(latent[start + 2 * i]), Fraction(latent[start + 2 * i + 1])
        fc, fs = Fraction(c), Fraction(s)
        out[start + 2 * i] = bf16_of_fraction(a * fc - b * fs)
        out[start + 2 * i + 1] = bf16_of_fraction(a * fs + b * fc)
    return out
