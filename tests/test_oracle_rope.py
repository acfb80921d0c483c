"""Pins of the RoPE oracle (CPU only): the YaRN frequencies against their
closed forms and limits (the YaRN paper's NTK-by-parts definition), the
rotation against an exact rational implementation (tests/brute.py), and the
invariants of a rotation."""
import math

import numpy as np
import pytest

import brute
import oracle
from oracle.rope import apply_rope, rope_table, yarn_inv_freq


def test_plain_frequencies_closed_form():
    f = yarn_inv_freq(64, 10000.0)
    assert f[0] == 1.0
    assert math.isclose(f[16], 10000.0 ** -0.5, rel_tol=1e-15)
    ratios = f[1:] / f[:-1]
    assert np.allclose(ratios, 10000.0 ** (-2.0 / 64), rtol=1e-14, atol=0)
    # factor 1 (no context extension) is plain RoPE whatever the other arguments
    assert np.array_equal(yarn_inv_freq(64, 10000.0, 1.0, 4096), f)


def test_yarn_ramp_limits():
    d, theta, L, s = 64, 10000.0, 4096.0, 40.0
    base = yarn_inv_freq(d, theta)
    f = yarn_inv_freq(d, theta, s, L, beta_fast=32.0, beta_slow=1.0)
    rotations = L * base / (2 * math.pi)
    fast = rotations > 32.0
    slow = rotations < 1.0
    assert fast[0] and slow[-1] and (~fast & ~slow).any()
    assert np.array_equal(f[fast], base[fast])                   # high frequencies kept
    assert np.allclose(f[slow], base[slow] / s, rtol=1e-15)      # low frequencies interpolated
    mid = ~fast & ~slow
    assert np.all(f[mid] < base[mid]) and np.all(f[mid] > base[mid] / s)
    # the blend weight is linear in the rotation count
    w = (f[mid] - base[mid] / s) / (base[mid] - base[mid] / s)
    assert np.allclose(w, (rotations[mid] - 1.0) / 31.0, rtol=1e-12)


def test_table_rows_are_unit_rotations():
    t = rope_table(np.arange(100), yarn_inv_freq(64, 10000.0, 8.0, 1024))
    assert t.shape == (100, 32, 2) and t.dtype == np.float32
    norm = t[..., 0].astype(np.float64) ** 2 + t[..., 1].astype(np.float64) ** 2
    assert np.allclose(norm, 1.0, atol=2e-7)
    assert np.array_equal(t[0, :, 0], np.ones(32, np.float32)) and np.array_equal(t[0, :, 1], np.zeros(32, np.float32))


def test_rotation_matches_exact_rationals():
    rng = np.random.default_rng(5)
    hd, rd, n = 16, 8, 40
    lat = oracle.bf16_round(rng.standard_normal((n, hd)).astype(np.float32) * 3)
    rows = rope_table(rng.integers(0, 10000, n), yarn_inv_freq(rd, 10000.0))
    got = apply_rope(lat, rows, rd)
    for e in range(n):
        ref = brute.rope([float(v) for v in lat[e]], [(float(c), float(s)) for c, s in rows[e]], rd)
        assert [float(v) for v in got[e]] == ref


def test_rotation_rounds_the_exact_value_at_a_midpoint():
    # a c is the bf16 midpoint 1 + 2^-8; b s = -2^-70 lies below float64's
    # resolution there, so a c - b s rounds to the midpoint in float64 while
    # the exact value is just above it: the bf16 result must be 1 + 2^-7
    lat = np.zeros((1, 4), np.float32)
    lat[0, 2], lat[0, 3] = 1.0, 2.0 ** -40
    rows = np.array([[[1.0 + 2.0 ** -8, -(2.0 ** -30)]]], np.float32)
    got = apply_rope(lat, rows, 2)
    assert got[0, 2] == np.float32(1.0 + 2.0 ** -7)
    assert brute.rope([0.0, 0.0, 1.0, 2.0 ** -40], [(1.0 + 2.0 ** -8, -(2.0 ** -30))], 2)[2] == 1.0 + 2.0 ** -7
    # the same with the opposite sign goes to the even neighbour below
    rows[0, 0, 1] = 2.0 ** -30
    assert apply_rope(lat, rows, 2)[0, 2] == np.float32(1.0)


def test_rotation_invariants():
    rng = np.random.default_rng(6)
    hd, rd = 64, 16
    lat = oracle.bf16_round(rng.standard_normal((50, hd)).astype(np.float32))
    inv = yarn_inv_freq(rd, 10000.0)
    pos = rng.integers(0, 5000, 50)
    got = apply_rope(lat, rope_table(pos, inv), rd)
    # features outside the rotary slice are untouched
    assert np.array_equal(got[:, :hd - rd], lat[:, :hd - rd])
    # position 0 is the identity
    assert np.array_equal(apply_rope(lat, rope_table(np.zeros(50), inv), rd), lat)
    # each pair keeps its length (up to the two bf16 roundings)
    a = lat[:, hd - rd:].reshape(50, -1, 2).astype(np.float64)
    b = got[:, hd - rd:].reshape(50, -1, 2).astype(np.float64)
    na, nb = np.hypot(a[..., 0], a[..., 1]), np.hypot(b[..., 0], b[..., 1])
    assert np.allclose(nb, na, rtol=2 ** -7, atol=1e-30)
    # turning by p then by q is turning by p + q, up to rounding
    q = rng.integers(0, 5000, 50)
    twice = apply_rope(got, rope_table(q, inv), rd)
    once = apply_rope(lat, rope_table(pos + q, inv), rd)
    assert np.allclose(twice[:, hd - rd:], once[:, hd - rd:], rtol=0, atol=0.05)


def test_rope_inside_prefill_and_decode():
    rng = np.random.default_rng(7)
    rd = 16
    cfg = oracle.Config(ratio=4, head_dim=64, rope_dim=rd)
    kv = rng.standard_normal((2, 22, 128)).astype(np.float32)
    sc = rng.standard_normal((2, 22, 128)).astype(np.float32)
    table = rope_table(np.arange(8) * 4 + 3, yarn_inv_freq(rd, 10000.0))
    w = oracle.Weights(rope_cs=table)
    out = oracle.prefill(cfg, w, oracle.State(cfg, 2), kv=kv, score=sc, quantize=True)
    # entry j turns by table row j; the compressor's latent stays unrotated
    ref = apply_rope(out["latent"], np.broadcast_to(table[:5], (2, 5, rd // 2, 2)), rd)
    assert np.array_equal(out["rotated"], ref)
    plain = oracle.prefill(oracle.Config(ratio=4, head_dim=64), oracle.Weights(), oracle.State(cfg, 2), kv=kv,
                           score=sc, quantize=True)
    assert np.array_equal(out["latent"], plain["latent"])
    # the cache form is that of the rotated latent
    codes, scales, deq = oracle.fp4_quant_e4m3(out["rotated"].reshape(-1, 64))
    assert np.array_equal(out["codes"].reshape(-1, 32), codes)
    # decode turns the entry it emits by the same row
    st = oracle.State(cfg, 2)
    dec = [oracle.decode_step(cfg, w, st, p, kv=kv[:, p:p + 1], score=sc[:, p:p + 1], quantize=True)
           for p in range(22)]
    rot = np.concatenate([d["rotated"] for d in dec if d is not None], axis=1)
    assert np.array_equal(rot, out["rotated"])
