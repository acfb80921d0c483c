"""Tolerance rules of the GPU-vs-oracle parity tests.

  pooled f32  : per entry, max |gpu - ref| <= 1e-5 * max |ref| (relative to
                the entry's largest value, so that values that cancel to
                nearly zero are judged against the entry's scale).
  latent bf16 : within 1 bf16 ulp of the oracle, the ulp taken at
                max(|ref|, 2^-8 * max |ref| of the entry), wherever the GPU's
                pooled value rounds to the same bf16 value as the oracle's.
                An f32 pooled value within the f32 tolerance of a bf16
                rounding midpoint may round the other way on the GPU (a
                "flip", explained by that tolerance); there the latent is
                within 2 ulps. (The floor follows from the pooled rule: an
                error of 1e-5 of the entry's largest value is below one bf16
                ulp only for elements above about 2^-8 of it.) Everywhere,
                the GPU latent is within 1 ulp, at each element's own
                magnitude with no floor, of the oracle's RMSNorm applied to
                the GPU's own pooled values.
  fp4         : (either form) codes and scales bit-exact against the oracle's fp4 round trip
                of the GPU's own bf16 latent (the decision is taken on the
                same input on both sides), and bit-exact against the oracle's
                end-to-end result on every block whose latent is bitwise equal.
  indices     : group counts and emit steps exact.
"""
from __future__ import annotations

import numpy as np

import oracle

POOLED_RTOL = 1e-5


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (2^(e - 7) for |v| in [2^e, 2^(e+1)))."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    v = np.maximum(v, 2.0 ** -126)
    return np.exp2(np.floor(np.log2(v)) - 7)


def check_pooled(gpu: np.ndarray, ref: np.ndarray, what="pooled"):
    gpu = gpu.reshape(-1, gpu.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    scale = np.abs(ref).max(axis=1, keepdims=True)
    err = np.abs(gpu - ref).max(axis=1, keepdims=True)
    bad = err > POOLED_RTOL * scale
    rel = np.where(scale > 0, err / np.where(scale > 0, scale, 1), 0)
    assert not bad.any(), f"{what}: {bad.sum()} entries beyond {POOLED_RTOL} relative, worst {rel.max():.3e}"
    return float(rel.max())


def check_latent(gpu_latent, gpu_pooled, ref_latent, ref_pooled, norm_w=None, eps=1e-6):
    """Returns (elements whose pooled value rounds to another bf16, total).

    Per element, with u = bf16(pooled):
      - where the GPU's u equals the oracle's, the latent is within 1 bf16 ulp;
      - where it differs (a "flip"), the oracle's f32 pooled value must lie
        within the pooled tolerance of the bf16 midpoint between the two u
        values, and the latent is within 2 ulps (one from u, one from the
        final rounding);
      - everywhere, the latent is within 1 ulp (its own, no floor) of the
        oracle's RMSNorm of the GPU's own pooled values.
    """
    hd = gpu_latent.shape[-1]
    gl = gpu_latent.reshape(-1, hd).astype(np.float64)
    rl = ref_latent.reshape(-1, hd).astype(np.float64)
    gp = gpu_pooled.reshape(-1, hd)
    rp = ref_pooled.reshape(-1, hd)
    ug = oracle.bf16_round(gp).astype(np.float64)
    ur = oracle.bf16_round(rp).astype(np.float64)
    flip = ug != ur
    if flip.any():
        scale = np.abs(rp.astype(np.float64)).max(axis=1, keepdims=True) * np.ones_like(ug)
        mid = (ug + ur) / 2
        near = np.abs(rp.astype(np.float64) - mid) <= POOLED_RTOL * scale
        assert np.all(near[flip]), f"{np.sum(flip & ~near)} bf16 flips not explained by the pooled tolerance"
    floor = 2.0 ** -8 * np.abs(rl).max(axis=1, keepdims=True)
    ulp = bf16_ulp(np.maximum(np.abs(rl), floor))
    allowed = np.where(flip, 2.0, 1.0) * ulp
    err = np.abs(gl - rl)
    bad = err > allowed
    assert not bad.any(), f"latent: {bad.sum()} values beyond the ulp bound in {bad.any(axis=1).sum()} entries"
    # every element: the GPU's norm step on its own pooled values
    # (no floor here: each element at its own bf16 ulp)
    own = oracle.rms_norm_bf16(gp, norm_w, eps).astype(np.float64)
    bad2 = np.abs(gl - own) > bf16_ulp(own)
    assert not bad2.any(), f"latent vs norm of own pooled: {bad2.sum()} values beyond 1 ulp of their own"
    return int(flip.sum()), flip.size


def check_fp4(gpu_codes, gpu_scales, gpu_latent, ref_codes=None, ref_scales=None, ref_latent=None,
              gpu_dequant=None, e8m0=False):
    hd = gpu_latent.shape[-1]
    blk = 32 if e8m0 else 16
    lat = gpu_latent.reshape(-1, hd).astype(np.float32)
    codes, scales, deq = (oracle.fp4_quant_e8m0 if e8m0 else oracle.fp4_quant_e4m3)(lat)
    gc = gpu_codes.reshape(-1, hd // 2)
    gs = gpu_scales.reshape(-1, hd // blk)
    assert np.array_equal(gc, codes), f"codes: {np.sum(gc != codes)} bytes differ"
    assert np.array_equal(gs, scales), f"scales: {np.sum(gs != scales)} differ"
    if gpu_dequant is not None:
        gd = gpu_dequant.reshape(-1, hd).astype(np.float32)
        assert np.array_equal(gd.view(np.uint32), deq.view(np.uint32))
    if ref_codes is not None:
        rl = ref_latent.reshape(-1, hd // blk, blk)
        same_block = np.all(lat.reshape(-1, hd // blk, blk) == rl, axis=2)
        rc = ref_codes.reshape(-1, hd // blk, blk // 2)
        assert np.array_equal(gc.reshape(-1, hd // blk, blk // 2)[same_block], rc[same_block])
        assert np.array_equal(gs[same_block], ref_scales.reshape(-1, hd // blk)[same_block])
        return int((~same_block).sum()), same_block.size
    return 0, 0
