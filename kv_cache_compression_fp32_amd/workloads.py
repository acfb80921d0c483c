"""Seeded synthetic inputs of the compressor workloads.

This module only draws random numbers with the shapes and distributions of the
workloads; it holds none of the compressor's arithmetic. Tests hand the same
arrays to the CPU oracle and to the HIP library, and the benchmark uses them as
its inputs.

Shapes follow the released Flash configuration ("Compressed Sparse Attention .
ratio m = 4", Released Flash configuration): hidden 4096, latent 512, ratio 4
(overlapped, projections of 2 x 512), ratio 128, and a 128-wide indexer
compressor. Values are N(0, std) with std the standard deviation: hidden states
N(0, 1), projection weights N(0, 0.02), positional bias N(0, 0.1); the
projection-free pair-pooling case draws k^c ~ N(0, 1) and g^c ~ N(0, 2).

The ratio-1 compressor (a plain bf16 projection) draws x and wkv the same
way; its callers hand the library the bf16 roundings of those arrays.

Every tensor is drawn in float32 by NumPy's PCG64 generator. Hidden states are
drawn in blocks of BLOCK_TOKENS tokens, each block from its own seed
(seed, stream, batch row, block index), so any token range of a long sequence
can be regenerated on its own without drawing the rest.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK_TOKENS = 256

# stream tags keep every tensor's random numbers independent
_TAG_X, _TAG_WKV, _TAG_WGATE, _TAG_APE, _TAG_KC, _TAG_GC = 1, 2, 3, 4, 5, 6
_TAG_IDX = 100  # added to the weight tags for the indexer compressor


@dataclass(frozen=True)
class Compressor:
    """One compressor of a workload."""
    ratio: int
    head_dim: int
    quantize: bool          # fp4 round trip of its latent
    weight_std: float = 0.02
    ape_std: float = 0.1
    tag: int = 0            # weight stream offset

    @property
    def proj(self) -> int:
        return 2 * self.head_dim if self.ratio == 4 else self.head_dim


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    dim: int                # 0: projections are given, no x
    compressors: tuple = field(default_factory=tuple)
    decode: bool = False    # stream the tokens one decode step at a time
    eps: float = 1e-6
    seed: int = 0
    kc_std: float = 1.0
    gc_std: float = 2.0

    @property
    def entries(self) -> int:
        """Compressed entries per pass (batch * seqlen // ratio of the first
        compressor)."""
        return self.batch * (self.seqlen // self.compressors[0].ratio)


MAIN4 = Compressor(ratio=4, head_dim=512, quantize=False)

WORKLOADS = {
    # pair pooling of given projections, ratio 2
    "pair_pool_r2": Workload("pair_pool_r2", batch=1, seqlen=64, dim=0,
                             compressors=(Compressor(ratio=2, head_dim=512, quantize=False),)),
    # ratio-4 overlapped prefill
    "prefill_r4_n4096": Workload("prefill_r4_n4096", batch=1, seqlen=4096, dim=4096,
                                 compressors=(MAIN4,)),
    # ratio-128 prefill
    "prefill_r128_b2_n16384": Workload("prefill_r128_b2_n16384", batch=2, seqlen=16384, dim=4096,
                                       compressors=(Compressor(ratio=128, head_dim=512, quantize=False),)),
    # ratio-4 decode streaming, 64 rows x 512 steps
    "decode_r4_b64_s512": Workload("decode_r4_b64_s512", batch=64, seqlen=512, dim=4096,
                                   compressors=(MAIN4,), decode=True),
    # long-context ratio-4 prefill, fp4 cache latent + 128-wide indexer compressor
    "prefill_r4_n65536_fp4_idx128": Workload(
        "prefill_r4_n65536_fp4_idx128", batch=1, seqlen=65536, dim=4096,
        compressors=(Compressor(ratio=4, head_dim=512, quantize=True),
                     Compressor(ratio=4, head_dim=128, quantize=False, tag=_TAG_IDX))),
    # ratio-1 compressor (bf16 projection + RMSNorm, fp4 cache form) over a long prefill
    "prefill_r1_n65536": Workload("prefill_r1_n65536", batch=1, seqlen=65536, dim=4096,
                                  compressors=(Compressor(ratio=1, head_dim=512, quantize=True),)),
}

# the order the workloads are listed in (smallest first)
ORDER = ["pair_pool_r2", "prefill_r4_n4096", "prefill_r128_b2_n16384",
         "decode_r4_b64_s512", "prefill_r4_n65536_fp4_idx128", "prefill_r1_n65536"]


def _normal(seed_words, shape, std) -> np.ndarray:
    rng = np.random.default_rng(list(seed_words))
    out = rng.standard_normal(shape, dtype=np.float32)
    out *= np.float32(std)
    return out


def weights(wl: Workload, comp: Compressor) -> dict:
    """wkv, wgate [proj, dim] and ape [ratio, proj], float32 (ratio 1: wkv
    only)."""
    s = wl.seed
    if comp.ratio == 1:
        return {"wkv": _normal((s, _TAG_WKV + comp.tag), (comp.proj, wl.dim), comp.weight_std)}
    return {
        "wkv": _normal((s, _TAG_WKV + comp.tag), (comp.proj, wl.dim), comp.weight_std),
        "wgate": _normal((s, _TAG_WGATE + comp.tag), (comp.proj, wl.dim), comp.weight_std),
        "ape": _normal((s, _TAG_APE + comp.tag), (comp.ratio, comp.proj), comp.ape_std),
    }


def hidden_rows(wl: Workload, b: int, t0: int, t1: int) -> np.ndarray:
    """Hidden states x[b, t0:t1, :] as float32 [t1 - t0, dim]."""
    if not (0 <= t0 <= t1 <= wl.seqlen and 0 <= b < wl.batch):
        raise IndexError("token range outside the workload")
    out = np.empty((t1 - t0, wl.dim), dtype=np.float32)
    k0, k1 = t0 // BLOCK_TOKENS, (t1 + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    for k in range(k0, k1):
        lo, hi = k * BLOCK_TOKENS, min((k + 1) * BLOCK_TOKENS, wl.seqlen)
        block = _normal((wl.seed, _TAG_X, b, k), (hi - lo, wl.dim), 1.0)
        a, z = max(lo, t0), min(hi, t1)
        if a < z:
            out[a - t0:z - t0] = block[a - lo:z - lo]
    return out


def hidden(wl: Workload) -> np.ndarray:
    """All hidden states x [batch, seqlen, dim], float32."""
    out = np.empty((wl.batch, wl.seqlen, wl.dim), dtype=np.float32)
    for b in range(wl.batch):
        out[b] = hidden_rows(wl, b, 0, wl.seqlen)
    return out


def given_projections(wl: Workload) -> tuple[np.ndarray, np.ndarray]:
    """The projection-free case: k^c ~ N(0, kc_std), g^c ~ N(0, gc_std),
    each [batch, seqlen, proj] float32."""
    comp = wl.compressors[0]
    shape = (wl.batch, wl.seqlen, comp.proj)
    return (_normal((wl.seed, _TAG_KC), shape, wl.kc_std),
            _normal((wl.seed, _TAG_GC), shape, wl.gc_std))


def scaled(wl: Workload, batch: int | None = None, seqlen: int | None = None,
           dim: int | None = None, head_dim: int | None = None) -> Workload:
    """The same workload at other sizes (for small parity cases)."""
    comps = wl.compressors
    if head_dim is not None:
        comps = tuple(Compressor(c.ratio, head_dim if i == 0 else c.head_dim, c.quantize,
                                 c.weight_std, c.ape_std, c.tag) for i, c in enumerate(comps))
    return Workload(wl.name + "_scaled", batch if batch is not None else wl.batch,
                    seqlen if seqlen is not None else wl.seqlen,
                    dim if dim is not None else wl.dim, comps, wl.decode, wl.eps, wl.seed,
                    wl.kc_std, wl.gc_std)
