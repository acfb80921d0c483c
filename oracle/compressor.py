"""CPU oracle of the DeepSeek-V4.1 compressed-attention Compressor (ratio > 1).

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check and the CPU-baseline leg
of the benchmark may import this module; the product path never does.

What it computes, step by step, in the pages' order:

1. Projections. x is taken in f32; kv = x . wkv^T and score = x . wgate^T with
   f32 weights of shape [out_dim, in_dim] ("Module compress", Functions,
   linear_f32; "DeepSeek V4.1 . Pool token pairs", Compressor listing,
   forward). Here each dot product is accumulated in float64 and rounded once
   to f32.
2. Positional bias. The gate logits are wgate(x) plus a positional bias
   ("Compressed Sparse Attention . ratio m = 4", Per-channel gated pooling).
   Reading: a table ape [ratio, proj]; token t gets row t mod ratio, added in
   f32 before anything else reads the logits.
3. Grouping. seqlen // ratio complete groups are pooled; the trailing
   seqlen % ratio tokens wait in the state; no group at all means no output
   (Compressor listing, forward, prefill branch).
   At ratio 4 the groups overlap ("Compressed Sparse Attention . ratio m = 4",
   Why one output uses eight candidates; Tensor-shape walkthrough): each token
   has two branches (kv and score are [.., 2*hd]); entry j takes 8 candidates,
   the previous block's branch B (tokens 4(j-1)..4j-1) then the current block's
   branch A (tokens 4j..4j+3). Reading: branch A is columns [0, hd), branch B
   is columns [hd, 2hd); entry 0's previous branch is padding with kv 0 and
   score -inf, the values the state starts from (Compressor listing,
   __init__).
4. Pooling. Per feature, a softmax over the candidates' logits weights the
   candidates' kv values, which are summed ("DeepSeek V4.1 . Pool token pairs",
   the pooling formula; Compressor listing, forward). Done in float64 and
   rounded once to f32.
5. Normalisation. The pooled f32 result is rounded to bf16 and RMS-normalised
   ("Module compress", Precision paragraph; Compressor listing, forward).
   Reading: y = bf16(w * u / sqrt(mean(u^2) + eps)) with u the bf16 values,
   computed in float64 and rounded once.
6. Decode. One token per call at start_pos > 0: it fills slot start_pos mod
   ratio, and a group is pooled only when (start_pos + 1) mod ratio == 0;
   start_pos == 0 always takes the prefill branch (Compressor listing,
   forward; "Compressed Sparse Attention . ratio m = 4", Prefill and decode use
   the same rule). Reading for the overlap: each state plane is
   [batch, 2*ratio, 2*hd]; rows [0, ratio) hold the previous complete block,
   rows [ratio, 2*ratio) the current one; after an emit the current rows move
   to the previous rows. A prefill leaves the last complete block (padding if
   none) in the previous rows and the trailing tokens in the first current
   rows.
7. Cache quantisation. Optionally the latent goes through the e4m3-scaled
   block-16 fp4 round trip of formats.fp4_quant_e4m3 (the KV latent's form),
   or the power-of-two-scaled block-32 one of formats.fp4_quant_e8m0 (the
   indexer's form).
8. RoPE (oracle/rope.py, optional, cfg.rope_dim > 0): "rotated" holds the
   latent with its rotary slice turned by the table row of the entry's index
   (w.rope_cs), and the fp4 cache form is taken from the rotated latent
   ("Compressed Sparse Attention . ratio m = 4", Normalize + RoPE + cache). The
   compressor's own output, "latent", stays unrotated.
9. Ratio 1 (plain_projection). No gate, no pooling, no state: every token is
   one entry, latent = RMSNorm(wkv(x)) in the checkpoint's bf16 (Compressor
   listing, __init__ and the ratio-1 branch of forward; "Module compress",
   CompressorWeights: wkv holds bf16 values at ratio 1). Reading: x and wkv
   hold bf16 values; the linear sums the exact products and rounds once to f32
   (the accumulator of a bf16 matrix product), which is rounded to bf16 (the
   linear's output dtype) and normalised as in step 5. "pooled" holds the f32
   projection.

Pins (tests/test_oracle_compressor.py): shape traces (16 tokens -> 4 entries,
32 candidate slots at ratio 4), softmax weights summing to one, the convex hull
of the pooled values, the ratio-2 closed form with the logistic function, equal
logits giving the mean, the first entry's padding, decode equal to prefill
bitwise, every prefill/decode split of a sequence, RMSNorm against torch's CPU
rms_norm, and an independent pure-Python implementation on tiny inputs.
Parity unpinned against the released model: which half is branch A, the
candidate order inside the window, the shape and indexing of the positional
bias, and the overlapped prefill-to-state hand-off are readings; no weights or
printed values exist to check them against.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import bf16_round, fp4_quant_e4m3, fp4_quant_e8m0
from .rope import apply_rope


@dataclass(frozen=True)
class Config:
    ratio: int          # compress ratio: 1 (plain projection), 2, 4 (overlapped) or 128
    head_dim: int       # latent width hd
    dim: int = 0        # hidden width of x (0 when projections are given)
    eps: float = 1e-6   # RMSNorm epsilon
    fp4: str = "e4m3"   # fp4 form of the output: "e4m3" (block 16) or "e8m0" (block 32)
    rope_dim: int = 0   # rotary slice width (last features of an entry); 0: no RoPE

    @property
    def overlap(self) -> bool:
        # "Overlap only when ratio = 4" ("Compressed Sparse Attention . ratio m = 4")
        return self.ratio == 4

    @property
    def proj(self) -> int:
        """Projection width per plane: two branches of hd when overlapped."""
        return 2 * self.head_dim if self.overlap else self.head_dim

    @property
    def state_rows(self) -> int:
        return 2 * self.ratio if self.overlap else self.ratio


@dataclass
class Weights:
    wkv: np.ndarray | None = None     # [proj, dim] f32
    wgate: np.ndarray | None = None   # [proj, dim] f32
    ape: np.ndarray | None = None     # [ratio, proj] f32, None = no bias
    norm_w: np.ndarray | None = None  # [hd] f32, None = ones
    rope_cs: np.ndarray | None = None  # [entries, rope_dim / 2, 2] f32 (cos, sin) per compressed entry


class State:
    """kv_state / score_state: f32 [batch, state_rows, proj], starting at kv 0
    and score -inf (Compressor listing, __init__)."""

    def __init__(self, cfg: Config, batch: int):
        self.kv = np.zeros((batch, cfg.state_rows, cfg.proj), dtype=np.float32)
        self.score = np.full((batch, cfg.state_rows, cfg.proj), -np.inf, dtype=np.float32)

    def copy(self) -> "State":
        other = object.__new__(State)
        other.kv = self.kv.copy()
        other.score = self.score.copy()
        return other


# --------------------------------------------------------------------------
# steps
# --------------------------------------------------------------------------
def project(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """linear_f32: x . w^T with w [out_dim, in_dim]; float64 sums, one f32
    rounding."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    w64 = np.asarray(w, dtype=np.float32).astype(np.float64)
    return (x64 @ w64.T).astype(np.float32)


def add_bias(score: np.ndarray, ape: np.ndarray | None, positions: np.ndarray, ratio: int) -> np.ndarray:
    """Gate logits plus the positional bias row of each token (position mod
    ratio), one f32 addition. score is [batch, tokens, proj]."""
    if ape is None:
        return score.astype(np.float32, copy=True)
    rows = np.asarray(ape, dtype=np.float32)[np.asarray(positions) % ratio]
    return (score.astype(np.float32) + rows[None, :, :]).astype(np.float32)


def softmax_weights(logits: np.ndarray) -> np.ndarray:
    """Softmax over axis 0 (the candidates) in float64, max-subtracted.
    A candidate with logit -inf gets weight exactly 0."""
    s = np.asarray(logits, dtype=np.float64)
    m = s.max(axis=0, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=0, keepdims=True)


def pool(kv_cand: np.ndarray, score_cand: np.ndarray) -> np.ndarray:
    """Per-feature softmax pooling over axis 0: sum_i softmax_i(score) * kv_i,
    in float64, rounded once to f32."""
    w = softmax_weights(score_cand)
    return (w * np.asarray(kv_cand, dtype=np.float64)).sum(axis=0).astype(np.float32)


def rms_norm_bf16(pooled: np.ndarray, norm_w: np.ndarray | None, eps: float) -> np.ndarray:
    """bf16 round, then RMSNorm over the last axis, rounded once to bf16.
    Returns float32 arrays holding bf16 values."""
    u = bf16_round(pooled).astype(np.float64)
    ms = (u * u).mean(axis=-1, keepdims=True)
    y = u / np.sqrt(ms + eps)
    if norm_w is not None:
        y = y * np.asarray(norm_w, dtype=np.float32).astype(np.float64)
    return bf16_round(y)


def entry_candidates(cfg: Config, kv: np.ndarray, score: np.ndarray, j: int):
    """Candidates of entry j from one batch row's kv/score [tokens, proj]
    (bias already added). Returns (kv_cand, score_cand), each [C, hd], in the
    order the pooling sums them."""
    r, hd = cfg.ratio, cfg.head_dim
    if not cfg.overlap:
        rows = slice(r * j, r * j + r)
        return kv[rows], score[rows]
    if j == 0:
        prev_kv = np.zeros((r, hd), dtype=np.float32)
        prev_sc = np.full((r, hd), -np.inf, dtype=np.float32)
    else:
        prev = slice(r * (j - 1), r * j)
        prev_kv, prev_sc = kv[prev, hd:2 * hd], score[prev, hd:2 * hd]
    cur = slice(r * j, r * j + r)
    return (np.concatenate([prev_kv, kv[cur, :hd]], axis=0),
            np.concatenate([prev_sc, score[cur, :hd]], axis=0))


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
def _projections(cfg: Config, w: Weights, x, kv, score):
    if x is not None:
        x = np.asarray(x, dtype=np.float32)
        return project(x, w.wkv), project(x, w.wgate)
    if kv is None or score is None:
        raise ValueError("need x, or kv and score")
    return np.asarray(kv, dtype=np.float32), np.asarray(score, dtype=np.float32)


def _finish(cfg: Config, w: Weights, pooled: np.ndarray, quantize: bool, entry_index=None) -> dict:
    """Norm, optional RoPE (entry_index [n]: the compressed index of each of
    the n entries along pooled's second-to-last axis) and optional fp4."""
    latent = rms_norm_bf16(pooled, w.norm_w, cfg.eps)
    out = {"pooled": pooled, "latent": latent}
    cached = latent
    if cfg.rope_dim:
        idx = np.asarray(entry_index)
        rows = np.asarray(w.rope_cs, dtype=np.float32)[idx]
        rows = np.broadcast_to(rows, latent.shape[:-1] + rows.shape[-2:])
        out["rotated"] = cached = apply_rope(latent, rows, cfg.rope_dim)
    if quantize:
        flat = cached.reshape(-1, cfg.head_dim)
        quant, block = (fp4_quant_e8m0, 32) if cfg.fp4 == "e8m0" else (fp4_quant_e4m3, 16)
        codes, scales, deq = quant(flat)
        lead = latent.shape[:-1]
        out["codes"] = codes.reshape(lead + (cfg.head_dim // 2,))
        out["scales"] = scales.reshape(lead + (cfg.head_dim // block,))
        out["dequant"] = deq.reshape(latent.shape)
    return out


def prefill(cfg: Config, w: Weights, state: State, x=None, kv=None, score=None,
            quantize: bool = False, entries=None) -> dict | None:
    """Compressor forward at start_pos == 0 over [batch, seqlen, dim] x (or
    given [batch, seqlen, proj] projections). Returns None when seqlen < ratio,
    else a dict with pooled f32 [batch, groups, hd], latent (bf16 values) and,
    with quantize, codes / scales / dequant. Updates `state` in place.

    `entries` (optional) restricts the pooled output to those group indices;
    the state is then left untouched (used to sample long sequences)."""
    kv, score = _projections(cfg, w, x, kv, score)
    batch, seqlen, proj = kv.shape
    if proj != cfg.proj:
        raise ValueError("projection width mismatch")
    r = cfg.ratio
    score = add_bias(score, w.ape, np.arange(seqlen), r)
    groups = seqlen // r
    rem = seqlen - groups * r

    if entries is None:
        # remainder into the state (Compressor listing, forward, prefill branch)
        cur0 = r if cfg.overlap else 0
        state.kv[:batch, cur0:cur0 + rem] = kv[:, groups * r:]
        state.score[:batch, cur0:cur0 + rem] = score[:, groups * r:]
        if cfg.overlap:
            if groups > 0:
                last = slice((groups - 1) * r, groups * r)
                state.kv[:batch, :r] = kv[:, last]
                state.score[:batch, :r] = score[:, last]
            else:
                state.kv[:batch, :r] = 0.0
                state.score[:batch, :r] = -np.inf
        entries = range(groups)
    if groups == 0:
        return None

    entries = list(entries)
    pooled = np.empty((batch, len(entries), cfg.head_dim), dtype=np.float32)
    for b in range(batch):
        for k, j in enumerate(entries):
            kc, sc = entry_candidates(cfg, kv[b], score[b], j)
            pooled[b, k] = pool(kc, sc)
    return _finish(cfg, w, pooled, quantize, np.array(entries))


def decode_step(cfg: Config, w: Weights, state: State, start_pos: int, x=None,
                kv=None, score=None, quantize: bool = False) -> dict | None:
    """Compressor forward for one token per batch row ([batch, 1, dim] x, or
    [batch, 1, proj] projections). Returns the emitted entry
    ([batch, 1, hd] arrays) when this token completes a group, else None."""
    if start_pos == 0:
        return prefill(cfg, w, state, x=x, kv=kv, score=score, quantize=quantize)
    kv, score = _projections(cfg, w, x, kv, score)
    batch = kv.shape[0]
    r, hd = cfg.ratio, cfg.head_dim
    slot = start_pos % r
    score = add_bias(score, w.ape, np.array([start_pos]), r)
    row = (r + slot) if cfg.overlap else slot
    state.kv[:batch, row] = kv[:, 0]
    state.score[:batch, row] = score[:, 0]
    if (start_pos + 1) % r != 0:
        return None
    pooled = np.empty((batch, 1, hd), dtype=np.float32)
    for b in range(batch):
        if cfg.overlap:
            kc = np.concatenate([state.kv[b, :r, hd:2 * hd], state.kv[b, r:, :hd]], axis=0)
            sc = np.concatenate([state.score[b, :r, hd:2 * hd], state.score[b, r:, :hd]], axis=0)
        else:
            kc, sc = state.kv[b], state.score[b]
        pooled[b, 0] = pool(kc, sc)
    if cfg.overlap:
        state.kv[:batch, :r] = state.kv[:batch, r:]
        state.score[:batch, :r] = state.score[:batch, r:]
    return _finish(cfg, w, pooled, quantize, np.array([(start_pos + 1) // r - 1]))


def plain_projection(cfg: Config, w: Weights, x: np.ndarray, quantize: bool = False) -> dict:
    """The ratio-1 compressor over [..., dim] x (bf16 values in float32
    arrays) with wkv [hd, dim] (bf16 values): every token gives one entry.
    Returns pooled (the f32 projection), latent and, with quantize, codes /
    scales / dequant, each with x's leading shape."""
    if cfg.ratio != 1:
        raise ValueError("plain_projection is the ratio-1 compressor")
    x = np.asarray(x, dtype=np.float32)
    wkv = np.asarray(w.wkv, dtype=np.float32)
    if not (np.array_equal(bf16_round(x), x) and np.array_equal(bf16_round(wkv), wkv)):
        raise ValueError("x and wkv must hold bf16 values at ratio 1")
    if wkv.shape != (cfg.head_dim, x.shape[-1]):
        raise ValueError("wkv must be [head_dim, dim]")
    if cfg.rope_dim:
        raise ValueError("RoPE is not offered at ratio 1")
    return _finish(cfg, w, project(x, wkv), quantize)
