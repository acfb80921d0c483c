"""Pins of the compressor oracle (CPU only).

The oracle is checked against facts fixed by the pages and by mathematics, not
against itself: the shape trace of "Compressed Sparse Attention . ratio m = 4"
(tests/golden/csa_ratio4_shape_trace.json), the softmax and pooling identities
of the pooling formula on "DeepSeek V4.1 . Pool token pairs", the emit rule of
the Compressor listing, decode equal to prefill ("Prefill and decode use the
same rule"), torch's CPU rms_norm, and the independent pure-Python
implementation in tests/brute.py.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import brute
import oracle
from oracle import Config, State, Weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_proj(rng, b, n, proj, kv_std=1.0, sc_std=2.0):
    kv = (rng.standard_normal((b, n, proj)) * kv_std).astype(np.float32)
    sc = (rng.standard_normal((b, n, proj)) * sc_std).astype(np.float32)
    return kv, sc


# ---------------------------------------------------------------- shapes
def test_shape_trace_matches_page_example():
    trace = json.load(open(os.path.join(GOLDEN, "csa_ratio4_shape_trace.json")))
    ex = trace["example"]
    hd = trace["branch_width"] // 64  # narrow features, same shape logic
    cfg = Config(ratio=trace["ratio"], head_dim=hd)
    assert cfg.proj == trace["branches"] * hd
    rng = np.random.default_rng(0)
    kv, sc = _rand_proj(rng, 1, ex["input_positions"], cfg.proj)
    out = oracle.prefill(cfg, Weights(), State(cfg, 1), kv=kv, score=sc)
    assert out["latent"].shape == (1, ex["compressed_positions"], hd)
    slots = sum(oracle.entry_candidates(cfg, kv[0], sc[0], j)[0].shape[0]
                for j in range(ex["compressed_positions"]))
    assert slots == ex["candidate_uses"]
    assert oracle.entry_candidates(cfg, kv[0], sc[0], 1)[0].shape == (trace["candidates_per_entry"], hd)


@pytest.mark.parametrize("ratio", [2, 4, 128])
def test_group_count_and_none_below_ratio(ratio):
    cfg = Config(ratio=ratio, head_dim=16)
    rng = np.random.default_rng(1)
    for n in (1, ratio - 1, ratio, ratio + 1, 3 * ratio + ratio // 2):
        kv, sc = _rand_proj(rng, 2, n, cfg.proj)
        out = oracle.prefill(cfg, Weights(), State(cfg, 2), kv=kv, score=sc)
        if n < ratio:
            assert out is None
        else:
            assert out["latent"].shape == (2, n // ratio, 16)


# ---------------------------------------------------------------- softmax pooling
def test_softmax_weights_sum_to_one_and_lie_in_unit_interval():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((8, 512)) * 5
    s[:4, :7] = -np.inf
    w = oracle.softmax_weights(s)
    assert np.all(np.abs(w.sum(axis=0) - 1) < 1e-15)
    assert np.all((w >= 0) & (w <= 1))
    assert np.all(w[:4, :7] == 0)


def test_pool_lies_in_convex_hull():
    rng = np.random.default_rng(3)
    kv = rng.standard_normal((8, 512)).astype(np.float32)
    sc = (rng.standard_normal((8, 512)) * 3).astype(np.float32)
    p = oracle.pool(kv, sc)
    assert np.all(p >= kv.min(axis=0)) and np.all(p <= kv.max(axis=0))


def test_pool_ratio2_closed_form():
    # pooling formula of "Pool token pairs": for a pair the softmax weights are
    # the logistic function of the logit difference
    rng = np.random.default_rng(4)
    kv = rng.standard_normal((2, 512)).astype(np.float32)
    sc = (rng.standard_normal((2, 512)) * 2).astype(np.float32)
    g0, g1 = sc[0].astype(np.float64), sc[1].astype(np.float64)
    ref = expit(g0 - g1) * kv[0] + expit(g1 - g0) * kv[1]
    assert np.allclose(oracle.pool(kv, sc), ref, rtol=0, atol=1e-6)
    assert np.all(np.abs(oracle.pool(kv, sc) - ref) <= np.spacing(np.abs(ref).astype(np.float32)) * 1.01 + 1e-12)


def test_pool_special_cases():
    rng = np.random.default_rng(5)
    kv = rng.standard_normal((8, 64)).astype(np.float32)
    # equal logits: the arithmetic mean
    eq = np.full((8, 64), 0.7, dtype=np.float32)
    assert np.allclose(oracle.pool(kv, eq), kv.astype(np.float64).mean(axis=0), rtol=1e-6, atol=1e-7)
    # one logit far above the others: that candidate alone
    sc = np.zeros((8, 64), dtype=np.float32)
    sc[3] = 1e4
    assert np.array_equal(oracle.pool(kv, sc), kv[3])
    # the same constant added to every candidate's logit changes nothing
    # (logits on a 2^-10 grid, so the f32 additions are exact)
    s2 = (np.round(rng.standard_normal((8, 64)) * 2 * 1024) / 1024).astype(np.float32)
    c = np.float32(16.0)
    assert np.allclose(oracle.pool(kv, s2 + c), oracle.pool(kv, s2), rtol=1e-12, atol=1e-12)


def test_overlap_first_entry_is_the_plain_pool_of_block_zero():
    # the first entry's padded previous branch gets weight exactly zero
    rng = np.random.default_rng(6)
    hd = 32
    cfg4 = Config(ratio=4, head_dim=hd)
    kv, sc = _rand_proj(rng, 1, 12, cfg4.proj)
    out = oracle.prefill(cfg4, Weights(), State(cfg4, 1), kv=kv, score=sc)
    plain = oracle.pool(kv[0, :4, :hd], sc[0, :4, :hd])
    assert np.array_equal(out["pooled"][0, 0], plain)
    # later entries do use the previous block's branch B
    kc, scc = oracle.entry_candidates(cfg4, kv[0], sc[0], 2)
    assert np.array_equal(kc[:4], kv[0, 4:8, hd:]) and np.array_equal(kc[4:], kv[0, 8:12, :hd])
    assert np.array_equal(scc[:4], sc[0, 4:8, hd:])


def test_positional_bias_is_added_by_position_mod_ratio():
    rng = np.random.default_rng(7)
    cfg = Config(ratio=4, head_dim=8)
    kv, sc = _rand_proj(rng, 1, 8, cfg.proj)
    ape = (rng.standard_normal((4, cfg.proj)) * 0.1).astype(np.float32)
    biased = oracle.add_bias(sc, ape, np.arange(8), 4)
    assert np.array_equal(biased[0, 5], (sc[0, 5] + ape[1]).astype(np.float32))
    # the same per-feature constant on every branch column of every row leaves
    # the pooled result unchanged (shift invariance of the softmax); logits on
    # a 2^-10 grid and constants on a 2^-4 grid keep the f32 additions exact
    sc = (np.round(sc * 1024) / 1024).astype(np.float32)
    c = (np.round(rng.standard_normal(8) * 3 * 16) / 16).astype(np.float32)
    ape_shift = np.tile(np.concatenate([c, c]), (4, 1)).astype(np.float32)
    a = oracle.prefill(cfg, Weights(), State(cfg, 1), kv=kv, score=sc)
    b = oracle.prefill(cfg, Weights(ape=ape_shift), State(cfg, 1), kv=kv, score=sc)
    assert np.allclose(a["pooled"], b["pooled"], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- RMSNorm
def test_rms_norm_matches_torch_cpu():
    rng = np.random.default_rng(8)
    p = (rng.standard_normal((64, 512)) * np.exp2(rng.integers(-6, 4, (64, 1)))).astype(np.float32)
    ours = oracle.rms_norm_bf16(p, None, 1e-6)
    u = torch.from_numpy(oracle.bf16_round(p))
    ref = torch.nn.functional.rms_norm(u, (512,), eps=1e-6).to(torch.bfloat16).float().numpy()
    ulp = np.spacing(np.abs(ref).astype(np.float32)) * 65536  # bf16 ulp
    assert np.all(np.abs(ours - ref) <= ulp)
    assert np.mean(ours == ref) > 0.999
    # weight scales each feature
    w = (rng.uniform(0.5, 2, 512)).astype(np.float32)
    refw = torch.nn.functional.rms_norm(u, (512,), weight=torch.from_numpy(w), eps=1e-6)
    refw = refw.to(torch.bfloat16).float().numpy()
    oursw = oracle.rms_norm_bf16(p, w, 1e-6)
    assert np.all(np.abs(oursw - refw) <= np.spacing(np.abs(refw).astype(np.float32)) * 65536)


def test_rms_norm_unit_mean_square():
    rng = np.random.default_rng(9)
    p = rng.standard_normal((16, 512)).astype(np.float32)
    y = oracle.rms_norm_bf16(p, None, 1e-6).astype(np.float64)
    u = oracle.bf16_round(p).astype(np.float64)
    ms_u = (u * u).mean(axis=1)
    # mean(y^2) = mean(u^2) / (mean(u^2) + eps), up to bf16 rounding of y
    assert np.allclose((y * y).mean(axis=1), ms_u / (ms_u + 1e-6), rtol=2 ** -7)


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("ratio", [2, 4, 128])
def test_decode_equals_prefill_bitwise(ratio):
    rng = np.random.default_rng(10 + ratio)
    hd = 16
    cfg = Config(ratio=ratio, head_dim=hd)
    n = 4 * ratio if ratio < 128 else 2 * ratio
    b = 3
    kv, sc = _rand_proj(rng, b, n, cfg.proj)
    ape = (rng.standard_normal((ratio, cfg.proj)) * 0.1).astype(np.float32)
    w = Weights(ape=ape)
    ref = oracle.prefill(cfg, w, State(cfg, b), kv=kv, score=sc, quantize=True)
    st = State(cfg, b)
    got = []
    for p in range(n):
        out = oracle.decode_step(cfg, w, st, p, kv=kv[:, p:p + 1], score=sc[:, p:p + 1], quantize=True)
        assert (out is not None) == ((p + 1) % ratio == 0 and p > 0)
        if out is not None:
            got.append(out)
    assert len(got) == n // ratio
    for key in ("pooled", "latent", "codes", "scales", "dequant"):
        cat = np.concatenate([g[key] for g in got], axis=1)
        assert np.array_equal(cat, ref[key]), key


@pytest.mark.parametrize("ratio", [2, 4])
def test_prefill_then_decode_equals_prefill_for_every_split(ratio):
    rng = np.random.default_rng(20 + ratio)
    hd = 8
    cfg = Config(ratio=ratio, head_dim=hd)
    n = 5 * ratio + 1
    kv, sc = _rand_proj(rng, 2, n, cfg.proj)
    ape = (rng.standard_normal((ratio, cfg.proj)) * 0.1).astype(np.float32)
    w = Weights(ape=ape)
    ref = oracle.prefill(cfg, w, State(cfg, 2), kv=kv, score=sc)["pooled"]
    for n0 in range(1, n + 1):
        st = State(cfg, 2)
        # stale state from an earlier sequence must not leak into the result
        st.kv[:] = 123.0
        st.score[:] = 7.0
        first = oracle.prefill(cfg, w, st, kv=kv[:, :n0], score=sc[:, :n0])
        parts = [] if first is None else [first["pooled"]]
        for p in range(n0, n):
            out = oracle.decode_step(cfg, w, st, p, kv=kv[:, p:p + 1], score=sc[:, p:p + 1])
            if out is not None:
                parts.append(out["pooled"])
        assert np.array_equal(np.concatenate(parts, axis=1), ref), n0


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("ratio,n", [(2, 1), (2, 7), (4, 3), (4, 4), (4, 13), (128, 293)])
def test_oracle_matches_pure_python_forward(ratio, n):
    rng = np.random.default_rng(30 + n)
    hd = 4 if ratio < 128 else 2
    dim = 8
    cfg = Config(ratio=ratio, head_dim=hd, dim=dim)
    x = rng.standard_normal((1, n, dim)).astype(np.float32)
    wkv = (rng.standard_normal((cfg.proj, dim)) * 0.3).astype(np.float32)
    wg = (rng.standard_normal((cfg.proj, dim)) * 0.3).astype(np.float32)
    ape = (rng.standard_normal((ratio, cfg.proj)) * 0.1).astype(np.float32)
    w = Weights(wkv=wkv, wgate=wg, ape=ape)
    n0 = n // 2
    st = State(cfg, 1)
    out = oracle.prefill(cfg, w, st, x=x[:, :n0])
    ours = [] if out is None else list(zip(out["pooled"][0], out["latent"][0]))
    for p in range(n0, n):
        o = oracle.decode_step(cfg, w, st, p, x=x[:, p:p + 1])
        if o is not None:
            ours.append((o["pooled"][0, 0], o["latent"][0, 0]))

    bc = brute.BruteCompressor(ratio, hd, wkv.tolist(), wg.tolist(), ape.tolist())
    xs = x[0].tolist()
    theirs = bc.prefill(xs[:n0])
    for p in range(n0, n):
        o = bc.decode(xs[p], p)
        if o is not None:
            theirs.append(o)
    assert len(ours) == len(theirs) == n // ratio
    for (p_o, y_o), (p_b, y_b) in zip(ours, theirs):
        p_b = np.array(p_b, dtype=np.float32)
        assert np.all(np.abs(p_o - p_b) <= np.spacing(np.abs(p_b))), (p_o, p_b)
        y_b = np.array(y_b, dtype=np.float32)
        assert np.all(np.abs(y_o - y_b) <= np.spacing(np.abs(y_b)) * 65536)


def test_projection_exact_cases():
    # one-hot rows select weight columns exactly; small integer rows give exact sums
    rng = np.random.default_rng(40)
    w = rng.standard_normal((6, 5)).astype(np.float32)
    eye = np.eye(5, dtype=np.float32)
    assert np.array_equal(oracle.project(eye, w), w.T)
    x = rng.standard_normal((3, 5)).astype(np.float32)
    ref = np.array([[brute.f32(brute.dot(xr, wr)) for wr in w.tolist()] for xr in x.tolist()], dtype=np.float32)
    assert np.array_equal(oracle.project(x, w), ref)


def test_fp4_output_of_prefill_matches_standalone_quant():
    rng = np.random.default_rng(41)
    cfg = Config(ratio=4, head_dim=64)
    kv, sc = _rand_proj(rng, 2, 20, cfg.proj)
    out = oracle.prefill(cfg, Weights(), State(cfg, 2), kv=kv, score=sc, quantize=True)
    codes, scales, deq = oracle.fp4_quant_e4m3(out["latent"].reshape(-1, 64))
    assert np.array_equal(out["codes"].reshape(-1, 32), codes)
    assert np.array_equal(out["scales"].reshape(-1, 4), scales)
    assert np.array_equal(out["dequant"].reshape(-1, 64), deq)


# ---------------------------------------------------------------- ratio 1
def _bf16_rand(rng, shape, std):
    return oracle.bf16_round((rng.standard_normal(shape) * std).astype(np.float32))


def test_plain_projection_matches_pure_python():
    rng = np.random.default_rng(41)
    hd, dim, n = 16, 24, 5
    x = _bf16_rand(rng, (n, dim), 1.0)
    wkv = _bf16_rand(rng, (hd, dim), 0.2)
    cfg = Config(ratio=1, head_dim=hd, dim=dim)
    out = oracle.plain_projection(cfg, Weights(wkv=wkv), x)
    ref = brute.plain_projection([[float(v) for v in row] for row in x], [[float(v) for v in row] for row in wkv])
    for t in range(n):
        assert [float(v) for v in out["pooled"][t]] == ref[t][0]
        assert [float(v) for v in out["latent"][t]] == ref[t][1]


def test_plain_projection_one_hot_token_reads_a_weight_column():
    rng = np.random.default_rng(42)
    hd, dim = 32, 64
    wkv = _bf16_rand(rng, (hd, dim), 0.02)
    x = np.zeros((3, dim), dtype=np.float32)
    for t, i in enumerate((0, 17, 63)):
        x[t, i] = 1.0
    out = oracle.plain_projection(Config(ratio=1, head_dim=hd, dim=dim), Weights(wkv=wkv), x)
    for t, i in enumerate((0, 17, 63)):
        assert np.array_equal(out["pooled"][t], wkv[:, i])
        # bf16 of a bf16 value is itself: the latent is the RMSNorm of the column
        u = wkv[:, i].astype(np.float64)
        ref = oracle.bf16_round(u / np.sqrt((u * u).mean() + 1e-6))
        assert np.array_equal(out["latent"][t], ref)


def test_plain_projection_scale_invariance_and_token_independence():
    rng = np.random.default_rng(43)
    hd, dim, n = 64, 128, 6
    x = _bf16_rand(rng, (n, dim), 1.0)
    wkv = _bf16_rand(rng, (hd, dim), 0.02)
    cfg = Config(ratio=1, head_dim=hd, dim=dim, eps=0.0)
    base = oracle.plain_projection(cfg, Weights(wkv=wkv), x)
    # x * 2^k: exact in bf16, projections scale exactly, RMSNorm (eps 0) is unchanged
    for k in (-5, 3):
        scaled = oracle.plain_projection(cfg, Weights(wkv=wkv), x * np.float32(2.0 ** k))
        assert np.array_equal(scaled["pooled"], base["pooled"] * np.float32(2.0 ** k))
        assert np.array_equal(scaled["latent"], base["latent"])
    # no state, no mixing: a permutation of the tokens permutes the entries
    perm = rng.permutation(n)
    moved = oracle.plain_projection(cfg, Weights(wkv=wkv), x[perm])
    assert np.array_equal(moved["latent"], base["latent"][perm])


def test_plain_projection_checks_its_inputs():
    cfg = Config(ratio=1, head_dim=16, dim=8)
    w = Weights(wkv=np.ones((16, 8), dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.plain_projection(cfg, w, np.full((2, 8), 0.1, dtype=np.float32))  # not a bf16 value
    with pytest.raises(ValueError):
        oracle.plain_projection(Config(ratio=4, head_dim=16, dim=8), w, np.ones((2, 8), dtype=np.float32))
