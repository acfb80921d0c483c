"""GPU parity of the HIP path against the CPU oracle on seeded inputs, at sizes
the oracle finishes in seconds that span several tiles and a ragged tail."""
import numpy as np
import pytest
import torch

import kv_cache_compression_fp32_amd.kvc as kvc
import oracle
from gpu_util import (bf16_inputs, dev, dev_x, host_bf16, note, oracle_cfg, oracle_weights, outputs_to_host,
                      prefill)
from parity import check_fp4, check_latent, check_pooled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvc.lib()


def test_single_hip_runtime_is_mapped():
    maps = open("/proc/self/maps").read()
    paths = set(line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line)
    assert len(paths) == 1, paths


# ---------------------------------------------------------------- fp4 quantiser
def _fp4_gpu(vals_bits: np.ndarray, width: int, inplace=False, e8m0=False):
    rows = vals_bits.size // width
    inp = torch.from_numpy(vals_bits.view(np.int16).reshape(rows, width).copy()).cuda()
    codes = torch.empty((rows, width // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, width // (32 if e8m0 else 16)), dtype=torch.uint8, device="cuda")
    out = inp if inplace else torch.empty_like(inp)
    (kvc.indexer_fp4_quant if e8m0 else kvc.latent_fp4_quant)(inp, codes, scales, out)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), host_bf16(out)


def test_fp4_quant_every_finite_bf16_value():
    note("fp4 every finite bf16, sorted blocks")
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[np.isfinite(oracle.bf16_from_bits(pats))]
    assert pats.size % 64 == 0
    codes, scales, deq = _fp4_gpu(pats, 64)
    rc, rs, rd = oracle.fp4_quant_e4m3(oracle.bf16_from_bits(pats).reshape(-1, 64))
    assert np.array_equal(codes, rc)
    assert np.array_equal(scales, rs)
    assert np.array_equal(deq.view(np.uint32), rd.view(np.uint32))


@pytest.mark.parametrize("inplace", [False, True])
def test_fp4_quant_shuffled_blocks(inplace):
    note(f"fp4 shuffled inplace={inplace}")
    rng = np.random.default_rng(11)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[np.isfinite(oracle.bf16_from_bits(pats))]
    pats = np.concatenate([rng.permutation(pats), np.zeros(256, dtype=np.uint16)])
    # plus rows of latent-like values of every scale
    lat = oracle.bf16_bits((rng.standard_normal((300, 512)) * np.exp2(rng.integers(-20, 8, (300, 1)))).astype(np.float32))
    allp = np.concatenate([pats, lat.reshape(-1)])
    codes, scales, deq = _fp4_gpu(allp, 512, inplace)
    rc, rs, rd = oracle.fp4_quant_e4m3(oracle.bf16_from_bits(allp).reshape(-1, 512))
    assert np.array_equal(codes, rc)
    assert np.array_equal(scales, rs)
    assert np.array_equal(deq.view(np.uint32), rd.view(np.uint32))


def test_fp4_quant_ragged_and_empty():
    note("fp4 ragged/empty")
    rng = np.random.default_rng(12)
    for rows, width in ((1, 16), (3, 48), (7, 128), (0, 512)):
        y = oracle.bf16_bits(rng.standard_normal((rows, width)).astype(np.float32)).reshape(-1)
        if rows == 0:
            kvc.latent_fp4_quant(torch.empty((0, width), dtype=torch.int16, device="cuda"))
            continue
        codes, scales, deq = _fp4_gpu(y, width)
        rc, rs, rd = oracle.fp4_quant_e4m3(oracle.bf16_from_bits(y).reshape(rows, width))
        assert np.array_equal(codes, rc) and np.array_equal(scales, rs)
        assert np.array_equal(deq, rd)


@pytest.mark.parametrize("inplace", [False, True])
def test_indexer_fp4_quant_every_finite_bf16_value(inplace):
    note(f"e8m0 fp4 every finite bf16 inplace={inplace}")
    rng = np.random.default_rng(13)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[np.isfinite(oracle.bf16_from_bits(pats))]
    for arr in (pats, rng.permutation(pats)):
        codes, scales, deq = _fp4_gpu(arr, 64, inplace, e8m0=True)
        rc, rs, rd = oracle.fp4_quant_e8m0(oracle.bf16_from_bits(arr).reshape(-1, 64))
        assert np.array_equal(codes, rc)
        assert np.array_equal(scales, rs)
        assert np.array_equal(deq.view(np.uint32), rd.view(np.uint32))


@pytest.mark.parametrize("ratio,hd,batch,seqlen", [(4, 128, 2, 4 * 33 + 2), (4, 512, 1, 64), (128, 128, 1, 256),
                                                   (2, 512, 2, 40)])
def test_pool_with_power_of_two_fp4(ratio, hd, batch, seqlen):
    note(f"pool e8m0 ratio={ratio} hd={hd}")
    rng = np.random.default_rng(ratio + hd + seqlen)
    cfg = kvc.Config(ratio, hd, 0, fp4_format=kvc.KVC_FP4_E8M0_B32)
    proj = kvc.kvc_proj_width(cfg)
    kv = rng.standard_normal((batch, seqlen, proj), dtype=np.float32)
    sc = rng.standard_normal((batch, seqlen, proj), dtype=np.float32) * np.float32(2)
    w = {"ape": rng.standard_normal((ratio, proj), dtype=np.float32) * np.float32(0.1)}
    g = prefill(cfg, w, batch, seqlen, kv=kv, sc=sc)
    ref = oracle.prefill(oracle_cfg(cfg), oracle_weights(w), oracle.State(oracle_cfg(cfg), batch), kv=kv,
                         score=sc, quantize=True)
    assert g["scales"].shape[-1] == hd // 32
    check_pooled(g["pooled"], ref["pooled"])
    check_latent(g["latent"], g["pooled"], ref["latent"], ref["pooled"])
    check_fp4(g["codes"], g["scales"], g["latent"], ref["codes"], ref["scales"], ref["latent"], g["dequant"],
              e8m0=True)


# ---------------------------------------------------------------- pooling from given projections
POOL_CASES = [
    # ratio, head_dim, batch, seqlen, bias, norm weight
    (2, 512, 1, 64, False, False),
    (2, 128, 3, 77, True, True),
    (4, 512, 2, 4 * 37 + 3, True, False),
    (4, 512, 1, 4, True, True),
    (4, 128, 3, 4 * 50 + 1, True, False),
    (4, 512, 2, 3, True, False),         # shorter than the ratio: no entry, carry only
    (128, 512, 2, 128 * 3 + 37, True, False),
    (128, 128, 1, 128 * 2, True, True),
]


@pytest.mark.parametrize("ratio,hd,batch,seqlen,bias,normw", POOL_CASES)
def test_pool_given_projections(ratio, hd, batch, seqlen, bias, normw):
    note(f"pool ratio={ratio} hd={hd} batch={batch} seqlen={seqlen}")
    rng = np.random.default_rng(ratio * 1000 + hd + seqlen)
    cfg = kvc.Config(ratio, hd, 0)
    proj = kvc.kvc_proj_width(cfg)
    kv = rng.standard_normal((batch, seqlen, proj), dtype=np.float32)
    sc = (rng.standard_normal((batch, seqlen, proj), dtype=np.float32) * np.float32(2.0))
    w = {}
    if bias:
        w["ape"] = (rng.standard_normal((ratio, proj), dtype=np.float32) * np.float32(0.1))
    if normw:
        w["norm_w"] = rng.uniform(0.5, 1.5, hd).astype(np.float32)
    g = prefill(cfg, w, batch, seqlen, kv=kv, sc=sc)
    st = oracle.State(oracle_cfg(cfg), batch)
    ref = oracle.prefill(oracle_cfg(cfg), oracle_weights(w), st, kv=kv, score=sc, quantize=True)
    assert g["n_groups"] == seqlen // ratio
    if ref is None:
        assert seqlen < ratio
    else:
        check_pooled(g["pooled"], ref["pooled"])
        check_latent(g["latent"], g["pooled"], ref["latent"], ref["pooled"], w.get("norm_w"), cfg.eps)
        check_fp4(g["codes"], g["scales"], g["latent"], ref["codes"], ref["scales"], ref["latent"], g["dequant"])
    # the carry is a copy of projection rows plus the bias: bit-exact
    assert np.array_equal(g["state_kv"], st.kv)
    assert np.array_equal(g["state_sc"], st.score)


# ---------------------------------------------------------------- projection GEMM
GEMM_CASES = [
    # ratio, head_dim, dim, batch, seqlen
    (4, 128, 256, 2, 300),
    (128, 512, 512, 1, 256 + 128 + 5),
    (2, 512, 128, 3, 61),
    (4, 512, 4096, 1, 130),
    (4, 512, 64, 1, 16384 + 37),   # 256 x 256 tiles, ragged last row tile
    (4, 512, 64, 1, 4096 + 37),    # 256 x 128 tiles, ragged last row tile
    (2, 128, 32, 2, 300),          # one 32-k stage
]


# (x format, projection): f32 rows split on the bf16 matrix cores, f32 rows
# on the f32 matrix cores, f32 rows as scaled f16 parts on the f16 matrix
# cores (the default for f32 rows), bf16 rows on the bf16 matrix cores (the
# default for bf16 rows)
PROJ_PATHS = [(kvc.KVC_X_F32, kvc.KVC_PROJ_BF16_SPLIT), (kvc.KVC_X_F32, kvc.KVC_PROJ_F32_MFMA),
              (kvc.KVC_X_F32, kvc.KVC_PROJ_F16_SPLIT), (kvc.KVC_X_BF16, kvc.KVC_PROJ_BF16_SPLIT)]


@pytest.mark.parametrize("x_format,projection", PROJ_PATHS)
@pytest.mark.parametrize("ratio,hd,dim,batch,seqlen", GEMM_CASES)
def test_projection_gemm_and_full_prefill(ratio, hd, dim, batch, seqlen, x_format, projection):
    note(f"gemm+prefill ratio={ratio} hd={hd} dim={dim} batch={batch} seqlen={seqlen} x_format={x_format} "
         f"projection={projection}")
    rng = np.random.default_rng(dim + seqlen)
    cfg = kvc.Config(ratio, hd, dim, x_format=x_format, projection=projection)
    proj = kvc.kvc_proj_width(cfg)
    x = rng.standard_normal((batch, seqlen, dim), dtype=np.float32)
    if x_format == kvc.KVC_X_BF16:  # the model's bf16 hidden state
        x = bf16_inputs(x)
    w = {"wkv": rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.02),
         "wgate": rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.02),
         "ape": rng.standard_normal((ratio, proj), dtype=np.float32) * np.float32(0.1)}
    g = prefill(cfg, w, batch, seqlen, x=x)
    # the projection planes of a GEMM-only call (a ratio-4 prefill with
    # outputs may pool inside the GEMM and write only the rows it needs)
    from gpu_util import weights
    ws = torch.empty(kvc.kvc_prefill_workspace_floats(cfg, batch, seqlen), dtype=torch.float32, device="cuda")
    kvc.compressor_prefill(cfg, weights(w), dev_x(cfg, x), batch, seqlen, ws)
    torch.cuda.synchronize()
    m = batch * seqlen * proj
    g["proj_kv"] = ws[:m].view(batch, seqlen, proj).cpu().numpy()
    g["proj_sc"] = ws[m:2 * m].view(batch, seqlen, proj).cpu().numpy()
    # projections: inside the worst-case bound of any f32 summation order,
    # dim * 2^-24 * sum |x| |w| (plus one rounding of the bias addition on the
    # score plane), and 1e-5 of each row's largest value
    for name, wname in (("proj_kv", "wkv"), ("proj_sc", "wgate")):
        ref = oracle.project(x.reshape(-1, dim), w[wname]).reshape(batch, seqlen, proj)
        if name == "proj_sc":  # the workspace's score plane carries the positional bias
            ref = oracle.add_bias(ref, w["ape"], np.arange(seqlen), ratio)
        absdot = (np.abs(x.reshape(-1, dim)).astype(np.float64) @ np.abs(w[wname]).astype(np.float64).T)
        bound = dim * 2.0 ** -24 * absdot.reshape(batch, seqlen, proj) + np.spacing(np.abs(ref)) + 1e-30
        err = np.abs(g[name].astype(np.float64) - ref)
        assert np.all(err <= bound), f"{name}: {np.sum(err > bound)} beyond the bound"
        check_pooled(g[name], ref, name)
    st = oracle.State(oracle_cfg(cfg), batch)
    ref = oracle.prefill(oracle_cfg(cfg), oracle_weights(w), st, x=x, quantize=True)
    check_pooled(g["pooled"], ref["pooled"])
    check_latent(g["latent"], g["pooled"], ref["latent"], ref["pooled"])
    check_fp4(g["codes"], g["scales"], g["latent"], ref["codes"], ref["scales"], ref["latent"], g["dequant"])
    # the carried rows are projections (+ bias): same tolerance as the projections
    fin = np.isfinite(st.score)
    assert np.array_equal(np.isfinite(g["state_sc"]), fin)
    check_pooled(np.where(fin, g["state_sc"], 0), np.where(fin, st.score, 0), "state score")
    check_pooled(g["state_kv"], st.kv, "state kv")


# ---------------------------------------------------------------- decode
def _decode_gpu(cfg, w, batch, xs=None, kvs=None, scs=None, start=0, state=None, fp4=True):
    """Run decode steps for positions start..; xs [batch, steps, dim] or the
    projections kvs/scs [batch, steps, proj]. Returns the emitted entries
    concatenated along the entry axis, and the final state."""
    proj = kvc.kvc_proj_width(cfg)
    steps = (xs if xs is not None else kvs).shape[1]
    ws = kvc.new_decode_workspace(cfg, batch)
    if state is None:
        state = kvc.new_state(cfg, batch)
    xd = dev_x(cfg, xs) if xs is not None else None
    kvd, scd = (dev(kvs), dev(scs)) if kvs is not None else (None, None)
    emitted = []
    for i in range(steps):
        p = start + i
        out = kvc.new_outputs(cfg, batch, 1, latent=True, pooled=True, fp4=fp4, dequant=fp4,
                              rotated=cfg.rope_dim > 0)
        if xd is None:
            ws[:batch * proj] = kvd[:, i].reshape(-1)
            ws[batch * proj:2 * batch * proj] = scd[:, i].reshape(-1)
            xi = None
        else:
            xi = xd[:, i].contiguous()
        e = kvc.compressor_decode_step(cfg, w, xi, batch, p, ws, state[0], state[1], out)
        assert e == (p > 0 and (p + 1) % cfg.ratio == 0)
        if e:
            emitted.append(out)
    torch.cuda.synchronize()
    from gpu_util import outputs_to_host
    res = [outputs_to_host(o) for o in emitted]
    cat = {k: np.concatenate([r[k] for r in res], axis=1) for k in res[0]} if res else {}
    cat["state_kv"] = state[0].cpu().numpy()
    cat["state_sc"] = state[1].cpu().numpy()
    return cat


def _live_rows(ratio, seqlen):
    rem = seqlen % ratio
    if ratio == 4:
        return list(range(ratio)) + [ratio + i for i in range(rem)]
    return list(range(rem))


@pytest.mark.parametrize("ratio,hd,batch,steps", [(4, 512, 3, 40), (4, 128, 2, 33), (2, 512, 2, 21),
                                                  (128, 512, 2, 256 + 9)])
def test_decode_equals_prefill_bitwise_given_projections(ratio, hd, batch, steps):
    note(f"decode==prefill bitwise ratio={ratio} hd={hd}")
    from gpu_util import weights
    rng = np.random.default_rng(ratio + steps)
    cfg = kvc.Config(ratio, hd, 0)
    proj = kvc.kvc_proj_width(cfg)
    kv = rng.standard_normal((batch, steps, proj), dtype=np.float32)
    sc = rng.standard_normal((batch, steps, proj), dtype=np.float32) * np.float32(2)
    w = {"ape": rng.standard_normal((ratio, proj), dtype=np.float32) * np.float32(0.1)}
    full = prefill(cfg, w, batch, steps, kv=kv, sc=sc)
    dec = _decode_gpu(cfg, weights(w), batch, kvs=kv, scs=sc)
    for k in ("pooled", "latent", "codes", "scales", "dequant"):
        assert np.array_equal(dec[k].view(np.uint8), full[k].view(np.uint8)), k
    # the rows a continuation reads next (other rows hold dead values)
    live = _live_rows(ratio, steps)
    assert np.array_equal(dec["state_kv"][:, live], full["state_kv"][:, live])
    assert np.array_equal(dec["state_sc"][:, live], full["state_sc"][:, live])
    # and the oracle agrees with both
    ref = oracle.prefill(oracle_cfg(cfg), oracle_weights(w), oracle.State(oracle_cfg(cfg), batch), kv=kv,
                         score=sc, quantize=True)
    check_pooled(dec["pooled"], ref["pooled"])


@pytest.mark.parametrize("ratio", [2, 4, 128])
def test_prefill_then_decode_continuation(ratio):
    note(f"continuation ratio={ratio}")
    from gpu_util import weights
    rng = np.random.default_rng(77 + ratio)
    hd, batch = 128, 2
    cfg = kvc.Config(ratio, hd, 0)
    proj = kvc.kvc_proj_width(cfg)
    n = 3 * ratio + 1
    kv = rng.standard_normal((batch, n, proj), dtype=np.float32)
    sc = rng.standard_normal((batch, n, proj), dtype=np.float32)
    w = {"ape": rng.standard_normal((ratio, proj), dtype=np.float32) * np.float32(0.1)}
    full = prefill(cfg, w, batch, n, kv=kv, sc=sc)
    splits = sorted(set([1, 2, ratio - 1, ratio, ratio + 1, 2 * ratio + 3, n - 1, n]) - {0})
    for n0 in splits:
        state = kvc.new_state(cfg, batch)
        state[0].fill_(5.0)  # stale values of an earlier sequence must not leak
        state[1].fill_(3.0)
        first = prefill(cfg, w, batch, n0, kv=kv[:, :n0], sc=sc[:, :n0], state=state)
        rest = _decode_gpu(cfg, weights(w), batch, kvs=kv[:, n0:], scs=sc[:, n0:], start=n0, state=state)
        parts = [p for p in (first.get("latent"), rest.get("latent")) if p is not None]
        got = np.concatenate(parts, axis=1)
        assert np.array_equal(got.view(np.uint32), full["latent"].view(np.uint32)), n0


@pytest.mark.parametrize("x_format", [kvc.KVC_X_F32, kvc.KVC_X_BF16])
def test_decode_with_projection_matches_oracle(x_format):
    note(f"decode with x, ratio 4, batch 64, dim 4096, 16 steps, x_format={x_format}")
    from gpu_util import weights
    rng = np.random.default_rng(5)
    cfg = kvc.Config(4, 512, 4096, x_format=x_format)
    proj = 1024
    batch, steps = 64, 16
    x = rng.standard_normal((batch, steps, 4096), dtype=np.float32)
    if x_format == kvc.KVC_X_BF16:
        x = bf16_inputs(x)
    w = {"wkv": rng.standard_normal((proj, 4096), dtype=np.float32) * np.float32(0.02),
         "wgate": rng.standard_normal((proj, 4096), dtype=np.float32) * np.float32(0.02),
         "ape": rng.standard_normal((4, proj), dtype=np.float32) * np.float32(0.1)}
    dec = _decode_gpu(cfg, weights(w), batch, xs=x)
    ref = oracle.prefill(oracle_cfg(cfg), oracle_weights(w), oracle.State(oracle_cfg(cfg), batch), x=x,
                         quantize=True)
    check_pooled(dec["pooled"], ref["pooled"])
    check_latent(dec["latent"], dec["pooled"], ref["latent"], ref["pooled"])
    check_fp4(dec["codes"], dec["scales"], dec["latent"], ref["codes"], ref["scales"], ref["latent"], dec["dequant"])
    # and the GPU prefill over the same tokens: from f32 x both sum each
    # projection in the same order, so every output is bit for bit the
    # prefill's; from bf16 x the prefill projects on the bf16 matrix cores
    full = prefill(cfg, w, batch, steps, x=x)
    if x_format == kvc.KVC_X_F32:
        for k in ("pooled", "latent", "codes", "scales", "dequant"):
            assert np.array_equal(dec[k].view(np.uint8), full[k].view(np.uint8)), k
        live = _live_rows(4, steps)
        assert np.array_equal(dec["state_kv"][:, live].view(np.uint32), full["state_kv"][:, live].view(np.uint32))
        assert np.array_equal(dec["state_sc"][:, live].view(np.uint32), full["state_sc"][:, live].view(np.uint32))
    else:
        check_pooled(dec["pooled"], full["pooled"], "decode vs prefill")


@pytest.mark.parametrize("ratio,batch,dim,steps", [(2, 8, 256, 21), (128, 4, 128, 2 * 128 + 3)])
def test_decode_streaming_with_projection_ratio_2_and_128(ratio, batch, dim, steps):
    note(f"decode with x, ratio {ratio}, batch {batch}, dim {dim}, {steps} steps")
    from gpu_util import weights
    rng = np.random.default_rng(ratio + steps)
    cfg = kvc.Config(ratio, 512, dim)
    proj = 512
    x = rng.standard_normal((batch, steps, dim), dtype=np.float32)
    w = {"wkv": rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.05),
         "wgate": rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.05),
         "ape": rng.standard_normal((ratio, proj), dtype=np.float32) * np.float32(0.1)}
    dec = _decode_gpu(cfg, weights(w), batch, xs=x)
    st = oracle.State(oracle_cfg(cfg), batch)
    ref = oracle.prefill(oracle_cfg(cfg), oracle_weights(w), st, x=x, quantize=True)
    assert dec["pooled"].shape[1] == steps // ratio
    check_pooled(dec["pooled"], ref["pooled"])
    check_latent(dec["latent"], dec["pooled"], ref["latent"], ref["pooled"])
    check_fp4(dec["codes"], dec["scales"], dec["latent"], ref["codes"], ref["scales"], ref["latent"], dec["dequant"])
    # the tail left in the state is the oracle's carry
    live = _live_rows(ratio, steps)
    check_pooled(dec["state_kv"][:, live], st.kv[:, live], "state kv")
    check_pooled(dec["state_sc"][:, live], st.score[:, live], "state score")


# ---------------------------------------------------------------- ratio 1
RATIO1_CASES = [
    # head_dim, dim, tokens, norm weight
    (512, 256, 300, False),         # 128 x 128 tiles, ragged
    (128, 128, 1000, True),
    (512, 64, 16384 + 37, False),   # 256 x 128 tiles, ragged
    (512, 64, 65536 + 37, True),    # 256 x 256 tiles, ragged
    (128, 64, 65536 + 5, False),    # 256 x 128 tiles at head_dim 128
]


def _bf16_pair(a: np.ndarray):
    """bf16 tensor (rounded from a) and the float32 array of its values."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t, t.float().numpy()


@pytest.mark.parametrize("hd,dim,tokens,normw", RATIO1_CASES)
def test_ratio1_forward_matches_oracle(hd, dim, tokens, normw):
    note(f"ratio 1 hd={hd} dim={dim} tokens={tokens}")
    rng = np.random.default_rng(hd + dim + tokens)
    cfg = kvc.Config(1, hd, dim)
    xt, x = _bf16_pair(rng.standard_normal((tokens, dim), dtype=np.float32))
    wt, wkv = _bf16_pair(rng.standard_normal((hd, dim), dtype=np.float32) * np.float32(0.05))
    nw = (1.0 + 0.1 * rng.standard_normal(hd)).astype(np.float32) if normw else None
    ws = torch.empty(kvc.kvc_ratio1_workspace_floats(cfg, tokens), dtype=torch.float32, device="cuda")
    out = kvc.new_outputs(cfg, 1, tokens, latent=True, pooled=True, fp4=True, dequant=True)
    kvc.compressor_ratio1_forward(cfg, wt.cuda(), xt.cuda(), tokens, ws, out, norm_w=dev(nw))
    torch.cuda.synchronize()
    g = {k: v[0] for k, v in outputs_to_host(out).items()}
    assert np.array_equal(ws.view(tokens, hd).cpu().numpy(), g["pooled"])  # the workspace holds it too
    # tokens are independent: large cases compare the first row tile, the
    # ragged last tiles and random rows, small cases every row
    if tokens > 20000:
        rows = np.array(sorted(set(range(256)) | set(range(tokens - 300, tokens)) |
                               set(rng.choice(tokens, 512, replace=False).tolist())))
    else:
        rows = np.arange(tokens)
    x, g = x[rows], {k: v[rows] for k, v in g.items()}
    ref = oracle.plain_projection(oracle.Config(ratio=1, head_dim=hd, dim=dim), oracle.Weights(wkv=wkv, norm_w=nw),
                                  x, quantize=True)
    # the f32 projection: inside the worst-case bound of any f32 summation
    # order of the (exact) bf16 products
    absdot = np.abs(x).astype(np.float64) @ np.abs(wkv).astype(np.float64).T
    bound = dim * 2.0 ** -24 * absdot + np.spacing(np.abs(ref["pooled"])) + 1e-30
    err = np.abs(g["pooled"].astype(np.float64) - ref["pooled"])
    assert np.all(err <= bound), f"projection: {np.sum(err > bound)} beyond the bound"
    check_pooled(g["pooled"], ref["pooled"], "projection")
    check_latent(g["latent"], g["pooled"], ref["latent"], ref["pooled"], nw, cfg.eps)
    check_fp4(g["codes"], g["scales"], g["latent"], ref["codes"], ref["scales"], ref["latent"], g["dequant"])


def test_ratio1_power_of_two_fp4_and_outputs_subset():
    note("ratio 1 hd=128 e8m0 fp4, latent-only call")
    rng = np.random.default_rng(91)
    hd, dim, tokens = 128, 192, 777
    cfg = kvc.Config(1, hd, dim, fp4_format=kvc.KVC_FP4_E8M0_B32)
    xt, x = _bf16_pair(rng.standard_normal((tokens, dim), dtype=np.float32))
    wt, wkv = _bf16_pair(rng.standard_normal((hd, dim), dtype=np.float32) * np.float32(0.05))
    ws = torch.empty(tokens * hd, dtype=torch.float32, device="cuda")
    full = kvc.new_outputs(cfg, 1, tokens, latent=True, pooled=True, fp4=True, dequant=True)
    kvc.compressor_ratio1_forward(cfg, wt.cuda(), xt.cuda(), tokens, ws, full)
    only = kvc.Outputs(latent=torch.empty((tokens, hd), dtype=torch.bfloat16, device="cuda"))
    kvc.compressor_ratio1_forward(cfg, wt.cuda(), xt.cuda(), tokens, ws, only)
    torch.cuda.synchronize()
    g = outputs_to_host(full)
    assert g["scales"].shape[-1] == hd // 32
    ref = oracle.plain_projection(oracle.Config(ratio=1, head_dim=hd, dim=dim, fp4="e8m0"),
                                  oracle.Weights(wkv=wkv), x, quantize=True)
    check_latent(g["latent"][0], g["pooled"][0], ref["latent"], ref["pooled"])
    check_fp4(g["codes"][0], g["scales"][0], g["latent"][0], ref["codes"], ref["scales"], ref["latent"],
              g["dequant"][0], e8m0=True)
    assert np.array_equal(only.latent.view(torch.int16).cpu().numpy(), full.latent[0].view(torch.int16).cpu().numpy())


# ---------------------------------------------------------------- RoPE
def _yarn_table(rows, rope_dim, ratio):
    # entry j stands for the last token of its group; YaRN-extended table
    pos = np.arange(rows) * ratio + ratio - 1
    return oracle.rope_table(pos, oracle.yarn_inv_freq(rope_dim, 10000.0, 16.0, 4096))


def test_latent_rope_matches_oracle_exactly():
    note("latent_rope: random rows, constructed bf16 midpoints, in place")
    rng = np.random.default_rng(21)
    rows, width, rd = 3000, 512, 64
    lat = oracle.bf16_round((rng.standard_normal((rows, width)) * np.exp2(rng.integers(-8, 8, (rows, 1))))
                            .astype(np.float32))
    table = oracle.rope_table(rng.integers(0, 1 << 20, rows + 7), oracle.yarn_inv_freq(rd, 10000.0, 40.0, 4096))
    # rows whose a c lands on a bf16 midpoint with b s below double resolution there
    for r, sign in ((0, 1.0), (1, -1.0), (2, 1.0)):
        lat[r, width - rd:] = 0.0
        lat[r, width - rd + 2 * np.arange(rd // 2)] = 1.0
        lat[r, width - rd + 1 + 2 * np.arange(rd // 2)] = 2.0 ** -40
        table[7 + r, :, 0] = np.float32(1.0 + 2.0 ** -8)
        table[7 + r, :, 1] = np.float32(-sign * 2.0 ** -30)
    ref = oracle.apply_rope(lat, table[7:7 + rows], rd)
    assert ref[0, width - rd] == np.float32(1.0 + 2.0 ** -7) and ref[1, width - rd] == np.float32(1.0)
    bits = lat.view(np.uint32) >> 16
    inp = torch.from_numpy(bits.astype(np.int32).astype(np.int16)).cuda()
    out = torch.empty_like(inp)
    tab = dev(table)
    kvc.latent_rope(inp, rd, tab, first_row=7, out=out)
    kvc.latent_rope(inp, rd, tab, first_row=7)  # in place
    torch.cuda.synchronize()
    for t in (out, inp):
        got = host_bf16(t)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{np.sum(got != ref)} values differ"


@pytest.mark.parametrize("ratio,hd,batch,seqlen", [(4, 512, 2, 4 * 37 + 1), (2, 128, 2, 50), (128, 512, 1, 384 + 3)])
def test_pool_with_rope_matches_oracle_and_decode(ratio, hd, batch, seqlen):
    note(f"pool + RoPE ratio={ratio} hd={hd}")
    from gpu_util import weights
    rng = np.random.default_rng(ratio + hd + seqlen)
    rd = 64
    cfg = kvc.Config(ratio, hd, 0, rope_dim=rd)
    proj = kvc.kvc_proj_width(cfg)
    kv = rng.standard_normal((batch, seqlen, proj), dtype=np.float32)
    sc = rng.standard_normal((batch, seqlen, proj), dtype=np.float32) * np.float32(2)
    groups = seqlen // ratio
    w = {"ape": rng.standard_normal((ratio, proj), dtype=np.float32) * np.float32(0.1),
         "rope_cs": _yarn_table(groups + 2, rd, ratio)}
    g = prefill(cfg, w, batch, seqlen, kv=kv, sc=sc)
    plain = prefill(kvc.Config(ratio, hd, 0), {"ape": w["ape"]}, batch, seqlen, kv=kv, sc=sc)
    # the compressor's own output is unrotated
    assert np.array_equal(g["latent"].view(np.uint32), plain["latent"].view(np.uint32))
    # entry j of every batch row turns by table row j, exactly as the oracle
    rows = np.broadcast_to(w["rope_cs"][:groups], (batch, groups, rd // 2, 2))
    ref_rot = oracle.apply_rope(g["latent"], rows, rd)
    assert np.array_equal(g["rotated"].view(np.uint32), ref_rot.view(np.uint32))
    # the cache form encodes the rotated entry
    check_fp4(g["codes"], g["scales"], g["rotated"], gpu_dequant=g["dequant"])
    # end to end against the oracle, and decode == prefill bitwise
    ref = oracle.prefill(oracle_cfg(cfg), oracle_weights(w), oracle.State(oracle_cfg(cfg), batch), kv=kv, score=sc,
                         quantize=True)
    same = np.all(g["latent"] == ref["latent"], axis=-1)
    assert np.array_equal(g["rotated"][same].view(np.uint32), ref["rotated"][same].view(np.uint32))
    dec = _decode_gpu(cfg, weights(w), batch, kvs=kv, scs=sc)
    for k in ("rotated", "codes", "scales", "dequant", "latent"):
        assert np.array_equal(dec[k].view(np.uint8), g[k].view(np.uint8)), k


# ---------------------------------------------------------------- fused projection + pooling
FUSED_CASES = [
    # head_dim, batch, seqlen, dim, options
    (512, 1, 16384 + 4 * 7 + 3, 64, "norm"),    # ragged last row tile, 3 tail tokens
    (512, 4, 4100, 64, "rope"),                  # row tiles straddle batch rows
    (128, 1, 65536 + 9, 64, "e8m0"),             # 128-wide: two column tiles
]


@pytest.mark.parametrize("x_format,projection", PROJ_PATHS)
@pytest.mark.parametrize("hd,batch,seqlen,dim,opt", FUSED_CASES)
def test_fused_pooling_equals_separate_kernels_bitwise(hd, batch, seqlen, dim, opt, x_format, projection):
    note(f"fused GEMM + pool hd={hd} batch={batch} seqlen={seqlen} {opt} x_format={x_format} projection={projection}")
    from gpu_util import weights
    rng = np.random.default_rng(hd + batch + seqlen)
    cfg = kvc.Config(4, hd, dim, rope_dim=64 if opt == "rope" else 0,
                     fp4_format=kvc.KVC_FP4_E8M0_B32 if opt == "e8m0" else kvc.KVC_FP4_E4M3_B16,
                     x_format=x_format, projection=projection)
    proj = 2 * hd
    groups = seqlen // 4
    x = rng.standard_normal((batch, seqlen, dim), dtype=np.float32)
    if x_format == kvc.KVC_X_BF16:
        x = bf16_inputs(x)
    w = {"wkv": rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.1),
         "wgate": rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.1),
         "ape": rng.standard_normal((4, proj), dtype=np.float32) * np.float32(0.1)}
    if opt == "norm":
        w["norm_w"] = (1.0 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    if opt == "rope":
        w["rope_cs"] = _yarn_table(groups, 64, 4)
    W = weights(w)
    xd = dev_x(cfg, x)
    outs = lambda: kvc.new_outputs(cfg, batch, groups, latent=True, pooled=True, fp4=True, dequant=True,  # noqa: E731
                                   rotated=cfg.rope_dim > 0)
    # fused: projection with pooling in the GEMM epilogue (NaN sentinel in the planes)
    ws = torch.full((kvc.kvc_prefill_workspace_floats(cfg, batch, seqlen),), float("nan"), device="cuda")
    st_f = kvc.new_state(cfg, batch)
    fused = outs()
    kvc.compressor_prefill(cfg, W, xd, batch, seqlen, ws, st_f[0], st_f[1], fused)
    # separate: the GEMM alone (planes with the bias), then the pool kernel on them
    ws2 = torch.empty_like(ws)
    kvc.compressor_prefill(cfg, W, xd, batch, seqlen, ws2)
    st_u = kvc.new_state(cfg, batch)
    sep = outs()
    kvc.compressor_prefill(cfg, kvc.Weights(norm_w=W.norm_w, rope_cs=W.rope_cs), None, batch, seqlen, ws2,
                           st_u[0], st_u[1], sep)
    torch.cuda.synchronize()
    # the fused path ran: it alone writes the pooled rows after the planes
    # (NaN sentinel everywhere else it leaves alone)
    pooled_rows = ws[2 * batch * seqlen * proj:2 * batch * seqlen * proj + batch * groups * hd]
    assert not torch.isnan(pooled_rows).any().item()
    if projection != kvc.KVC_PROJ_F32_MFMA:  # (there interior rows hold the first k half's sums)
        planes = ws[:2 * batch * seqlen * proj].view(2, batch * seqlen, proj)
        assert torch.isnan(planes[0, 100, 0]).item() and torch.isnan(planes[1, 1000, hd]).item()
    a, b = outputs_to_host(fused), outputs_to_host(sep)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    live = _live_rows(4, seqlen)
    assert np.array_equal(st_f[0][:, live].cpu().numpy(), st_u[0][:, live].cpu().numpy())
    assert np.array_equal(st_f[1][:, live].cpu().numpy(), st_u[1][:, live].cpu().numpy())
    # and sampled entries against the oracle
    ent = np.array(sorted(set([0, 1, 63, 64, 65, 127, 128, groups - 1]) | set(rng.choice(groups, 40).tolist())))
    ocfg = oracle_cfg(cfg)
    for bb in range(batch):
        ref = oracle.prefill(ocfg, oracle_weights(w), oracle.State(ocfg, 1), x=x[bb:bb + 1], quantize=True,
                             entries=ent)
        check_pooled(a["pooled"][bb][ent], ref["pooled"][0])
        check_latent(a["latent"][bb][ent], a["pooled"][bb][ent], ref["latent"][0], ref["pooled"][0],
                     w.get("norm_w"), cfg.eps)


# ---------------------------------------------------------------- bf16 hidden states: exact weight split
SPLIT_CASES = [
    # ratio, head_dim, dim, batch, seqlen
    (4, 128, 256, 1, 256 + 64),    # 256 x 256 tiles, ragged last row tile
    (2, 128, 128, 2, 130),         # 128-wide halves: 256 x 128 tiles
    (128, 512, 256, 1, 300),
]


@pytest.mark.parametrize("x_format", [kvc.KVC_X_BF16, kvc.KVC_X_F32])
@pytest.mark.parametrize("ratio,hd,dim,batch,seqlen", SPLIT_CASES)
def test_one_hot_rows_reproduce_the_f32_weights_exactly(ratio, hd, dim, batch, seqlen, x_format):
    """x row r = the unit vector e_(r mod dim): each output is then one f32
    weight times 1, i.e. 1 * hi + 1 * mid + 1 * lo of its three bf16 parts
    (f32 x: 1 splits into 1 + 0 + 0), which must give the weight back bit
    for bit (the score plane then adds the positional bias in one f32
    addition). Weights span the f32 exponent range whose parts are all normal
    numbers, with zeros, the largest finite value and values whose low parts
    have leading zeros."""
    note(f"one-hot x ratio={ratio} hd={hd} dim={dim} batch={batch} seqlen={seqlen} x_format={x_format}")
    from gpu_util import weights
    rng = np.random.default_rng(ratio + dim + seqlen)
    cfg = kvc.Config(ratio, hd, dim, x_format=x_format, projection=kvc.KVC_PROJ_BF16_SPLIT)
    proj = kvc.kvc_proj_width(cfg)
    m = batch * seqlen
    x = np.zeros((m, dim), np.float32)
    x[np.arange(m), np.arange(m) % dim] = 1.0

    def wide(shape):
        v = rng.choice([-1.0, 1.0], shape) * np.ldexp(rng.uniform(1.0, 2.0, shape), rng.integers(-100, 127, shape))
        v = v.astype(np.float32)
        flat = v.reshape(-1)
        special = np.array([0.0, -0.0, np.finfo(np.float32).max, -np.finfo(np.float32).max, 1 + 2.0 ** -23,
                            -(1 + 2.0 ** -16), 1 + 2.0 ** -8 + 2.0 ** -23, np.float32(0.1)], np.float32)
        flat[rng.choice(flat.size, special.size, replace=False)] = special
        return v

    w = {"wkv": wide((proj, dim)), "wgate": wide((proj, dim)),
         "ape": rng.standard_normal((ratio, proj)).astype(np.float32)}
    ws = torch.full((kvc.kvc_prefill_workspace_floats(cfg, batch, seqlen),), float("nan"), device="cuda")
    kvc.compressor_prefill(cfg, weights(w), dev_x(cfg, x.reshape(batch, seqlen, dim)), batch, seqlen, ws)
    torch.cuda.synchronize()
    kv = ws[:m * proj].view(m, proj).cpu().numpy()
    sc = ws[m * proj:2 * m * proj].view(m, proj).cpu().numpy()
    col = np.arange(m) % dim
    # a sum accumulated from +0 turns a -0 weight into +0 (as any f32 dot product does)
    want = w["wkv"].T[col] + np.float32(0.0)
    bad = kv.view(np.uint32) != want.view(np.uint32)
    assert not bad.any(), f"{bad.sum()} differ, e.g. weights {want[bad][:4]} -> {kv[bad][:4]}"
    pos = np.arange(m) % seqlen
    want = w["wgate"].T[col] + w["ape"][pos % ratio]   # one f32 rounding, as on the GPU
    bad = sc.view(np.uint32) != want.view(np.uint32)
    assert not bad.any(), f"{bad.sum()} differ, e.g. {want[bad][:4]} -> {sc[bad][:4]}"


@pytest.mark.parametrize("ratio,hd,dim,batch,seqlen", SPLIT_CASES)
def test_f32_x_split_gives_faithfully_rounded_products(ratio, hd, dim, batch, seqlen):
    """f32 x rows v_r e_(r mod dim) with bf16-valued weights (mid = lo = 0):
    the kernel sums xh w, xm w and xl w, each product exact, where xh w + xm w
    is still exact in f32 and only the last addition rounds. Every output
    must therefore be one of the two f32 neighbours of the exact v_r w
    (computed in float64). The matrix cores' addition is not always the
    nearest one (a few percent of these outputs land on the other
    neighbour), so nearest-even rounding is counted, not required."""
    note(f"f32 x split ratio={ratio} hd={hd} dim={dim} batch={batch} seqlen={seqlen}")
    from gpu_util import bf16_inputs, weights
    rng = np.random.default_rng(7 + ratio + dim)
    cfg = kvc.Config(ratio, hd, dim, projection=kvc.KVC_PROJ_BF16_SPLIT)
    proj = kvc.kvc_proj_width(cfg)
    m = batch * seqlen
    v = (rng.standard_normal(m) * np.exp2(rng.integers(-30, 30, m))).astype(np.float32)
    x = np.zeros((m, dim), np.float32)
    x[np.arange(m), np.arange(m) % dim] = v
    w = {"wkv": bf16_inputs(rng.standard_normal((proj, dim)).astype(np.float32)),
         "wgate": bf16_inputs(rng.standard_normal((proj, dim)).astype(np.float32))}
    ws = torch.full((kvc.kvc_prefill_workspace_floats(cfg, batch, seqlen),), float("nan"), device="cuda")
    kvc.compressor_prefill(cfg, weights(w), dev(x.reshape(batch, seqlen, dim)), batch, seqlen, ws)
    torch.cuda.synchronize()
    col = np.arange(m) % dim
    for plane, name in ((0, "wkv"), (1, "wgate")):
        got = ws[plane * m * proj:(plane + 1) * m * proj].view(m, proj).cpu().numpy()
        exact = v[:, None].astype(np.float64) * w[name].T[col].astype(np.float64)  # exact: 24 x 8 bits
        lo = exact.astype(np.float32)                      # nearest; then its neighbour on the other side
        other = np.where(lo.astype(np.float64) < exact, np.nextafter(lo, np.float32(np.inf)),
                         np.nextafter(lo, np.float32(-np.inf)))
        faithful = (got == lo) | (got == other) | ((exact == 0) & (got == 0))
        assert faithful.all(), f"{name}: {(~faithful).sum()} not within one rounding of v w"
        note(f"  {name}: {(got != lo).sum()} of {got.size} outputs on the farther neighbour")


# ---------------------------------------------------------------- the scaled f16 split
def _f16_parts_sum(w):
    """h + l of each weight row scaled by 2^b (b brings the row's largest
    magnitude into [2^14, 2^15)), scaled back: what one-hot x rows give."""
    amax = np.abs(w).max(axis=1, keepdims=True).astype(np.float64)
    b = np.where(amax > 0, 15 - np.frexp(np.where(amax > 0, amax, 1.0))[1], 0)
    y = np.ldexp(w.astype(np.float64), b).astype(np.float32)   # exact: a power-of-two scaling
    h = y.astype(np.float16)
    l = (y - h.astype(np.float32)).astype(np.float16)          # y - h is exact in f32
    return np.ldexp(h.astype(np.float32) + l.astype(np.float32), -b).astype(np.float32)


@pytest.mark.parametrize("ratio,hd,dim,batch,seqlen", SPLIT_CASES)
def test_f16_split_one_hot_rows_give_the_two_part_weights(ratio, hd, dim, batch, seqlen):
    """x row r = e_(r mod dim) (scaled to 2^14, split into 2^14 + 0) picks
    one weight: the output is its two f16 parts' sum scaled back, bit for bit,
    and that sum is within 2^-22 relative of the f32 weight. Weight rows have
    scales 2^-100 .. 2^100 (each row's exponent is its own) and values
    spanning 2^9 inside a row."""
    note(f"f16 split one-hot ratio={ratio} hd={hd} dim={dim} batch={batch} seqlen={seqlen}")
    from gpu_util import weights
    rng = np.random.default_rng(11 + ratio + dim + seqlen)
    cfg = kvc.Config(ratio, hd, dim, projection=kvc.KVC_PROJ_F16_SPLIT)
    proj = kvc.kvc_proj_width(cfg)
    m = batch * seqlen
    x = np.zeros((m, dim), np.float32)
    x[np.arange(m), np.arange(m) % dim] = 1.0

    def rows(shape):
        shift = rng.integers(-100, 100, (shape[0], 1))
        shift[0] = 0   # row 0 also holds the special values below
        v = rng.choice([-1.0, 1.0], shape) * np.ldexp(rng.uniform(1.0, 2.0, shape), shift + rng.integers(-8, 1, shape))
        v = v.astype(np.float32)
        v[0, :4] = [0.0, -0.0, 1 + 2.0 ** -23, -(1 + 2.0 ** -12)]
        return v

    w = {"wkv": rows((proj, dim)), "wgate": rows((proj, dim)),
         "ape": rng.standard_normal((ratio, proj)).astype(np.float32)}
    ws = torch.full((kvc.kvc_prefill_workspace_floats(cfg, batch, seqlen),), float("nan"), device="cuda")
    kvc.compressor_prefill(cfg, weights(w), dev(x.reshape(batch, seqlen, dim)), batch, seqlen, ws)
    torch.cuda.synchronize()
    kv = ws[:m * proj].view(m, proj).cpu().numpy()
    sc = ws[m * proj:2 * m * proj].view(m, proj).cpu().numpy()
    col = np.arange(m) % dim
    for name in ("wkv", "wgate"):
        parts = _f16_parts_sum(w[name])
        rel = np.abs(parts.astype(np.float64) - w[name]) / np.maximum(np.abs(w[name]).astype(np.float64), 1e-300)
        assert rel.max() <= 2.0 ** -22, f"{name}: two-part sum off by {rel.max():.3e} relative"
        want = parts.T[col] + np.float32(0.0)
        if name == "wgate":
            want = want + w["ape"][(np.arange(m) % seqlen) % ratio]   # one f32 rounding, as on the GPU
        got = kv if name == "wkv" else sc
        bad = got.view(np.uint32) != want.view(np.uint32)
        assert not bad.any(), f"{name}: {bad.sum()} differ, e.g. {want[bad][:4]} -> {got[bad][:4]}"


@pytest.mark.parametrize("fused", [False, True])
def test_f16_split_rows_of_any_scale(fused):
    """x rows and weight rows with scales 2^-60 .. 2^60 (N(0,1) values times
    the row's power of two) through the plain kernel (projections inside the
    f32 bound of the GEMM tests), and x rows of 2^-4 .. 2^4 with weight rows
    of 2^-10 .. 2^10 through the pooling kernel (sampled entries inside the
    pooled tolerance): each row's own exponent scales it into the f16 range
    and back."""
    note(f"f16 split wide row scales fused={fused}")
    from gpu_util import weights
    rng = np.random.default_rng(5 + fused)
    ratio, batch = 4, 1
    hd, dim, seqlen = (512, 64, 16384 + 5) if fused else (128, 256, 300)
    cfg = kvc.Config(ratio, hd, dim, projection=kvc.KVC_PROJ_F16_SPLIT)
    proj = kvc.kvc_proj_width(cfg)
    m = batch * seqlen
    # the pooled check needs gate logits of moderate size (a softmax over
    # logits of size 2^60 turns on their last bits): narrower scales there
    xs, ws_ = (4, 10) if fused else (60, 60)
    x = (rng.standard_normal((m, dim)) * np.exp2(rng.integers(-xs, xs, (m, 1)))).astype(np.float32)
    x[3] = 0.0   # a row of zeros keeps exponent 0
    if not fused:  # a row of f32 subnormals: exponent above 127, results scaled back into the subnormal range
        x[5] = (rng.standard_normal(dim) * 2.0 ** -135).astype(np.float32)
    w = {"wkv": (rng.standard_normal((proj, dim)) * np.exp2(rng.integers(-ws_, ws_, (proj, 1)))).astype(np.float32),
         "wgate": (rng.standard_normal((proj, dim)) * 0.02).astype(np.float32),
         "ape": (rng.standard_normal((ratio, proj)) * 0.1).astype(np.float32)}
    xd = dev(x.reshape(batch, seqlen, dim))
    ws = torch.empty(kvc.kvc_prefill_workspace_floats(cfg, batch, seqlen), dtype=torch.float32, device="cuda")
    kvc.compressor_prefill(cfg, weights(w), xd, batch, seqlen, ws)
    torch.cuda.synchronize()
    rows = np.arange(m) if m <= 4096 else np.unique(np.concatenate([np.arange(300), rng.choice(m, 700)]))
    for plane, name in ((0, "wkv"), (1, "wgate")):
        got = ws[plane * m * proj:(plane + 1) * m * proj].view(m, proj).cpu().numpy()[rows].astype(np.float64)
        ref = oracle.project(x[rows], w[name])
        if name == "wgate":
            ref = oracle.add_bias(ref[None], w["ape"], rows % seqlen, ratio)[0]
        absdot = np.abs(x[rows]).astype(np.float64) @ np.abs(w[name]).astype(np.float64).T
        bound = dim * 2.0 ** -24 * absdot + np.spacing(np.abs(ref)) + 1e-300
        err = np.abs(got - ref)
        assert np.all(err <= bound), f"{name}: {np.sum(err > bound)} beyond the bound, worst {np.max(err / bound):.3g}"
    if fused:
        groups = seqlen // ratio
        out = kvc.new_outputs(cfg, batch, groups, latent=True, pooled=True)
        kvc.compressor_prefill(cfg, weights(w), xd, batch, seqlen, ws, None, None, out)
        torch.cuda.synchronize()
        pooled = out.pooled.cpu().numpy()
        ent = np.array(sorted(set([0, 1, 63, 64, 65, groups - 1]) | set(rng.choice(groups, 40).tolist())))
        ocfg = oracle_cfg(cfg)
        ref = oracle.prefill(ocfg, oracle_weights(w), oracle.State(ocfg, 1), x=x.reshape(batch, seqlen, dim),
                             quantize=False, entries=ent)
        check_pooled(pooled[0][ent], ref["pooled"][0])


@pytest.mark.parametrize("ratio,hd,dim,batch,seqlen", SPLIT_CASES)
def test_f16_split_of_f32_rows_is_the_two_part_sum(ratio, hd, dim, batch, seqlen):
    """x rows v_r e_(r mod dim) (v_r any f32 of scale 2^-40 .. 2^40) with
    weights that are powers of two (their low parts zero): each output is
    then (h + l) w of x's two f16 parts scaled back, every step exact, so it
    must equal that value bit for bit, and lie within 2^-22 relative of the
    exact v_r w. This pins the split the kernel does in registers."""
    note(f"f16 split of x rows ratio={ratio} hd={hd} dim={dim} batch={batch} seqlen={seqlen}")
    from gpu_util import weights
    rng = np.random.default_rng(23 + ratio + dim)
    cfg = kvc.Config(ratio, hd, dim, projection=kvc.KVC_PROJ_F16_SPLIT)
    proj = kvc.kvc_proj_width(cfg)
    m = batch * seqlen
    v = (rng.standard_normal(m) * np.exp2(rng.integers(-40, 40, m))).astype(np.float32)
    v[:3] = [1 + 2.0 ** -23, -(2.0 ** -30) * (1 + 2.0 ** -11 + 2.0 ** -23), 0.0]
    x = np.zeros((m, dim), np.float32)
    x[np.arange(m), np.arange(m) % dim] = v
    pow2 = lambda: (rng.choice([-1.0, 1.0], (proj, dim)) * np.exp2(rng.integers(-8, 1, (proj, dim)))).astype(np.float32)  # noqa: E731
    w = {"wkv": pow2(), "wgate": pow2()}
    ws = torch.full((kvc.kvc_prefill_workspace_floats(cfg, batch, seqlen),), float("nan"), device="cuda")
    kvc.compressor_prefill(cfg, weights(w), dev(x.reshape(batch, seqlen, dim)), batch, seqlen, ws)
    torch.cuda.synchronize()
    xs = _f16_parts_sum(v[:, None])[:, 0]           # x's two parts, scaled back
    rel = np.abs(xs.astype(np.float64) - v) / np.maximum(np.abs(v).astype(np.float64), 1e-300)
    assert rel.max() <= 2.0 ** -22
    col = np.arange(m) % dim
    for plane, name in ((0, "wkv"), (1, "wgate")):
        got = ws[plane * m * proj:(plane + 1) * m * proj].view(m, proj).cpu().numpy()
        want = (xs[:, None] * w[name].T[col]).astype(np.float32) + np.float32(0.0)  # exact: times a power of two
        bad = got.view(np.uint32) != want.view(np.uint32)
        assert not bad.any(), f"{name}: {bad.sum()} differ, e.g. {want[bad][:4]} -> {got[bad][:4]}"


@pytest.mark.parametrize("batch,dim,hd", [(70, 2048, 128), (5, 4096, 512), (33, 1536, 512)])
def test_decode_projection_tiles(batch, dim, hd):
    """Decode from f32 rows: batches that are not a multiple of the 32-row
    tile (70: three row tiles; 5; 33), k segments of 16, 32 and 12 stages of
    64 k; the emitted entries and the carried state against the oracle over
    the same tokens, and bit for bit against the GPU prefill."""
    note(f"decode projection tiles batch={batch} dim={dim} hd={hd}")
    from gpu_util import weights
    rng = np.random.default_rng(batch + dim + hd)
    cfg = kvc.Config(4, hd, dim)
    proj = kvc.kvc_proj_width(cfg)
    steps = 6
    x = rng.standard_normal((batch, steps, dim), dtype=np.float32)
    w = {"wkv": rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.02),
         "wgate": rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.02),
         "ape": rng.standard_normal((4, proj), dtype=np.float32) * np.float32(0.1)}
    dec = _decode_gpu(cfg, weights(w), batch, xs=x)
    st = oracle.State(oracle_cfg(cfg), batch)
    ref = oracle.prefill(oracle_cfg(cfg), oracle_weights(w), st, x=x, quantize=True)
    check_pooled(dec["pooled"], ref["pooled"])
    check_latent(dec["latent"], dec["pooled"], ref["latent"], ref["pooled"])
    # the carry after 6 tokens: the previous block (rows 0..3) and 2 current rows
    live = _live_rows(4, steps)
    fin = np.isfinite(st.score[:, live])
    assert np.array_equal(np.isfinite(dec["state_sc"][:, live]), fin)
    check_pooled(dec["state_kv"][:, live], st.kv[:, live], "state kv")
    check_pooled(np.where(fin, dec["state_sc"][:, live], 0), np.where(fin, st.score[:, live], 0), "state score")
    full = prefill(cfg, w, batch, steps, x=x)
    for k in ("pooled", "latent", "codes", "scales"):
        assert np.array_equal(dec[k].view(np.uint8), full[k].view(np.uint8)), k
    assert np.array_equal(dec["state_kv"][:, live].view(np.uint32), full["state_kv"][:, live].view(np.uint32))
    assert np.array_equal(dec["state_sc"][:, live].view(np.uint32), full["state_sc"][:, live].view(np.uint32))


# ratio, head_dim, dim, batch, steps: k segments of whole 64-k stages (dim %
# 128 == 0), of 32-k stages (segments 64 and 96 at dim 160, 224 and 256 at
# dim 480, 32 and 64 at dim 96), one segment (dim 32), ragged batches, every
# ratio
DECODE_BITWISE_CASES = [
    (4, 512, 4096, 64, 12),
    (4, 128, 160, 5, 9),
    (2, 512, 32, 3, 6),
    (128, 128, 256, 2, 130),
    (4, 512, 480, 33, 8),
    (2, 128, 1024, 97, 5),
    (4, 128, 96, 70, 6),
    (4, 512, 256, 256, 6),   # eight 32-row tiles
]


@pytest.mark.parametrize("ratio,hd,dim,batch,steps", DECODE_BITWISE_CASES)
def test_decode_equals_prefill_bitwise_from_x(ratio, hd, dim, batch, steps):
    """From f32 hidden states a decode step sums each projection exactly as
    the prefill's f32 matrix cores do (two k segments, the same MFMA order,
    p0 + p1), so a decode stream and a prefill over the same tokens write the
    same bits: entries, fp4 codes and the carried state. Also a
    continuation: prefill of the first tokens, decode of the rest."""
    note(f"decode == prefill bitwise from x ratio={ratio} hd={hd} dim={dim} batch={batch} steps={steps}")
    from gpu_util import weights
    rng = np.random.default_rng(ratio * 7 + hd + dim + batch)
    cfg = kvc.Config(ratio, hd, dim)
    proj = kvc.kvc_proj_width(cfg)
    x = rng.standard_normal((batch, steps, dim), dtype=np.float32)
    w = {"wkv": rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.05),
         "wgate": rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.05),
         "ape": rng.standard_normal((ratio, proj), dtype=np.float32) * np.float32(0.1)}
    dec = _decode_gpu(cfg, weights(w), batch, xs=x)
    full = prefill(cfg, w, batch, steps, x=x)
    live = _live_rows(ratio, steps)
    if steps >= ratio:
        for k in ("pooled", "latent", "codes", "scales", "dequant"):
            assert np.array_equal(dec[k].view(np.uint8), full[k].view(np.uint8)), k
    assert np.array_equal(dec["state_kv"][:, live].view(np.uint32), full["state_kv"][:, live].view(np.uint32))
    assert np.array_equal(dec["state_sc"][:, live].view(np.uint32), full["state_sc"][:, live].view(np.uint32))
    # prefill of n0 tokens, then decode: the same entries as the full prefill
    n0 = steps // 2 + 1
    state = kvc.new_state(cfg, batch)
    first = prefill(cfg, w, batch, n0, x=x[:, :n0], state=state)
    rest = _decode_gpu(cfg, weights(w), batch, xs=x[:, n0:], start=n0, state=state)
    parts = [p for p in (first.get("latent"), rest.get("latent")) if p is not None]
    if parts:
        got = np.concatenate(parts, axis=1)
        assert np.array_equal(got.view(np.uint16), full["latent"].view(np.uint16))
    assert np.array_equal(rest["state_kv"][:, live].view(np.uint32), full["state_kv"][:, live].view(np.uint32))


def test_decode_workspace_counters_rest_at_zero_and_a_dirty_one_poisons():
    """The decode workspace's arrival counters are zero after every step (so
    any number of steps and graph replays can share it); a workspace that was
    not zero-filled makes the affected state rows NaN instead of silently
    wrong values, and once it is zero-filled again the steps are correct."""
    note("decode arrival counters")
    from gpu_util import weights
    rng = np.random.default_rng(17)
    cfg = kvc.Config(4, 128, 256)
    batch, proj = 40, 256
    w = {"wkv": rng.standard_normal((proj, 256), dtype=np.float32) * np.float32(0.05),
         "wgate": rng.standard_normal((proj, 256), dtype=np.float32) * np.float32(0.05)}
    x = dev(rng.standard_normal((3, batch, 256), dtype=np.float32))
    ws = kvc.new_decode_workspace(cfg, batch)
    tiles = ((batch + 31) // 32) * (2 * proj // 32)
    counters = ws[-((tiles + 63) // 64 * 64):]
    st = kvc.new_state(cfg, batch)
    kvc.compressor_decode_step(cfg, weights(w), x[0], batch, 0, ws, st[0], st[1])
    torch.cuda.synchronize()
    assert torch.all(counters.view(torch.int32) == 0).item()
    good = st[0][:, 4].clone()
    assert torch.isfinite(good).all().item()
    # a dirty counter (tile 0: batch rows 0..31, kv columns 0..31)
    counters.view(torch.int32)[0] = 9
    kvc.compressor_decode_step(cfg, weights(w), x[0], batch, 0, ws, st[0], st[1])
    torch.cuda.synchronize()
    assert torch.isnan(st[0][:32, 4, :32]).all().item()
    assert torch.equal(st[0][:, 4, 32:], good[:, 32:]) and torch.equal(st[0][32:, 4], good[32:])
    ws.zero_()
    kvc.compressor_decode_step(cfg, weights(w), x[0], batch, 0, ws, st[0], st[1])
    torch.cuda.synchronize()
    assert torch.equal(st[0][:, 4], good)
