"""GPU parity at the five workload sizes, in the launch configuration the
benchmark times. Where the oracle cannot compute everything in seconds, it
computes sampled entries one by one from the token rows they depend on."""
import functools

import numpy as np
import pytest
import torch

import kv_cache_compression_fp32_amd.kvc as kvc
import kv_cache_compression_fp32_amd.workloads as W
import oracle
from gpu_util import bf16_inputs, dev, dev_x, note, oracle_cfg, oracle_weights, outputs_to_host, prefill, weights
from parity import check_fp4, check_latent, check_pooled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvc.lib()


def _cfg(wl, comp, x_format=kvc.KVC_X_F32, projection=kvc.KVC_PROJ_AUTO):
    return kvc.Config(comp.ratio, comp.head_dim, wl.dim, wl.eps, x_format=x_format, projection=projection)


def _sample_entries(groups, n=24, seed=0):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, 2, groups // 2, groups - 2, groups - 1}
    rand = set(rng.choice(groups, size=min(n, groups), replace=False).tolist())
    return sorted(e for e in fixed | rand if 0 <= e < groups)


def _oracle_entry(wl, comp, w, b, j, fp4="e4m3", x_bf16=False):
    """One entry from only the token rows it depends on: ratio 4 needs the
    previous block too (the slice then starts at a multiple of 4, so the bias
    rows line up), other ratios only the group itself. With x_bf16 the rows
    are the bf16 hidden states the GPU received."""
    cfg = oracle.Config(comp.ratio, comp.head_dim, wl.dim, wl.eps, fp4=fp4)
    r = comp.ratio
    if r == 4 and j > 0:
        t0, idx = r * (j - 1), 1
    else:
        t0, idx = r * j, 0
    x = W.hidden_rows(wl, b, t0, r * j + r)[None]
    if x_bf16:
        x = bf16_inputs(x)
    out = oracle.prefill(cfg, oracle_weights(w), oracle.State(cfg, 1), x=x, quantize=comp.quantize or fp4 == "e8m0")
    return {k: v[0, idx] for k, v in out.items()}


def _check_sampled(wl, comp, w, got, entries, batch_rows, fp4="e4m3", x_bf16=False):
    ref = {}
    for b in batch_rows:
        for j in entries:
            e = _oracle_entry(wl, comp, w, b, j, fp4, x_bf16)
            for k, v in e.items():
                ref.setdefault(k, []).append(v)
    ref = {k: np.stack(v) for k, v in ref.items()}
    sel = lambda a: np.stack([a[b, j] for b in batch_rows for j in entries])  # noqa: E731
    worst = check_pooled(sel(got["pooled"]), ref["pooled"])
    flips, total = check_latent(sel(got["latent"]), sel(got["pooled"]), ref["latent"], ref["pooled"], eps=wl.eps)
    note(f"    pooled worst {worst:.2e} of the entry's scale; latent bf16 flips {flips} of {total}")
    if comp.quantize or fp4 == "e8m0":
        check_fp4(sel(got["codes"]), sel(got["scales"]), sel(got["latent"]), ref["codes"], ref["scales"],
                  ref["latent"], sel(got["dequant"]), e8m0=fp4 == "e8m0")


def test_pair_pool_r2_full():
    wl = W.WORKLOADS["pair_pool_r2"]
    comp = wl.compressors[0]
    note(f"{wl.name}")
    kc, gc = W.given_projections(wl)
    cfg = _cfg(wl, comp)
    g = prefill(cfg, {}, wl.batch, wl.seqlen, kv=kc, sc=gc, fp4=False)
    ref = oracle.prefill(oracle_cfg(cfg), oracle.Weights(), oracle.State(oracle_cfg(cfg), wl.batch), kv=kc,
                         score=gc)
    assert g["latent"].shape == (1, 32, 512)
    worst = check_pooled(g["pooled"], ref["pooled"])
    flips, total = check_latent(g["latent"], g["pooled"], ref["latent"], ref["pooled"], eps=wl.eps)
    note(f"    every entry: pooled worst {worst:.2e} of the entry's scale; latent bf16 flips {flips} of {total}")


@functools.lru_cache(maxsize=1)
def _oracle_r4_n4096():
    wl = W.WORKLOADS["prefill_r4_n4096"]
    cfg = oracle.Config(4, 512, wl.dim, wl.eps)
    w = W.weights(wl, wl.compressors[0])
    return oracle.prefill(cfg, oracle_weights(w), oracle.State(cfg, wl.batch), x=W.hidden(wl), quantize=True)


# the f32 matrix cores (the default for f32 x) and the two opt-in emulations
@pytest.mark.parametrize("projection", [kvc.KVC_PROJ_F32_MFMA, kvc.KVC_PROJ_F16_SPLIT, kvc.KVC_PROJ_BF16_SPLIT])
def test_prefill_r4_n4096_full_oracle(projection):
    wl = W.WORKLOADS["prefill_r4_n4096"]
    comp = wl.compressors[0]
    note(f"{wl.name} projection={projection}")
    w = W.weights(wl, comp)
    x = W.hidden(wl)
    cfg = _cfg(wl, comp, projection=projection)
    g = prefill(cfg, w, wl.batch, wl.seqlen, x=x, fp4=True)
    ref = _oracle_r4_n4096()
    assert g["n_groups"] == 1024
    worst = check_pooled(g["pooled"], ref["pooled"])
    flips, total = check_latent(g["latent"], g["pooled"], ref["latent"], ref["pooled"], eps=wl.eps)
    differ, blocks = check_fp4(g["codes"], g["scales"], g["latent"], ref["codes"], ref["scales"], ref["latent"],
                               g["dequant"])
    note(f"    every entry: pooled worst {worst:.2e} of the entry's scale; latent bf16 flips {flips} of {total}; "
         f"fp4 blocks with a differing latent {differ} of {blocks}")


@pytest.mark.parametrize("projection", [kvc.KVC_PROJ_F32_MFMA])
@pytest.mark.parametrize("seqlen", [16384, 16384 + 37])
def test_prefill_r128_sampled(seqlen, projection):
    wl = W.scaled(W.WORKLOADS["prefill_r128_b2_n16384"], seqlen=seqlen)
    comp = wl.compressors[0]
    note(f"{wl.name} seqlen={seqlen} projection={projection}")
    w = W.weights(wl, comp)
    cfg = _cfg(wl, comp, projection=projection)
    g = prefill(cfg, w, wl.batch, wl.seqlen, x_dev=dev(W.hidden(wl)), fp4=True)
    groups = seqlen // 128
    assert g["n_groups"] == groups
    # 64 random entries of the 128 of each batch row, plus the first and last ones
    _check_sampled(wl, comp, w, g, _sample_entries(groups, 64), range(wl.batch))
    # the carried tail: rows [0, seqlen mod 128) are the last tokens' projections
    rem = seqlen % 128
    if rem:
        ocfg = oracle.Config(128, 512, wl.dim, wl.eps)
        for b in range(wl.batch):
            xt = W.hidden_rows(wl, b, groups * 128, seqlen)
            kv = oracle.project(xt, w["wkv"])
            sc = oracle.add_bias(oracle.project(xt, w["wgate"])[None], w["ape"], np.arange(rem), 128)[0]
            check_pooled(g["state_kv"][b, :rem], kv, "state kv")
            check_pooled(g["state_sc"][b, :rem], sc, "state score")
        del ocfg
    assert np.all(g["state_kv"][:, rem:] == 0) and np.all(np.isneginf(g["state_sc"][:, rem:]))


def test_decode_r4_b64_s512_equals_prefill():
    wl = W.WORKLOADS["decode_r4_b64_s512"]
    comp = wl.compressors[0]
    note(f"{wl.name}")
    w = W.weights(wl, comp)
    cfg = _cfg(wl, comp)
    x = W.hidden(wl)
    xd = dev(x)
    full = prefill(cfg, w, wl.batch, wl.seqlen, x_dev=xd, fp4=True)
    wts = weights(w)
    ws = kvc.new_decode_workspace(cfg, wl.batch)
    state = kvc.new_state(cfg, wl.batch)
    outs = []
    for p in range(wl.seqlen):
        out = kvc.new_outputs(cfg, wl.batch, 1, latent=True, pooled=True, fp4=True, dequant=True)
        e = kvc.compressor_decode_step(cfg, wts, xd[:, p].contiguous(), wl.batch, p, ws, state[0], state[1], out)
        assert e == (p > 0 and (p + 1) % 4 == 0)
        if e:
            outs.append(out)
    torch.cuda.synchronize()
    assert len(outs) == 128
    hs = [outputs_to_host(o) for o in outs]
    dec = {k: np.concatenate([h[k] for h in hs], axis=1) for k in hs[0]}
    # decode sums each projection as the prefill's f32 matrix cores do: all
    # 64 rows x 128 entries bit for bit, and the carried state
    for k in ("pooled", "latent", "codes", "scales", "dequant"):
        assert np.array_equal(dec[k].view(np.uint8), full[k].view(np.uint8)), k
    st_kv, st_sc = state[0].cpu().numpy(), state[1].cpu().numpy()
    assert np.array_equal(st_kv[:, :4].view(np.uint32), full["state_kv"][:, :4].view(np.uint32))
    assert np.array_equal(st_sc[:, :4].view(np.uint32), full["state_sc"][:, :4].view(np.uint32))
    # and 16 of the 64 rows, every entry, against the oracle
    ocfg = oracle_cfg(cfg)
    rows = sorted(set([0, 31, 32, 63]) | set(np.random.default_rng(4).choice(64, 12, replace=False).tolist()))
    assert len(rows) >= 16
    flips = total = differ = blocks = 0
    worst = 0.0
    for b in rows:
        ref = oracle.prefill(ocfg, oracle_weights(w), oracle.State(ocfg, 1), x=x[b:b + 1], quantize=True)
        worst = max(worst, check_pooled(dec["pooled"][b:b + 1], ref["pooled"]))
        f, t = check_latent(dec["latent"][b:b + 1], dec["pooled"][b:b + 1], ref["latent"], ref["pooled"], eps=wl.eps)
        d, n = check_fp4(dec["codes"][b], dec["scales"][b], dec["latent"][b], ref["codes"][0], ref["scales"][0],
                         ref["latent"][0], dec["dequant"][b])
        flips, total, differ, blocks = flips + f, total + t, differ + d, blocks + n
    note(f"    {len(rows)} rows x 128 entries: pooled worst {worst:.2e}; latent bf16 flips {flips} of {total}; "
         f"fp4 blocks with a differing latent {differ} of {blocks}")


@pytest.mark.parametrize("projection", [kvc.KVC_PROJ_BF16_SPLIT, kvc.KVC_PROJ_F32_MFMA, kvc.KVC_PROJ_F16_SPLIT])
def test_prefill_r4_n65536_fp4_idx128_sampled(projection):
    wl = W.WORKLOADS["prefill_r4_n65536_fp4_idx128"]
    note(f"{wl.name} projection={projection}")
    xd = dev(W.hidden(wl))
    for comp in wl.compressors:
        w = W.weights(wl, comp)
        cfg = _cfg(wl, comp, projection=projection)
        note(f"  compressor ratio={comp.ratio} hd={comp.head_dim} fp4={comp.quantize}")
        g = prefill(cfg, w, wl.batch, wl.seqlen, x_dev=xd, fp4=True)
        assert g["n_groups"] == 16384
        _check_sampled(wl, comp, w, g, _sample_entries(16384, 40), [0])
        if comp.quantize:
            # every entry: the fp4 codes of the GPU's latent, bit-exact
            check_fp4(g["codes"], g["scales"], g["latent"], gpu_dequant=g["dequant"])
        del g


def test_prefill_r4_n65536_bf16_hidden_states_sampled():
    # the long workload with the model's bf16 hidden states (the projection
    # on the bf16 matrix cores from the weights' three exact bf16 parts),
    # both compressors, fused pooling: the benchmark's launch configuration
    wl = W.WORKLOADS["prefill_r4_n65536_fp4_idx128"]
    note(f"{wl.name} bf16 x")
    for comp in wl.compressors:
        w = W.weights(wl, comp)
        cfg = _cfg(wl, comp, kvc.KVC_X_BF16)
        xd = dev_x(cfg, bf16_inputs(W.hidden(wl)))
        note(f"  compressor ratio={comp.ratio} hd={comp.head_dim} fp4={comp.quantize}")
        g = prefill(cfg, w, wl.batch, wl.seqlen, x_dev=xd, fp4=True)
        assert g["n_groups"] == 16384
        _check_sampled(wl, comp, w, g, _sample_entries(16384, 40, seed=2), [0], x_bf16=True)
        if comp.quantize:
            check_fp4(g["codes"], g["scales"], g["latent"], gpu_dequant=g["dequant"])
        del g, xd


def test_prefill_r4_n65536_index_keys_power_of_two_fp4_sampled():
    # the 128-wide indexer compressor of the long workload with its keys in
    # the indexer's fp4 form (power-of-two scales, blocks of 32), fused
    wl = W.WORKLOADS["prefill_r4_n65536_fp4_idx128"]
    comp = wl.compressors[1]
    assert comp.head_dim == 128
    note(f"{wl.name} indexer keys e8m0")
    xd = dev(W.hidden(wl))
    w = W.weights(wl, comp)
    cfg = kvc.Config(comp.ratio, comp.head_dim, wl.dim, wl.eps, fp4_format=kvc.KVC_FP4_E8M0_B32)
    g = prefill(cfg, w, wl.batch, wl.seqlen, x_dev=xd, fp4=True)
    assert g["scales"].shape == (1, 16384, 4)
    _check_sampled(wl, comp, w, g, _sample_entries(16384, 40, seed=1), [0], fp4="e8m0")
    check_fp4(g["codes"], g["scales"], g["latent"], gpu_dequant=g["dequant"], e8m0=True)


def test_prefill_r1_n65536_sampled():
    # the ratio-1 compressor over the long sequence, in the benchmark's launch
    # configuration; tokens are independent, so sampled rows are checked
    wl = W.WORKLOADS["prefill_r1_n65536"]
    comp = wl.compressors[0]
    note(f"{wl.name}")
    cfg = kvc.Config(1, comp.head_dim, wl.dim, wl.eps)
    xt = torch.from_numpy(W.hidden(wl)[0]).cuda().to(torch.bfloat16)
    wt = torch.from_numpy(W.weights(wl, comp)["wkv"]).cuda().to(torch.bfloat16)
    tokens = wl.seqlen
    ws = torch.empty(kvc.kvc_ratio1_workspace_floats(cfg, tokens), dtype=torch.float32, device="cuda")
    out = kvc.new_outputs(cfg, 1, tokens, latent=True, pooled=True, fp4=True, dequant=True)
    kvc.compressor_ratio1_forward(cfg, wt, xt, tokens, ws, out)
    torch.cuda.synchronize()
    rows = np.array(_sample_entries(tokens, 200, seed=3) + list(range(tokens - 256, tokens - 200)))
    rows_t = torch.from_numpy(rows).cuda()
    x = xt[rows_t].float().cpu().numpy()
    wkv = wt.float().cpu().numpy()
    g = outputs_to_host(kvc.Outputs(latent=out.latent[0][rows_t], pooled=out.pooled[0][rows_t],
                                    codes=out.codes[0][rows_t], scales=out.scales[0][rows_t],
                                    dequant=out.dequant[0][rows_t]))
    ref = oracle.plain_projection(oracle.Config(ratio=1, head_dim=comp.head_dim, dim=wl.dim, eps=wl.eps),
                                  oracle.Weights(wkv=wkv), x, quantize=True)
    check_pooled(g["pooled"], ref["pooled"], "projection")
    check_latent(g["latent"], g["pooled"], ref["latent"], ref["pooled"], eps=wl.eps)
    check_fp4(g["codes"], g["scales"], g["latent"], ref["codes"], ref["scales"], ref["latent"], g["dequant"])
