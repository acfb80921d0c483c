"""Helpers of the GPU tests: run the HIP library through its binding on NumPy
inputs and bring the results back as NumPy arrays. No arithmetic of the
method happens here."""
from __future__ import annotations

import sys

import numpy as np
import torch

import kv_cache_compression_fp32_amd.kvc as kvc
import oracle


def note(msg: str) -> None:
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def dev(a: np.ndarray | None) -> torch.Tensor | None:
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_inputs(a: np.ndarray) -> np.ndarray:
    """Hidden states as the model holds them: the bf16 rounding of `a`
    (torch's conversion), returned as float32 values."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).float().numpy()


def dev_x(cfg: kvc.Config, x: np.ndarray | None) -> torch.Tensor | None:
    """x on the GPU in the element type cfg.x_format names (bf16 x must hold
    bf16 values already: the conversion is then exact)."""
    if x is None:
        return None
    t = dev(x)
    if cfg.x_format == kvc.KVC_X_BF16:
        b = t.to(torch.bfloat16)
        assert torch.equal(b.float(), t), "x is not bf16-valued"
        return b
    return t


def host_bf16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> float32 NumPy array of the same values."""
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return oracle.bf16_from_bits(bits)


def weights(w: dict) -> kvc.Weights:
    return kvc.Weights(wkv=dev(w.get("wkv")), wgate=dev(w.get("wgate")), ape=dev(w.get("ape")),
                       norm_w=dev(w.get("norm_w")), rope_cs=dev(w.get("rope_cs")))


def outputs_to_host(o: kvc.Outputs) -> dict:
    res = {}
    if o.latent is not None:
        res["latent"] = host_bf16(o.latent)
    if o.pooled is not None:
        res["pooled"] = o.pooled.cpu().numpy()
    if o.codes is not None:
        res["codes"] = o.codes.cpu().numpy()
        res["scales"] = o.scales.cpu().numpy()
    if o.dequant is not None:
        res["dequant"] = host_bf16(o.dequant)
    if o.rotated is not None:
        res["rotated"] = host_bf16(o.rotated)
    return res


def prefill(cfg: kvc.Config, w: dict, batch: int, seqlen: int, x=None, kv=None, sc=None,
            fp4=True, state=None, x_dev=None) -> dict:
    """GPU prefill. x (NumPy or x_dev) or given projections kv/sc. `state`
    (a (kv, sc) pair of device tensors) is updated in place when given."""
    proj = kvc.kvc_proj_width(cfg)
    ws = torch.empty(kvc.kvc_prefill_workspace_floats(cfg, batch, seqlen), dtype=torch.float32, device="cuda")
    if x is None and x_dev is None:
        m = batch * seqlen * proj
        ws[:m] = dev(kv).reshape(-1)
        ws[m:2 * m] = dev(sc).reshape(-1)
    xd = x_dev if x_dev is not None else dev_x(cfg, x)
    if state is None:
        state = kvc.new_state(cfg, batch)
    groups = seqlen // cfg.ratio
    out = kvc.new_outputs(cfg, batch, groups, latent=True, pooled=True, fp4=fp4, dequant=fp4,
                          rotated=cfg.rope_dim > 0)
    n = kvc.compressor_prefill(cfg, weights(w), xd, batch, seqlen, ws, state[0], state[1], out)
    torch.cuda.synchronize()
    res = outputs_to_host(out) if groups > 0 else {}
    res["n_groups"] = n
    res["state_kv"] = state[0].cpu().numpy()
    res["state_sc"] = state[1].cpu().numpy()
    res["proj_kv"] = ws[:batch * seqlen * proj].reshape(batch, seqlen, proj).cpu().numpy()
    res["proj_sc"] = ws[batch * seqlen * proj:2 * batch * seqlen * proj].reshape(batch, seqlen, proj).cpu().numpy()
    return res


def oracle_cfg(cfg: kvc.Config) -> oracle.Config:
    return oracle.Config(ratio=cfg.ratio, head_dim=cfg.head_dim, dim=cfg.dim, eps=cfg.eps,
                         fp4="e8m0" if cfg.fp4_format == kvc.KVC_FP4_E8M0_B32 else "e4m3", rope_dim=cfg.rope_dim)


def oracle_weights(w: dict) -> oracle.Weights:
    return oracle.Weights(wkv=w.get("wkv"), wgate=w.get("wgate"), ape=w.get("ape"), norm_w=w.get("norm_w"),
                          rope_cs=w.get("rope_cs"))
