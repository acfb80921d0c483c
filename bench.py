"""Benchmark of the compressor hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole path over one batch: for the default
workload (ratio-4 prefill of 65536 tokens, hidden 4096) that is the 512-wide
compressor (f32 projections, pooling + RMSNorm + fp4 cache codes) and the
128-wide indexer compressor (projections, pooling + RMSNorm, bf16 latent),
with the hidden states resident in HBM: x f32 [1, 65536, 4096] ~ N(0, 1). The
projections run on the f32 matrix cores (the library's default for f32 x).
Beside the headline (`workloads`): the same step on the library's opt-in
emulations of the f32 products on 16-bit matrix cores (each with its own
dtype label), from the model's bf16 hidden states, the other prefill
workloads, the decode stream, the standalone quantisers and the ratio-1
compressor. Prints one JSON line.

Timing: HIP events on the launch stream. Inside the timed steps the bench
records an event before and after each compressor call, and the library
records a pair right around its projection kernel (kvc_time_next_projection),
so the dominant kernel's duration in the roofline is that of the kernel the
step runs, measured live; the time before it (the split weights of an
emulation) and after it (the pooling epilogue kernels and the state store)
is reported per compressor. Reference launches of single stages (the plain
projection, the pooling of given projections) are timed before the warmup.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed KV entries/sec + achieved HBM GB/s, ratio-4 prefill N=65536"
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_16BIT_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 / f16 matrix
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
TRAFFIC_SOURCE = ("profiles/traffic.json: rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, of this benchmark's own "
                  "command, each scaled by the same counter on a 1 GiB copy kernel; null once the kernel's "
                  "sources differ from those the counters were taken on")
CSRC = "kv_cache_compression_fp32_amd/csrc/"
# the sources each counted kernel is built from (the traffic figures turn
# null as soon as any of them changes)
KERNEL_SOURCES = {
    "gemm_f32": [CSRC + f for f in ("gemm_common.h", "gemm_f32_kernel.h", "gemm_f32.hip", "kvc_device.h",
                                    "gemm_epilogue.h", "kvc_launch.h")],
    "decode_f32": [CSRC + f for f in ("gemm_common.h", "decode_f32.hip", "kvc_launch.h")],
    "pool": [CSRC + f for f in ("pool.hip", "kvc_device.h", "kvc_launch.h")],
}

# projection paths: (x format, projection, dtype label, description)
PATHS = {
    "f32-mfma": ("f32", "f32-mfma", "f32", "f32 rows, N(0,1); f32 matrix cores (the library's default)"),
    "f16-split": ("f32", "f16-split", "f16x3-split",
                  "f32 rows, N(0,1); opt-in emulation: rows of x and of the weights scaled by powers of two and "
                  "split into two f16 parts, three part products on the f16 matrix cores, f32 accumulation"),
    "bf16-split": ("f32", "bf16-split", "bf16x6-split",
                   "f32 rows, N(0,1); opt-in emulation: x and the weights split into three bf16 parts, six part "
                   "products on the bf16 matrix cores, f32 accumulation"),
    "x-bf16": ("bf16", "auto", "bf16x3-split",
               "bf16 rows (the bf16 rounding of the N(0,1) draws, the model's hidden-state type); the exact "
               "three-part bf16 split of the f32 weights on the bf16 matrix cores (exact products), f32 "
               "accumulation"),
}


def source_sha(name: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(key: str, sources: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel's sources changed since."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = data.get(key)
    if not entry or entry.get("source_sha") != source_sha(sources):
        return None
    return entry.get("bytes_per_launch")


def pool_bytes(batch, seqlen, ratio, hd, quantize, latent, block=16):
    """Algorithmic HBM bytes of one pooling launch: every projection value
    read once (kv and score planes), outputs written once."""
    proj = 2 * hd if ratio == 4 else hd
    groups = seqlen // ratio
    read = 2 * batch * groups * ratio * proj * 4
    write = 0
    if latent:
        write += batch * groups * hd * 2
    if quantize:
        write += batch * groups * (hd // 2 + hd // block)
    return read + write


def post_projection_bytes(batch, seqlen, hd, quantize):
    """Algorithmic bytes of the kernels after the fused ratio-4 projection:
    the row tiles' first entries (8 candidate rows of both planes read, the
    pooled entry written), the per-entry epilogue (pooled f32 entries read,
    the outputs written) and the state store (the last block's rows of both
    planes read and written)."""
    proj, groups = 2 * hd, seqlen // 4
    tiles = (batch * seqlen + 255) // 256
    boundary = (tiles - 1) * (8 * hd * 2 * 4 + hd * 4)
    out = batch * groups * ((hd // 2 + hd // 16) if quantize else hd * 2)
    finish = batch * groups * hd * 4 + out
    state = batch * 4 * proj * 2 * 4 * 2
    return boundary + finish + state


def bf16_hidden(torch, x: np.ndarray) -> np.ndarray:
    """The bf16 rounding of synthetic hidden states (torch's conversion), as
    float32 values."""
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(wl, W, seconds=10.0, x_bf16=False):
    """The oracle, as it stands, on the first tokens of the workload: doubles
    the sample until it takes `seconds` or covers the whole sequence."""
    import torch
    import oracle
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        pass
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    tokens = 512
    while True:
        x = np.stack([W.hidden_rows(wl, b, 0, tokens) for b in range(wl.batch)])
        if x_bf16:
            x = bf16_hidden(torch, x)
        t0 = time.perf_counter()
        entries = 0
        for comp in wl.compressors:
            w = W.weights(wl, comp)
            cfg = oracle.Config(comp.ratio, comp.head_dim, wl.dim, wl.eps)
            out = oracle.prefill(cfg, oracle.Weights(w["wkv"], w["wgate"], w["ape"]), oracle.State(cfg, wl.batch),
                                 x=x, quantize=comp.quantize)
            entries = max(entries, out["latent"].shape[0] * out["latent"].shape[1])
        dt = time.perf_counter() - t0
        if dt >= seconds or tokens >= wl.seqlen:
            break
        tokens = min(2 * tokens, wl.seqlen)
    return {"value": round(entries / dt, 1), "unit": "entries/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "blas_threads": threads,
            "blas": ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in blas) or "none found",
            "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"first {tokens} tokens of each of {wl.batch} batch rows through all "
                      f"{len(wl.compressors)} compressor(s) of the workload ({entries} entries, {dt:.2f} s; "
                      f"float64 NumPy, the projection a BLAS matmul on {threads} threads, the rest one thread)"}


def _timed(torch, stream, fn, reps):
    """Average time of `reps` back-to-back calls of `fn`. The calls are
    queued behind a GPU sleep, so that the host-side cost of a call (the
    binding's checks, ctypes) never leaves the GPU idle between launches."""
    fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e8))
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _events(torch, stream, n):
    """n timing events that exist (recorded once), so that their handles can
    be handed to the library."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record(stream)
    torch.cuda.synchronize()
    return ev


def _kernel_ms(torch, kvc, stream, fn, reps):
    """Average duration of the projection kernel of `fn` (one library call),
    from the library's own events around it."""
    fn()
    ev = _events(torch, stream, 2 * reps)
    for r in range(reps):
        kvc.time_next_projection(ev[2 * r], ev[2 * r + 1])
        fn()
    torch.cuda.synchronize()
    return sum(ev[2 * r].elapsed_time(ev[2 * r + 1]) for r in range(reps)) / reps


def _cold_ms(torch, stream, fn, reps):
    """Average duration of single launches of `fn`, each after a 1 GiB read
    that evicts its inputs from the caches (a true HBM measurement even
    where the inputs would fit in the 256 MB last-level cache; a read leaves
    no dirty lines whose write-back the launch would pay for)."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    fn()
    ev = _events(torch, stream, 2 * reps)
    for r in range(reps):
        flush.sum()
        ev[2 * r].record(stream)
        fn()
        ev[2 * r + 1].record(stream)
    torch.cuda.synchronize()
    del flush
    return sum(ev[2 * r].elapsed_time(ev[2 * r + 1]) for r in range(reps)) / reps


def x_format_of(kvc, name):
    return kvc.KVC_X_BF16 if name == "bf16" else kvc.KVC_X_F32


def projection_of(kvc, name):
    return {"auto": kvc.KVC_PROJ_AUTO, "f32-mfma": kvc.KVC_PROJ_F32_MFMA, "f16-split": kvc.KVC_PROJ_F16_SPLIT,
            "bf16-split": kvc.KVC_PROJ_BF16_SPLIT}[name]


def resolved(kvc, x_format, projection):
    """The projection the library runs for KVC_PROJ_AUTO."""
    if projection != kvc.KVC_PROJ_AUTO:
        return projection
    return kvc.KVC_PROJ_F32_MFMA if x_format == kvc.KVC_X_F32 else kvc.KVC_PROJ_BF16_SPLIT


def mfma_passes(kvc, x_format, projection):
    """16-bit matrix-core passes per f32 product (bf16 or f16, both at the
    same peak; 0: the f32 matrix cores)."""
    projection = resolved(kvc, x_format, projection)
    if projection == kvc.KVC_PROJ_F32_MFMA:
        return 0
    if projection == kvc.KVC_PROJ_F16_SPLIT:
        return 3
    return 3 if x_format == kvc.KVC_X_BF16 else 6


def gemm_kernel_name(kvc, x_format, projection, fused):
    p = resolved(kvc, x_format, projection)
    if p == kvc.KVC_PROJ_F32_MFMA:
        return f"gemm_f32_kernel<256, 256, 64, 128, 8, 1, true, {'true' if fused else 'false'}>"
    if p == kvc.KVC_PROJ_F16_SPLIT:
        return f"gemm_x6_kernel<{'true' if fused else 'false'}, true, 256, 128>"
    if x_format == kvc.KVC_X_BF16:
        return f"gemm_mc_kernel<256, 256, 128, 64, 8, 1, {'true' if fused else 'false'}, true>"
    return f"gemm_x6_kernel<{'true' if fused else 'false'}, false, 128, 64>"


def gemm_roofline(kvc, ms, flop, x_format, projection, traffic):
    """Roofline object of the 512-wide projection kernel: on the f32 matrix
    cores its flops against the fp32 peak; an emulation's 16-bit part
    products against the 16-bit peak, with the f32-equivalent rate beside it."""
    passes = mfma_passes(kvc, x_format, projection)
    tflops = flop / ms / 1e9
    if passes:
        work = passes * flop
        return {"bound": "mfma", "achieved": round(work / ms / 1e9, 2), "peak": PEAK_16BIT_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(work / ms / 1e9 / PEAK_16BIT_MFMA_TFLOPS, 4),
                "traffic": None, "per_launch": work, "avg_ms": round(ms, 4),
                "work": f"{passes} 16-bit part products per f32 product",
                "f32_equivalent_tflops": round(tflops, 2)}
    return {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_FP32_MFMA_TFLOPS, 4), "traffic": traffic, "traffic_source": TRAFFIC_SOURCE,
            "per_launch": flop, "avg_ms": round(ms, 4)}


def _rounded(d):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}


def run_prefill(wl, steps, warmup, reps, torch, kvc, W, x_format, projection, cold_pool=False):
    """Reference launches of single stages, then W warmup steps and K timed
    steps of `wl` with the per-compressor breakdown. x is the workload's f32
    draws, or (x_format bf16) their bf16 rounding as bf16 rows."""
    dev = "cuda"
    print(f"[bench] {wl.name}: generating inputs (x_format {x_format}, projection {projection})",
          file=sys.stderr, flush=True)
    x = torch.from_numpy(W.hidden(wl)).to(dev)
    if x_format == kvc.KVC_X_BF16:
        x = x.to(torch.bfloat16)
    torch.cuda.synchronize()
    comps = []
    for comp in wl.compressors:
        cfg = kvc.Config(comp.ratio, comp.head_dim, wl.dim, wl.eps, x_format=x_format, projection=projection)
        w = {k: torch.from_numpy(v).to(dev) for k, v in W.weights(wl, comp).items()}
        wts = kvc.Weights(wkv=w["wkv"], wgate=w["wgate"], ape=w["ape"])
        groups = wl.seqlen // comp.ratio
        ws = torch.empty(kvc.kvc_prefill_workspace_floats(cfg, wl.batch, wl.seqlen), dtype=torch.float32,
                         device=dev)
        state = kvc.new_state(cfg, wl.batch)
        out = kvc.new_outputs(cfg, wl.batch, groups, latent=not comp.quantize, fp4=comp.quantize)
        comps.append((comp, cfg, wts, ws, state, out, groups))
    stream = torch.cuda.current_stream()

    def call(c):
        comp, cfg, wts, ws, state, out, groups = c
        kvc.compressor_prefill(cfg, wts, x, wl.batch, wl.seqlen, ws, state[0], state[1], out)

    # reference launches of single stages (also bring the clocks up)
    print(f"[bench] {wl.name}: single-stage launches", file=sys.stderr, flush=True)
    kernels = {}
    for comp, cfg, wts, ws, state, out, groups in comps:
        tag = f"hd{comp.head_dim}"
        proj = comp.proj
        flops = 2.0 * wl.batch * wl.seqlen * wl.dim * 2 * proj
        plain = lambda: kvc.compressor_prefill(cfg, wts, x, wl.batch, wl.seqlen, ws)  # noqa: E731
        plain_ms = _kernel_ms(torch, kvc, stream, plain, reps)
        kernels[f"gemm_{tag}_plain"] = {"ms": plain_ms, "tflops": flops / plain_ms / 1e9, "flop": flops,
                                        "note": "projection-only call: the GEMM without the pooling epilogue"}
        # ws now holds this compressor's projections, the bias in the score
        # plane: the separate pool kernel on them
        given = lambda: kvc.compressor_prefill(cfg, kvc.Weights(), None, wl.batch, wl.seqlen, ws,  # noqa: E731
                                               None, None, out)
        pool_ms = _timed(torch, stream, given, reps)
        pbytes = pool_bytes(wl.batch, wl.seqlen, comp.ratio, comp.head_dim, comp.quantize, not comp.quantize)
        kernels[f"pool_{tag}"] = {"ms": pool_ms, "gbps": pbytes / pool_ms / 1e6, "bytes": pbytes,
                                  "note": "pooling of given projections (the separate pool kernel), back-to-back "
                                          "launches"}
        if cold_pool:
            cold_ms = _cold_ms(torch, stream, given, reps)
            kernels[f"pool_{tag}_cold"] = {"ms": cold_ms, "gbps": pbytes / cold_ms / 1e6, "bytes": pbytes,
                                           "note": "the same launch, each after a 1 GiB read that evicts the "
                                                   "planes from every cache"}
        if comp.head_dim == 128 and not comp.quantize:
            # the same pooling with the index keys' fp4 form (power-of-two
            # scales, blocks of 32) fused in place of the bf16 latent
            cfg8 = kvc.Config(comp.ratio, comp.head_dim, wl.dim, wl.eps, fp4_format=kvc.KVC_FP4_E8M0_B32)
            out8 = kvc.new_outputs(cfg8, wl.batch, groups, latent=False, fp4=True)
            ms8 = _timed(torch, stream, lambda: kvc.compressor_prefill(cfg8, kvc.Weights(), None, wl.batch,
                                                                       wl.seqlen, ws, None, None, out8), reps)
            b8 = pool_bytes(wl.batch, wl.seqlen, comp.ratio, comp.head_dim, True, False, block=32)
            kernels[f"pool_{tag}_e8m0"] = {"ms": ms8, "gbps": b8 / ms8 / 1e6, "bytes": b8}
            del out8

    print(f"[bench] {wl.name}: {warmup} warmup + {steps} timed steps", file=sys.stderr, flush=True)
    for _ in range(warmup):
        for c in comps:
            call(c)
    torch.cuda.synchronize()
    nc = len(comps)
    ev = _events(torch, stream, 4 * nc * steps + 2)
    ev[-2].record(stream)
    for i in range(steps):
        for j, c in enumerate(comps):
            e = ev[4 * (i * nc + j):4 * (i * nc + j) + 4]
            e[0].record(stream)
            kvc.time_next_projection(e[1], e[2])
            call(c)
            e[3].record(stream)
    ev[-1].record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev[-2].elapsed_time(ev[-1]) / steps
    for j, c in enumerate(comps):
        tag = f"hd{c[0].head_dim}"
        parts = [ev[4 * (i * nc + j):4 * (i * nc + j) + 4] for i in range(steps)]
        gemm = sum(p[1].elapsed_time(p[2]) for p in parts) / steps
        pre = sum(p[0].elapsed_time(p[1]) for p in parts) / steps
        post = sum(p[2].elapsed_time(p[3]) for p in parts) / steps
        flops = 2.0 * wl.batch * wl.seqlen * wl.dim * 2 * c[0].proj
        kernels[f"gemm_{tag}"] = {"ms": gemm, "tflops": flops / gemm / 1e9, "flop": flops,
                                  "note": "the projection kernel of the timed steps (HIP events the library "
                                          "records around it)"}
        kernels[f"step_{tag}"] = {"before_projection_ms": pre, "projection_ms": gemm, "after_projection_ms": post}
    entries = comps[0][6] * wl.batch
    fused = [c[0].ratio == 4 and c[6] > 0 for c in comps]
    del comps, x
    torch.cuda.empty_cache()
    return {"ms_per_step": ms_per_step, "entries_per_step": entries,
            "entries_per_s": entries / (ms_per_step / 1e3), "kernels": kernels, "fused": fused}


def run_decode(wl, passes, torch, kvc, W, x_format):
    """Whole decode passes (every row streams all its tokens from start_pos
    0, one decode step per token), captured once in a HIP graph so that host
    launch overhead is not measured; then one eager pass behind a long sleep
    kernel (so the launches queue up) with the library's events around each
    step's projection kernel."""
    dev = "cuda"
    comp = wl.compressors[0]
    cfg = kvc.Config(comp.ratio, comp.head_dim, wl.dim, wl.eps, x_format=x_format)
    print(f"[bench] {wl.name}: generating inputs", file=sys.stderr, flush=True)
    x = torch.from_numpy(W.hidden(wl)).to(dev)
    if x_format == kvc.KVC_X_BF16:
        x = x.to(torch.bfloat16)
    x = x.transpose(0, 1).contiguous()  # [steps, batch, dim]
    w = {k: torch.from_numpy(v).to(dev) for k, v in W.weights(wl, comp).items()}
    wts = kvc.Weights(wkv=w["wkv"], wgate=w["wgate"], ape=w["ape"])
    ws = kvc.new_decode_workspace(cfg, wl.batch)
    state = kvc.new_state(cfg, wl.batch)
    groups = wl.seqlen // comp.ratio
    lat = torch.empty((groups, wl.batch, comp.head_dim), dtype=torch.bfloat16, device=dev)
    outs = [kvc.Outputs(latent=lat[e]) for e in range(groups)]
    stream = torch.cuda.current_stream()

    def one_pass(ev=None):
        e = 0
        for p in range(wl.seqlen):
            emits = p > 0 and (p + 1) % comp.ratio == 0
            if ev is not None:
                kvc.time_next_projection(ev[3 * p], ev[3 * p + 1])
            kvc.compressor_decode_step(cfg, wts, x[p], wl.batch, p, ws, state[0], state[1],
                                       outs[e] if emits else None)
            if ev is not None:
                ev[3 * p + 2].record(stream)
            e += emits

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: {passes} timed graph replays", file=sys.stderr, flush=True)
    ms = _timed(torch, stream, graph.replay, passes)
    ev = _events(torch, stream, 3 * wl.seqlen)
    torch.cuda._sleep(int(3e8))  # the queue fills while the GPU sleeps
    one_pass(ev)
    torch.cuda.synchronize()
    kern = [ev[3 * p].elapsed_time(ev[3 * p + 1]) for p in range(wl.seqlen)]
    after = [ev[3 * p + 1].elapsed_time(ev[3 * p + 2]) for p in range(wl.seqlen)]
    emit = [p for p in range(wl.seqlen) if p > 0 and (p + 1) % comp.ratio == 0]
    # the same steps repeated back to back (queued behind a sleep): a step
    # that completes no group (the projection kernel alone) and one that does
    # (the projection kernel, then the pooling of the state window)
    plain_ms = _timed(torch, stream, lambda: kvc.compressor_decode_step(
        cfg, wts, x[1], wl.batch, 1, ws, state[0], state[1], None), 256)
    emit_ms = _timed(torch, stream, lambda: kvc.compressor_decode_step(
        cfg, wts, x[comp.ratio - 1], wl.batch, comp.ratio - 1, ws, state[0], state[1], outs[0]), 256)
    proj = comp.proj
    flop_step = 2.0 * wl.batch * wl.dim * 2 * proj
    entries = wl.batch * groups
    kern_us = 1e3 * plain_ms
    del graph, x, outs, lat
    torch.cuda.empty_cache()
    return {"ms_per_pass": ms, "entries_per_pass": entries, "entries_per_s": entries / (ms / 1e3),
            "us_per_step": ms * 1e3 / wl.seqlen, "tflops": flop_step * wl.seqlen / ms / 1e9,
            "projection_kernel_us": kern_us,
            "projection_kernel": "decode_f32_kernel<32, 64, 4> (projection + state ingest)"
            if x_format == kvc.KVC_X_F32 else "decode_gemm_kernel<4, uint16_t> (projection)",
            "projection_kernel_timing": "a step that completes no group, repeated back to back (its one launch)",
            "projection_kernel_us_hook": 1e3 * sum(kern) / len(kern),
            "projection_roofline": {"bound": "mfma", "achieved": round(flop_step / kern_us / 1e6, 2),
                                    "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                                    "frac": round(flop_step / kern_us / 1e6 / PEAK_FP32_MFMA_TFLOPS, 4),
                                    "per_launch": flop_step},
            "emit_pool_us": 1e3 * (emit_ms - plain_ms),
            "emit_pool_timing": "a step that completes a group minus one that does not, both repeated back to back",
            "emit_pool_us_hook": 1e3 * sum(after[p] for p in emit) / max(1, len(emit)),
            "note": "ms_per_pass from graph replays; *_hook: one eager pass queued behind a sleep with the "
                    "library's events around each step's projection kernel (the events add their own latency)"}


def run_ratio1(wl, steps, warmup, reps, torch, kvc, W):
    """Time the ratio-1 compressor over the whole workload (every token one
    entry), then its projection alone."""
    comp = wl.compressors[0]
    cfg = kvc.Config(1, comp.head_dim, wl.dim, wl.eps)
    print(f"[bench] {wl.name}: generating inputs", file=sys.stderr, flush=True)
    tokens = wl.batch * wl.seqlen
    x = torch.from_numpy(W.hidden(wl).reshape(tokens, wl.dim)).cuda().to(torch.bfloat16)
    wkv = torch.from_numpy(W.weights(wl, comp)["wkv"]).cuda().to(torch.bfloat16)
    ws = torch.empty(kvc.kvc_ratio1_workspace_floats(cfg, tokens), dtype=torch.float32, device="cuda")
    out = kvc.new_outputs(cfg, 1, tokens, latent=not comp.quantize, fp4=comp.quantize)
    stream = torch.cuda.current_stream()

    def step():
        kvc.compressor_ratio1_forward(cfg, wkv, x, tokens, ws, out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = _timed(torch, stream, step, steps)
    gemm_ms = _timed(torch, stream, lambda: kvc.compressor_ratio1_forward(cfg, wkv, x, tokens, ws), reps)
    flop = 2.0 * tokens * wl.dim * comp.head_dim
    hd = comp.head_dim
    fin_bytes = tokens * hd * 4 + (tokens * (hd // 2 + hd // 16) if comp.quantize else tokens * hd * 2)
    fin_ms = ms - gemm_ms
    del x, ws, out
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "entries_per_s": round(tokens / (ms / 1e3), 1), "dtype": "bf16",
            "kernels": {"gemm_bf16": {"ms": round(gemm_ms, 4), "tflops": round(flop / gemm_ms / 1e9, 2),
                                      "flop": flop,
                                      "frac_of_bf16_peak": round(flop / gemm_ms / 1e9 / PEAK_16BIT_MFMA_TFLOPS, 4)},
                        "rows_finish": {"ms": round(fin_ms, 4), "gbps": round(fin_bytes / fin_ms / 1e6, 1),
                                        "bytes": fin_bytes, "note": "step minus projection"}}}


def run_fp4_quant(rows, width, reps, torch, kvc):
    """Time the standalone fp4 round trips over rows x width bf16 values
    (codes, scales and the dequantised copy written)."""
    g = torch.Generator(device="cuda").manual_seed(7)
    inp = torch.randn((rows, width), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(inp)
    res = {}
    for name, fn, blk in (("latent_e4m3_b16", kvc.latent_fp4_quant, 16),
                          ("indexer_e8m0_b32", kvc.indexer_fp4_quant, 32)):
        codes = torch.empty((rows, width // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((rows, width // blk), dtype=torch.uint8, device="cuda")
        ms = _timed(torch, torch.cuda.current_stream(), lambda: fn(inp, codes, scales, out), reps)
        nbytes = rows * width * (2 + 0.5 + 2) + rows * (width // blk)
        res[name] = {"rows": rows, "width": width, "ms": round(ms, 4), "gbps": round(nbytes / ms / 1e6, 1),
                     "frac_of_hbm_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBPS, 4), "bytes": int(nbytes)}
    # the read + write ceiling on the same box: a plain 1 GiB copy
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    cms = _timed(torch, torch.cuda.current_stream(), lambda: dst.copy_(src), reps)
    res["copy_1GiB"] = {"ms": round(cms, 4), "gbps": round(2 * (1 << 30) / cms / 1e6, 1)}
    del inp, out, src, dst
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_r4_n65536_fp4_idx128")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--x-format", choices=("f32", "bf16"), default="f32",
                    help="hidden states handed to the library: the f32 draws, or their bf16 rounding as bf16 rows")
    ap.add_argument("--projection", choices=("auto", "f32-mfma", "f16-split", "bf16-split"), default="auto",
                    help="prefill projection: the library's default (the f32 matrix cores for f32 x, the exact "
                         "bf16 split for bf16 x), or one of the opt-in emulations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads")
    ap.add_argument("--only-decode", action="store_true", help="run the decode stream only (for profiling)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain copy kernel (read + write) of this many MiB")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_compression_fp32_amd.kvc as kvc
    import kv_cache_compression_fp32_amd.workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kvc.lib()  # fails loudly if the HIP library is missing
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # reads n * 4 bytes, writes n * 4 bytes
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    x_format = x_format_of(kvc, args.x_format)
    projection = resolved(kvc, x_format, projection_of(kvc, args.projection))
    if args.only_decode:
        d = run_decode(W.WORKLOADS["decode_r4_b64_s512"], 5, torch, kvc, W, x_format)
        print(json.dumps({"decode_r4_b64_s512": _rounded(d)}), flush=True)
        return
    wl = W.WORKLOADS[args.workload]
    if wl.decode or wl.dim == 0:
        print("bench.py's headline is a prefill workload with hidden states", file=sys.stderr)
        sys.exit(2)

    head = run_prefill(wl, args.steps, args.warmup, args.kernel_reps, torch, kvc, W, x_format, projection)
    kernels = head["kernels"]
    main = wl.compressors[0]
    tag = f"hd{main.head_dim}"
    g = kernels[f"gemm_{tag}"]
    fused = head["fused"][0]
    dtype = {(kvc.KVC_X_F32, kvc.KVC_PROJ_F32_MFMA): "f32", (kvc.KVC_X_F32, kvc.KVC_PROJ_F16_SPLIT): "f16x3-split",
             (kvc.KVC_X_F32, kvc.KVC_PROJ_BF16_SPLIT): "bf16x6-split",
             (kvc.KVC_X_BF16, kvc.KVC_PROJ_BF16_SPLIT): "bf16x3-split"}[(x_format, projection)]
    traffic = measured_traffic("gemm_f32_pool" if fused else "gemm_f32", "gemm_f32")
    roofline = gemm_roofline(kvc, g["ms"], g["flop"], x_format, projection, traffic)
    roofline["kernel"] = (gemm_kernel_name(kvc, x_format, projection, fused) +
                          f" ({main.head_dim}-wide projection" + (" with the pooling epilogue" if fused else "") + ")")
    roofline["timing"] = ("HIP events the library records on the launch stream around this kernel in each timed "
                          "step (kvc_time_next_projection), averaged over the timed steps")
    p = kernels[f"pool_{tag}"]
    pool = {"bound": "hbm", "achieved": round(p["gbps"], 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(p["gbps"] / PEAK_HBM_GBPS, 4), "traffic": measured_traffic("pool", "pool"),
            "traffic_source": TRAFFIC_SOURCE,
            "kernel": f"pool_small_kernel<{main.head_dim},4,true> (pooling + RMSNorm + fp4 of given projections)",
            "workload": "the same step's projections handed over (x NULL): the library's separate pool path, "
                        "which the fused step replaces by the GEMM epilogue",
            "per_launch": p["bytes"], "avg_ms": round(p["ms"], 4)}
    st = kernels[f"step_{tag}"]
    post_b = post_projection_bytes(wl.batch, wl.seqlen, main.head_dim, main.quantize)
    step_pooling = {
        "fused_epilogue_ms": round(g["ms"] - kernels[f"gemm_{tag}_plain"]["ms"], 4),
        "after_projection_ms": round(st["after_projection_ms"], 4),
        "after_projection_kernels": f"pool_boundary_kernel<{main.head_dim}> + rows_finish_kernel<{main.head_dim}> "
                                    "+ state_store_kernel",
        "after_projection_bytes": post_b,
        "after_projection_gbps": round(post_b / st["after_projection_ms"] / 1e6, 1),
        "note": "the pooling the timed step runs: the pooling epilogue inside the projection kernel (its cost: "
                "that kernel minus the plain projection) and the kernels after it"} if fused else None
    result = {
        "metric": METRIC, "value": round(head["entries_per_s"], 1), "unit": "entries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "seqlen": wl.seqlen, "dim": wl.dim,
                   "x": ("bf16 rows: the bf16 rounding of the N(0,1) draws" if x_format == kvc.KVC_X_BF16
                         else "f32 rows, N(0,1)"),
                   "projection": {"f32": "f32 matrix cores", "f16x3-split": PATHS["f16-split"][3],
                                  "bf16x6-split": PATHS["bf16-split"][3], "bf16x3-split": PATHS["x-bf16"][3]}[dtype],
                   "weights": "f32",
                   "compressors": [{"ratio": c.ratio, "head_dim": c.head_dim, "fp4": c.quantize}
                                   for c in wl.compressors],
                   "entries_per_step": head["entries_per_step"]},
        "hbm_gbps": pool["achieved"],
        "hbm_gbps_kernel": pool["kernel"] + "; " + pool["workload"],
        "roofline": roofline,
        "pool": pool,
        "step_pooling": step_pooling,
        "kernels": {k: _rounded(v) for k, v in kernels.items()},
    }
    if not args.no_extras:
        extras = {}
        # the same step on the opt-in emulations and from bf16 rows
        for name in ("f16-split", "bf16-split", "x-bf16"):
            xf_name, pr_name, dt, desc = PATHS[name]
            xf, pr = x_format_of(kvc, xf_name), resolved(kvc, x_format_of(kvc, xf_name), projection_of(kvc, pr_name))
            if (xf, pr) == (x_format, projection):
                continue
            r = run_prefill(wl, 20, 20, args.kernel_reps, torch, kvc, W, xf, pr)
            rg = r["kernels"][f"gemm_{tag}"]
            roof = gemm_roofline(kvc, rg["ms"], rg["flop"], xf, pr, None)
            roof["kernel"] = gemm_kernel_name(kvc, xf, pr, r["fused"][0])
            extras[f"{wl.name}_{name}"] = {
                "dtype": dt, "x": desc, "ms_per_step": round(r["ms_per_step"], 4),
                "entries_per_s": round(r["entries_per_s"], 1), "roofline": roof,
                "kernels": {k: _rounded(v) for k, v in r["kernels"].items()}}
        for name, cold in (("prefill_r4_n4096", False), ("prefill_r128_b2_n16384", True)):
            r = run_prefill(W.WORKLOADS[name], 5, 3, 5, torch, kvc, W, x_format, projection, cold_pool=cold)
            extras[name] = {"dtype": dtype, "ms_per_step": round(r["ms_per_step"], 4),
                            "entries_per_s": round(r["entries_per_s"], 1),
                            "kernels": {k: _rounded(v) for k, v in r["kernels"].items()}}
            if cold:
                pk, pc = r["kernels"]["pool_hd512"], r["kernels"]["pool_hd512_cold"]
                extras[name]["pool"] = {
                    "bound": "hbm", "achieved": round(pk["gbps"], 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(pk["gbps"] / PEAK_HBM_GBPS, 4), "kernel": "pool_long_kernel<512, 128>",
                    "per_launch": pk["bytes"], "avg_ms": round(pk["ms"], 4),
                    "note": "back-to-back launches: the 134 MB of planes stay in the 256 MB last-level cache, as "
                            "in the step, where the projection has just written them",
                    "cold": {"achieved": round(pc["gbps"], 1), "frac": round(pc["gbps"] / PEAK_HBM_GBPS, 4),
                             "avg_ms": round(pc["ms"], 4),
                             "note": "single launches, each after a 1 GiB read that evicts the planes: every "
                                     "byte from HBM"}}
        d = run_decode(W.WORKLOADS["decode_r4_b64_s512"], 5, torch, kvc, W, x_format)
        extras["decode_r4_b64_s512"] = {"dtype": dtype, **_rounded(d)}
        extras["fp4_quant_262144x512"] = run_fp4_quant(262144, 512, 10, torch, kvc)
        extras["prefill_r1_n65536"] = run_ratio1(W.WORKLOADS["prefill_r1_n65536"], 10, 3, 10, torch, kvc, W)
        result["workloads"] = extras
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, W, x_bf16=x_format == kvc.KVC_X_BF16)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
