"""Benchmark of the compressor hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole path over one batch: for the default
workload (ratio-4 prefill of 65536 tokens, hidden 4096) that is the 512-wide
compressor (f32 projections, pooling + RMSNorm + fp4 cache codes) and the
128-wide indexer compressor (projections, pooling + RMSNorm, bf16 latent),
with the hidden states resident in HBM: x f32 [1, 65536, 4096] ~ N(0, 1).
The projections are f32 products on the f16 matrix cores by default (each
row of x and each weight row scaled by a power of two and split into two f16
parts, three part products summed in f32; the step computes x's row
exponents once for both compressors); --projection bf16-split (six bf16 part
products) and f32-mfma (the f32 matrix cores) select the others. Beside the
headline (`workloads`) the same step on the other projection paths, and from
the model's bf16 hidden states (the bf16 rounding of the same draws as bf16
rows: exact products from the weights' three parts; --x-format bf16 makes
that the headline). Prints one JSON line.

Kernel durations are measured with HIP events on the launch stream around
repeated launches of each kernel alone (the same library calls with the other
stages switched off through their arguments: no outputs = projection only,
which with a split projection is the weight split (under 1% of it) and the
GEMM; projections given = pooling only). The roofline object reports the
dominant kernel (the 512-wide projection GEMM, matrix-core bound: the f16 or
bf16 part products against the 16-bit matrix-core peak, with the
f32-equivalent rate beside it; the f32 matrix cores against the fp32 peak);
`pool` reports the pooling kernel against HBM bandwidth.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed KV entries/sec + achieved HBM GB/s, ratio-4 prefill N=65536"
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 matrix
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the sources each counted kernel is built from (the traffic figures turn
# null as soon as any of them changes)
KERNEL_SOURCES = {
    "gemm": ["kv_cache_compression_fp32_amd/csrc/gemm_common.h", "kv_cache_compression_fp32_amd/csrc/gemm_f32_kernel.h",
             "kv_cache_compression_fp32_amd/csrc/gemm_f32.hip", "kv_cache_compression_fp32_amd/csrc/kvc_device.h",
             "kv_cache_compression_fp32_amd/csrc/gemm_epilogue.h"],
    "gemm_x6": ["kv_cache_compression_fp32_amd/csrc/gemm_common.h", "kv_cache_compression_fp32_amd/csrc/gemm_bf16.hip",
                "kv_cache_compression_fp32_amd/csrc/kvc_device.h", "kv_cache_compression_fp32_amd/csrc/gemm_epilogue.h"],
    "gemm_x3": ["kv_cache_compression_fp32_amd/csrc/gemm_common.h", "kv_cache_compression_fp32_amd/csrc/gemm_bf16.hip",
                "kv_cache_compression_fp32_amd/csrc/kvc_device.h", "kv_cache_compression_fp32_amd/csrc/gemm_epilogue.h"],
    "gemm_h3": ["kv_cache_compression_fp32_amd/csrc/gemm_common.h", "kv_cache_compression_fp32_amd/csrc/gemm_bf16.hip",
                "kv_cache_compression_fp32_amd/csrc/kvc_device.h", "kv_cache_compression_fp32_amd/csrc/gemm_epilogue.h"],
    "pool": ["kv_cache_compression_fp32_amd/csrc/pool.hip", "kv_cache_compression_fp32_amd/csrc/kvc_device.h"],
}


def source_sha(name: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel source changed since it was taken."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = data.get(name)
    if not entry or entry.get("source_sha") != source_sha(name):
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


def bf16_hidden(torch, x: np.ndarray) -> np.ndarray:
    """The bf16 rounding of synthetic hidden states (torch's conversion), as
    float32 values."""
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


def cpu_baseline(wl, W, seconds=10.0, x_bf16=False):
    """The oracle, as it stands, on the first tokens of the workload: doubles
    the sample until it takes `seconds` or covers the whole sequence."""
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
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
    return {"value": entries / dt, "unit": "entries/s", "cores": threads, "kind": "oracle",
            "sample": f"first {tokens} tokens of each of {wl.batch} batch rows through all "
                      f"{len(wl.compressors)} compressor(s) of the workload ({entries} entries, {dt:.2f} s)"}


def _timed(torch, stream, fn, reps):
    fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def gemm_roofline(kvc, g, x_format, projection):
    """Roofline object of the 512-wide projection launch `g`: on the bf16 or
    f16 matrix cores its passes against that peak (with the f32-equivalent
    rate beside it), on the f32 matrix cores its flops against the fp32 peak."""
    passes = mfma_passes(kvc, x_format, projection)
    if passes:
        if resolved(kvc, x_format, projection) == kvc.KVC_PROJ_F16_SPLIT:
            what = ("f32 x and f32 weights, rows scaled by powers of two and split into two f16 parts, three part "
                    "products on the f16 matrix cores")
            kernel, traffic = "gemm_x6_kernel<*, F16>", "gemm_h3"
        elif passes == 3:
            what = "bf16 x times the three bf16 parts of the f32 weights"
            kernel, traffic = "gemm_mc_kernel", "gemm_x3"
        else:
            what = "f32 x split into three bf16 parts times the three parts of the f32 weights, six part products"
            kernel, traffic = "gemm_x6_kernel", "gemm_x6"
        return {"bound": "mfma", "achieved": round(g["mfma_tflops"], 2), "peak": PEAK_BF16_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(g["mfma_tflops"] / PEAK_BF16_MFMA_TFLOPS, 4),
                "traffic": measured_traffic(traffic),
                "kernel": f"{kernel} (512-wide projection, {what}, f32 accumulation)",
                "per_launch": g["mfma_flop"], "avg_ms": round(g["ms"], 4),
                "f32_equivalent_tflops": round(g["tflops"], 2),
                "f32_equivalent_frac_of_fp32_peak": round(g["tflops"] / PEAK_FP32_MFMA_TFLOPS, 4)}
    return {"bound": "mfma", "achieved": round(g["tflops"], 2), "peak": PEAK_FP32_MFMA_TFLOPS,
            "unit": "TFLOP/s", "frac": round(g["tflops"] / PEAK_FP32_MFMA_TFLOPS, 4),
            "traffic": measured_traffic("gemm"), "kernel": "gemm_f32_kernel (512-wide projection, f32 matrix cores)",
            "per_launch": g["flop"], "avg_ms": round(g["ms"], 4)}


def _rounded(d):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}


def resolved(kvc, x_format, projection):
    """The projection the library runs for KVC_PROJ_AUTO."""
    if projection != kvc.KVC_PROJ_AUTO:
        return projection
    return kvc.KVC_PROJ_F16_SPLIT if x_format == kvc.KVC_X_F32 else kvc.KVC_PROJ_BF16_SPLIT


def mfma_passes(kvc, x_format, projection):
    """16-bit matrix-core passes per f32 product (bf16 or f16, both at the
    same peak; 0: the f32 matrix cores)."""
    projection = resolved(kvc, x_format, projection)
    if projection == kvc.KVC_PROJ_F32_MFMA:
        return 0
    if projection == kvc.KVC_PROJ_F16_SPLIT:
        return 3
    return 3 if x_format == kvc.KVC_X_BF16 else 6


def run_prefill(wl, steps, warmup, reps, torch, kvc, W, x_format, projection):
    """Time whole prefill steps of `wl`, then each kernel alone. x is the
    workload's f32 draws, or (x_format bf16) their bf16 rounding as bf16 rows."""
    dev = "cuda"
    print(f"[bench] {wl.name}: generating inputs (x_format {x_format})", file=sys.stderr, flush=True)
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
    m = wl.batch * wl.seqlen
    # the f16 split scales each row of x by its own power of two: both
    # compressors read the same hidden states, so the step computes the
    # row exponents once and hands them to both
    shared = resolved(kvc, x_format, projection) == kvc.KVC_PROJ_F16_SPLIT
    exps = torch.empty(m, dtype=torch.int32, device=dev) if shared else None

    def step():
        if shared:
            kvc.x_row_exponents(x, m, wl.dim, exps)
        for comp, cfg, wts, ws, state, out, groups in comps:
            kvc.compressor_prefill(cfg, wts, x, wl.batch, wl.seqlen, ws, state[0], state[1], out, x_exponents=exps)

    print(f"[bench] {wl.name}: warmup + {steps} timed steps", file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms_per_step = _timed(torch, stream, step, steps)
    entries = comps[0][6] * wl.batch

    kernels = {}
    if shared:
        xe_ms = _timed(torch, stream, lambda: kvc.x_row_exponents(x, m, wl.dim, exps), reps)
        xe_bytes = m * wl.dim * 4 + m * 4
        kernels["x_exponents"] = {"ms": xe_ms, "gbps": xe_bytes / xe_ms / 1e6, "bytes": xe_bytes}
    for comp, cfg, wts, ws, state, out, groups in comps:
        tag = f"hd{comp.head_dim}"
        gemm_ms = _timed(torch, stream, lambda: kvc.compressor_prefill(cfg, wts, x, wl.batch, wl.seqlen, ws,
                                                                       x_exponents=exps), reps)
        # ws now holds this compressor's projections, the bias already in the
        # score plane: pool them alone, exactly as the step's pooling launch
        pool_ms = _timed(torch, stream, lambda: kvc.compressor_prefill(cfg, kvc.Weights(), None, wl.batch,
                                                                       wl.seqlen, ws, None, None, out), reps)
        proj = 2 * comp.head_dim if comp.ratio == 4 else comp.head_dim
        flops = 2.0 * wl.batch * wl.seqlen * wl.dim * 2 * proj
        pbytes = pool_bytes(wl.batch, wl.seqlen, comp.ratio, comp.head_dim, comp.quantize, not comp.quantize)
        kernels[f"gemm_{tag}"] = {"ms": gemm_ms, "tflops": flops / gemm_ms / 1e9, "flop": flops}
        passes = mfma_passes(kvc, x_format, projection)
        if passes:
            # the bf16 matrix-core work: one pass per part product
            kernels[f"gemm_{tag}"].update({"mfma_flop": passes * flops, "mfma_tflops": passes * flops / gemm_ms / 1e9})
        kernels[f"pool_{tag}"] = {"ms": pool_ms, "gbps": pbytes / pool_ms / 1e6, "bytes": pbytes}
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
    del comps, x
    torch.cuda.empty_cache()
    return {"ms_per_step": ms_per_step, "entries_per_step": entries,
            "entries_per_s": entries / (ms_per_step / 1e3), "kernels": kernels}


def run_decode(wl, passes, torch, kvc, W, x_format):
    """Time whole decode passes (every row streams all its tokens from
    start_pos 0, one decode step per token), captured once in a HIP graph so
    that host launch overhead is not measured."""
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
    ws = torch.empty(kvc.kvc_decode_workspace_floats(cfg, wl.batch), dtype=torch.float32, device=dev)
    state = kvc.new_state(cfg, wl.batch)
    groups = wl.seqlen // comp.ratio
    lat = torch.empty((groups, wl.batch, comp.head_dim), dtype=torch.bfloat16, device=dev)
    outs = [kvc.Outputs(latent=lat[e]) for e in range(groups)]

    def one_pass():
        e = 0
        for p in range(wl.seqlen):
            emits = p > 0 and (p + 1) % comp.ratio == 0
            kvc.compressor_decode_step(cfg, wts, x[p], wl.batch, p, ws, state[0], state[1],
                                       outs[e] if emits else None)
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
    stream = torch.cuda.current_stream()
    print(f"[bench] {wl.name}: {passes} timed graph replays", file=sys.stderr, flush=True)
    ms = _timed(torch, stream, graph.replay, passes)
    eager_ms = _timed(torch, stream, one_pass, 1)
    proj = 2 * comp.head_dim if comp.ratio == 4 else comp.head_dim
    flop_step = 2.0 * wl.batch * wl.dim * 2 * proj
    entries = wl.batch * groups
    del graph, x, outs, lat
    torch.cuda.empty_cache()
    return {"ms_per_pass": ms, "entries_per_pass": entries, "entries_per_s": entries / (ms / 1e3),
            "us_per_step": ms * 1e3 / wl.seqlen, "tflops": flop_step * wl.seqlen / ms / 1e9,
            "eager_ms_per_pass": eager_ms}


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
    # the epilogue kernel reads the f32 projections and writes the outputs
    hd = comp.head_dim
    fin_bytes = tokens * hd * 4 + (tokens * (hd // 2 + hd // 16) if comp.quantize else tokens * hd * 2)
    fin_ms = ms - gemm_ms
    del x, ws, out
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "entries_per_s": round(tokens / (ms / 1e3), 1),
            "kernels": {"gemm_bf16": {"ms": round(gemm_ms, 4), "tflops": round(flop / gemm_ms / 1e9, 2),
                                      "flop": flop, "frac_of_bf16_peak": round(flop / gemm_ms / 1e9 / PEAK_BF16_MFMA_TFLOPS, 4)},
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
                     "bytes": int(nbytes)}
    del inp, out
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the clock climbs for about 100 ms of sustained matrix-core load: the
    # default warmup (about 60 ms of steps) times the loaded state
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_r4_n65536_fp4_idx128")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--x-format", choices=("f32", "bf16"), default="f32",
                    help="hidden states handed to the library: the f32 draws, or their bf16 rounding as bf16 rows")
    ap.add_argument("--projection", choices=("auto", "f16-split", "bf16-split", "f32-mfma"), default="auto",
                    help="prefill projection: the library's default (f16 split for f32 x, bf16 split for bf16 x), "
                         "the f16 matrix cores on scaled two-part f16 splits, the bf16 matrix cores on exact bf16 "
                         "parts, or the f32 matrix cores")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads")
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
    wl = W.WORKLOADS[args.workload]
    if wl.decode or wl.dim == 0:
        print("bench.py's headline is a prefill workload with hidden states", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # reads n * 4 bytes, writes n * 4 bytes
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    x_format = kvc.KVC_X_BF16 if args.x_format == "bf16" else kvc.KVC_X_F32
    projection = {"auto": kvc.KVC_PROJ_AUTO, "bf16-split": kvc.KVC_PROJ_BF16_SPLIT, "f32-mfma": kvc.KVC_PROJ_F32_MFMA,
                  "f16-split": kvc.KVC_PROJ_F16_SPLIT}[args.projection]
    projection = resolved(kvc, x_format, projection)
    head = run_prefill(wl, args.steps, args.warmup, args.kernel_reps, torch, kvc, W, x_format, projection)
    kernels = head["kernels"]
    main_tag = f"hd{wl.compressors[0].head_dim}"
    g = kernels[f"gemm_{main_tag}"]
    p = kernels[f"pool_{main_tag}"]
    roofline = gemm_roofline(kvc, g, x_format, projection)
    pool = {"bound": "hbm", "achieved": round(p["gbps"], 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(p["gbps"] / PEAK_HBM_GBPS, 4), "traffic": measured_traffic("pool"),
            "kernel": "pool_small_kernel<512,4,true>", "per_launch": p["bytes"], "avg_ms": round(p["ms"], 4)}
    result = {
        "metric": METRIC, "value": round(head["entries_per_s"], 1), "unit": "entries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "seqlen": wl.seqlen, "dim": wl.dim,
                   "x": ("bf16 rows: the bf16 rounding of the N(0,1) draws" if x_format == kvc.KVC_X_BF16
                         else "f32 rows, N(0,1)"),
                   "projection": {kvc.KVC_PROJ_F32_MFMA: "f32 matrix cores",
                                  kvc.KVC_PROJ_BF16_SPLIT: "bf16 matrix cores on exact bf16 parts, f32 accumulation",
                                  kvc.KVC_PROJ_F16_SPLIT: "f16 matrix cores on row-scaled two-part f16 splits, "
                                                          "f32 accumulation"}[projection],
                   "weights": "f32",
                   "compressors": [{"ratio": c.ratio, "head_dim": c.head_dim, "fp4": c.quantize}
                                   for c in wl.compressors],
                   "entries_per_step": head["entries_per_step"]},
        "hbm_gbps": pool["achieved"],
        "roofline": roofline,
        "pool": pool,
        "kernels": {k: _rounded(v) for k, v in kernels.items()},
    }
    if not args.no_extras:
        extras = {}
        # the same step by the other projection paths
        for name, xf, pr, desc in (
                ("f32_mfma", kvc.KVC_X_F32, kvc.KVC_PROJ_F32_MFMA, "f32 rows, N(0,1); f32 matrix cores"),
                ("f16_split", kvc.KVC_X_F32, kvc.KVC_PROJ_F16_SPLIT,
                 "f32 rows, N(0,1); f16 matrix cores on row-scaled two-part f16 splits (three part products)"),
                ("bf16_split", kvc.KVC_X_F32, kvc.KVC_PROJ_BF16_SPLIT,
                 "f32 rows, N(0,1); bf16 matrix cores on exact bf16 parts (six part products)"),
                ("x_bf16", kvc.KVC_X_BF16, kvc.KVC_PROJ_BF16_SPLIT,
                 "bf16 rows: the bf16 rounding of the N(0,1) draws, the model's hidden-state type; bf16 matrix "
                 "cores on the exact bf16 parts of the weights")):
            if (xf, pr) == (x_format, projection):
                continue
            r = run_prefill(wl, 20, 20, args.kernel_reps, torch, kvc, W, xf, pr)
            extras[f"{wl.name}_{name}"] = {
                "x": desc, "ms_per_step": round(r["ms_per_step"], 4), "entries_per_s": round(r["entries_per_s"], 1),
                "roofline": gemm_roofline(kvc, r["kernels"][f"gemm_{main_tag}"], xf, pr),
                "kernels": {k: _rounded(v) for k, v in r["kernels"].items()}}
        for name in ("prefill_r4_n4096", "prefill_r128_b2_n16384"):
            r = run_prefill(W.WORKLOADS[name], 5, 2, 5, torch, kvc, W, x_format, projection)
            extras[name] = {"ms_per_step": round(r["ms_per_step"], 4), "entries_per_s": round(r["entries_per_s"], 1),
                            "kernels": {k: _rounded(v) for k, v in r["kernels"].items()}}
        d = run_decode(W.WORKLOADS["decode_r4_b64_s512"], 5, torch, kvc, W, x_format)
        extras["decode_r4_b64_s512"] = _rounded(d)
        extras["fp4_quant_262144x512"] = run_fp4_quant(262144, 512, 10, torch, kvc)
        extras["prefill_r1_n65536"] = run_ratio1(W.WORKLOADS["prefill_r1_n65536"], 10, 3, 10, torch, kvc, W)
        result["workloads"] = extras
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, W, x_bf16=x_format == kvc.KVC_X_BF16)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
