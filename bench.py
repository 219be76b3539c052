#!/usr/bin/env python3
"""LatentMoE layer forward benchmark on one MI355X (gfx950).

One step = one whole forward of the layer (projection + router, top-k,
permutation, both expert GEMMs, combine, up-projection + shared expert) over
one batch of seeded synthetic inputs already resident in HBM.  The default
workload is the Ultra-shape prefill layer: T=8192 tokens, d=8192, l=2048,
E=512, top-22, f=2048, shared expert 8192, bf16 with fp32 accumulation.
bf16 expert weights are packed once into the tiled layout before timing
(lmoe_pack_expert_weights; --expert-layout rowmajor skips that).

Prints one JSON line:
  value         whole-layer tokens/s over the K timed steps
  roofline      the dominant kernel (the grouped expert GEMM): algorithmic
                FLOPs per launch / its average launch time from hipEvents on
                the launch stream, against the bf16 dense MFMA peak
  decode        the weight-streaming decode layer (T=64, skewed routing):
                tokens/s and algorithmic HBM bytes / time against 8 TB/s
  other_workloads  the NVFP4-expert prefill layer and the mid-size layer:
                tokens/s, layer TFLOP/s and the grouped GEMM's rate
  cpu_baseline  the CPU oracle on a bounded token sample of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-extra]
       python bench.py --vendor-gemm-calibration   (the vendor library's GEMMs on the prefill shapes,
                                                    and this library's kernels in isolation)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LatentMoE fwd tokens/s + % MFMA peak (prefill) / % HBM BW (decode), d=8192"
PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA
PEAK_FP8_FLOPS = 5.0e15    # MI355X dense fp8 MFMA
PEAK_HBM_BYTES = 8.0e12    # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_gemm_prefill_bf16_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def code_only(text: str) -> str:
    """C++ source without its comments, whitespace runs folded to one space
    (string and character literals kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest() -> str:
    """sha256 of the GEMM kernel sources' code (comments and layout left
    out, so re-wording a comment does not void counters taken on the same
    kernels)."""
    h = hashlib.sha256()
    for f in ("gemm_mfma.hip", "device_common.hpp", "lmoe_internal.hpp"):
        with open(os.path.join(ROOT, "sparse_moe_layer_06_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per grouped-GEMM launch from the committed rocprofv3 counter
    runs, only if they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return t.get("bytes_per_launch")


def time_steps(call, steps, torch):
    """Average ms per call over `steps` back-to-back calls (hipEvents on the stream)."""
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(s)
    for _ in range(steps):
        call()
    b.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return a.elapsed_time(b) / steps, wall


def prepared(cfg, inp, layout, B):
    """The config and inputs the GPU runs: bf16 expert stacks packed once into
    the tiled layout (weight preparation, outside every timed region)."""
    if layout == "tiled" and cfg.experts == "bf16":
        return B.pack_experts(cfg, inp)
    return cfg, inp


def captured(make_call, torch):
    """One forward recorded into a HIP graph on torch's capture stream.  The
    library allocates nothing and enqueues only kernels, so a replay is the
    same launches without the host-side work of the call."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        make_call()()
    torch.cuda.synchronize()
    return g


def graph_matches(g, out, torch):
    """Replay once and compare with what the eager call left in `out`."""
    ref = out.clone()
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    return bool(torch.equal(out, ref))


def prefill(cfg, steps, warmup, torch, B, synth, layout="tiled", graph=False):
    log(f"bench: generating inputs {cfg.name}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    ws = B.alloc_workspace(cfg)
    pcfg, pinp = prepared(cfg, inp, layout, B)
    call = B.Call(pcfg, pinp, out, ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    log(f"bench: timing {steps} steps")
    ms, wall = time_steps(call, steps, torch)
    log(f"bench: {ms:.3f} ms/step")
    if graph:  # the same step replayed from a HIP graph (reported, not the headline)
        g = captured(lambda: B.Call(pcfg, pinp, out, ws), torch)
        same = graph_matches(g, out, torch)
        gms, _ = time_steps(g.replay, steps, torch)
        graph = dict(ms_per_step=gms, matches_eager=same)
        log(f"bench: {gms:.3f} ms/step replayed from a HIP graph")
        del g

    # Per-kernel durations over the same number of steps (separate pass, so the
    # headline timing has no extra events between launches).
    with B.KernelTimer(capacity=64 * steps) as kt:
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
    per = kt.by_kernel()
    kernels = {n: dict(avg_ms=sum(v) / len(v), launches_per_step=len(v) / steps,
                       ms_per_step=sum(v) / steps) for n, v in per.items()}
    return inp, out, ms, wall, kernels, graph


def decode(cfg, steps, torch, B, synth, layout="tiled", graph=False):
    log(f"bench: generating inputs {cfg.name}")
    inp = synth.make_inputs(cfg, 0, "cuda")
    out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    ws = B.alloc_workspace(cfg)
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    pcfg, pinp = prepared(cfg, inp, layout, B)
    call = B.Call(pcfg, pinp, out, ws, debug=dict(counts=counts))
    # Reading 1 GiB between steps evicts L2 and the 256 MB Infinity Cache; a read
    # leaves only clean lines, so the timed step pays no write-back of flush data.
    flush = torch.ones(1 << 29, dtype=torch.float16, device="cuda")
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    times = []
    for _ in range(steps):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        call()
        b.record(s)
        times.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in times)[len(times) // 2]
    if graph:  # the same step replayed from a HIP graph, same eviction between steps
        g = captured(lambda: B.Call(pcfg, pinp, out, ws), torch)
        same = graph_matches(g, out, torch)
        gtimes = []
        for _ in range(steps):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            g.replay()
            b.record(s)
            gtimes.append((a, b))
        torch.cuda.synchronize()
        graph = dict(ms_per_step=sorted(a.elapsed_time(b) for a, b in gtimes)[len(gtimes) // 2],
                     matches_eager=same)
        del g
    # per-kernel durations, a separate pass with the same eviction between steps
    n_k = min(steps, 20)
    with B.KernelTimer(capacity=64 * n_k) as kt:
        for _ in range(n_k):
            flush.sum()
            call()
        torch.cuda.synchronize()
    kernels = {n: dict(avg_us=round(1e3 * sum(v) / len(v), 2), launches_per_step=len(v) / n_k)
               for n, v in kt.by_kernel().items()}
    touched = int((counts > 0).sum().item())
    l, f, d, E, T = cfg.l, cfg.f, cfg.d, cfg.E, cfg.T
    r_in = l if cfg.router_latent else d  # router weights W_r [E][r_in]
    # W_down and W_up: bf16, or E4M3 codes plus one fp32 scale per row
    proj = (0 if cfg.standard_moe else 2 * d * l + 4 * (l + d) if cfg.proj_fp8
            else 2 * d * l + 2 * d * l // 32 if cfg.proj_mxfp8 else 2 * d * l * 2)
    bytes_alg = (touched * 2 * l * f * 2 + proj + r_in * E * 2 + 2 * T * d * 2
                 + (E * 4 if cfg.zipf_bias else 0))
    gbs = bytes_alg / (ms * 1e-3) / 1e9
    return dict(workload=f"{cfg.name} T={T} d={d} l={l} E={E} k={cfg.k} f={f}, {cfg.experts} experts "
                         f"({layout if cfg.experts == 'bf16' else 'as stored'}), router reads "
                         f"{'z (latent)' if cfg.router_latent else 'x'}"
                         f"{', standard MoE (experts in d)' if cfg.standard_moe else ''}"
                         f"{', FP8 projections' if cfg.proj_fp8 else ''}"
                         f"{', MXFP8 projections' if cfg.proj_mxfp8 else ''}", tokens_per_s=T / (ms * 1e-3),
                ms_per_step=ms, experts_touched=touched, alg_bytes=bytes_alg, achieved_GBps=gbs,
                hbm_frac=gbs * 1e9 / PEAK_HBM_BYTES, timing="median of %d single-step hipEvent timings, "
                "1 GiB buffer read between steps (cache eviction)" % steps, kernels=kernels,
                **({"hipgraph": graph} if graph else {}))


def grouped_bytes_per_launch(cfg):
    """Algorithmic HBM bytes of one expert GEMM, the two launches averaged:
    every expert's weights once (bf16, or NVFP4 codes plus one E4M3 scale
    byte per 16 weights or per 16 x 16 block), the T k gathered input rows
    and the T k output rows.  Only for unbiased routing, where T k >= 16 E
    leaves no expert without rows (the chance is below e^-16 per expert);
    None otherwise."""
    if cfg.zipf_bias or cfg.T * cfg.k < 16 * cfg.E:
        return None
    per_weight = {"bf16": 2.0, "nvfp4": 0.5 + 1 / 16, "nvfp4_2d": 0.5 + 1 / 256}.get(cfg.experts)
    if per_weight is None:
        return None
    weights = cfg.E * cfg.l * cfg.f * per_weight
    rows = cfg.T * cfg.k * (cfg.l + cfg.f) * 2
    return weights + rows


def secondary(cfg, steps, warmup, torch, B, synth, layout="tiled"):
    """The other MFMA-bound workloads (same metric, reported beside the headline)."""
    inp, out, ms, _, kernels, _ = prefill(cfg, steps, warmup, torch, B, synth, layout)
    gname = "grouped_gemm_nvfp4" if cfg.experts in ("nvfp4", "nvfp4_2d") else "grouped_gemm"
    g = kernels.get(gname)
    res = dict(workload=f"{cfg.name}: T={cfg.T} d={cfg.d} l={cfg.l} E={cfg.E} k={cfg.k} f={cfg.f} f_s={cfg.f_s}, "
                        f"{cfg.experts} experts, router reads {'z (latent)' if cfg.router_latent else 'x'}"
                        f"{', FP8 shared expert (E4M3 x E4M3 MFMA)' if cfg.shared_fp8 else ''}"
                        f"{', FP8 down- and up-projections' if cfg.proj_fp8 else ''}"
                        f"{', MXFP8 down- and up-projections' if cfg.proj_mxfp8 else ''}"
                        f"{', standard MoE (experts in d, no latent projections)' if cfg.standard_moe else ''}",
               ms_per_step=ms, tokens_per_s=cfg.T / (ms * 1e-3),
               layer_tflops=cfg.flops / (ms * 1e-3) / 1e12, layer_mfma_frac=cfg.flops / (ms * 1e-3) / PEAK_BF16_FLOPS)
    if g:
        ach = 2.0 * cfg.T * cfg.k * cfg.l * cfg.f / (g["avg_ms"] * 1e-3)
        res["grouped"] = dict(kernel=gname, avg_launch_ms=g["avg_ms"], achieved_tflops=ach / 1e12,
                              mfma_frac=ach / PEAK_BF16_FLOPS)
        nbytes = grouped_bytes_per_launch(cfg)
        if nbytes:
            res["grouped"].update(alg_bytes_per_launch=nbytes,
                                  hbm_frac=nbytes / (g["avg_ms"] * 1e-3) / PEAK_HBM_BYTES)
    f8 = kernels.get("fp8_gemm")
    # the fp8 products: the shared expert's two (2 T d f_s FLOPs each) and
    # the two projections (2 T d l each)
    f8_flops = (4.0 * cfg.T * cfg.d * cfg.f_s if cfg.shared_fp8 else 0.0) + \
        (4.0 * cfg.T * cfg.d * cfg.l if cfg.proj_fp8 or cfg.proj_mxfp8 else 0.0)
    if f8 and f8_flops > 0:
        ach = f8_flops / (f8["ms_per_step"] * 1e-3)
        res["fp8_gemm"] = dict(avg_launch_ms=f8["avg_ms"], launches_per_step=f8["launches_per_step"],
                               achieved_tflops=ach / 1e12, mfma_frac_fp8=ach / PEAK_FP8_FLOPS)
    del inp, out
    torch.cuda.empty_cache()
    return res


def oracle_seconds(cfg, inp, tokens, synth, threads=None):
    """Wall time of the CPU oracle on the given token rows of a layer (their
    routing, experts, up-projection and shared expert), with numpy's BLAS
    limited to `threads` threads (all by default).  The experts those rows
    use are copied to the host first: device-to-host copies are not oracle
    work."""
    import contextlib

    import numpy as np
    from oracle import latentmoe_oracle as O
    from threadpoolctl import threadpool_limits
    h = {}
    for k, v in inp.items():
        if v is None:
            h[k] = None
        elif k in ("W1", "W2"):
            h[k] = synth.LazyExperts(v)
        else:
            h[k] = synth.host_view(v)
    _, idx, _ = O.route({"x": h["x"][tokens], "W_r": h["W_r"], "b_r": h.get("b_r"),
                         "W_down": h.get("W_down")}, cfg.k)
    for e in np.unique(idx):
        h["W1"][e], h["W2"][e]
    limit = threadpool_limits(limits=threads) if threads else contextlib.nullcontext()
    with limit:
        t0 = time.perf_counter()
        O.forward(h, cfg.k, tokens=tokens, experts=O.ExpertWeights(h, cache_size=len(np.unique(idx))))
        return time.perf_counter() - t0


def cpu_baseline(cfg, inp, n_tokens, synth, torch):
    """The oracle timed on the host: the headline workload on a bounded token
    sample with every host core, and single-threaded on the tiny workload
    (all 64 tokens), the mid-size one (a 32-token sample) and the decode
    workload (all 64 tokens)."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    tokens = np.linspace(0, cfg.T - 1, n_tokens).astype(np.int64)
    dt = oracle_seconds(cfg, inp, tokens, synth)
    single = {}
    for name, n in (("tiny_f32", 64), ("mid_bf16", 32), ("decode_bf16_zipf", 64)):
        c = synth.CONFIGS[name]
        sub = synth.make_inputs(c, 0, "cuda")
        t = np.linspace(0, c.T - 1, min(n, c.T)).astype(np.int64)
        s1 = oracle_seconds(c, sub, t, synth, threads=1)
        single[name] = dict(tokens=int(len(t)), seconds=s1, tokens_per_s=len(t) / s1)
        del sub
        torch.cuda.empty_cache()
    return dict(value=n_tokens / dt, unit="tokens/s", cores=cores, blas_threads=blas_threads, kind="oracle",
                sample=f"{n_tokens} evenly spaced tokens of {cfg.name} (routing, experts, up-projection "
                       f"and shared expert of those tokens), {dt:.1f} s, float64 numpy on {cores} host cores "
                       f"(BLAS threads {blas_threads})",
                single_thread=single)


def vendor_gemm_calibration(torch, steps):
    """torch's bf16 GEMMs on the prefill layer's products, random operands,
    all contiguous: the two dense projections as plain GEMMs, and the expert
    GEMM as a batched GEMM of 512 experts with 352 rows each (the mean rows
    per expert at T = 8192, top-22; the same FLOPs, without the row gather
    and the ragged tiles).  Not part of the layer: a measure of what the
    vendor library sustains on this chip under the same clocks."""
    dev, bf = "cuda", torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(0)

    def rnd(*shape):
        return torch.randn(*shape, device=dev, dtype=bf, generator=g)

    cases = {
        "down_projection_router_shared": (lambda a, b: torch.matmul(a, b), (8192, 8192), (8192, 10752)),
        "up_projection_shared": (lambda a, b: torch.matmul(a, b), (8192, 10240), (10240, 8192)),
        "experts_batched": (lambda a, b: torch.bmm(a, b), (512, 352, 2048), (512, 2048, 2048)),
    }
    out = {}
    for name, (fn, sa, sb) in cases.items():
        a, b = rnd(*sa), rnd(*sb)
        flops = 2.0 * a.numel() * sb[-1]
        for _ in range(3):
            fn(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out[name] = dict(a=list(sa), b=list(sb), ms=ms, tflops=flops / (ms * 1e-3) / 1e12,
                         mfma_frac=flops / (ms * 1e-3) / PEAK_BF16_FLOPS)
        del a, b
    torch.cuda.empty_cache()
    return {"vendor_gemm_calibration": out, "own_kernels_in_isolation": own_kernels_in_isolation(torch, steps)}


def own_kernels_in_isolation(torch, steps):
    """The library's staged calls on the prefill workload, each repeated back
    to back as the vendor GEMMs are above: the per-launch time of every
    kernel of one call, in launch order (the layer's own timing runs them in
    sequence, where the clock follows the whole step's power draw)."""
    from sparse_moe_layer_06_amd import binding as B
    from sparse_moe_layer_06_amd import synth
    cfg = synth.CONFIGS["prefill_bf16"]
    inp = synth.make_inputs(cfg, 0, "cuda")
    ws = B.alloc_workspace(cfg)
    pcfg, pinp = prepared(cfg, inp, "tiled", B)
    r = B.project_route(pcfg, pinp, ws)
    pm = B.permute(pcfg, r["idx"], ws)
    Y = B.experts_ffn(pcfg, pinp, r["z"], pm["offsets"], pm["perm"], ws)
    stages = {
        "project_route": lambda: B.project_route(pcfg, pinp, ws),
        "experts_ffn": lambda: B.experts_ffn(pcfg, pinp, r["z"], pm["offsets"], pm["perm"], ws),
        "combine_up": lambda: B.combine_up(pcfg, pinp, Y, pm["inv"], r["gate"], r["hs"], ws, cfg.T),
    }
    res = {}
    for name, fn in stages.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        with B.KernelTimer(capacity=16 * steps) as kt:
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
        recs = kt.records
        n = len(recs) // steps
        res[name] = [dict(kernel=recs[i][0], avg_ms=sum(recs[i + j * n][1] for j in range(steps)) / steps)
                     for i in range(n)]
    del inp, ws, pinp, r, pm, Y
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_bf16")
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--cpu-tokens", type=int, default=2048)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replays (profiling runs: every launch is then an eager one)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (NVFP4 and mid prefill, latent router)")
    ap.add_argument("--expert-layout", choices=("tiled", "rowmajor"), default="tiled",
                    help="bf16 expert weights as packed by lmoe_pack_expert_weights (default) or row-major")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device-to-device 3 times (scale for HBM byte counters) and exit")
    ap.add_argument("--vendor-gemm-calibration", action="store_true",
                    help="only time torch's bf16 GEMMs (the ROCm BLAS libraries) on the prefill layer's "
                         "product shapes and exit: what the vendor library sustains on this chip")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the layer is benchmarked on a single MI355X "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        # A plain copy of known size: under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
        # it gives the factor between those counters and bytes moved.
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return

    if args.vendor_gemm_calibration:
        print(json.dumps(vendor_gemm_calibration(torch, args.steps)), flush=True)
        return

    from sparse_moe_layer_06_amd import binding as B
    from sparse_moe_layer_06_amd import synth

    B.lib()
    cfg = synth.CONFIGS[args.workload]
    inp, out, ms, wall, kernels, graph = prefill(cfg, args.steps, args.warmup, torch, B, synth,
                                                 args.expert_layout, graph=not args.no_graph)
    tokens_per_s = cfg.T / (ms * 1e-3)
    layer_tflops = cfg.flops / (ms * 1e-3) / 1e12

    # Dominant kernel: the grouped expert GEMM (two launches per step, equal FLOPs).
    gname = "grouped_gemm_nvfp4" if cfg.experts in ("nvfp4", "nvfp4_2d") else "grouped_gemm"
    g = kernels.get(gname)
    flops_per_launch = 2.0 * cfg.T * cfg.k * cfg.l * cfg.f
    roofline = None
    if g:
        achieved = flops_per_launch / (g["avg_ms"] * 1e-3) / 1e12
        roofline = dict(kernel=gname, bound="mfma", achieved=achieved, peak=PEAK_BF16_FLOPS / 1e12,
                        unit="TFLOP/s", frac=achieved * 1e12 / PEAK_BF16_FLOPS, traffic=measured_traffic(),
                        avg_launch_ms=g["avg_ms"], alg_flops_per_launch=flops_per_launch)
    for v in kernels.values():
        v["avg_ms"] = round(v["avg_ms"], 4)
        v["ms_per_step"] = round(v["ms_per_step"], 4)

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: LatentMoE layer T={cfg.T} d={cfg.d} l={cfg.l} E={cfg.E} "
                               f"k={cfg.k} f={cfg.f} f_s={cfg.f_s}, {cfg.experts} experts"
                               f"{' (' + args.expert_layout + ' layout)' if cfg.experts == 'bf16' else ''}, seed 0",
                   "global_batch": cfg.T, "parallelism": "single GPU"},
        "layer_tflops": layer_tflops,
        "layer_mfma_frac": layer_tflops * 1e12 / PEAK_BF16_FLOPS,
        "wall_s_timed": wall,
        "roofline": roofline,
        "kernels": kernels,
        # the graded figure is the eager one above; this is the same step replayed from a HIP graph
        "hipgraph": graph,
    }
    if not args.no_decode:
        result["decode"] = decode(synth.CONFIGS["decode_bf16_zipf"], args.decode_steps, torch, B, synth,
                                  args.expert_layout, graph=not args.no_graph)
    if not args.no_extra:
        C = synth.CONFIGS
        extra = [C[n] for n in ("prefill_nvfp4", "mid_bf16") if n != args.workload]
        extra.append(C["prefill_nvfp4"].with_(name="prefill_nvfp4_2d", experts="nvfp4_2d"))
        extra.append(C["prefill_bf16"].with_(name="prefill_bf16_latent_router", router_latent=True))
        extra.append(C["prefill_bf16"].with_(name="prefill_bf16_fp8_shared", shared_fp8=True))
        extra.append(C["prefill_bf16"].with_(name="prefill_bf16_fp8_proj_shared", shared_fp8=True, proj_fp8=True))
        extra.append(C["prefill_bf16"].with_(name="prefill_bf16_mxfp8_proj_fp8_shared", shared_fp8=True,
                                             proj_mxfp8=True))
        # the standard MoE the overview compares against: 128 experts of d, top-6
        extra.append(C["prefill_bf16"].with_(name="prefill_standard_moe", l=C["prefill_bf16"].d, E=128, k=6,
                                             standard_moe=True))
        result["other_workloads"] = {c.name: secondary(c, max(args.steps // 2, 3), args.warmup, torch, B, synth,
                                                       args.expert_layout) for c in extra}
        if not args.no_decode:
            result["other_workloads"]["decode_latent_router"] = decode(
                C["decode_bf16_zipf"].with_(name="decode_latent_router", router_latent=True),
                args.decode_steps, torch, B, synth, args.expert_layout)
            result["other_workloads"]["decode_fp8_proj"] = decode(
                C["decode_bf16_zipf"].with_(name="decode_fp8_proj", proj_fp8=True),
                args.decode_steps, torch, B, synth, args.expert_layout)
            result["other_workloads"]["decode_mxfp8_proj"] = decode(
                C["decode_bf16_zipf"].with_(name="decode_mxfp8_proj", proj_mxfp8=True),
                args.decode_steps, torch, B, synth, args.expert_layout)
            result["other_workloads"]["decode_standard_moe"] = decode(
                C["decode_bf16_zipf"].with_(name="decode_standard_moe", l=C["decode_bf16_zipf"].d, E=128, k=6,
                                            standard_moe=True),
                args.decode_steps, torch, B, synth, args.expert_layout)
    if not args.no_cpu:
        log("bench: cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_tokens, synth, torch)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
