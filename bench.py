"""Benchmark of the batched CFM sampler on one MI355X.

One bench step = one cfm_sample call: the whole hot path (timestep MLP and
modulation set-up, S Euler steps of the DiT estimator over the CFG-expanded
batch, guidance combine and Euler update) over one batch of synthetic input,
with inputs resident in HBM. Default workload: the Mel DiT generator
(22 layers, d=1024, 16 heads, FFN 2048, 100-channel latent, 1000 frames,
8 requests x CFG = 16 rows, text condition 1000x512, 32 Euler steps, s=2).

Prints ONE JSON line on stdout:
  value            estimator evals/s = rows * S / t_sample
  frames           latent frame-steps/s and generated frames/s
  gemm_attn_frac   GEMM + attention FLOPs / their kernel time / 2.5 PFLOP/s (bf16 dense)
  roofline         the dominant kernel class: algorithmic FLOPs (or bytes) per launch /
                   its mean launch duration (HIP events on the launch stream); traffic =
                   HBM-side bytes per launch from the committed rocprofv3 counter summary
                   (profiles/traffic_mel_dit.txt), null once the GEMM sources differ
  cpu_baseline     the fp64 CPU oracle on a bounded sample of the same workload
  cfg_euler_cold   the CFG + Euler kernel alone with the last-level cache flushed before each launch
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, B/s
MFMA_CLASSES = ["gemm_qkv", "gemm_proj", "gemm_fc1", "gemm_fc2", "attention", "gemm_in", "gemm_out",
                "xattn", "gemm_xattn"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_model(s, lengths):
    """Algorithmic work per launch of each kernel class (valid tokens only) and launches per sample."""
    R, Tx, C, d, f, H = s.n_requests, s.n_frames, s.latent_dim, s.d_model, s.ffn_dim, s.n_heads
    P = s.n_prefix if s.cond_mode == "prefix" else 0
    nb, L, S = s.n_branches, s.n_layers, s.n_steps
    Lv = np.minimum(np.asarray(lengths), Tx)
    tok_v = nb * float(np.sum(Lv + P))                  # valid tokens over all rows
    x_v = float(np.sum(Lv))                              # valid latent frames over all requests
    attn = 4.0 * s.head_dim * H * nb * float(np.sum((Lv + P) ** 2))
    f1 = 2 * f if s.mlp == "swiglu" else f               # fused gate-up FC1 width
    cross = s.cond_mode == "cross"
    w = {
        "gemm_qkv": (2.0 * tok_v * 3 * d * d, L * S),
        "gemm_proj": (2.0 * tok_v * d * d, L * S),
        "gemm_fc1": (2.0 * tok_v * f1 * d, L * S),
        "gemm_fc2": (2.0 * tok_v * d * f, L * S),
        "attention": (attn, L * S),
        "gemm_in": (2.0 * x_v * d * C, S),
        "gemm_out": (2.0 * nb * x_v * C * d, S),
        # bytes: LN reads h fp32, writes bf16 (valid tokens); CFG+Euler reads x, writes x, reads nb v
        "adaln": (tok_v * d * (4 + 2), (3 if cross else 2) * L * S + S),
        "cfg_euler": (x_v * C * 4 * (2 + nb), S),
    }
    if cross:   # queries of every valid token against the row's n_prefix context keys
        w["xattn"] = (4.0 * s.head_dim * H * nb * float(np.sum(Lv)) * s.n_prefix, L * S)
        w["gemm_xattn"] = (2.0 * tok_v * d * d, 2 * L * S)       # query and output projections
    return w


def cfg_euler_cold(s, reps: int = 20):
    """The CFG + Euler kernel alone on the workload's shapes with the 256 MiB last-level cache flushed
    (a 512 MiB device write) before every launch: per-launch time (HIP events around the launch on the
    current stream) and algorithmic bytes over it. The in-pipeline figure is in kernels["cfg_euler"]."""
    import torch
    import flow_matching_tts_amd as F
    R, Tx, C, nb = s.n_requests, s.n_frames, s.latent_dim, s.n_branches
    g = torch.Generator(device="cuda").manual_seed(7)
    v = torch.randn(nb, R, Tx, C, device="cuda", generator=g)
    x = torch.randn(R, Tx, C, device="cuda", generator=g)
    w = [1.0] if nb == 1 else ([1 - s.guidance[0], s.guidance[0]] if nb == 2 else
                               [1 - s.guidance[0], s.guidance[0] - s.guidance[1], s.guidance[1]])
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        scratch.fill_(i & 0xFF)
        ev[i][0].record()
        F.cfg_euler(v, w, 1.0 / s.n_steps, x)
        ev[i][1].record()
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
    nbytes = R * Tx * C * 4 * (2 + nb)
    del scratch
    return {"bytes": nbytes, "mean_us": us, "rate": nbytes / us / 1e3, "rate_unit": "GB/s",
            "frac": nbytes / (us * 1e-6) / PEAK_HBM, "flush": "512 MiB device write before each launch",
            "reps": reps}


def host_description():
    """CPU model and the numpy BLAS build the oracle runs on."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or blas
    except Exception:
        pass
    return model, f"numpy {np.__version__}, BLAS {blas}"


def cpu_baseline(s, W, I, max_workers: int):
    """The fp64 oracle on a bounded sample of the workload: one Euler step (of the
    workload's S) for as many requests as there are worker processes (one request per
    process, one BLAS thread each), scaled to estimator evals/s like the GPU figure."""
    from oracle import sampler as O
    variant = (s.norm, s.mlp, s.rope, s.cond_mode == "cross") != ("layer", "gelu", False, False)
    cores = 1 if variant else max(1, min(O.host_cores(), max_workers, s.n_requests))
    reqs = list(range(cores))
    t0 = time.perf_counter()
    if variant:     # the block-variant oracle runs its requests in one process
        from oracle import variants as V
        V.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], 1, s.guidance, requests=reqs)
    else:
        O.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], 1, s.guidance, requests=reqs, workers=cores)
    t = time.perf_counter() - t0
    evals = len(reqs) * s.n_branches * 1
    model, blas = host_description()
    return {"value": evals / t, "unit": "estimator evals/s", "cores": cores, "kind": "oracle",
            "sample": f"{s.name}: 1 of {s.n_steps} Euler steps for {len(reqs)} of {s.n_requests} requests = "
                      f"{evals} row-evaluations of {s.seq_len} frames; fp64 numpy oracle, one process per "
                      f"request with 1 BLAS thread; {t:.1f} s wall",
            "cpu": model, "numpy_blas": blas, "host_cores": O.host_cores(), "seconds": t}


PROBE_BYTES = 1 << 30     # bytes read (and written) by one launch of the copy probe
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_mel_dit.txt")
TRAFFIC_SOURCES = ["gemm_bf16.hip", "epilogue.h", "kernels.h", "common.h", "tile_map.h"]


def traffic_probe():
    """A plain device copy of PROBE_BYTES, three launches: the HBM counters of this kernel,
    divided into the bytes it must move, give the scale of FETCH_SIZE and WRITE_SIZE."""
    import torch
    src = torch.ones(PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "copy", "bytes_read": PROBE_BYTES, "bytes_written": PROBE_BYTES}), flush=True)


def gemm_kscan(reps: int = 10):
    """The block GEMMs of the Mel DiT workload (16 000 tokens) through the GEMM entry point at
    K = 256 .. 4096 with the library's own tile choice: the slope of time over K is the main
    loop's rate, the intercept the fixed cost of a launch (prologue, epilogue, ramp)."""
    import torch
    import flow_matching_tts_amd as F
    M, d, f = 16000, 1024, 2048
    shapes = {"qkv (bf16 out)": (3 * d, 1), "proj / fc2 (gated residual)": (d, 3), "fc1 (GELU)": (f, 2)}
    Ks = [256, 512, 1024, 2048, 4096]
    rng = np.random.default_rng(0)
    A = torch.from_numpy(rng.standard_normal((M, max(Ks)), dtype=np.float32)).to(torch.bfloat16).cuda()
    res = {}
    for name, (N, epi) in shapes.items():
        W = torch.from_numpy(rng.standard_normal((N, max(Ks)), dtype=np.float32) * 0.02).to(torch.bfloat16).cuda()
        bias = torch.zeros(N, dtype=torch.float32, device="cuda")
        gate = torch.ones(N, dtype=torch.float32, device="cuda")
        out = torch.zeros((M, N), dtype=torch.bfloat16 if epi in (1, 2) else torch.float32, device="cuda")
        rows = []
        for K in Ks:
            Ak, Wk = A[:, :K].contiguous(), W[:, :K].contiguous()
            call = lambda: F.gemm_bf16(Ak, Wk, bias, epilogue=epi, out=out, gate=gate)
            call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            rows.append({"K": K, "us": us, "tflops": 2.0 * M * N * K / us / 1e6})
        x = np.array([r["K"] for r in rows], float)
        y = np.array([r["us"] for r in rows])
        slope, icpt = np.polyfit(x, y, 1)
        res[name] = {"N": N, "points": rows, "main_loop_pflops": 2.0 * M * N / slope / 1e9,
                     "fixed_us": float(icpt)}
        log(f"[kscan] {name}: main loop {res[name]['main_loop_pflops']:.3f} PFLOP/s, fixed {icpt:.1f} us")
    print(json.dumps({"gemm_kscan": res, "M": M}), flush=True)


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "flow_matching_tts_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel_class, workload):
    """HBM bytes per launch of the kernel class, from the committed counter summary, or None
    when there is none for this kernel and workload or the kernel sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#") and "=" in line:
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_class") != kernel_class or kv.get("workload") != workload:
        return None
    if kv.get("sources_sha256") != sources_sha256():
        return None
    return float(kv["traffic_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="mel_dit", choices=list(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=16)
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only copy a known number of bytes (calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--gemm-kscan", action="store_true",
                    help="only time the block GEMM shapes at several K (main-loop rate and fixed cost)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one sampling call in a HIP graph and time its replays")
    ap.add_argument("--schedule", default="uniform", choices=["uniform", "quadratic", "trailing", "native"])
    ap.add_argument("--native-steps", type=int, default=None)
    ap.add_argument("--solver", default="euler", choices=["euler", "midpoint"])
    ap.add_argument("--guidance-mode", default="full", choices=["full", "interval", "adaptive"])
    ap.add_argument("--interval", type=float, nargs=2, default=(0.10, 0.70))
    ap.add_argument("--adaptive", type=float, nargs=3, default=(0.015, 4, 2),
                    help="threshold, warm-up steps, patience")
    ap.add_argument("--cache", action="store_true", help="block-residual cache with its default settings")
    args = ap.parse_args()
    if args.gemm_kscan:
        gemm_kscan()
        return
    if args.traffic_probe:
        traffic_probe()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the sampler shards by request "
              f"with no communication during sampling, so a multi-GPU figure is not measured here.",
              file=sys.stderr)
        sys.exit(2)

    s = synth.workload(args.workload)
    nondefault = (args.schedule != "uniform" or args.solver != "euler" or args.guidance_mode != "full"
                  or args.cache)
    if nondefault:   # the per-kernel work model assumes every row at every step
        args.no_kernel_timing = True
    t0 = time.perf_counter()
    W, I = synth.make_weights(s), synth.make_inputs(s)
    log(f"[bench] {s.name}: inputs drawn in {time.perf_counter() - t0:.1f} s")
    base = None
    if not args.no_cpu_baseline:      # before any GPU work: the oracle forks worker processes
        base = cpu_baseline(s, W, I, args.cpu_workers)
        log(f"[bench] cpu baseline: {base['value']:.3f} evals/s ({base['sample']})")

    import torch
    import flow_matching_tts_amd as F
    torch.cuda.set_device(0)
    per_eval = 2 if args.solver == "midpoint" else 1
    smp = F.Sampler(F.config_from_shape(s, max_steps=per_eval * s.n_steps), W)
    x0 = torch.from_numpy(I["x0"]).cuda()
    cond = torch.from_numpy(I["cond"]).cuda()
    spk = None if I["spk"] is None else torch.from_numpy(I["spk"]).cuda()
    mask = None if I["mask"] is None else torch.from_numpy(I["mask"]).cuda()
    out = torch.empty_like(x0)
    guided = torch.zeros(s.n_requests, dtype=torch.int32, device="cuda")
    hits = torch.zeros(1, dtype=torch.int32, device="cuda")
    options = dict(schedule=args.schedule, native_steps=args.native_steps, solver=args.solver,
                   guidance_mode=args.guidance_mode, interval=tuple(args.interval),
                   adaptive=(args.adaptive[0], int(args.adaptive[1]), int(args.adaptive[2])),
                   cache={} if args.cache else None)
    eager = lambda: smp.sample(x0, cond, mask=mask, spk=spk, n_steps=s.n_steps, guidance=s.guidance, out=out,
                               guided_evals=guided, cache_hits=hits, **options)
    run = eager
    if args.graph:
        # the call synchronises nothing and allocates nothing, so one call can be
        # captured whole and replayed on fixed buffers
        eager()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                eager()
        torch.cuda.current_stream().wait_stream(stream)
        run = graph.replay

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run()
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    log(f"[bench] first call {first_ms:.1f} ms; warmup {args.warmup} done")

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] {args.steps} timed steps: {ms:.3f} ms per sampling call")

    torch.cuda.synchronize()
    guided_evals = guided.cpu().tolist()
    cache_hits = int(hits.cpu()[0])
    lengths = I["lengths"]
    rows = s.n_rows
    # estimator row-evaluations actually run: all rows at each evaluation, except the
    # unconditional rows of unguided evaluations and the evaluations cached whole
    n_eval = per_eval * s.n_steps
    row_evals = s.n_requests * n_eval + (s.n_branches - 1) * sum(guided_evals) if s.n_branches > 1 \
        else s.n_requests * n_eval
    evals_s = rows * s.n_steps / (ms / 1e3)
    valid_frames = float(np.sum(np.minimum(lengths, s.n_frames)))
    model = work_model(s, lengths)

    kernels = {}
    if not args.no_kernel_timing:
        # per-class kernel time: one instrumented call per class (events around each launch)
        for cls, (work, launches) in model.items():
            smp.profile_enable(cls, launches + 8)
            eager()
            tot, n, dropped = smp.profile_read()
            smp.profile_disable()
            kernels[cls] = {"ms_per_sample": tot, "launches": n, "mean_us": 1e3 * tot / max(n, 1)}
        dom = max((c for c in kernels), key=lambda c: kernels[c]["ms_per_sample"])
        # the dominant class again, live over the timed steps
        work, launches = model[dom]
        smp.profile_enable(dom, launches * args.steps + 8)
        for _ in range(args.steps):
            eager()
        tot, n, dropped = smp.profile_read()
        smp.profile_disable()
        mean_s = tot / 1e3 / n
        mfma = dom in MFMA_CLASSES
        achieved = work / mean_s
        peak = PEAK_BF16 if mfma else PEAK_HBM
        roofline = {"kernel_class": dom, "bound": "mfma" if mfma else "hbm",
                    "achieved": achieved / (1e12 if mfma else 1e9), "peak": peak / (1e12 if mfma else 1e9),
                    "unit": "TFLOP/s" if mfma else "GB/s", "frac": achieved / peak,
                    "traffic": measured_traffic(dom, s.name),
                    "mean_launch_us": mean_s * 1e6, "launches": n,
                    "work_per_launch": work}
        mf = sum(model[c][0] * model[c][1] for c in MFMA_CLASSES if c in model)
        mt = sum(kernels[c]["ms_per_sample"] for c in MFMA_CLASSES if c in kernels) / 1e3
        gemm_attn_frac = mf / mt / PEAK_BF16
        for c, k in kernels.items():
            work_c, launches_c = model.get(c, (None, None))
            if work_c is None or k["launches"] == 0:
                continue
            rate = work_c * k["launches"] / (k["ms_per_sample"] / 1e3)
            k["rate"] = rate / (1e12 if c in MFMA_CLASSES else 1e9)
            k["rate_unit"] = "TFLOP/s" if c in MFMA_CLASSES else "GB/s"
            k["frac"] = rate / (PEAK_BF16 if c in MFMA_CLASSES else PEAK_HBM)
    else:
        roofline, gemm_attn_frac = None, None
        mf = sum(model[c][0] * model[c][1] for c in MFMA_CLASSES if c in model)
    k1_cold = None if args.no_kernel_timing or s.dtype != "bf16" else cfg_euler_cold(s)

    res = {
        "metric": "estimator evals/sec and latent frames/sec per step; % bf16 MFMA peak",
        "value": evals_s,
        "unit": "estimator evals/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": s.name, "requests": s.n_requests, "branches": s.n_branches, "rows": rows,
                   "frames": s.n_frames, "layers": s.n_layers, "d_model": s.d_model,
                   "heads": s.n_heads, "ffn": s.ffn_dim, "latent": s.latent_dim,
                   "euler_steps": s.n_steps, "guidance": list(s.guidance), "launch": "graph" if args.graph else "eager",
                   "block": {"cond_mode": s.cond_mode, "context_tokens": s.n_prefix if s.cond_mode == "cross" else 0,
                             "norm": s.norm, "mlp": s.mlp, "rope": s.rope},
                   "sampler": {k: (list(v) if isinstance(v, tuple) else v) for k, v in options.items()}},
        "row_evaluations_run": row_evals, "guided_evaluations_per_request": guided_evals, "cache_hits": cache_hits,
        "latent_frame_steps_per_s": valid_frames * s.n_steps / (ms / 1e3),
        "generated_frames_per_s": valid_frames / (ms / 1e3),
        "gemm_attn_frac_bf16_peak": gemm_attn_frac,
        "end_to_end_frac_bf16_peak": mf / (ms / 1e3) / PEAK_BF16,
        "first_call_ms": first_ms,
        "roofline": roofline,
        "cpu_baseline": base,
        "kernels": kernels,
        "cfg_euler_cold": k1_cold,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
