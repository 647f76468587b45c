#!/usr/bin/env python3
"""Benchmark of the EXL3 decode-matmul on one MI355X.

Workload (the headline GEMV case): the Llama-3.1-8B-shaped MLP at m=1 -
gate and up 4096->14336 and down 14336->4096 - at K = 2, 3 and 4 bits per
weight.  One step = those 9 GEMVs through exl3_gemv, inputs resident in HBM.
The weight buffers are replicated so that consecutive steps read different
memory (more than 1 GiB in rotation), so the 256 MB Infinity Cache cannot
serve the stream.  Steps run as HIP graphs replayed on one stream.

value = algorithmic bytes of a step / time of a step (GB/s):
  per GEMV: K/8 bytes per weight + x (2 m n_in) + sign (2 n_in) + out_scale
  (2 n_out) + y (2 m n_out).
roofline: the dominant kernel (gemv at K=4), algorithmic bytes per launch over
its average launch time from HIP events around each launch.
cpu_baseline: the CPU oracle on a bounded sample of the same workload.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def gemv_bytes(n_in, n_out, K, m):
    return n_in * n_out * K // 8 + 2 * m * n_in + 2 * n_in + 2 * n_out + 2 * m * n_out


def build_mlp(torch, ex, m, Ks=(2, 3, 4), replicas=7, seed_base=0):
    """Device tensors for the MLP GEMVs: per K, gate/up/down, `replicas` copies each."""
    import synth
    cases = []
    for K in Ks:
        for name, n_in, n_out in (("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)):
            seed = [seed_base, 2, K, {"gate": 0, "up": 1, "down": 2}[name]]
            w = synth.words_only(n_in, n_out, K, seed)
            rng = np.random.default_rng(seed + [1])
            x = rng.standard_normal((m, n_in)).astype(np.float16)
            sign = (2 * rng.integers(0, 2, n_in) - 1).astype(np.float16)
            scale = (rng.uniform(0.5, 1.5, n_out) * 0.02).astype(np.float16)
            wd = torch.from_numpy(w.view(np.int16)).cuda()
            reps = [wd] + [wd.clone() for _ in range(replicas - 1)]
            cases.append(dict(name=f"{name}_k{K}", K=K, n_in=n_in, n_out=n_out, m=m, words=reps,
                              x=torch.from_numpy(x).cuda(), sign=torch.from_numpy(sign).cuda(),
                              scale=torch.from_numpy(scale).cuda(),
                              y=torch.empty((m, n_out), dtype=torch.float16, device="cuda"),
                              bytes=gemv_bytes(n_in, n_out, K, m)))
    ws = ex.Workspace(14336, 14336, 8, 8)
    return cases, ws


def run_step(ex, cases, ws, rep):
    for c in cases:
        ex.gemv(c["x"], c["words"][rep], c["sign"], c["scale"], c["K"], workspace=ws, y=c["y"])


def time_graphs(torch, ex, cases, ws, replicas, steps, warmup):
    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        run_step(ex, cases, ws, 0)  # first call caches device properties outside capture
    torch.cuda.synchronize()
    for r in range(replicas):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run_step(ex, cases, ws, r)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % replicas].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            graphs[i % replicas].replay()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def per_kernel_events(torch, ex, cases, ws, replicas, steps):
    """Average duration of each launch, from events on the launching stream."""
    stream = torch.cuda.current_stream()
    ev = []
    for i in range(steps):
        for c in cases:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            ex.gemv(c["x"], c["words"][i % replicas], c["sign"], c["scale"], c["K"], workspace=ws, y=c["y"])
            b.record(stream)
            ev.append((c["name"], c["K"], a, b))
    torch.cuda.synchronize()
    dur = {}
    for name, K, a, b in ev:
        dur.setdefault((name, K), []).append(a.elapsed_time(b))
    return {k: float(np.mean(v)) for k, v in dur.items()}


def copy_bandwidth(torch, nbytes=1 << 30, iters=10):
    a = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9


def gemm_tflops(torch, ex, iters=5):
    """Prefill GEMM: m=2048, 8192->8192 at K=4 (context figure for the second metric)."""
    import synth
    m, n_in, n_out, K = 2048, 8192, 8192, 4
    w = torch.from_numpy(synth.words_only(n_in, n_out, K, [0, 4, 9]).view(np.int16)).cuda()
    x = torch.randn((m, n_in), device="cuda").half()
    sign = torch.ones(n_in, dtype=torch.float16, device="cuda")
    scale = torch.full((n_out,), 0.02, dtype=torch.float16, device="cuda")
    y = torch.empty((m, n_out), dtype=torch.float16, device="cuda")
    ws = ex.Workspace(n_in, n_out, K, m)
    ex.gemm(x, w, sign, scale, K, workspace=ws, y=y)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        ex.gemm(x, w, sign, scale, K, workspace=ws, y=y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    return 2.0 * m * n_in * n_out / (ms * 1e-3) / 1e12, ms


def cpu_baseline(strips=896):
    """CPU oracle on a bounded sample: gate 4096->14336 at K=4, m=1, `strips` 16-row strips."""
    import synth
    from oracle import exl3_oracle as O
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    n_in, n_out, K, m = 4096, 14336, 4, 1
    w = synth.words_only(n_in, n_out, K, [0, 2, K, 0])[:strips]
    rng = np.random.default_rng([0, 2, K, 0, 1])
    x = rng.standard_normal((m, n_in)).astype(np.float16)
    sign = (2 * rng.integers(0, 2, n_in) - 1).astype(np.float16)
    scale = (rng.uniform(0.5, 1.5, 16 * strips) * 0.02).astype(np.float16)
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    t0 = time.perf_counter()
    O.linear(x, w, sign, scale, K)
    dt = time.perf_counter() - t0
    if ctx is not None:
        ctx.unregister() if hasattr(ctx, "unregister") else None
    nbytes = gemv_bytes(n_in, 16 * strips, K, m)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"gate 4096->{16 * strips} (first {strips} of 896 strips) K=4 m=1, "
                      f"{dt:.1f} s, numpy fp64, BLAS limited to 1 thread"}


def kernel_sources_hash() -> str:
    """Hash of the GEMV kernel sources: counter-derived traffic is valid only for them."""
    import hashlib
    h = hashlib.sha256()
    for f in ("exl3_device.hpp", "exl3_kernels.hip"):
        with open(os.path.join(ROOT, "decode_gemm_exl3_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    profile (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when the
    kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "gemv_k4_llama8b_mlp_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_hash") != kernel_sources_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def only_mode(what, steps, replicas):
    """Short runs for the profiler: the dominant GEMV alone, or a plain copy."""
    import torch
    import decode_gemm_exl3_amd as ex
    if what == "copy":
        nbytes = 256 << 20
        a = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda")
        b = torch.empty_like(a)
        for _ in range(steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each": nbytes, "copies": steps}), flush=True)
        return
    cases, ws = build_mlp(torch, ex, 1, Ks=(4,), replicas=replicas)
    for i in range(steps):
        run_step(ex, cases, ws, i % replicas)
    torch.cuda.synchronize()
    print(json.dumps({"gemv_k4_launches": steps * len(cases),
                      "bytes_per_launch": [c["bytes"] for c in cases]}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=7)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--only", choices=["gemv_k4", "copy"], help="profiling runs: one kernel family only")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_gemm_exl3_amd as ex
    ex.load()
    torch.cuda.init()
    if args.only:
        only_mode(args.only, args.steps, args.replicas)
        return

    cases, ws = build_mlp(torch, ex, 1, replicas=args.replicas)
    step_bytes = sum(c["bytes"] for c in cases)
    ms, wall = time_graphs(torch, ex, cases, ws, args.replicas, args.steps, args.warmup)
    value = step_bytes / (ms * 1e-3) / 1e9

    kdur = per_kernel_events(torch, ex, cases, ws, args.replicas, max(10, min(args.steps, 50)))
    per_k = {}
    for K in (2, 3, 4):
        names = [c for c in cases if c["K"] == K]
        b = sum(c["bytes"] for c in names)
        t = sum(kdur[(c["name"], K)] for c in names)
        per_k[f"k{K}"] = {"gbs": round(b / (t * 1e-3) / 1e9, 1), "us_per_launch": round(1e3 * t / len(names), 2)}
    dom = [c for c in cases if c["K"] == 4]
    dom_bytes = float(np.mean([c["bytes"] for c in dom]))
    dom_ms = float(np.mean([kdur[(c["name"], 4)] for c in dom]))
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9

    extra = {"per_bits_m1": per_k, "copy_gbs": round(copy_bandwidth(torch), 1),
             "step_bytes": step_bytes, "wall_s": round(wall, 3)}
    for m in (4, 8):
        del cases
        torch.cuda.empty_cache()
        cases, ws = build_mlp(torch, ex, m, replicas=args.replicas)
        msm, _ = time_graphs(torch, ex, cases, ws, args.replicas, max(20, args.steps // 4), 5)
        extra[f"m{m}_gbs"] = round(sum(c["bytes"] for c in cases) / (msm * 1e-3) / 1e9, 1)
    del cases
    torch.cuda.empty_cache()
    if not args.no_gemm:
        tf, gms = gemm_tflops(torch, ex)
        extra["gemm_m2048_8192x8192_k4"] = {"tflops": round(tf, 1), "ms": round(gms, 3),
                                            "frac_of_mfma_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}

    rec = {
        "metric": "EXL3 GEMV achieved HBM GB/s at m=1 (Llama-3.1-8B MLP, K=2,3,4)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "llama3.1-8b-mlp-gemv: gate/up 4096->14336, down 14336->4096, "
                               "K in {2,3,4}, m=1, 9 GEMVs per step",
                   "m": 1, "bits": [2, 3, 4], "weight_replicas": args.replicas},
        "roofline": {"bound": "hbm", "kernel": "gemv_kernel<K=4>", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic()},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "extra": extra,
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
