#!/usr/bin/env python3
"""Benchmark of the EXL3 decode-matmul on one MI355X.

Workload (the headline GEMV case): the Llama-3.1-8B-shaped MLP at m=1 -
gate and up 4096->14336 and down 14336->4096 - at K = 2, 3 and 4 bits per
weight.  One step = those 9 projections, inputs resident in HBM: per K, gate
and up in one exl3_gemv_multi launch (they read the same input) and down
through exl3_gemv.
The weight buffers are replicated so that consecutive steps read different
memory (more than 1 GiB in rotation), so the 256 MB Infinity Cache cannot
serve the stream.  Steps run as HIP graphs replayed on one stream.

value = algorithmic bytes of a step / time of a step (GB/s):
  per launch: K/8 bytes per weight + x (2 m n_in) + sign (2 n_in) once, and
  per projection out_scale (2 n_out) + y (2 m n_out).
roofline: the dominant kernel (the fused gate+up launch at K=4), algorithmic
bytes per launch over its average launch time from HIP events around a batch
of back-to-back launches; alu_roofline: the same launch's vector instructions
(committed counters) against the vector-ALU issue peak.
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


def call_bytes(c):
    """Algorithmic bytes of one launch: each projection's weights, scale and y,
    plus x and sign once (they are read once for the whole launch)."""
    b = 2 * c["m"] * c["n_in"] + 2 * c["n_in"]
    for n_out in c["n_outs"]:
        b += c["n_in"] * n_out * c["K"] // 8 + 2 * n_out + 2 * c["m"] * n_out
    return b


def make_call(torch, name, K, n_in, n_outs, m, words_list, x, sign, scales, replicas):
    """Device tensors of one launch (one or more projections of one input)."""
    reps = []
    for w in words_list:
        wd = torch.from_numpy(w.view(np.int16)).cuda()
        reps.append([wd] + [wd.clone() for _ in range(replicas - 1)])
    c = dict(name=name, K=K, n_in=n_in, n_outs=list(n_outs), m=m, words=reps,
             x=torch.from_numpy(x).cuda(), sign=torch.from_numpy(sign).cuda(),
             scales=[torch.from_numpy(sc).cuda() for sc in scales],
             ys=[torch.empty((m, n_out), dtype=torch.float16, device="cuda") for n_out in n_outs])
    c["bytes"] = call_bytes(c)
    return c


def build_mlp(torch, ex, m, Ks=(2, 3, 4), replicas=7, seed_base=0):
    """The MLP launches per K: gate and up in one fused launch (they read the
    same input), then down; `replicas` copies of every weight matrix."""
    import synth
    calls = []
    for K in Ks:
        seeds = {nm: [seed_base, 2, K, i] for i, nm in enumerate(("gate", "up", "down"))}
        words = {nm: synth.words_only(n_in, n_out, K, seeds[nm])
                 for nm, n_in, n_out in (("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096))}
        for name, n_in, members in (("gate_up", 4096, ("gate", "up")), ("down", 14336, ("down",))):
            rng = np.random.default_rng(seeds[members[0]] + [1])
            x = rng.standard_normal((m, n_in)).astype(np.float16)
            sign = (2 * rng.integers(0, 2, n_in) - 1).astype(np.float16)
            n_outs = [words[nm].shape[0] * 16 for nm in members]
            scales = [(rng.uniform(0.5, 1.5, n) * 0.02).astype(np.float16) for n in n_outs]
            calls.append(make_call(torch, f"{name}_k{K}", K, n_in, n_outs, m, [words[nm] for nm in members],
                                   x, sign, scales, replicas))
    return calls


def launch(ex, c, rep):
    cb = c.get("codebook", 0)
    if len(c["n_outs"]) == 1:
        ex.gemv(c["x"], c["words"][0][rep], c["sign"], c["scales"][0], c["K"], y=c["ys"][0], codebook=cb)
    else:
        ex.gemv_multi(c["x"], [(w[rep], sc) for w, sc in zip(c["words"], c["scales"])], c["sign"], c["K"],
                      ys=c["ys"], codebook=cb)


def run_step(ex, calls, rep):
    for c in calls:
        launch(ex, c, rep % len(c["words"][0]))


def time_graphs(torch, ex, calls, replicas, steps, warmup, per_graph=1):
    """ms per step from HIP graphs replayed on one stream.  Graph r holds
    `per_graph` steps on weight replicas r, r+1, ...; short steps need several
    per graph so that the host's replay rate does not set the time."""
    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        run_step(ex, calls, 0)  # first call caches device properties outside capture
    torch.cuda.synchronize()
    for r in range(replicas):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for k in range(per_graph):
                run_step(ex, calls, r + k)
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
    return e0.elapsed_time(e1) / (steps * per_graph), wall


def per_kernel_events(torch, ex, calls, replicas, steps):
    """Average duration of each launch shape: HIP events on the stream the
    library launches on (the current stream) around `steps` back-to-back
    launches of that shape (weight replicas rotating), divided by `steps`."""
    stream = torch.cuda.current_stream()
    ev = []
    for c in calls:
        # a long GPU sleep before each batch, so that all its launches are
        # queued before the GPU reaches them and the events time the GPU, not
        # the host's launch rate
        torch.cuda._sleep(int(5e7))
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            launch(ex, c, i % replicas)
        b.record(stream)
        ev.append((c["name"], a, b))
    torch.cuda.synchronize()
    return {name: a.elapsed_time(b) / steps for name, a, b in ev}


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


def gemm_tflops(torch, ex, iters=5, codebook=0, n_out=8192, K=4):
    """Prefill GEMM: m=2048, 8192->8192 at K=4, or 8192->n_out at K (the second metric)."""
    import synth
    m, n_in = 2048, 8192
    w = torch.from_numpy(synth.words_only(n_in, n_out, K, [0, 4, 9] if (n_out, K) == (8192, 4) else [0, K, 9, n_out])
                         .view(np.int16)).cuda()
    x = torch.randn((m, n_in), device="cuda").half()
    sign = torch.ones(n_in, dtype=torch.float16, device="cuda")
    scale = torch.full((n_out,), 0.02, dtype=torch.float16, device="cuda")
    y = torch.empty((m, n_out), dtype=torch.float16, device="cuda")
    ws = ex.Workspace(n_in, n_out, K, m)
    ex.gemm(x, w, sign, scale, K, workspace=ws, y=y, codebook=codebook)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        ex.gemm(x, w, sign, scale, K, workspace=ws, y=y, codebook=codebook)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    return 2.0 * m * n_in * n_out / (ms * 1e-3) / 1e12, ms


def fp16_matmul_tflops(torch, iters=10):
    """Context for the GEMM: a plain fp16 matrix product of the same shape
    (2048 x 8192 by 8192 x 8192, no decode) through torch's BLAS on the same
    GPU: what the vendor library reaches on this part, at the clock the matrix
    cores hold on random data."""
    m, k, n = 2048, 8192, 8192
    a = torch.randn((m, k), device="cuda").half()
    b = torch.randn((k, n), device="cuda").half()
    c = a @ b
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del a, b, c
    return 2.0 * m * k * n / (ms * 1e-3) / 1e12, ms


def cpu_baseline():
    """The CPU oracle on a bounded sample of the workload: the K=4 MLP at m=1
    (gate and up 4096->14336, down 14336->4096), one BLAS thread."""
    import synth
    from oracle import exl3_oracle as O
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    K, m = 4, 1
    mats = [(nm, n_in, n_out, [0, 2, K, i]) for i, (nm, n_in, n_out) in
            enumerate((("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)))]
    inputs = []
    for nm, n_in, n_out, seed in mats:
        w = synth.words_only(n_in, n_out, K, seed)
        rng = np.random.default_rng(seed + [1])
        x = rng.standard_normal((m, n_in)).astype(np.float16)
        sign = (2 * rng.integers(0, 2, n_in) - 1).astype(np.float16)
        scale = (rng.uniform(0.5, 1.5, n_out) * 0.02).astype(np.float16)
        inputs.append((w, x, sign, scale, gemv_bytes(n_in, n_out, K, m)))
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    t0 = time.perf_counter()
    for w, x, sign, scale, _ in inputs:
        O.linear(x, w, sign, scale, K)
    dt = time.perf_counter() - t0
    if ctx is not None and hasattr(ctx, "unregister"):
        ctx.unregister()
    nbytes = sum(i[-1] for i in inputs)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the K=4 MLP at m=1 (gate, up 4096->14336, down 14336->4096; 3 of the 9 projections "
                      f"of a step), {dt:.1f} s, numpy fp64, BLAS limited to 1 thread"}


def kernel_sources_hash() -> str:
    """Hash of the GEMV kernel and launch-plan sources with their comments and
    blank lines removed: counter-derived figures are valid only for this code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("exl3_device.hpp", "exl3_internal.hpp", "exl3_kernels.hip", "exl3_api.hip"):
        with open(os.path.join(ROOT, "decode_gemm_exl3_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln.strip()).encode())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    profile (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when the
    kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "gemv_gate_up_k4_llama8b_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_hash") != kernel_sources_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


# Vector-ALU issue peak of MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# (one 32-bit lane-operation per lane and clock; a wave64 instruction takes
# four clocks of a SIMD).
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9


def alu_roofline(ms_per_launch):
    """The same launch against the vector-ALU issue peak: the decode makes the
    GEMV issue-bound at K <= 4, so this is the roofline that binds."""
    n = recorded_valu_insts()
    if n is None:
        return None
    achieved = n * 64 / (ms_per_launch * 1e-3)
    return {"bound": "alu", "kernel": "gemv_kernel<K=4> gate+up 4096->2x14336",
            "achieved": round(achieved / 1e12, 2), "peak": round(VALU_PEAK_LANE_OPS / 1e12, 2),
            "unit": "T lane-ops/s", "frac": round(achieved / VALU_PEAK_LANE_OPS, 4),
            "valu_insts_per_launch": int(n)}


def recorded_valu_insts():
    """Vector-ALU instructions (MFMAs excluded) per launch of the dominant
    kernel from the committed counter profile, or None when the kernel
    sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "gemv_gate_up_k4_llama8b_issue.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_hash") != kernel_sources_hash():
        return None
    return rec.get("valu_insts_without_mfma")


def stack_tokens_per_s(torch, ex, fused=True, reps=20):
    """32-layer Llama-3.1-8B-shaped stack at m=1: tokens/s = 1 / (one graph
    replay of every projection of every layer, in model order, on one stream).
    fused: q/k/v and gate/up each in one launch (128 launches), else one launch
    per matmul (224).  The stack's weights (about 4 GB) exceed every cache."""
    import synth
    groups = synth.llama8b_stack_groups()
    calls = []
    for grp in groups:
        parts = [grp] if fused else [[mm] for mm in grp]
        for part in parts:
            words, x, sign, scales = synth.draw_group(part)
            calls.append(make_call(torch, "+".join(mm.name for mm in part), part[0].K, part[0].n_in,
                                   [mm.n_out for mm in part], 1, words, x, sign, scales, 1))
    nbytes = sum(c["bytes"] for c in calls)
    ms, _ = time_graphs(torch, ex, calls, 1, reps, 3)
    out = {"tokens_per_s": round(1e3 / ms, 1), "ms_per_token": round(ms, 4), "launches": len(calls),
           "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes_per_token": nbytes}
    del calls
    torch.cuda.empty_cache()
    return out


def llama70b_rates(torch, ex, replicas=3, steps=20):
    """70B-shaped decode GEMVs at m=1: GB/s of each launch shape."""
    import synth
    out = {}
    for name, n_in, n_outs, K in (("gate_up_k2", 8192, (28672, 28672), 2), ("gate_up_k3", 8192, (28672, 28672), 3),
                                  ("down_k2", 28672, (8192,), 2), ("down_k3", 28672, (8192,), 3),
                                  ("attn_k4", 8192, (8192,), 4)):
        words = [synth.words_only(n_in, n, K, [0, 3, 100 + i, K]) for i, n in enumerate(n_outs)]
        rng = np.random.default_rng([0, 3, 200, K, n_in])
        x = rng.standard_normal((1, n_in)).astype(np.float16)
        sign = (2 * rng.integers(0, 2, n_in) - 1).astype(np.float16)
        scales = [(rng.uniform(0.5, 1.5, n) * 0.02).astype(np.float16) for n in n_outs]
        c = make_call(torch, name, K, n_in, n_outs, 1, words, x, sign, scales, replicas)
        ms, _ = time_graphs(torch, ex, [c], replicas, steps, 3, per_graph=12)
        out[name] = {"gbs": round(c["bytes"] / (ms * 1e-3) / 1e9, 1), "us": round(ms * 1e3, 2)}
        del c
        torch.cuda.empty_cache()
    return out


def medium_m(torch, ex, ms=(16, 32, 64, 128, 256), n_in=4096, n_out=14336, K=4, replicas=4):
    """Batched decode and chunked prefill sizes through exl3_linear (the GEMV or
    the split GEMM, as its table picks): us per call, weight GB/s and TFLOP/s."""
    import synth
    w = torch.from_numpy(synth.words_only(n_in, n_out, K, [0, 8, K]).view(np.int16)).cuda()
    reps = [w] + [w.clone() for _ in range(replicas - 1)]
    sign = torch.ones(n_in, dtype=torch.float16, device="cuda")
    scale = torch.full((n_out,), 0.02, dtype=torch.float16, device="cuda")
    ws = ex.Workspace(n_in, n_out, K, max(ms))
    out = {}
    for m in ms:
        x = torch.randn((m, n_in), device="cuda").half()
        y = torch.empty((m, n_out), dtype=torch.float16, device="cuda")
        for i in range(2):
            ex.linear(x, reps[i % replicas], sign, scale, K, workspace=ws, y=y)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=st):
            for i in range(8):
                ex.linear(x, reps[i % replicas], sign, scale, K, workspace=ws, y=y)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 40 * 1e3
        out[f"m{m}"] = {"us": round(us, 1), "weight_gbs": round(n_in * n_out * K / 8 / us / 1e3, 1),
                        "tflops": round(2.0 * m * n_in * n_out / us / 1e6, 1)}
    return out


def encode_rates(torch, ex, n_tiles=2048, Ks=(2, 3, 4)):
    """Tail-biting Viterbi encoder: tiles/s on unit-Gaussian tiles and the mean
    squared error per weight it reaches."""
    out = {}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    for K in Ks:
        w = torch.randn((n_tiles, 256), device="cuda", generator=gen)
        ws = torch.empty(ex.encode_slot_bytes(K) * min(n_tiles, 1024), dtype=torch.uint8, device="cuda")
        ex.encode_tiles(w[:64], K, workspace=ws)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        _, costs = ex.encode_tiles(w, K, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        out[f"k{K}"] = {"tiles_per_s": round(n_tiles / ms * 1e3), "mse": round(float(costs.mean()) / 256, 5),
                        "s_per_4096x4096": round(65536 / n_tiles * ms / 1e3, 3)}
        del w, ws
    return out


def only_mode(what, steps, replicas):
    """Short runs for the profiler: the fused gate+up launch at K=4 alone (the
    dominant kernel), the m=2048 8192->8192 K=4 GEMM, or a plain copy of known
    size."""
    import torch
    import decode_gemm_exl3_amd as ex
    if what == "gemm":
        tf, ms = gemm_tflops(torch, ex, iters=steps)
        print(json.dumps({"gemm_m2048_8192x8192_k4": {"launches": steps + 1, "tflops": round(tf, 1)}}), flush=True)
        return
    if what == "copy":
        nbytes = 256 << 20
        a = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda")
        b = torch.empty_like(a)
        for _ in range(steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each": nbytes, "copies": steps}), flush=True)
        return
    calls = [c for c in build_mlp(torch, ex, 1, Ks=(4,), replicas=replicas) if c["name"] == "gate_up_k4"]
    for i in range(steps):
        run_step(ex, calls, i % replicas)
    torch.cuda.synchronize()
    print(json.dumps({"launches": {c["name"]: steps for c in calls},
                      "bytes_per_launch": {c["name"]: c["bytes"] for c in calls}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=7)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="headline line only (no m=4/8, GEMM, 70B, stack)")
    ap.add_argument("--only", choices=["gate_up_k4", "gemm", "copy"], help="profiling runs: one launch shape only")
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

    calls = build_mlp(torch, ex, 1, replicas=args.replicas)
    step_bytes = sum(c["bytes"] for c in calls)
    ms, wall = time_graphs(torch, ex, calls, args.replicas, args.steps, args.warmup)
    value = step_bytes / (ms * 1e-3) / 1e9

    kdur = per_kernel_events(torch, ex, calls, args.replicas, max(10, min(args.steps, 50)))
    launches = {c["name"]: {"us": round(1e3 * kdur[c["name"]], 2),
                            "gbs": round(c["bytes"] / (kdur[c["name"]] * 1e-3) / 1e9, 1)} for c in calls}
    per_k = {}
    for K in (2, 3, 4):
        sel = [c for c in calls if c["K"] == K]
        b = sum(c["bytes"] for c in sel)
        t = sum(kdur[c["name"]] for c in sel)
        per_k[f"k{K}"] = {"gbs": round(b / (t * 1e-3) / 1e9, 1)}
    dom = next(c for c in calls if c["name"] == "gate_up_k4")
    dom_ms = kdur[dom["name"]]
    achieved = dom["bytes"] / (dom_ms * 1e-3) / 1e9

    extra = {"launches_m1": launches, "per_bits_m1": per_k, "copy_gbs": round(copy_bandwidth(torch), 1),
             "step_bytes": step_bytes, "wall_s": round(wall, 3)}
    del calls
    torch.cuda.empty_cache()
    if not args.no_extra:
        for m in (4, 8):
            calls = build_mlp(torch, ex, m, replicas=args.replicas)
            msm, _ = time_graphs(torch, ex, calls, args.replicas, max(20, args.steps // 4), 5)
            extra[f"m{m}_gbs"] = round(sum(c["bytes"] for c in calls) / (msm * 1e-3) / 1e9, 1)
            del calls
            torch.cuda.empty_cache()
        tf, gms = gemm_tflops(torch, ex)
        tfr, rms = fp16_matmul_tflops(torch)
        extra["gemm_m2048_8192x8192_k4"] = {"tflops": round(tf, 1), "ms": round(gms, 3),
                                            "frac_of_mfma_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                                            "plain_fp16_matmul_same_shape": {"tflops": round(tfr, 1),
                                                                             "ms": round(rms, 3)}}
        tf3, gms3 = gemm_tflops(torch, ex, n_out=28672, K=3)
        extra["gemm_m2048_8192x28672_k3"] = {"tflops": round(tf3, 1), "ms": round(gms3, 3),
                                             "frac_of_mfma_f16_peak": round(tf3 / MFMA_F16_PEAK_TFLOPS, 4)}
        extra["llama70b_m1"] = llama70b_rates(torch, ex)
        extra["encode"] = encode_rates(torch, ex)
        extra["medium_m_4096x14336_k4"] = medium_m(torch, ex)
        # the byte-sum (dp4a) codebook on the K=4 MLP launches and the GEMM
        calls = build_mlp(torch, ex, 1, Ks=(4,), replicas=args.replicas)
        for c in calls:
            c["codebook"] = 1
        kd1 = per_kernel_events(torch, ex, calls, args.replicas, 20)
        tf1, gms1 = gemm_tflops(torch, ex, codebook=1)
        extra["codebook1"] = {c["name"]: {"us": round(1e3 * kd1[c["name"]], 2),
                                          "gbs": round(c["bytes"] / (kd1[c["name"]] * 1e-3) / 1e9, 1)} for c in calls}
        extra["codebook1"]["gemm_m2048_8192x8192_k4"] = {"tflops": round(tf1, 1), "ms": round(gms1, 3)}
        del calls
        torch.cuda.empty_cache()
        extra["llama8b_stack_m1"] = {"fused": stack_tokens_per_s(torch, ex, True),
                                     "unfused": stack_tokens_per_s(torch, ex, False)}

    rec = {
        "metric": "EXL3 GEMV achieved HBM GB/s at m=1 (Llama-3.1-8B MLP, K=2,3,4)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "llama3.1-8b-mlp-gemv: gate/up 4096->14336 (one fused launch), down 14336->4096, "
                               "K in {2,3,4}, m=1, 6 launches (9 projections) per step",
                   "m": 1, "bits": [2, 3, 4], "weight_replicas": args.replicas},
        "roofline": {"bound": "hbm", "kernel": "gemv_kernel<K=4> gate+up 4096->2x14336",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic()},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "alu_roofline": alu_roofline(dom_ms),
        "extra": extra,
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
