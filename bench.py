#!/usr/bin/env python3
"""Benchmark of the EXL3 decode-matmul on one MI355X.

Headline workload: the 32-layer Llama-3.1-8B-shaped linear stack at m=1 (per
layer q 4096->4096, k/v 4096->1024, o 4096->4096, gate/up 4096->14336, down
14336->4096; per-layer K drawn from {2..6}, attention +1 bit; 224 matmuls, about
4 GB of packed weights).  One step = one token: every matmul of every layer, in
model order, on one stream, q/k/v and gate/up each in one exl3_gemv_multi launch
(128 launches), replayed as one HIP graph.  Inputs are resident in HBM; the
stack's weights exceed every cache, so each step streams them from HBM.

value = algorithmic bytes of a step / time of a step (GB/s):
  per launch: K/8 bytes per weight + x (2 m n_in) + sign (2 n_in) once, and per
  projection out_scale (2 n_out) + y (2 m n_out).
roofline: the launch shape with the largest share of the step's time (count in
  the step x its average duration), its algorithmic bytes per launch over its
  average duration from HIP events around back-to-back launches on the stream
  they run on, with at least 1 GiB of distinct weights in rotation; beside it
  the median of the committed rocprofv3 kernel trace of the same launch shape
  and the HBM traffic from the committed counters (both only while the kernel
  sources are those they were taken on).
cpu_baseline: the CPU oracle on a bounded sample of every workload (decode and
  contraction timed apart, all host cores), run before the GPU is touched.
extra: every other workload (the single 4096x4096 layer, the 8B MLP at m = 1,
  4, 8, the 70B launches, the m=2048 GEMMs, medium m, codebook 1, the encoder,
  the unfused stack, a device copy), each per-launch figure over at least 1 GiB
  of distinct weights in rotation.

Prints one JSON line.  --only runs one launch shape for the profiler;
--trace-summary summarises a rocprofv3 kernel trace.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
GIB = 1 << 30
# Vector-ALU issue peak of MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# (one 32-bit lane-operation per lane and clock; a wave64 instruction takes
# four clocks of a SIMD).
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9


# ----------------------------------------------------------------- launches --
def launch_bytes(launch) -> int:
    """Algorithmic bytes of one launch: each projection's weights, scale and y,
    plus x and sign once (they are read once for the whole launch)."""
    m, n_in, K = launch.m, launch.n_in, launch.K
    b = 2 * m * n_in + 2 * n_in
    for n_out in launch.n_outs:
        b += n_in * n_out * K // 8 + 2 * n_out + 2 * m * n_out
    return b


def weight_bytes(launch) -> int:
    return sum(mm.trellis_bytes for mm in launch.members)


def replicas_for(launch, min_bytes=GIB) -> int:
    """Copies of the weights so that at least min_bytes of distinct weights
    rotate (the 256 MB Infinity Cache then cannot serve a repeated launch)."""
    return max(1, math.ceil(min_bytes / weight_bytes(launch)))


def stack_kind(launch) -> str:
    names = [mm.name.split(".")[1].split("_k")[0] for mm in launch.members]
    return {"q+k+v": "qkv"}.get("+".join(names), "+".join(names).replace("gate+up", "gate_up"))


class DevLaunch:
    """Device tensors of one launch: `replicas` copies of every weight matrix,
    one input, scales and outputs; `fn` is the binding call that runs it."""

    def __init__(self, torch, ex, launch, fn, replicas=1, workspace=None, codebook=0, name=None):
        import synth
        words, x, sign, scales = synth.draw_group(launch.members)
        self.launch, self.fn, self.cb, self.ws = launch, fn, codebook, workspace
        self.name = name or launch.name
        self.words = []
        for w in words:
            wd = torch.from_numpy(w.view(np.int16)).cuda()
            self.words.append([wd] + [wd.clone() for _ in range(replicas - 1)])
        self.replicas = replicas
        self.x = torch.from_numpy(x).cuda()
        self.sign = torch.from_numpy(sign).cuda()
        self.scales = [torch.from_numpy(sc).cuda() for sc in scales]
        self.ys = [torch.empty((launch.m, n), dtype=torch.float16, device="cuda") for n in launch.n_outs]
        self.bytes = launch_bytes(launch)

    def call(self, ex, rep=0):
        r = rep % self.replicas
        if self.fn == "gemv_multi":
            ex.gemv_multi(self.x, [(w[r], sc) for w, sc in zip(self.words, self.scales)], self.sign, self.launch.K,
                          ys=self.ys, workspace=self.ws, codebook=self.cb)
        else:
            getattr(ex, self.fn)(self.x, self.words[0][r], self.sign, self.scales[0], self.launch.K,
                                 workspace=self.ws, y=self.ys[0], codebook=self.cb)


def gemv_fn(launch) -> str:
    return "gemv_multi" if len(launch.members) > 1 else "gemv"


def time_events(torch, ex, dl, n):
    """Average ms per launch: HIP events on the stream the library launches on
    (the current stream) around n back-to-back launches, weight replicas
    rotating.  A GPU sleep first, so that every launch is queued before the GPU
    reaches it and the events time the GPU, not the host's launch rate."""
    dl.call(ex, 0)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    torch.cuda._sleep(int(5e7))
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        dl.call(ex, i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def time_graphs(torch, ex, step_fn, variants, steps, warmup, per_graph=1):
    """ms per step from HIP graphs replayed on one stream.  Graph v holds
    `per_graph` steps on weight replicas v, v+1, ...; short steps need several
    per graph so that the host's replay rate does not set the time.  The timed
    region is bracketed by synchronisations and HIP events on the replay
    stream."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step_fn(0)  # first call caches device properties outside capture
    torch.cuda.synchronize()
    graphs = []
    for v in range(variants):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for k in range(per_graph):
                step_fn(v + k)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % variants].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            graphs[i % variants].replay()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / (steps * per_graph), wall


def gbs(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


# -------------------------------------------------------- the 8B stack ------
def stack_launches(fused=True):
    import synth
    if fused:
        return [synth.Launch("+".join(mm.name for mm in g), g) for g in synth.llama8b_stack_groups()]
    return [synth.Launch(mm.name, [mm]) for mm in synth.llama8b_stack()]


def stack_shapes(launches):
    """Distinct launch shapes of the stack: key -> (count, first launch)."""
    shapes = {}
    for lc in launches:
        key = f"{stack_kind(lc)}_k{lc.K}"
        cnt, first = shapes.get(key, (0, lc))
        shapes[key] = (cnt + 1, first)
    return shapes


def stack_run(torch, ex, steps, warmup, fused=True):
    """Tokens/s of the stack: one HIP graph of every launch of a token."""
    launches = stack_launches(fused)
    dls = [DevLaunch(torch, ex, lc, gemv_fn(lc)) for lc in launches]
    nbytes = sum(d.bytes for d in dls)

    def step(_v):
        for d in dls:
            d.call(ex, 0)

    ms, wall = time_graphs(torch, ex, step, 1, steps, warmup)
    del dls
    torch.cuda.empty_cache()
    return {"tokens_per_s": round(1e3 / ms, 1), "ms_per_token": round(ms, 5), "launches": len(launches),
            "gbs": round(gbs(nbytes, ms), 1), "bytes_per_token": nbytes, "wall_s": round(wall, 3)}


def stack_shape_times(torch, ex, n=50):
    """Average duration of every distinct launch shape of the fused stack, over
    >= 1 GiB of weights in rotation, and its share of a token's time."""
    out = {}
    for key, (cnt, lc) in stack_shapes(stack_launches(True)).items():
        dl = DevLaunch(torch, ex, lc, gemv_fn(lc), replicas=replicas_for(lc))
        ms = time_events(torch, ex, dl, max(n, dl.replicas))
        out[key] = {"count": cnt, "us": round(ms * 1e3, 3), "bytes_per_launch": dl.bytes,
                    "gbs": round(gbs(dl.bytes, ms), 1), "rotation_bytes": dl.replicas * weight_bytes(lc),
                    "n_in": lc.n_in, "n_outs": lc.n_outs, "K": lc.K, "total_us": round(cnt * ms * 1e3, 2)}
        del dl
        torch.cuda.empty_cache()
    total = sum(v["total_us"] for v in out.values())
    for v in out.values():
        v["share"] = round(v["total_us"] / total, 4)
    return out


# -------------------------------------------------------------- profiles ----
GEMV_SOURCES = ("exl3_device.hpp", "exl3_internal.hpp", "exl3_kernels.hip", "exl3_api.hip")
GEMM_SOURCES = ("exl3_device.hpp", "exl3_internal.hpp", "exl3_kernels.hip", "exl3_api.hip", "exl3_gemm.hip")
ENCODE_SOURCES = ("exl3_device.hpp", "exl3_internal.hpp", "exl3_api.hip", "exl3_encode.hip")


def kernel_sources_hash(files=GEMV_SOURCES) -> str:
    """Hash of the kernel and launch-plan sources (the GEMV's by default, the
    GEMM's with its rotation pre-pass otherwise) with comments and blank lines
    removed: profile-derived figures are valid only for this code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "decode_gemm_exl3_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln.strip()).encode())
    return h.hexdigest()[:16]


def profile_record(name):
    """A committed profile summary (JSON) of the current sources, or None."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("kernel_sources_hash") == kernel_sources_hash() else None


# ----------------------------------------------------------- other configs --
def single_layer_rate(torch, ex, n=128):
    """The single 4096x4096 layer at K=4, m=1 through exl3_gemv, 128 copies of
    its 8 MiB of weights in rotation."""
    import synth
    mm = synth.single_layer()[0]
    lc = synth.Launch(mm.name, [mm])
    dl = DevLaunch(torch, ex, lc, "gemv", replicas=replicas_for(lc))
    ms = time_events(torch, ex, dl, max(n, dl.replicas))
    out = {"us": round(ms * 1e3, 3), "gbs": round(gbs(dl.bytes, ms), 1), "bytes": dl.bytes,
           "rotation_bytes": dl.replicas * weight_bytes(lc)}
    del dl
    torch.cuda.empty_cache()
    return out


def mlp_rates(torch, ex, m, steps, n=50):
    """The 8B MLP at m rows, K = 2, 3, 4 (gate+up fused, down): per-launch
    figures over >= 1 GiB of rotation, and the step of all six launches as
    graphs over enough replicas to rotate >= 1 GiB."""
    import synth
    ws = ex.Workspace(14336, 14336, 8, m)
    launches = [lc for K in (2, 3, 4) for lc in synth.mlp_launches(K, m)]
    per = {}
    for lc in launches:
        dl = DevLaunch(torch, ex, lc, gemv_fn(lc), replicas=replicas_for(lc), workspace=ws)
        ms = time_events(torch, ex, dl, max(n, dl.replicas))
        per[lc.name] = {"us": round(ms * 1e3, 3), "gbs": round(gbs(dl.bytes, ms), 1),
                        "rotation_bytes": dl.replicas * weight_bytes(lc)}
        del dl
        torch.cuda.empty_cache()
    step_w = sum(weight_bytes(lc) for lc in launches)
    reps = max(1, math.ceil(GIB / step_w))
    dls = [DevLaunch(torch, ex, lc, gemv_fn(lc), replicas=reps, workspace=ws) for lc in launches]
    nbytes = sum(d.bytes for d in dls)

    def step(v):
        for d in dls:
            d.call(ex, v)

    ms, _ = time_graphs(torch, ex, step, reps, steps, 5)
    del dls
    torch.cuda.empty_cache()
    return {"step_gbs": round(gbs(nbytes, ms), 1), "step_us": round(ms * 1e3, 2),
            "step_rotation_bytes": reps * step_w, "launches": per}


def llama70b_rates(torch, ex, n=40):
    import synth
    ws = ex.Workspace(28672, 28672, 8, 1)
    out = {}
    for lc in synth.llama70b_launches():
        dl = DevLaunch(torch, ex, lc, gemv_fn(lc), replicas=replicas_for(lc), workspace=ws)
        ms = time_events(torch, ex, dl, max(n, dl.replicas))
        out[lc.name] = {"us": round(ms * 1e3, 2), "gbs": round(gbs(dl.bytes, ms), 1),
                        "rotation_bytes": dl.replicas * weight_bytes(lc)}
        del dl
        torch.cuda.empty_cache()
    return out


def gemm_rate(torch, ex, which, codebook=0, n=None):
    """Prefill GEMM at m=2048 (8192->8192 K=4 or 8192->28672 K=3), the whole
    call (rotation pre-pass and GEMM) timed by events, weights rotating over
    >= 1 GiB."""
    import synth
    mm = synth.prefill_gemm()[0 if which == "8192_k4" else 1]
    lc = synth.Launch(mm.name, [mm])
    ws = ex.Workspace(mm.n_in, mm.n_out, mm.K, mm.m)
    dl = DevLaunch(torch, ex, lc, "gemm", replicas=replicas_for(lc), workspace=ws, codebook=codebook)
    ms = time_events(torch, ex, dl, n or max(20, dl.replicas))
    tf = 2.0 * mm.m * mm.n_in * mm.n_out / (ms * 1e-3) / 1e12
    out = {"tflops": round(tf, 1), "us": round(ms * 1e3, 1), "frac_of_mfma_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
           "rotation_bytes": dl.replicas * weight_bytes(lc)}
    del dl, ws
    torch.cuda.empty_cache()
    return out


def fp16_matmul_tflops(torch, iters=10):
    """Context for the GEMM: a plain fp16 matrix product of the same shape
    (2048 x 8192 by 8192 x 8192, no decode) through torch's BLAS on the same
    GPU: what the vendor library reaches on this part."""
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
    return {"tflops": round(2.0 * m * k * n / (ms * 1e-3) / 1e12, 1), "us": round(ms * 1e3, 1)}


def medium_m_rates(torch, ex, ms=(16, 32, 64, 128, 256), n=40):
    """Batched decode and chunked prefill sizes of the 8B gate projection
    (4096->14336, K=4) through exl3_linear (the GEMV or the split GEMM, as its
    table picks)."""
    import synth
    ws = ex.Workspace(4096, 14336, 4, max(ms))
    out = {}
    for m in ms:
        mm = synth.medium_m(m)
        lc = synth.Launch(mm.name, [mm])
        dl = DevLaunch(torch, ex, lc, "linear", replicas=replicas_for(lc), workspace=ws)
        t = time_events(torch, ex, dl, max(n, dl.replicas))
        out[f"m{m}"] = {"us": round(t * 1e3, 1), "weight_gbs": round(gbs(weight_bytes(lc), t), 1),
                        "tflops": round(2.0 * m * mm.n_in * mm.n_out / (t * 1e-3) / 1e12, 1)}
        del dl
        torch.cuda.empty_cache()
    return out


def codebook1_rates(torch, ex, n=50):
    """The byte-sum codebook on the K=4 MLP launches at m=1 and the 8192x8192 GEMM."""
    import synth
    out = {}
    for lc in synth.mlp_launches(4, 1):
        dl = DevLaunch(torch, ex, lc, gemv_fn(lc), replicas=replicas_for(lc), codebook=1)
        ms = time_events(torch, ex, dl, max(n, dl.replicas))
        out[lc.name] = {"us": round(ms * 1e3, 2), "gbs": round(gbs(dl.bytes, ms), 1)}
        del dl
        torch.cuda.empty_cache()
    out["gemm_m2048_8192x8192_k4"] = gemm_rate(torch, ex, "8192_k4", codebook=1)
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


def copy_bandwidth(torch, nbytes=GIB, iters=10):
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
    out = 2 * nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return round(out, 1)


# ------------------------------------------------------------ CPU oracle ----
def _decode_chunk(args):
    from oracle import exl3_oracle as O
    words, K = args
    return O.dequant(words, K)


def cpu_baseline(workers=None):
    """The CPU oracle, as it stands, on a bounded sample of every workload.
    Decode (the oracle's exact dequantisation, strip blocks spread over all
    host cores by a process pool) and contraction (the rotation and the
    float64 product through NumPy's BLAS, all cores) are timed apart; the
    single 4096x4096 layer also on one core.  Runs before the GPU is touched
    (the pool forks)."""
    import multiprocessing as mp

    import synth
    from oracle import exl3_oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    workers = workers or min(cores, 16)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    blas = None
    if threadpool_info:
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in threadpool_info()]
    pool = mp.get_context("fork").Pool(workers)

    def decode(words, K, strips_per_task=16):
        tasks = [(words[a:a + strips_per_task], K) for a in range(0, words.shape[0], strips_per_task)]
        return np.concatenate(pool.map(_decode_chunk, tasks), axis=0)

    def one(mm, strips=None, rows=None):
        """Decode + contraction seconds of one matmul, on its first `strips`
        strips and first `rows` rows of x (sample), scaled to the whole."""
        words, x, sign, scale = synth.draw(mm)
        s = strips or words.shape[0]
        r = rows or mm.m
        w = np.ascontiguousarray(words[:s])
        t0 = time.perf_counter()
        W = decode(w, mm.K)
        t1 = time.perf_counter()
        xr = O.rotate(x[:r].astype(np.float64), sign.astype(np.float64))
        y = (xr @ W.astype(np.float64).T) * scale[:16 * s].astype(np.float64)
        t2 = time.perf_counter()
        assert np.isfinite(y).all()
        fs, fr = words.shape[0] / s, mm.m / r
        return {"decode_s": (t1 - t0) * fs, "contract_s": (t2 - t1) * fs * fr, "bytes": mm.trellis_bytes,
                "sampled": f"{s} of {words.shape[0]} strips" + (f", {r} of {mm.m} rows" if r != mm.m else "")}

    def total(parts):
        d = sum(p["decode_s"] for p in parts)
        c = sum(p["contract_s"] for p in parts)
        b = sum(p["bytes"] for p in parts)
        return {"decode_s": round(d, 3), "contract_s": round(c, 3), "gbs": round(b / (d + c) / 1e9, 4)}

    t_start = time.perf_counter()
    out = {}
    c1 = synth.single_layer()[0]
    out["single_4096x4096_k4_m1"] = total([one(c1)])
    words, x, sign, scale = synth.draw(c1)
    if threadpool_limits:
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            O.linear(x, words, sign, scale, c1.K)
            t1 = time.perf_counter()
        out["single_4096x4096_k4_m1"]["one_core_s"] = round(t1 - t0, 3)
        out["single_4096x4096_k4_m1"]["one_core_gbs"] = round(c1.trellis_bytes / (t1 - t0) / 1e9, 4)
    out["mlp_k4_m1"] = total([one(mm) for lc in synth.mlp_launches(4, 1) for mm in lc.members])
    out["llama70b_gate_k3_m1"] = total([one(synth.llama70b_launches()[1].members[0], strips=224)])
    g = synth.prefill_gemm()[0]
    out["gemm_m2048_8192x8192_k4"] = total([one(g, rows=256)])
    t = out["gemm_m2048_8192x8192_k4"]
    t["tflops"] = round(2.0 * g.m * g.n_in * g.n_out / (t["decode_s"] + t["contract_s"]) / 1e12, 5)
    layer0 = synth.llama8b_stack()[:4 * 7]  # the first four layers
    part = total([one(mm) for mm in layer0])
    all_bytes = sum(mm.trellis_bytes for mm in synth.llama8b_stack())
    l0_bytes = sum(mm.trellis_bytes for mm in layer0)
    scale_up = all_bytes / l0_bytes
    stack = {"decode_s": round(part["decode_s"] * scale_up, 2), "contract_s": round(part["contract_s"] * scale_up, 2),
             "gbs": part["gbs"]}
    stack["tokens_per_s"] = round(1.0 / (stack["decode_s"] + stack["contract_s"]), 5)
    out["stack_m1"] = stack
    pool.close()
    pool.join()
    wall = time.perf_counter() - t_start
    return {"value": stack["gbs"], "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": ("the 32-layer stack at m=1, from its first four layers' 28 matmuls scaled by the stack's bytes; "
                       "decode over a fork pool of %d processes, float64 contraction through NumPy's BLAS; "
                       "other workloads in per_config (70B gate: 224 of 1792 strips; GEMM: 256 of 2048 rows)"
                       % workers),
            "host_cores": cores, "cpu_model": model, "blas": blas, "wall_s": round(wall, 1), "per_config": out}


# --------------------------------------------------------------- profiling --
def only_mode(args):
    """Short runs for the profiler: one launch shape back to back over >= 1 GiB
    of weights in rotation (stack:<shape>, mlp<m>:<launch>, 70b:<launch>,
    single), the whole stack step as graph replays (stack), a GEMM
    (gemm:8192_k4 | gemm:28672_k3), or a plain copy of known size (copy)."""
    import torch

    import decode_gemm_exl3_amd as ex
    import synth
    ex.load()
    what = args.only
    steps = args.steps
    if what == "copy":
        nbytes = 256 << 20
        a = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda")
        b = torch.empty_like(a)
        for _ in range(steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each": nbytes, "copies": steps}), flush=True)
        return
    if what == "stack":
        r = stack_run(torch, ex, steps, 3)
        print(json.dumps({"stack": r}), flush=True)
        return
    if what.startswith("encode:"):
        K = int(what.split(":")[1])
        r = encode_rates(torch, ex, Ks=(K,))
        print(json.dumps({"encode": r}), flush=True)
        return
    if what == "fp16mm":
        r = fp16_matmul_tflops(torch, iters=steps)
        print(json.dumps({"plain_fp16_matmul_2048x8192x8192": r, "launches": steps + 1}), flush=True)
        return
    kind, _, name = what.partition(":")
    if kind == "gemm":
        r = gemm_rate(torch, ex, name, n=steps)
        print(json.dumps({f"gemm_{name}": r, "launches": steps + 1}), flush=True)
        return
    lc = _spec_launch(what)
    ws = None
    if kind.startswith("mlp"):
        ws = ex.Workspace(14336, 14336, 8, lc.m)
    elif kind == "70b":
        ws = ex.Workspace(28672, 28672, 8, 1)
    dl = DevLaunch(torch, ex, lc, gemv_fn(lc), replicas=replicas_for(lc), workspace=ws)
    ms = time_events(torch, ex, dl, steps)
    print(json.dumps({"launch": what, "launches": steps + 1, "bytes_per_launch": dl.bytes,
                      "rotation_bytes": dl.replicas * weight_bytes(lc), "event_us": round(ms * 1e3, 3)}), flush=True)


def trace_summary(path, top=12, kernel=None):
    """Per-kernel count, median, mean, min and max duration (ns) from a
    rocprofv3 kernel_trace.csv; with `kernel` (a substring of its name) one
    JSON object for that kernel instead."""
    import csv
    durs = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            d = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
            durs.setdefault(row["Kernel_Name"], []).append(d)
    if kernel:
        name = next(k for k in durs if kernel in k)
        v = np.asarray(durs[name])
        print(json.dumps({"kernel": name, "dispatches": int(v.size), "median_ns": int(np.median(v)),
                          "mean_ns": int(v.mean()), "min_ns": int(v.min()), "max_ns": int(v.max()),
                          "kernel_sources_hash": kernel_sources_hash()}))
        return
    rows = sorted(durs.items(), key=lambda kv: -sum(kv[1]))
    total = sum(sum(v) for v in durs.values())
    print("# columns: kernel | calls | median ns | mean ns | min ns | max ns | percent of GPU time")
    for k, v in rows[:top]:
        v = np.asarray(v)
        print(f"{k} | {v.size} | {int(np.median(v))} | {int(v.mean())} | {int(v.min())} | {int(v.max())} | "
              f"{100.0 * v.sum() / total:.2f}")


def _median_counters(path, kernel, largest=False):
    """Median over the dispatches of `kernel` of every counter in a rocprofv3
    counter_collection.csv (with `largest`, the largest value instead: the
    timed launch of a run whose warm-up launch is smaller)."""
    import csv
    vals = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Kernel_Name"] == kernel:
                vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    pick = (lambda v: float(np.max(v))) if largest else (lambda v: float(np.median(v)))
    return {k: pick(v) for k, v in vals.items()}, max((len(v) for v in vals.values()), default=0)


STALL_COUNTERS = ("SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
                  "SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS")
SQ_COUNTERS = ("SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_SALU SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES "
               "SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")


def make_profile(prof_dir, tag, spec):
    """The committed profile summary of one launch shape (JSON on stdout) from
    the rocprofv3 outputs of the passes listed under "commands": the kernel
    trace (durations), FETCH_SIZE and WRITE_SIZE (HBM traffic, scaled by what
    the same counters read for a plain 256 MiB device copy) and the SQ and GRBM
    counters (instructions, matrix-core busy cycles, clock)."""
    import csv
    trace = os.path.join(prof_dir, f"{tag}_trace_kernel_trace.csv")
    durs = {}
    with open(trace) as f:
        for row in csv.DictReader(f):
            if "exl3::" in row["Kernel_Name"] or (spec == "fp16mm" and "Cijk" in row["Kernel_Name"]):
                durs.setdefault(row["Kernel_Name"], []).append(int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    kernel = max(durs, key=lambda k: sum(durs[k]))
    v = np.asarray(durs[kernel])
    is_gemm = spec.startswith("gemm:") or spec == "fp16mm"
    files = GEMM_SOURCES if is_gemm else (ENCODE_SOURCES if spec.startswith("encode:") else GEMV_SOURCES)
    rec = {"launch": spec, "kernel": kernel, "kernel_sources_hash": kernel_sources_hash(files),
           "dispatches": int(v.size),
           "median_ns": int(np.median(v)), "mean_ns": int(v.mean()), "min_ns": int(v.min()), "max_ns": int(v.max())}
    others = {k: {"dispatches": len(d), "median_ns": int(np.median(d))} for k, d in durs.items() if k != kernel}
    if others:
        rec["other_kernels"] = others
    med_s = rec["median_ns"] * 1e-9
    if spec.startswith("encode:"):
        # one warm-up launch of 64 tiles, then the timed launch of 2048 tiles
        longest = int(v.max())
        rec["workload"] = f"tail-biting Viterbi encoder, K={spec.split(':')[1]}, 2048 unit-Gaussian tiles"
        rec["timed_launch_ns"] = longest
        rec["tiles_per_s"] = round(2048 / (longest * 1e-9))
        med_s = longest * 1e-9
    elif is_gemm:
        import synth
        mm = synth.prefill_gemm()[0 if spec in ("gemm:8192_k4", "fp16mm") else 1]
        flops = 2.0 * mm.m * mm.n_in * mm.n_out
        rec["workload"] = (f"prefill GEMM m={mm.m}, {mm.n_in}->{mm.n_out}, K={mm.K}" if spec != "fp16mm" else
                           "plain fp16 matrix product 2048x8192 by 8192x8192 through torch's BLAS (no decode)")
        rec["flops"] = flops
        rec["median_tflops"] = round(flops / med_s / 1e12, 1)
        rec["frac_of_mfma_f16_peak"] = round(flops / med_s / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
    else:
        lc = _spec_launch(spec)
        b = launch_bytes(lc)
        rec["workload"] = f"{lc.name}: {lc.n_in}->{'+'.join(map(str, lc.n_outs))}, K={lc.K}, m={lc.m}"
        rec["algorithmic_bytes_per_launch"] = b
        rec["median_gbs"] = round(b / med_s / 1e9, 1)
        rec["frac_of_hbm_peak"] = round(b / med_s / 1e9 / HBM_PEAK_GBS, 4)
    fpath = os.path.join(prof_dir, f"{tag}_fetch_counter_collection.csv")
    if os.path.exists(fpath):
        cf, _ = _median_counters(os.path.join(prof_dir, "copy_fetch_counter_collection.csv"), "__amd_rocclr_copyBuffer")
        cw, _ = _median_counters(os.path.join(prof_dir, "copy_write_counter_collection.csv"), "__amd_rocclr_copyBuffer")
        copy_bytes = 256 << 20
        fs = copy_bytes / (cf["FETCH_SIZE"] * 1024)
        ws = copy_bytes / (cw["WRITE_SIZE"] * 1024)
        kf, nf = _median_counters(fpath, kernel)
        kw, _ = _median_counters(os.path.join(prof_dir, f"{tag}_write_counter_collection.csv"), kernel)
        hbm = kf["FETCH_SIZE"] * 1024 * fs + kw["WRITE_SIZE"] * 1024 * ws
        rec["traffic"] = {"fetch_size_kib_median": kf["FETCH_SIZE"], "write_size_kib_median": kw["WRITE_SIZE"],
                          "dispatches": nf, "copy_fetch_scale": round(fs, 4), "copy_write_scale": round(ws, 4),
                          "hbm_bytes_per_launch": int(hbm),
                          "traffic_over_algorithmic": round(hbm / rec.get("algorithmic_bytes_per_launch", hbm), 4)}
    qpath = os.path.join(prof_dir, f"{tag}_sq_counter_collection.csv")
    if os.path.exists(qpath):
        q, nq = _median_counters(qpath, kernel, largest=spec.startswith("encode:"))
        valu = q["SQ_INSTS_VALU"] - q["SQ_INSTS_MFMA"]  # SQ_INSTS_VALU counts the MFMAs too
        se_cycles = q["SQ_BUSY_CYCLES"] / 32           # summed over the 32 shader engines
        clock = se_cycles / med_s                        # shader clock while the kernel ran (a lower bound)
        mfma_cycles = q["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024
        rec["issue"] = {"dispatches": nq, "sq_insts_valu": q["SQ_INSTS_VALU"], "sq_insts_mfma": q["SQ_INSTS_MFMA"],
                        "sq_insts_salu": q["SQ_INSTS_SALU"], "valu_insts_without_mfma": valu,
                        "mfma_busy_cycles_per_simd": mfma_cycles,
                        "valu_coexec_frac_of_mfma_busy": round(q["SQ_VALU_MFMA_COEXEC_CYCLES"]
                                                               / max(q["SQ_VALU_MFMA_BUSY_CYCLES"], 1), 4),
                        "sq_busy_cycles_per_se": se_cycles, "grbm_gui_active": q["GRBM_GUI_ACTIVE"],
                        "clock_ghz_est": round(clock / 1e9, 3),
                        "mfma_busy_frac_at_est_clock": round(mfma_cycles / se_cycles, 4),
                        "valu_lane_ops_per_s": valu * 64 / med_s,
                        "valu_frac_of_issue_peak": round(valu * 64 / med_s / VALU_PEAK_LANE_OPS, 4)}
        if "flops" in rec:
            peak_at_clock = MFMA_F16_PEAK_TFLOPS * (clock / 2.4e9)
            rec["issue"]["mfma_f16_peak_at_est_clock_tflops"] = round(peak_at_clock, 1)
            rec["issue"]["frac_of_peak_at_est_clock"] = round(rec["median_tflops"] / peak_at_clock, 4)
    spath = os.path.join(prof_dir, f"{tag}_stall_counter_collection.csv")
    if os.path.exists(spath):
        q, ns = _median_counters(spath, kernel, largest=spec.startswith("encode:"))
        wc = max(q["SQ_WAVE_CYCLES"], 1)
        rec["stalls"] = {"dispatches": ns, **{k.lower(): q[k] for k in sorted(q)},
                         "wait_any_frac_of_wave_cycles": round(q["SQ_WAIT_ANY"] / wc, 4),
                         "wait_inst_any_frac_of_wave_cycles": round(q["SQ_WAIT_INST_ANY"] / wc, 4),
                         "lds_bank_conflict_frac_of_lds_active": round(q["SQ_LDS_BANK_CONFLICT"]
                                                                       / max(q["SQ_ACTIVE_INST_LDS"], 1), 4)}
    nsteps = 1 if spec.startswith("encode:") else (30 if is_gemm else 60)
    cmds = [f"cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o {tag}_trace -- "
            f"python3 <repo>/bench.py --only {spec} --steps {nsteps}"]
    if os.path.exists(fpath):
        cmds += [f"cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out> -o {tag}_fetch -- "
                 f"python3 <repo>/bench.py --only {spec} --steps 20",
                 f"cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out> -o {tag}_write -- "
                 f"python3 <repo>/bench.py --only {spec} --steps 20",
                 "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out> -o copy_fetch -- "
                 "python3 <repo>/bench.py --only copy --steps 20   (and WRITE_SIZE into copy_write)"]
    if os.path.exists(qpath):
        cmds.append(f"cd /tmp && rocprofv3 --pmc {SQ_COUNTERS} --output-format csv -d <out> -o {tag}_sq -- "
                    f"python3 <repo>/bench.py --only {spec} --steps {nsteps if nsteps == 1 else (10 if is_gemm else 20)}")
    if os.path.exists(spath):
        cmds.append(f"cd /tmp && rocprofv3 --pmc {STALL_COUNTERS} --output-format csv -d <out> -o {tag}_stall -- "
                    f"python3 <repo>/bench.py --only {spec} --steps {1 if nsteps == 1 else 10}")
    cmds.append(f"python3 <repo>/bench.py --make-profile {tag} --prof-dir <out> --only {spec}")
    rec["commands"] = cmds
    rec["derivation"] = ("durations: End - Start of the kernel's dispatches in the trace; traffic: FETCH_SIZE and "
                         "WRITE_SIZE medians (KiB) times the bytes a 256 MiB copy moves over what the same counter "
                         "reads for it; SQ_INSTS_VALU counts MFMAs, so vector instructions = SQ_INSTS_VALU - "
                         "SQ_INSTS_MFMA (64 lane-operations each); SQ_BUSY_CYCLES is read as summed over the 32 "
                         "shader engines, so SQ_BUSY_CYCLES / 32 / median duration estimates the shader clock the "
                         "kernel ran at (a lower bound: cycles with no wave resident do not count); MFMA busy "
                         "fraction = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (SQ_BUSY_CYCLES / 32)")
    print(json.dumps(rec, indent=1))


def _spec_launch(spec):
    import synth
    kind, _, name = spec.partition(":")
    if kind == "stack":
        return stack_shapes(stack_launches(True))[name][1]
    if kind.startswith("mlp"):
        return next(x for x in synth.mlp_launches(int(name.split("_k")[1]), int(kind[3:] or 1)) if x.name == name)
    if kind == "70b":
        return next(x for x in synth.llama70b_launches() if x.name == name)
    if kind == "single":
        mm = synth.single_layer()[0]
        return synth.Launch(mm.name, [mm])
    raise SystemExit(f"unknown launch {spec}")


# -------------------------------------------------------------------- main --
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="headline, roofline and baseline only")
    ap.add_argument("--only", help="profiling runs: one launch shape only (see only_mode)")
    ap.add_argument("--trace-summary", help="summarise a rocprofv3 kernel_trace.csv and exit")
    ap.add_argument("--trace-kernel", help="with --trace-summary: one kernel (name substring) as JSON")
    ap.add_argument("--make-profile", help="profile summary of a launch shape (tag of the rocprofv3 outputs)")
    ap.add_argument("--prof-dir", help="with --make-profile: the rocprofv3 output folder")
    args = ap.parse_args()
    if args.make_profile:
        make_profile(args.prof_dir, args.make_profile, args.only)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, kernel=args.trace_kernel)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.only:
        only_mode(args)
        return

    # the CPU oracle first: its process pool forks before the GPU is touched
    cpu = None if args.no_cpu else cpu_baseline()

    import torch

    import decode_gemm_exl3_amd as ex
    ex.load()
    torch.cuda.init()

    head = stack_run(torch, ex, args.steps, args.warmup, fused=True)
    ms = head["ms_per_token"]
    value = gbs(head["bytes_per_token"], ms)

    shapes = stack_shape_times(torch, ex)
    dom_key = max(shapes, key=lambda k: shapes[k]["total_us"])
    dom = shapes[dom_key]
    achieved = gbs(dom["bytes_per_launch"], dom["us"] * 1e-3)
    prof = profile_record(f"gemv_stack8b_{dom_key}.json")
    traffic = prof.get("traffic") if prof else None
    issue = prof.get("issue") if prof else None
    kernel = f"gemv_kernel<K={dom['K']}> {dom_key}: {dom['n_in']}->{'+'.join(map(str, dom['n_outs']))}, m=1"
    roofline = {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic.get("hbm_bytes_per_launch") if traffic else None,
                "bytes_per_launch": dom["bytes_per_launch"], "event_us": dom["us"],
                "share_of_step": dom["share"], "rotation_bytes": dom["rotation_bytes"]}
    if prof:
        med = prof["median_ns"] * 1e-6
        roofline["profile_median_us"] = round(prof["median_ns"] * 1e-3, 3)
        roofline["profile_frac"] = round(gbs(dom["bytes_per_launch"], med) / HBM_PEAK_GBS, 4)
    alu = None
    if issue:
        n = issue["valu_insts_without_mfma"]
        a = n * 64 / (dom["us"] * 1e-6)
        alu = {"bound": "alu", "kernel": kernel, "achieved": round(a / 1e12, 2),
               "peak": round(VALU_PEAK_LANE_OPS / 1e12, 2), "unit": "T lane-ops/s",
               "frac": round(a / VALU_PEAK_LANE_OPS, 4), "valu_insts_per_launch": int(n)}

    extra = {"stack_launch_shapes": shapes, "copy_gbs": copy_bandwidth(torch)}
    # what a plain device copy reaches on this part, beside the spec peak
    roofline["frac_of_copy_rate"] = round(achieved / extra["copy_gbs"], 4)
    if not args.no_extra:
        extra["single_4096x4096_k4_m1"] = single_layer_rate(torch, ex)
        for m in (1, 4, 8):
            extra[f"mlp_m{m}"] = mlp_rates(torch, ex, m, max(20, args.steps // 4))
        # the vector-ALU roofline of each m = 1 launch (K = 2, 3, 4): its committed
        # issue counters over the duration measured here
        for name, r in extra["mlp_m1"]["launches"].items():
            p1 = profile_record(f"gemv_mlp8b_m1_{name}.json")
            if p1 and p1.get("issue"):
                n = p1["issue"]["valu_insts_without_mfma"]
                r["alu_frac"] = round(n * 64 / (r["us"] * 1e-6) / VALU_PEAK_LANE_OPS, 4)
                r["valu_insts_per_launch"] = int(n)
        extra["llama70b_m1"] = llama70b_rates(torch, ex)
        extra["gemm_m2048_8192x8192_k4"] = gemm_rate(torch, ex, "8192_k4")
        extra["gemm_m2048_8192x8192_k4"]["plain_fp16_matmul_same_shape"] = fp16_matmul_tflops(torch)
        extra["gemm_m2048_8192x28672_k3"] = gemm_rate(torch, ex, "28672_k3")
        extra["medium_m_4096x14336_k4"] = medium_m_rates(torch, ex)
        extra["codebook1"] = codebook1_rates(torch, ex)
        extra["encode"] = encode_rates(torch, ex)
        extra["stack_unfused"] = stack_run(torch, ex, max(20, args.steps // 4), 3, fused=False)

    rec = {
        "metric": "EXL3 GEMV achieved HBM GB/s at m=1 (32-layer Llama-3.1-8B-shaped stack, 224 matmuls)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "llama3.1-8b-shaped 32-layer linear stack at m=1: q 4096->4096, k/v 4096->1024, "
                               "o 4096->4096, gate/up 4096->14336, down 14336->4096 per layer, K_b from {2..6} "
                               "(attention +1), q/k/v and gate/up fused, 128 launches per token as one HIP graph",
                   "m": 1, "tokens_per_s": head["tokens_per_s"], "bytes_per_token": head["bytes_per_token"]},
        "roofline": roofline,
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "alu_roofline": alu,
        "extra": extra,
    }
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
