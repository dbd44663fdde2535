#!/usr/bin/env python3
"""Throughput of the fused GPTQ W4A16 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--eager]

A step is one pass of the hot path over one batch: the seven quantized linear
layers of a Llama-7B-shaped decoder block (q, k, v, o 4096x4096; gate, up
4096x11008; down 11008x4096; groupsize 128; bias on q) at M = 1, run back to
back through the C ABI (q4_matmul_bias). The value is effective HBM
bandwidth: bytes of packed weights + scales + packed zeros per step divided by
the time per step. Inputs are resident in HBM before timing starts. To keep
the 256 MB last-level cache from serving the weights, the steps rotate over
ten handle copies of the block (1.05 GB). By default the steps are replayed
from HIP graphs captured on the timing stream (one graph of ten consecutive
steps, one per copy for a remainder) so that neither the host launch rate nor
a per-graph launch cost bounds a ~35 us step; --eager launches directly.

Also reported on the same JSON line:
  roofline      the skinny kernel's achieved bandwidth: algorithmic bytes per
                launch / mean launch duration, from HIP events around graph
                replays of each layer's launches on the launch stream (each
                layer rotating over >= 1 GiB of weight copies, so the weights
                come from HBM as in the block steps); traffic comes from
                committed rocprofv3 counter runs, when their kernel source hash
                matches the current source, else null;
  cpu_baseline  the CPU oracle's fused route on whole layers of the block;
  secondary     the same block with q/k/v and gate/up fused into one call each
                (4 launches a step); the 70B-shaped MLP layers at M = 1, 2, 4,
                8, 16, the 7B MLP layers at M = 17 .. 256 and the act-order
                7B MLP layers at M = 1, 4 (GB/s, each layer over >= 1 GiB of
                copies); the 7B MLP layers with 8-bit
                weights at M = 1, 4; the seven-layer block with bfloat16
                activations; the prefill GEMM at M = 2048 on the 7B MLP
                shapes, groupsize 128 and 32, act-order, bfloat16 and 8-bit
                weights (TFLOPS against the dense fp16/bf16 MFMA peak).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMV effective HBM GB/s (% peak) at M=1; TFLOPS (% MFMA peak) at M=2048"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA
MALL_DEFEAT_BYTES = 1 << 30     # rotate at least this much distinct weight memory
WARM_S = 0.1                    # seconds of replays before a timed region


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources that decide what the skinny kernel does and how it is launched
# (its code, the shared device helpers and geometry, the weight layout the
# repack writes, the launch plan and the dispatch): counter figures taken for
# it stay valid while their code (comments aside) is unchanged.
GEMV_SOURCES = ("q4_gemv.hip", "q4_device.h", "q4_internal.h", "q4_prep.hip", "q4_plan.cpp",
                "q4_api.hip")


def _code_only(text: str) -> str:
    """Source text without comments and blank-line or trailing-space changes,
    so that editing a comment does not invalidate recorded counters."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gptq_bit_weight_amd", "csrc")
    for name in GEMV_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


class Layer:
    """Device-resident layer: C handle copies, x, bias, out, raw pointers."""

    def __init__(self, q4, torch, name, L, copies):
        dev = torch.device("cuda", 0)
        self.q4 = q4
        self.src = (torch.from_numpy(L.qweight).to(dev), torch.from_numpy(L.qzeros).to(dev),
                    torch.from_numpy(L.scales).to(dev),
                    torch.from_numpy(L.g_idx).to(dev) if L.g_idx is not None else None)
        self.name, self.K, self.N, self.G, self.M = name, L.K, L.N, L.G, L.M
        self.bits = L.bits
        self.mats = [self._make() for _ in range(copies)]
        self.bf16 = L.xfmt == "bf16"
        act = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)) if self.bf16 \
            else torch.from_numpy
        self.x = act(L.x).to(dev)
        self.bias = act(L.bias).to(dev) if L.bias is not None else None
        self.out = torch.empty((L.M, L.N), dtype=self.x.dtype, device=dev)
        self.bytes = L.metric_bytes()
        self.flops = 2 * L.M * L.K * L.N
        self.xp = ctypes.c_void_p(self.x.data_ptr())
        self.bp = ctypes.c_void_p(self.bias.data_ptr()) if self.bias is not None else None
        self.op = ctypes.c_void_p(self.out.data_ptr())

    def _make(self):
        qw, qz, sc, gi = self.src
        return self.q4.Q4Matrix(qw, qz, sc, gi, groupsize=self.G, bits=self.bits)

    def grow(self, copies):
        """Make handle copies until there are `copies` of them."""
        while len(self.mats) < copies:
            self.mats.append(self._make())

    def shrink(self, copies):
        while len(self.mats) > copies:
            self.mats.pop().close()

    def launch(self, lib, copy, stream_ptr):
        fn = lib.q4_matmul_bf16 if self.bf16 else lib.q4_matmul_bias
        st = fn(self.mats[copy]._h, self.xp, self.bp, self.op, self.M, stream_ptr)
        if st:
            raise RuntimeError(f"q4_matmul({self.name}) failed: {lib.q4_last_error()}")

    def close(self):
        for m in self.mats:
            m.close()
        self.mats = []


def build_layers(q4, torch, synth, specs, G, M, workload, copies, xfmt="f16"):
    layers = []
    for name, K, N, bias in specs:
        L = synth.make_layer(K, N, G, M, seed=synth.layer_seed(workload, name, M), bias=bias, xfmt=xfmt)
        layers.append(Layer(q4, torch, name, L, copies))
    return layers


def per_launch_times(lib, torch, layers, min_launches, stream):
    """Mean kernel duration of each layer, with its weights coming from HBM:
    the layer's launches rotate over ceil(1 GiB / layer bytes) handle copies
    (made for this measurement and freed after it), at least `min_launches`
    of them, captured in one HIP graph on the launch stream. The graph is
    replayed for about WARM_S seconds first (clocks ramp up over some
    milliseconds after the host-side set-up left the GPU idle), then three
    times between two events each; the median replay gives the time.
    Consecutive kernels of a graph start back to back, so elapsed / launches
    is the mean launch duration (the figure the kernel trace of rocprofv3
    reports for the same launches)."""
    out = []
    for ly in layers:
        base = len(ly.mats)
        copies = max(base, math.ceil(MALL_DEFEAT_BYTES / ly.bytes))
        ly.grow(copies)
        n = copies * max(1, math.ceil(min_launches / copies))
        with torch.cuda.stream(stream):
            sp = ctypes.c_void_p(stream.cuda_stream)
            for c in range(copies):
                ly.launch(lib, c, sp)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for r in range(n):
                ly.launch(lib, r % copies, cap)
        def timed_replay():
            # one untimed replay ahead keeps the GPU busy while the timed one
            # is enqueued, so the events do not include the host's launch
            # latency
            with torch.cuda.stream(stream):
                g.replay()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
            stream.synchronize()
            return a.elapsed_time(b) * 1e-3

        first = timed_replay()
        with torch.cuda.stream(stream):
            for _ in range(max(1, math.ceil(WARM_S / first))):
                g.replay()
        stream.synchronize()
        out.append(sorted(timed_replay() for _ in range(3))[1] / n)
        del g
        ly.shrink(base)
        torch.cuda.empty_cache()
    return out


def time_steps(lib, torch, layers, copies, steps, warmup, stream, use_graph):
    sp = ctypes.c_void_p(stream.cuda_stream)

    def eager_step(s):
        c = s % copies
        for ly in layers:
            ly.launch(lib, c, sp)

    graphs = None
    if use_graph:
        with torch.cuda.stream(stream):
            for s in range(copies):         # first calls happen eagerly (allocations, if any)
                eager_step(s)
        stream.synchronize()
        # one graph per copy (one step each) and one graph of `copies`
        # consecutive steps, so that a graph launch is not paid per step
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                for ly in layers:
                    ly.launch(lib, c, cap)
            graphs.append(g)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for c in range(copies):
                for ly in layers:
                    ly.launch(lib, c, cap)
        graphs.append(g)

    def run(first, count):
        """Steps first .. first+count-1 (step s uses weight copy s % copies)."""
        s = first
        while s < first + count:
            if graphs is None:
                eager_step(s)
                s += 1
            elif s % copies == 0 and s + copies <= first + count:
                graphs[copies].replay()
                s += copies
            else:
                graphs[s % copies].replay()
                s += 1

    with torch.cuda.stream(stream):
        # Clocks ramp over milliseconds after the host-side set-up left the
        # GPU idle: replay for at least WARM_S seconds whatever `warmup` is,
        # then the `warmup` steps themselves.
        w0 = time.perf_counter()
        while time.perf_counter() - w0 < WARM_S:
            run(0, copies)
            stream.synchronize()
        torch.cuda.synchronize()
        # The `warmup` steps (at least one graph of `copies` steps) are
        # enqueued without waiting, so the GPU is still running them when the
        # start event and the timed steps are enqueued: the events then time
        # the K steps back to back on the GPU, not the host's graph launch
        # latency in front of them (tens of microseconds, a large part of a
        # short timed region).
        run(0, max(warmup, copies))
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        t0.record(stream)
        run(max(warmup, copies), steps)
        t1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    return t0.elapsed_time(t1) * 1e-3, wall, graphs


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(oracle, L, budget_s):
    """Whole-layer oracle runs of L (fused route) repeated for about budget_s
    seconds (at least once): (GB/s of metric bytes, GFLOP/s, runs, seconds)."""
    runs, elapsed = 0, 0.0
    while runs == 0 or elapsed < budget_s:
        t = time.perf_counter()
        oracle.matmul(L.x, L.qweight, L.qzeros, L.scales, L.g_idx, L.K, L.N, L.G, bias=L.bias)
        elapsed += time.perf_counter() - t
        runs += 1
    return (L.metric_bytes() * runs / elapsed / 1e9, 2.0 * L.M * L.K * L.N * runs / elapsed / 1e9,
            runs, elapsed)


def cpu_baseline(synth, oracle, specs, G, workload, budget_s):
    """The oracle's fused route on whole layers of the block at M = 1, layers
    in block order and repeated (at least one whole block), until budget_s of
    CPU time has passed, on all the threads the oracle is given; then single
    threaded on one layer of each decode workload (tiny 512x512; the block's
    q projection 4096x4096; the act-order 4096x11008 layer at M = 1)."""
    done_bytes, done_flops, elapsed, layers_done = 0, 0, 0.0, 0
    cache = {}
    i = 0
    while elapsed < budget_s or layers_done < len(specs):
        name, K, N, bias = specs[i % len(specs)]
        if name not in cache:
            cache[name] = synth.make_layer(K, N, G, 1, seed=synth.layer_seed(workload, name, 1),
                                           bias=bias)
        L = cache[name]
        t = time.perf_counter()
        oracle.matmul(L.x, L.qweight, L.qzeros, L.scales, None, K, N, G, bias=L.bias)
        elapsed += time.perf_counter() - t
        done_bytes += L.metric_bytes()
        done_flops += 2 * L.K * L.N
        layers_done += 1
        i += 1
    threads = oracle.num_threads()
    single = {}
    prev = oracle.set_num_threads(1)
    try:
        for label, L in (
                ("tiny_512x512_m1", synth.make_layer(512, 512, 128, 1, seed=synth.layer_seed("tiny", 1))),
                ("llama7b_q_proj_4096x4096_m1", cache.get("q_proj") or synth.make_layer(
                    4096, 4096, G, 1, seed=synth.layer_seed(workload, "q_proj", 1), bias=True)),
                ("llama7b_actorder_4096x11008_m1", synth.make_layer(
                    4096, 11008, 128, 1, seed=synth.layer_seed("llama7b_actorder", 4096, 11008, 1),
                    act_order=True))):
            gbs, gfl, runs, secs = _oracle_rate(oracle, L, 1.0)
            single[label] = {"GB/s": round(gbs, 4), "GFLOP/s": round(gfl, 3), "runs": runs,
                             "seconds": round(secs, 2)}
    finally:
        oracle.set_num_threads(prev)
    return {
        "value": round(done_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{layers_done} whole M=1 layers of the block in order (fused route, double "
                  f"accumulation), {elapsed:.1f} s on {threads} threads",
        "GFLOP/s": round(done_flops / elapsed / 1e9, 3),
        "cpu_model": cpu_model(),
        "single_thread": single,
    }


def gpu_environment(torch):
    """Clocks and software versions of the run (best effort: missing tools
    give null)."""
    env = {"rocm": None, "torch_hip": getattr(torch.version, "hip", None), "sclk_mhz": None,
           "mclk_mhz": None, "device": torch.cuda.get_device_name(0)}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        pass
    try:
        import subprocess
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        data = json.loads(r.stdout[r.stdout.index("{"):]) if "{" in r.stdout else {}
        card = next(iter(data.values()), {}) if data else {}
        env["smi_clocks"] = {k: v for k, v in card.items() if "clk" in k.lower()} or None
        for key, val in card.items():
            m = re.search(r"\(?(\d+)\s*Mhz", str(val), re.I)
            if not m:
                continue
            k = key.lower()
            if k.startswith("sclk") and env["sclk_mhz"] is None:
                env["sclk_mhz"] = int(m.group(1))
            elif k.startswith("mclk") and env["mclk_mhz"] is None:
                env["mclk_mhz"] = int(m.group(1))
    except Exception:   # noqa: BLE001 -- a missing or odd tool leaves nulls
        pass
    return env


def read_ceiling(lib, torch, stream, sizes):
    """Achievable read rate of one launch of each size in `sizes` (bytes,
    rounded down to a multiple of 16 KiB): q4_read_probe launches, captured
    in a graph that rotates over at least 1 GiB of distinct memory (so the
    bytes come from HBM, as the weights do), replayed for WARM_S seconds and
    then three times between events; the median replay gives the mean launch
    time. Returns {size: {"GB/s", "us"}}."""
    pool_bytes = max(MALL_DEFEAT_BYTES, max(sizes)) + (16 << 20)
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    out = {}
    for size in sizes:
        size = size - size % 16384
        # (at most 4096 copies: the 16 KiB probe then cycles over 64 MiB,
        # which is what a near-empty launch needs; every layer-sized probe
        # still rotates over >= 1 GiB)
        copies = max(1, min(pool_bytes // size, math.ceil(MALL_DEFEAT_BYTES / size), 4096))
        offs = [(c * size) - (c * size) % 256 for c in range(copies)]
        n = copies * max(1, math.ceil(200 / copies)) if size < (256 << 20) else max(copies, 10)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for r in range(n):
                st = lib.q4_read_probe(ctypes.c_void_p(pool.data_ptr() + offs[r % copies]), size,
                                       ctypes.c_void_p(sink.data_ptr()), cap)
                if st:
                    raise RuntimeError(f"q4_read_probe failed: {lib.q4_last_error()}")
        with torch.cuda.stream(stream):
            w0 = time.perf_counter()
            while time.perf_counter() - w0 < WARM_S:
                g.replay()
                stream.synchronize()
            times = []
            for _ in range(3):
                g.replay()      # untimed, ahead of the timed replay (host launch latency)
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
                stream.synchronize()
                times.append(a.elapsed_time(b) * 1e-3 / n)
        t = sorted(times)[1]
        out[size] = {"GB/s": round(size / t / 1e9, 1), "us": round(t * 1e6, 3)}
        del g
    del pool, sink
    torch.cuda.empty_cache()
    return out


def traffic_for(kernel: str, src_hash: str):
    """HBM bytes per launch from committed counter runs, if they were taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def fused_block(q4, torch, synth, lib, stream, G, M, workload, copies, steps=500):
    """The same block with the layers that take the same input fused into one
    call each (q/k/v and gate/up concatenated along N: 4 launches a step), the
    same weights, copies rotated and graphs replayed as in the main figure."""
    specs = {name: (K, N, bias) for name, K, N, bias in synth.LLAMA7B_BLOCK}
    layers = []
    for gname, names in synth.LLAMA7B_FUSED:
        parts = [synth.make_layer(specs[n][0], specs[n][1], G, M, seed=synth.layer_seed(workload, n, M),
                                  bias=specs[n][2]) for n in names]
        layers.append(Layer(q4, torch, gname, synth.concat_layers(parts), copies))
    step_bytes = sum(ly.bytes for ly in layers)
    elapsed, _, graphs = time_steps(lib, torch, layers, copies, steps, 1000, stream, use_graph=True)
    del graphs
    lt = per_launch_times(lib, torch, layers, min_launches=200, stream=stream)
    for ly in layers:
        ly.close()
    torch.cuda.empty_cache()
    gbs = step_bytes / (elapsed / steps) / 1e9
    return {"GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
            "us_per_step": round(elapsed / steps * 1e6, 2), "launches_per_step": len(layers),
            "per_layer_us": {ly.name: round(t * 1e6, 3) for ly, t in zip(layers, lt)}}


def decode_sweep(q4, torch, synth, lib, stream, workload, specs, Ms, act_order=False, bits=4):
    """GB/s of each layer in `specs` ((name, K, N)) at each M: one layer's
    handles rotate over >= 1 GiB of copies (per_launch_times), the same
    handles serve every M (only the activations change)."""
    out = {}
    for name, K, N in specs:
        L = synth.make_layer(K, N, 128, max(Ms), seed=synth.layer_seed(workload, name, act_order),
                             act_order=act_order, bits=bits)
        ly = Layer(q4, torch, name, L, 1)
        x_all = ly.x
        for M in Ms:
            ly.x = x_all[:M].contiguous()
            ly.M = M
            ly.out = torch.empty((M, N), dtype=torch.float16, device=x_all.device)
            ly.xp = ctypes.c_void_p(ly.x.data_ptr())
            ly.op = ctypes.c_void_p(ly.out.data_ptr())
            t = per_launch_times(lib, torch, [ly], min_launches=200, stream=stream)[0]
            gbs = ly.bytes / t / 1e9
            out[f"{name}_m{M}"] = {"GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "us": round(t * 1e6, 2), "TFLOP/s": round(2 * M * K * N / t / 1e12, 1)}
        ly.close()
        del ly
        torch.cuda.empty_cache()
    return out


def bf16_block(q4, torch, synth, lib, stream, G, M, workload, copies, steps=500):
    """The seven-layer block with bfloat16 activations, bias and outputs:
    the same weights' shapes, copies rotated and graphs replayed as in the
    main figure."""
    layers = build_layers(q4, torch, synth, synth.LLAMA7B_BLOCK, G, M, workload + "_bf16", copies,
                          xfmt="bf16")
    step_bytes = sum(ly.bytes for ly in layers)
    elapsed, _, graphs = time_steps(lib, torch, layers, copies, steps, 1000, stream, use_graph=True)
    del graphs
    lt = per_launch_times(lib, torch, layers, min_launches=200, stream=stream)
    for ly in layers:
        ly.close()
    torch.cuda.empty_cache()
    gbs = step_bytes / (elapsed / steps) / 1e9
    return {"GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
            "us_per_step": round(elapsed / steps * 1e6, 2),
            "per_layer_us": {ly.name: round(t * 1e6, 3) for ly, t in zip(layers, lt)}}


def prefill_rates(q4, torch, synth, lib, stream, M=2048):
    """TFLOP/s of the prefill GEMM on the 7B MLP shapes: groupsize 128 and 32,
    and act-order at 128 (the weights are 23-26 MB; compute, not memory,
    bounds these). Twenty launches are captured in one graph, replayed for
    WARM_S seconds, then three times (each behind an untimed replay); the
    median replay gives the time."""
    out = {}
    reps = 20
    for K, N, G, act, xfmt, bits in ((4096, 11008, 128, False, "f16", 4), (11008, 4096, 128, False, "f16", 4),
                                     (4096, 11008, 32, False, "f16", 4), (11008, 4096, 32, False, "f16", 4),
                                     (4096, 11008, 128, True, "f16", 4), (4096, 11008, 128, False, "bf16", 4),
                                     (11008, 4096, 128, False, "bf16", 4), (4096, 11008, 128, False, "f16", 8),
                                     (11008, 4096, 128, False, "f16", 8)):
        L = synth.make_layer(K, N, G, M, seed=synth.layer_seed("prefill", K, N, G, act), act_order=act,
                             xfmt=xfmt, bits=bits)
        ly = Layer(q4, torch, f"prefill_{K}x{N}", L, 1)
        with torch.cuda.stream(stream):
            ly.launch(lib, 0, ctypes.c_void_p(stream.cuda_stream))   # sizes the act-order workspace
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for _ in range(reps):
                ly.launch(lib, 0, cap)
        times = []
        with torch.cuda.stream(stream):
            w0 = time.perf_counter()
            while time.perf_counter() - w0 < WARM_S:
                g.replay()
                stream.synchronize()
            for _ in range(3):
                g.replay()      # untimed, ahead of the timed replay (host launch latency)
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
                stream.synchronize()
                times.append(a.elapsed_time(b) * 1e-3 / reps)
        t = sorted(times)[1]
        tf = ly.flops / t / 1e12
        out[f"{K}x{N}_g{G}{'_act' if act else ''}{'_bf16' if xfmt == 'bf16' else ''}"
            f"{'_w8' if bits == 8 else ''}_m{M}"] = {
            "TFLOP/s": round(tf, 1), "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "us": round(t * 1e6, 1)}
        del g
        ly.close()
        del ly
    torch.cuda.empty_cache()
    return out


def prefill_counter_run(q4, torch, synth, lib, M=2048, launches=10):
    """Launches for counter runs (rocprofv3 --pmc): `launches` eager prefill
    GEMMs on each 7B MLP shape (groupsize 128, the planned schedule), then 5
    plain copies of 256 MiB as a reference of known size. Prints one JSON
    line describing the launches to stderr."""
    stream = torch.cuda.Stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    meta = {"prefill_counters_run": True, "launches_per_shape": launches, "copy_bytes": 256 << 20,
            "shapes": []}
    for K, N in ((4096, 11008), (11008, 4096)):
        L = synth.make_layer(K, N, 128, M, seed=synth.layer_seed("prefill", K, N, 128, False))
        ly = Layer(q4, torch, f"prefill_{K}x{N}", L, 1)
        with torch.cuda.stream(stream):
            for _ in range(launches):
                ly.launch(lib, 0, sp)
        stream.synchronize()
        meta["shapes"].append({"K": K, "N": N, "M": M, "flops": ly.flops, "weight_bytes": ly.bytes,
                               "x_bytes": 2 * M * K, "out_bytes": 2 * M * N,
                               "workers": q4.plan_gemm(M, N, K, torch.cuda.get_device_properties(0)
                                                       .multi_processor_count)})
        ly.close()
    with torch.cuda.stream(stream):
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
    torch.cuda.synchronize()
    log(json.dumps(meta))


def secondary(q4, torch, synth, lib, stream):
    """Figures on the other workloads: the 7B block with projection fusion
    and with bfloat16 activations, the 70B MLP layers at M = 1, 2, 4, 8, 16
    (where the skinny kernel stops being bandwidth-bound), the 7B MLP layers
    at M = 17 .. 256 (small batches: the skinny kernel's two row blocks up
    to 32, the GEMM above), the 8-bit and act-order 7B MLP layers at M = 1
    and 4, and the prefill GEMM at M = 2048."""
    out = {}
    out["llama7b_block_fused_m1"] = fused_block(q4, torch, synth, lib, stream, 128, 1,
                                                "llama7b_block_decode", 10)
    out["llama7b_block_bf16_m1"] = bf16_block(q4, torch, synth, lib, stream, 128, 1,
                                              "llama7b_block_decode", 10)
    out["llama70b_mlp_decode"] = decode_sweep(q4, torch, synth, lib, stream, "llama70b_mlp_decode",
                                              synth.LLAMA70B_MLP, (1, 2, 4, 8, 16))
    # batches past 16 rows: the skinny kernel's two row blocks up to 32,
    # then the GEMM's 64-row tiles
    out["llama7b_mlp_small_batch"] = decode_sweep(
        q4, torch, synth, lib, stream, "llama7b_mlp_small_batch",
        (("gate_proj", 4096, 11008), ("down_proj", 11008, 4096)), (17, 24, 32, 33, 64, 128, 256))
    out["llama7b_mlp_w8_decode"] = decode_sweep(
        q4, torch, synth, lib, stream, "llama7b_mlp_w8_decode",
        (("gate_proj", 4096, 11008), ("down_proj", 11008, 4096)), (1, 4), bits=8)
    out["llama7b_actorder_decode"] = decode_sweep(
        q4, torch, synth, lib, stream, "llama7b_actorder_decode",
        (("gate_proj", 4096, 11008), ("down_proj", 11008, 4096)), (1, 4), act_order=True)
    out["prefill"] = prefill_rates(q4, torch, synth, lib, stream)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--eager", action="store_true", help="launch each step directly (no graph)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-eager", action="store_true",
                    help="skip the eager (no graph) reference figure, e.g. so that the last skinny-kernel "
                         "launches of a profiled run are the timed steps")
    ap.add_argument("--secondary-only", action="store_true",
                    help="print only the secondary figures (one JSON line), e.g. to profile their kernels")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--counters", action="store_true",
                    help="no timing: run 20 eager steps of the block, then 5 plain copies of "
                         "256 MiB (a reference of known size for HBM counters), for rocprofv3 --pmc")
    ap.add_argument("--prefill-counters", action="store_true",
                    help="no timing: 10 eager launches of the prefill GEMM at M = 2048 on each 7B MLP "
                         "shape (groupsize 128), then 5 plain copies of 256 MiB, for rocprofv3 --pmc")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (one GPU's share of a "
              "sharded layer is the same kernel at a smaller shape). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gptq_bit_weight_amd as q4
    import synth
    if not os.path.exists(q4.library_path()):
        from gptq_bit_weight_amd import build as libbuild
        libbuild.build()

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    lib = q4.load_library()
    if args.secondary_only:
        print(json.dumps({"secondary": secondary(q4, torch, synth, lib, torch.cuda.Stream())}), flush=True)
        return
    if args.prefill_counters:
        prefill_counter_run(q4, torch, synth, lib)
        return
    workload = "llama7b_block_decode"
    G, M = 128, 1
    copies = 10
    log(f"[bench] building {copies} copies of the {len(synth.LLAMA7B_BLOCK)}-layer block")
    layers = build_layers(q4, torch, synth, synth.LLAMA7B_BLOCK, G, M, workload, copies)
    block_bytes = sum(ly.bytes for ly in layers)
    assert copies * block_bytes >= MALL_DEFEAT_BYTES * 0.97
    stream = torch.cuda.Stream()
    assert all(ly.mats[0].path_for(M) == q4.PATH_GEMV for ly in layers)

    if args.counters:
        sp = ctypes.c_void_p(stream.cuda_stream)
        with torch.cuda.stream(stream):
            for s in range(20):
                for ly in layers:
                    ly.launch(lib, s % copies, sp)
            src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(5):
                dst.copy_(src)
        torch.cuda.synchronize()
        log(json.dumps({"counters_run": True, "launches_per_layer": 20, "copy_bytes": 256 << 20,
                        "layers": [[ly.name, ly.bytes] for ly in layers],
                        "source_hash": kernel_source_hash()}))
        return

    log("[bench] per-launch event timing")
    lt = per_launch_times(lib, torch, layers, min_launches=200, stream=stream)
    kern_bytes = sum(ly.bytes for ly in layers)
    layer_bytes = [ly.bytes for ly in layers]
    n_layers = len(layers)
    kern_time = sum(lt)
    achieved = kern_bytes / kern_time / 1e9

    log(f"[bench] timing {args.steps} steps after {args.warmup} warmup "
        f"({'eager' if args.eager else 'graph replay'})")
    elapsed, wall, graphs = time_steps(lib, torch, layers, copies, args.steps, args.warmup, stream,
                                       use_graph=not args.eager)
    ms_per_step = elapsed / args.steps * 1e3
    value = block_bytes / (elapsed / args.steps) / 1e9
    # eager figure for reference (the host launch path, no graph)
    eager_gbs = None
    if not args.no_eager:
        e_elapsed, _, _ = time_steps(lib, torch, layers, copies, min(args.steps, 500), 20, stream,
                                     use_graph=False)
        eager_gbs = round(block_bytes / (e_elapsed / min(args.steps, 500)) / 1e9, 1)

    del graphs
    for ly in layers:
        ly.close()
    del layers
    torch.cuda.empty_cache()

    sec = {} if args.no_secondary else secondary(q4, torch, synth, lib, stream)

    log("[bench] read ceiling")
    # (16 KiB: one workgroup reading one chunk, the time of a launch that
    # does almost nothing, in the same chain of dependent launches)
    sizes = sorted({ly_bytes for ly_bytes in (8716288, 23425024, 122028032)} | {2 << 30, 16384})
    ceiling = read_ceiling(lib, torch, stream, sizes)
    launch_floor_us = ceiling[16384]["us"]

    def probe_us(nbytes):
        """Read-probe time for nbytes, from the probe of the nearest size."""
        size = min((k for k in ceiling if k > 16384), key=lambda k: abs(k - nbytes))
        return ceiling[size]["us"] * nbytes / size

    block_read_us = sum(probe_us(b) for b in layer_bytes)
    src_hash = kernel_source_hash()
    traffic = traffic_for("q4_gemv_kernel", src_hash)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "layers": [f"{n}:{K}x{N}" for n, K, N, _ in synth.LLAMA7B_BLOCK],
            "M": M, "groupsize": G, "bias": "q_proj", "bytes_per_step": block_bytes,
            "weight_copies_rotated": copies, "launch": "eager" if args.eager else "hip_graph",
            "parallelism": "none",
        },
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "eager_GB/s": eager_gbs,
        "roofline": {
            "bound": "hbm",
            "kernel": "q4_gemv_kernel",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": round(kern_bytes / n_layers),
            "per_layer_us": {ly_name: round(t * 1e6, 3)
                             for (ly_name, _, _, _), t in zip(synth.LLAMA7B_BLOCK, lt)},
            "source_hash": src_hash,
        },
        "read_ceiling": {
            "what": "one q4_read_probe launch of each size (16-byte non-temporal loads, nothing "
                    "else), rotating over >= 1 GiB (the 16 KiB launch over 64 MiB), mean launch "
                    "time in a chain of dependent launches; launch_floor_us is the 16 KiB one",
            "by_bytes": {str(k): v for k, v in ceiling.items()},
            "block_us": round(block_read_us, 2),
            "block_GB/s": round(block_bytes / block_read_us / 1e3, 1),
            "value_frac_of_ceiling": round(block_read_us / (ms_per_step * 1e3), 4),
            "launch_floor_us": launch_floor_us,
            "block_launch_floor_us": round(n_layers * launch_floor_us, 2),
        },
        "environment": gpu_environment(torch),
        "secondary": sec,
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        import oracle
        result["cpu_baseline"] = cpu_baseline(synth, oracle, synth.LLAMA7B_BLOCK, G, workload,
                                              args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    log(f"[bench] wall {wall:.2f} s for the timed steps")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
