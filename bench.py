#!/usr/bin/env python3
"""GVA decode benchmark on one MI355X.

A step is one pass of the decode hot path for one layer's compact cache:
append one new token per sequence (RoPE on its positional key), rotate the
query's positional slice, decode (absorbed scores over V and k_r, online
softmax, P.V, split-K merge). The headline runs it as gva_decode_step (one
launch); the same step as three calls (gva_append, gva_rope_query,
gva_decode) is reported beside it.
Consecutive steps visit R distinct cache replicas (layers) so every decode
reads data that has not been touched for more than the 256 MB last-level
cache; the default workload is B=16, S=4096, H=16, G=4, d_v=d_n=64, d_r=16,
bf16 (the mid workload), on seeded synthetic data.

Prints one JSON line. `value` = steps/s of the whole path: K steps launched
back to back on one stream, queued behind a spin kernel that outlasts the
host's launch loop, so the HIP events around them measure the device running
the K steps, not the host launching them (a graph replay of the same steps is
reported beside it; it adds a fixed start cost of its own per replay).
`roofline` describes the one kernel of the timed region (the fused step):
algorithmic cache bytes per step over its average launch duration, from the
events on the stream the kernels run on. gva_decode alone (one kernel, no
append) is timed the same way and reported beside it.

`--mode gqa` instead times gva_decode against the same-shape GQA reference
(gva_gqa_ref_decode, K and V caches) on the wide workload and reports the
time ratio beside the ratio of the bytes each must read. `--mode folded`,
`multi`, `lifecycle`, `prefill` and `ragged` time the maps folded into the
query projection, several queries per sequence, the paged-cache block
operations, the causal prefill (against the matrix-core peak) and the ragged
paged batch.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of the MI355X
METRIC = "GVA decode steps/s + effective cache-read GB/s (% HBM peak), B=16 S=4096 bf16"


def hold_device():
    """Keep the GPU busy for about a millisecond (a spin kernel on the current
    stream) while the host enqueues a graph replay, so that the events bracket
    the replay as the device runs it, not the host's submission of the graph
    before its first kernel."""
    import torch
    torch.cuda._sleep(2_000_000)


def cache_capacity(tokens: int) -> int:
    """Cache capacity for at least `tokens` tokens, rounded up to a multiple
    of 512 so that each (sequence, group) slab of the contiguous value cache
    (capacity x 64 bf16 channels) starts on a 64 KiB multiple. Strides just
    past a power of two make the concurrent partition streams of many slabs
    collide in the memory channels: at B=32, S=8192 (128 slabs) a decode
    took 26.2 us with capacity 8192, 29.2 us with 8240 and 35.0 us with 8256,
    and 26.5 us with 8704 or 10240; at the mid and long shapes the capacity
    made no difference."""
    return -(-tokens // 512) * 512


def queued_time(launch, n_warm: int, K: int, host_us: float, before_timed=None):
    """Device time per call (ms) of K calls of `launch()` run back to back on
    the current stream, HIP events around them on that stream.

    The calls are enqueued behind a spin kernel that outlasts the host's
    enqueueing, after `n_warm` untimed calls queued right before them, so the
    events bracket the device's back-to-back execution of exactly K calls and
    not the host's launch loop. If the device reached the first timed call
    before the host had enqueued the last one (the start event completed
    early), the spin is lengthened from the measured host rate and the
    measurement repeated (up to three runs; if the host never stays ahead,
    the last run's figure is returned with a negative attempt count); host
    gaps could only have made the time longer.
    The spin is sized from `host_us`, the host's time per launch call, with a
    30% margin: a much longer one lets the clocks drop while one wave spins,
    and the first timed steps then run slower (measured: 10.8-10.9 us per
    mid step after a 0.5-1 ms spin, 11.0-11.1 us after 2-4 ms).
    Returns (ms per call, attempts)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for attempt in range(1, 4):
        torch.cuda.synchronize()
        torch.cuda._sleep(int((n_warm + K) * host_us * 2.4e3 * 1.3) + 300_000)  # GPU clock cycles
        t0 = time.perf_counter()
        for _ in range(n_warm):
            launch()
        if before_timed is not None:
            before_timed()
        e0.record()
        for _ in range(K):
            launch()
        e1.record()
        ahead = not e0.query()
        host_us = max(host_us, 1.5 * (time.perf_counter() - t0) * 1e6 / (n_warm + K))
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / K
        if ahead:
            return ms, attempt
    # the host never stayed ahead: the last figure may include launch gaps,
    # which can only lengthen it; reported with a negative attempt count
    return ms, -attempt


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="mid_bf16")
    p.add_argument("--replicas", type=int, default=0, help="cache replicas (0 = enough for 512 MB)")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the graph-replay figure, the GQA comparison and the ceilings")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--split", type=int, default=-1,
                   help="split-K partition length in tokens (-1 = the workload's, 0 = automatic)")
    p.add_argument("--profile-decode", type=int, default=0,
                   help="only run N eager decodes (for rocprofv3 runs) and exit")
    p.add_argument("--profile-step", type=int, default=0,
                   help="only run N eager fused steps (for rocprofv3 runs) and exit")
    p.add_argument("--profile-copy-mb", type=int, default=0,
                   help="with --profile-step/--profile-decode: first run a plain elementwise copy "
                        "(read N MiB, write N MiB) three times, the reference for traffic counters")
    p.add_argument("--mode", choices=["step", "gqa", "folded", "multi", "lifecycle", "prefill", "ragged",
                                      "ceiling"],
                   default="step")
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "this decode path has no multi-GPU mode; see the sharding notes in the design doc.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import compact_kv_cache_amd as gva
    import workloads as W
    from compact_kv_cache_amd.cache import GvaCache

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.mode == "gqa":
        gqa_compare(args)
        return
    if args.mode == "folded":
        folded_compare(args)
        return
    if args.mode == "multi":
        multi_compare(args)
        return
    if args.mode == "lifecycle":
        lifecycle_bench(args)
        return
    if args.mode == "prefill":
        prefill_bench(args)
        return
    if args.mode == "ragged":
        ragged_bench(args)
        return
    if args.mode == "ceiling":
        ceiling_bench(args)
        return
    wl = W.WORKLOADS[args.workload]
    if args.split >= 0:
        wl = wl.replace(split_tokens=args.split)
    assert not wl.ragged, "bench drives uniform-length workloads"
    base = wl.rope_base
    bpt = gva.gva_cache_bytes_per_token(wl.G, wl.d_v, wl.d_r, wl.dtype)
    cache_bytes = wl.B * wl.S * bpt
    R = args.replicas or max(2, math.ceil(512e6 / cache_bytes))
    K, Wm = args.steps, args.warmup
    # every step appends a token; the queued regions may run up to three times
    # (queued_time): 2 eager + 3 (W - 2 + K) fused + 3 K three-call + (W - 2 + K)
    # graph + K eager steps at most
    total_steps = 4 * Wm + 8 * K + 8
    per_rep = math.ceil(total_steps / R) + 1
    cap = cache_capacity(wl.S + per_rep)

    # ---- inputs (seeded, synthetic) -------------------------------------
    inp = W.make_gva_inputs(wl)
    rng = np.random.Generator(np.random.PCG64(wl.seed + 77))
    v_new = W.round_storage(rng.standard_normal((total_steps, wl.B, wl.G, 1, wl.d_v)), wl.dtype)
    kr_new = W.round_storage(rng.standard_normal((total_steps, wl.B, 1, wl.d_r)), wl.dtype)
    td = W.torch_dtype(wl.dtype)
    to = lambda x: W.to_torch(x, wl.dtype).to(dev)  # noqa: E731
    q_nope, q_rope, M0 = to(inp.q_nope), to(inp.q_rope), to(inp.M)
    v_new_d, kr_new_d = to(v_new), to(kr_new)
    q_rot = torch.empty_like(q_rope)
    out = torch.empty(wl.B, wl.H, wl.d_v, dtype=td, device=dev)

    caches = []
    first = GvaCache(wl.B, wl.H, wl.G, wl.d_n, wl.d_v, wl.d_r, dtype=wl.dtype, capacity=cap,
                     device=dev)
    first.append(to(np.stack(inp.V)), to(np.stack(inp.kr)), base)
    caches.append(first)
    for _ in range(R - 1):
        c = GvaCache(wl.B, wl.H, wl.G, wl.d_n, wl.d_v, wl.d_r, dtype=wl.dtype, capacity=cap,
                     device=dev)
        c.v_cache.copy_(first.v_cache)
        c.kr_cache.copy_(first.kr_cache)
        c.seq_lens.copy_(first.seq_lens)
        caches.append(c)
    del inp
    # every replica stands for one layer and carries its own reconstruction maps
    Ms = [M0] + [M0.clone() for _ in range(R - 1)]
    n_host = [wl.S] * R
    ws_bytes = max(gva.gva_decode_workspace_bytes(caches[0].shape(n, wl.split_tokens))
                   for n in range(wl.S, cap + 1))
    ws = torch.zeros(max(ws_bytes, 4) // 4 + 1, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def shape_at(r, n):
        return caches[r].shape(n, wl.split_tokens)

    def decode(r):
        c = caches[r]
        gva.gva_decode(shape_at(r, n_host[r]), q_nope, q_rot, Ms[r], c.v_cache, c.kr_cache,
                       c.seq_lens, None, wl.scale, out, ws)

    step_bytes = []
    ws_step_bytes = max(gva.gva_decode_step_workspace_bytes(caches[0].shape(n, wl.split_tokens))
                        for n in range(wl.S, cap + 1))
    ws_step = torch.zeros(ws_step_bytes // 4 + 1, dtype=torch.float32, device=dev)

    def fused_step(i):
        r = i % R
        c = caches[r]
        n_host[r] += 1
        gva.gva_decode_step(shape_at(r, n_host[r]), v_new_d[i].view(wl.B, wl.G, wl.d_v),
                            kr_new_d[i].view(wl.B, wl.d_r), q_nope, q_rope, Ms[r], c.v_cache,
                            c.kr_cache, c.seq_lens, None, wl.scale, base, out, ws_step)
        step_bytes.append(wl.B * n_host[r] * bpt)

    def step(i):
        r = i % R
        c = caches[r]
        gva.gva_append(shape_at(r, c.capacity), v_new_d[i], kr_new_d[i], 1, c.seq_lens,
                       c.v_cache, c.kr_cache, None, base)
        n_host[r] += 1
        gva.gva_rope_query(shape_at(r, n_host[r]), q_rope, q_rot, c.seq_lens, base)
        decode(r)
        step_bytes.append(wl.B * n_host[r] * bpt)

    if args.profile_copy_mb and (args.profile_decode or args.profile_step):
        nb = args.profile_copy_mb << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.profile_decode:
        for i in range(args.profile_decode):
            decode(i % R)
        torch.cuda.synchronize()
        print(json.dumps({"profile_decode": args.profile_decode, "replicas": R}))
        return
    if args.profile_step:
        for i in range(args.profile_step):
            fused_step(i)
        torch.cuda.synchronize()
        print(json.dumps({"profile_step": args.profile_step, "replicas": R}))
        return

    # Warm-up: the W untimed steps. The first two run eagerly, one of each
    # form of the step (loading both paths), then synchronized; the rest are
    # queued right before the timed steps, so those start on a busy device in
    # steady state.
    use_graph = not args.no_graph
    n_eager = min(Wm, 2)
    counter = [0]

    def next_index():
        counter[0] += 1
        return counter[0] - 1

    for k in range(n_eager):
        (fused_step if k % 2 == 0 else step)(next_index())
    torch.cuda.synchronize()
    # host time per launch call through the Python binding (the first calls
    # above include one-time loading, so not measured there); queued_time
    # lengthens the spin from the measured rate if the host falls behind
    host_us_fused, host_us_three = 25.0, 75.0

    def graph_time(fn, warm=0):
        """The same K steps captured in one graph (after `warm` untimed steps
        in a graph of their own) and replayed behind the spin kernel: the
        replay's fixed start cost (about 13 us) lands inside the events."""
        gw = None
        if warm > 0:
            gw = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gw):
                for k in range(warm):
                    fn(next_index())
        step_bytes.clear()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(K):
                fn(next_index())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hold_device()
        if gw is not None:
            gw.replay()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    # ---- timed region 1: the whole step, one launch (gva_decode_step), K
    # launches back to back behind the spin kernel --------------------------
    n_queued_warm = Wm - n_eager
    ms_step, step_attempts = queued_time(lambda: fused_step(next_index()), n_queued_warm, K, host_us_fused,
                                         before_timed=step_bytes.clear)
    mean_step_bytes = float(np.mean(step_bytes))
    ms_per_step = ms_step
    # the same step as three calls (append, rope_query, decode)
    ms_three, _ = queued_time(lambda: step(next_index()), 0, K, host_us_three)
    # the fused step replayed from a graph (the former timing method)
    ms_graph = graph_time(fused_step, n_queued_warm) if use_graph else None
    # eager (host-launched) fused steps, host clock: the Python launch rate
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        fused_step(next_index())
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / K

    # ---- timed region 2: decode kernel alone, HIP events around each call --
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    dec_bytes = []
    torch.cuda.synchronize()
    for k in range(K):
        r = k % R
        evs[k][0].record(stream)
        decode(r)
        evs[k][1].record(stream)
        dec_bytes.append(wl.B * n_host[r] * bpt)
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in evs]
    dec_ms_mean = float(np.mean(dec_ms))
    dec_bytes_mean = float(np.mean(dec_bytes))

    # ---- timed region 3: K decode launches back to back behind the spin
    # kernel, HIP events around the whole run on the launch stream: the
    # average launch duration without per-call event overhead (the figure the
    # kernel trace's average reproduces)
    dec_i = [0]

    def next_decode():
        decode(dec_i[0] % R)
        dec_i[0] += 1

    ms_dec_queued, _ = queued_time(next_decode, R, K, 20.0)
    ms_launch = ms_dec_queued
    dec_gbps = dec_bytes_mean / (ms_launch * 1e-3) / 1e9
    # the timed region launches one kernel per step (the fused step)
    achieved = mean_step_bytes / (ms_step * 1e-3) / 1e9

    traffic = recorded_traffic(wl.name)

    # partition length(s) of the lengths the recorded steps ran at (the
    # automatic choice depends on the number of 64-token tiles)
    splits = sorted({gva.gva_decode_split_tokens(shape_at(0, int(round(b / (wl.B * bpt)))))
                     for b in step_bytes})
    split_used = splits[0] if len(splits) == 1 else splits
    result = {
        "metric": METRIC,
        "value": round(1e3 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) caches and queries, M ~ N(0,1/64))",
        "config": {"workload": f"{wl.name}: GVA decode step B={wl.B} S={wl.S} H={wl.H} "
                               f"G={wl.G} d_n={wl.d_n} d_v={wl.d_v} d_r={wl.d_r} {wl.dtype}, "
                               f"contiguous cache, {R} cold replicas",
                   "B": wl.B, "S": wl.S, "H": wl.H, "G": wl.G, "d_v": wl.d_v, "d_r": wl.d_r,
                   "replicas": R, "split_tokens": split_used,
                   "timing": "K launches back to back, queued behind a spin kernel",
                   "step": "gva_decode_step (one launch)"},
        "cache_read_GBps": round(mean_step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_kernel_us": round(ms_step * 1e3, 3),
        "decode_us": round(ms_launch * 1e3, 3),
        "decode_cache_read_GBps": round(dec_gbps, 1),
        "decode_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "decode_event_per_call_us": round(dec_ms_mean * 1e3, 3),
        "decode_event_per_call_median_us": round(float(np.median(dec_ms)) * 1e3, 3),
        "graph_ms_per_step": None if ms_graph is None else round(ms_graph, 6),
        "timing_attempts": step_attempts,
        "eager_ms_per_step": round(ms_eager, 6),
        "three_call_steps_per_s": round(1e3 / ms_three, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "fused decode step",
                     "bytes_per_launch": mean_step_bytes},
    }

    if use_graph:
        # speed-up of the decode over the same-shape GQA reference (decode
        # kernels only, each timed back to back over its own cold replicas)
        caches.clear()  # the step replicas are no longer needed
        Ms.clear()
        torch.cuda.empty_cache()
        cmp = measure_gva_vs_gqa(wl, K)
        result["gqa_decode_us"] = cmp["gqa"]["us"]
        result["gva_decode_us_same_pass"] = cmp["gva"]["us"]
        result["speedup_vs_gqa"] = cmp["time_ratio_gqa_over_gva"]
        result["gqa_byte_ratio"] = cmp["byte_ratio_gqa_over_gva"]

    if use_graph:
        # the same GPU's ceilings for this many bytes, measured in this process
        ceil = measure_ceilings(mean_step_bytes)
        result["ceiling"] = ceil
        result["ceiling_GBps"] = ceil["read_GBps"]
        result["frac_of_ceiling"] = round(achieved / ceil["read_GBps"], 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def measure_ceilings(read_bytes: int, replicas: int = 16):
    """Ceilings on this GPU, timed in this process (libgva_ceiling.so) as K
    launches back to back behind a spin kernel, like the decode step:
    the per-launch floor of an empty kernel, a plain read of `read_bytes` in
    the decode's load pattern (256 workgroups, 1 KB per load instruction,
    `replicas` cold buffers), and a 2 GiB streaming read."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "compact_kv_cache_amd", "libgva_ceiling.so"))
    lib.ceiling_empty_us.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.ceiling_read_us.argtypes = [ctypes.c_ulonglong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_double)]
    us = ctypes.c_double()

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")
        return us.value

    wgs = 256
    unit = wgs * 1024
    rb = max(unit, (int(read_bytes) // unit) * unit)
    empty = check(lib.ceiling_empty_us(100, ctypes.byref(us)), "empty-launch ceiling")
    mid = check(lib.ceiling_read_us(rb, replicas, wgs, 64, ctypes.byref(us)), "read ceiling")
    big_bytes = 2 << 30
    big = check(lib.ceiling_read_us(big_bytes, 2, 2048, 20, ctypes.byref(us)), "2 GiB read ceiling")
    return {"empty_launch_us": round(empty, 3),
            "read_bytes": rb, "read_us": round(mid, 3), "read_GBps": round(rb / (mid * 1e-6) / 1e9, 1),
            "read_2GiB_us": round(big, 2), "read_2GiB_GBps": round(big_bytes / (big * 1e-6) / 1e9, 1),
            "kernel": "plain read, 1 KB per load instruction, 256 workgroups x 8 waves, "
                      "every load of a wave requested at once; cold replicas; K launches back to back behind a spin kernel"}


def ceiling_bench(args):
    """`--mode ceiling`: the ceilings alone (empty launch, plain read of the
    mid cache's bytes, 2 GiB read), one JSON line."""
    import workloads as W
    wl = W.WORKLOADS["mid_bf16"]
    bpt = (wl.G * wl.d_v + wl.d_r) * 2
    res = measure_ceilings(wl.B * wl.S * bpt)
    res["mode"] = "ceiling"
    print(json.dumps(res), flush=True)


KERNEL_SOURCES = ("compact_kv_cache_amd/csrc/decode_mfma.hip", "compact_kv_cache_amd/csrc/gva_device.hpp",
                  "compact_kv_cache_amd/csrc/launch.hpp", "compact_kv_cache_amd/csrc/mfma_common.hpp")


def recorded_traffic(workload: str):
    """HBM bytes per fused-step launch from the committed counter summary, or
    None when there is none for this workload or the kernel sources changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"step_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].strip().split(": ", 1)
            rec[k] = v
    if rec.get("workload") != workload or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return int(rec["traffic_bytes_per_launch"])


def kernel_source_hash() -> str:
    """sha256 of the decode kernel's sources with // comments, trailing blanks
    and empty lines removed (comment edits do not change the kernel)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            for line in fh:
                line = re.sub(r"//.*$", "", line).rstrip()
                if line:
                    h.update(line.encode() + b"\n")
    return h.hexdigest()


def gqa_compare(args):
    """`--mode gqa`: gva_decode against gva_gqa_ref_decode on the wide workload
    (or the one named), one JSON line."""
    import workloads as W
    wl = W.WORKLOADS["wide_dr24" if args.workload == "mid_bf16" else args.workload]
    res = measure_gva_vs_gqa(wl, args.steps)
    res["config"] = {"workload": f"{wl.name}: B={wl.B} S={wl.S} H={wl.H} G={wl.G} d_v={wl.d_v} "
                                 f"d_r={wl.d_r} {wl.dtype}, contiguous caches, cold replicas",
                     "steps": args.steps}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_gqa(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def folded_compare(args):
    """`--mode folded`: one layer's decode step from hidden states x [B, d_model]
    (d_model = H * d_n), with and without the maps folded into the query
    projection. unfolded: projection to q_nope, q_rope, then the fused step
    with M; folded: projection to q' = (M W_q,nope) x, q_rope, then the fused
    step without M. Every replica (layer) has its own weights and cache; each
    variant is timed as K steps in one graph."""
    import numpy as np
    import torch

    import compact_kv_cache_amd as gva
    import workloads as W
    from compact_kv_cache_amd.cache import GvaCache

    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[args.workload]
    K = args.steps
    d_model = wl.H * wl.d_n
    bpt = gva.gva_cache_bytes_per_token(wl.G, wl.d_v, wl.d_r, wl.dtype)
    R = max(2, math.ceil(512e6 / (wl.B * wl.S * bpt)))
    n_steps = 6 * K + 8
    cap = cache_capacity(wl.S + math.ceil(n_steps / R) + 2)
    inp = W.make_gva_inputs(wl)
    to = lambda a: W.to_torch(a, wl.dtype).to(dev)  # noqa: E731
    first = GvaCache(wl.B, wl.H, wl.G, wl.d_n, wl.d_v, wl.d_r, dtype=wl.dtype, capacity=cap, device=dev)
    first.append(to(np.stack(inp.V)), to(np.stack(inp.kr)), wl.rope_base)
    caches = [first]
    for _ in range(R - 1):
        c = GvaCache(wl.B, wl.H, wl.G, wl.d_n, wl.d_v, wl.d_r, dtype=wl.dtype, capacity=cap, device=dev)
        c.v_cache.copy_(first.v_cache)
        c.kr_cache.copy_(first.kr_cache)
        c.seq_lens.copy_(first.seq_lens)
        caches.append(c)
    x_h, wq_nope_h, wq_rope_h = W.make_projection_inputs(wl, d_model)
    M = to(inp.M)
    layers = []
    for r in range(R):
        wq = to(wq_nope_h) if r == 0 else layers[0]["wq"].clone()
        wr = to(wq_rope_h) if r == 0 else layers[0]["wr"].clone()
        wf = torch.empty(wl.H, wl.d_v, d_model, dtype=W.torch_dtype(wl.dtype), device=dev)
        gva.gva_fold_query_projection(M, wq, wf)
        layers.append({"wq": wq, "wr": wr, "wf": wf, "M": M.clone()})
    del inp
    x = to(x_h)
    td = W.torch_dtype(wl.dtype)
    q_a = torch.empty(wl.B, wl.H, wl.d_v, dtype=td, device=dev)
    q_r = torch.empty(wl.B, wl.H, wl.d_r, dtype=td, device=dev)
    out = torch.empty(wl.B, wl.H, wl.d_v, dtype=td, device=dev)
    v_new = torch.randn(wl.B, wl.G, wl.d_v, device=dev).to(td)
    k_new = torch.randn(wl.B, wl.d_r, device=dev).to(td)
    n_host = [wl.S] * R
    ws = torch.zeros(gva.gva_decode_step_workspace_bytes(caches[0].shape(cap)) // 4 + 1,
                     dtype=torch.float32, device=dev)

    def project(i, folded):
        r = i % R
        L = layers[r]
        gva.gva_query_projection(caches[r].shape(cap), x, L["wf"] if folded else L["wq"], L["wr"], q_a, q_r)

    def fstep(i, folded):
        r = i % R
        n_host[r] += 1
        caches[r].step(v_new, k_new, q_a, q_r, None if folded else layers[r]["M"], wl.scale, out, n_host[r],
                       workspace=ws, rope_base=wl.rope_base)

    def layer_step(i, folded):
        project(i, folded)
        fstep(i, folded)

    def gtime(fn, first_i):
        for k in range(2 * R):
            fn(first_i + k)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(K):
                fn(first_i + 2 * R + k)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K * 1e3

    # lengths grow by one per step and replica; every variant steps the same caches
    res = {}
    res["unfolded_layer_step_us"] = gtime(lambda i: layer_step(i, False), 0)
    res["folded_layer_step_us"] = gtime(lambda i: layer_step(i, True), 0)
    res["fused_step_with_M_us"] = gtime(lambda i: fstep(i, False), 0)
    res["fused_step_folded_us"] = gtime(lambda i: fstep(i, True), 0)
    res["projection_us"] = gtime(lambda i: project(i, True), 0)
    res = {k: round(v, 3) for k, v in res.items()}
    res.update({
        "mode": "folded_compare",
        "config": {"workload": f"{wl.name}: B={wl.B} S={wl.S}.. H={wl.H} G={wl.G} d_v=d_n={wl.d_v} "
                               f"d_r={wl.d_r} d_model={d_model} {wl.dtype}, {R} cold replicas with their own "
                               f"weights", "steps": K},
        "layer_steps_per_s": {"unfolded": round(1e6 / res["unfolded_layer_step_us"], 1),
                              "folded": round(1e6 / res["folded_layer_step_us"], 1)},
        "projection_weight_bytes": wl.H * (wl.d_v + wl.d_r) * d_model * 2,
    })
    print(json.dumps(res), flush=True)


def multi_compare(args):
    """`--mode multi`: gva_decode_multi with n_q = 1, 2, 4 queries per sequence
    (the last n_q tokens, causal among them) on the mid shape, K launches in a
    graph over cold replicas. The cache bytes per launch are the same; the
    query tokens served per launch grow with n_q."""
    import numpy as np
    import torch

    import compact_kv_cache_amd as gva
    import workloads as W

    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[args.workload]
    K = args.steps
    n = wl.S + 4
    bpt = gva.gva_cache_bytes_per_token(wl.G, wl.d_v, wl.d_r, wl.dtype)
    nbytes = wl.B * n * bpt
    R = max(2, math.ceil(512e6 / nbytes))
    rng = np.random.Generator(np.random.PCG64(wl.seed + 5))
    V0 = torch.from_numpy(rng.standard_normal((wl.B, wl.G, n, wl.d_v), dtype=np.float32)).to(dev).bfloat16()
    K0 = torch.from_numpy(rng.standard_normal((wl.B, n, wl.d_r), dtype=np.float32)).to(dev).bfloat16()
    reps = [(V0.clone(), K0.clone(), (torch.randn(wl.H, wl.d_v, wl.d_n, device=dev) / 8).bfloat16())
            for _ in range(R)]
    del V0, K0
    seq = torch.full((wl.B,), n, dtype=torch.int32, device=dev)
    shape = gva.make_shape(wl.B, wl.H, wl.G, wl.d_n, wl.d_v, wl.d_r, capacity=n, max_seq_len=n, dtype=wl.dtype)
    res = {"mode": "multi_compare",
           "config": {"workload": f"{wl.name}: B={wl.B} n={n} H={wl.H} G={wl.G} d_v=d_n={wl.d_v} d_r={wl.d_r} "
                                  f"{wl.dtype}, contiguous, {R} cold replicas", "steps": K},
           "cache_bytes_per_launch": nbytes}
    for nq in (1, 2, 4):
        q = torch.randn(wl.B, nq, wl.H, wl.d_n, device=dev).bfloat16()
        qr = torch.randn(wl.B, nq, wl.H, wl.d_r, device=dev).bfloat16()
        out = torch.empty(wl.B, nq, wl.H, wl.d_v, dtype=torch.bfloat16, device=dev)
        ws = torch.zeros(max(gva.gva_decode_multi_workspace_bytes(shape, nq), 4) // 4 + 1,
                         dtype=torch.float32, device=dev)

        def call(i):
            v, k, M = reps[i % R]
            gva.gva_decode_multi(shape, nq, q, qr, M, v, k, seq, None, wl.scale, out, ws)

        host = []
        for i in range(2 * R):
            t0 = time.perf_counter()
            call(i)
            host.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        ci = [0]

        def next_call():
            call(ci[0])
            ci[0] += 1

        ms, _ = queued_time(next_call, R, K, 1e6 * float(np.median(host)))
        us = ms * 1e3
        res[f"nq{nq}"] = {"us": round(us, 3), "cache_GBps": round(nbytes / us / 1e3, 1),
                          "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4),
                          "query_tokens_per_s": round(wl.B * nq / us * 1e6, 1)}
    print(json.dumps(res), flush=True)


def prefill_flops(B: int, H: int, n: int, nq: int, d_v: int, d_r: int, d_n: int, absorb: bool) -> float:
    """Algorithmic flops of a causal prefill: per (sequence, head, query j at
    position n - n_q + j, cached token t <= that position) a score over the
    absorbed key width and the positional slice (2*(d_v + d_r)) and the
    probability-weighted value row (2*d_v); plus the absorption q' = M q
    (2*d_n*d_v per query and head) when the maps are given."""
    pos = [n - nq + j for j in range(nq)]
    pairs = sum(p + 1 for p in pos if p >= 0)
    f = B * H * pairs * (2.0 * (d_v + d_r) + 2.0 * d_v)
    if absorb:
        f += B * nq * H * 2.0 * d_n * d_v
    return f


def prefill_bench(args):
    """`--mode prefill`: gva_prefill on the mid shape (B=16, a 4096-token
    prompt, H=16, G=4, d_r=16), the whole prompt as queries, and the last
    512-token chunk of a chunked prefill of the same prompt; K launches in one
    graph, HIP events around the replay. Compute-bound: reported against the
    dense bf16 matrix-core peak."""
    import numpy as np
    import torch

    import compact_kv_cache_amd as gva
    import workloads as W

    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[args.workload]
    K = args.steps
    n = wl.S
    rng = np.random.Generator(np.random.PCG64(wl.seed + 9))
    V = torch.from_numpy(rng.standard_normal((wl.B, wl.G, n, wl.d_v), dtype=np.float32)).to(dev).bfloat16()
    Kr = torch.from_numpy(rng.standard_normal((wl.B, n, wl.d_r), dtype=np.float32)).to(dev).bfloat16()
    M = (torch.randn(wl.H, wl.d_v, wl.d_n, device=dev) / 8).bfloat16()
    seq = torch.full((wl.B,), n, dtype=torch.int32, device=dev)
    shape = gva.make_shape(wl.B, wl.H, wl.G, wl.d_n, wl.d_v, wl.d_r, capacity=n, max_seq_len=n, dtype=wl.dtype)
    res = {"mode": "prefill",
           "config": {"workload": f"{wl.name} prefill: B={wl.B} prompt n={n} H={wl.H} G={wl.G} d_v=d_n={wl.d_v} "
                                  f"d_r={wl.d_r} {wl.dtype}, contiguous cache, maps M in the kernel",
                      "steps": K}}
    for label, nq in (("full_prompt", n), ("last_chunk_512", 512)):
        q = torch.randn(wl.B, nq, wl.H, wl.d_n, device=dev).bfloat16()
        qr = torch.randn(wl.B, nq, wl.H, wl.d_r, device=dev).bfloat16()
        out = torch.empty(wl.B, nq, wl.H, wl.d_v, dtype=torch.bfloat16, device=dev)

        def call():
            gva.gva_prefill(shape, nq, q, qr, M, V, Kr, seq, None, wl.scale, out)

        # warm-up long enough (about half a second) for the clocks to settle
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < 0.5:
            for _ in range(5):
                call()
            torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(K):
                call()
        torch.cuda.synchronize()
        g.replay()  # once untimed, straight into the timed replay: no idle gap for the clocks to drop
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / K * 1e3
        fl = prefill_flops(wl.B, wl.H, n, nq, wl.d_v, wl.d_r, wl.d_n, True)
        tf = fl / us / 1e6
        res[label] = {"n_q": nq, "us": round(us, 2), "flops": fl, "TFLOPs": round(tf, 1),
                      "frac_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                      "query_tokens_per_s": round(wl.B * nq / us * 1e6, 1)}
        del q, qr, out, g
    full = res["full_prompt"]
    res["roofline"] = {"bound": "mfma", "achieved": full["TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": full["frac_bf16_peak"], "traffic": None,
                       "kernel": "prefill_mfma_kernel (whole prompt)"}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def ragged_bench(args):
    """`--mode ragged`: the ragged paged workload (B=64, lengths uniform in
    [1024, 32768] from the workload's seed, 64-token blocks in a shuffled
    table): gva_decode and the fused step (one appended token per sequence),
    K launches in one graph over R cold replicas of the page pool."""
    import numpy as np
    import torch

    import compact_kv_cache_amd as gva
    import workloads as W

    dev = torch.device("cuda:0")
    wl = W.WORKLOADS["ragged_paged"]
    K = args.steps
    ROUNDS = 5
    lens = W.ragged_lens(wl)
    extra = K + 8
    table, nblk = W.paged_pool(lens + extra, 64, wl.seed)
    bpt = gva.gva_cache_bytes_per_token(wl.G, wl.d_v, wl.d_r, wl.dtype)
    pool_bytes = nblk * 64 * bpt
    R = max(2, math.ceil(512e6 / pool_bytes))
    reps = []
    for _ in range(R):
        v = torch.randn(nblk, wl.G, 64, wl.d_v, device=dev).bfloat16()
        k = torch.randn(nblk, 64, wl.d_r, device=dev).bfloat16()
        reps.append((v, k, (torch.randn(wl.H, wl.d_v, wl.d_n, device=dev) / 8).bfloat16(),
                     torch.tensor(lens.astype(np.int32), device=dev)))
    tab = torch.tensor(table, device=dev)
    q = torch.randn(wl.B, wl.H, wl.d_n, device=dev).bfloat16()
    qr = torch.randn(wl.B, wl.H, wl.d_r, device=dev).bfloat16()
    out = torch.empty(wl.B, wl.H, wl.d_v, dtype=torch.bfloat16, device=dev)
    v_new = torch.randn(wl.B, wl.G, wl.d_v, device=dev).bfloat16()
    k_new = torch.randn(wl.B, wl.d_r, device=dev).bfloat16()
    n_max = int(lens.max()) + extra

    def shape_at(n):
        return gva.make_shape(wl.B, wl.H, wl.G, wl.d_n, wl.d_v, wl.d_r, max_seq_len=n, block_size=64,
                              num_blocks=nblk, max_blocks_per_seq=table.shape[1],
                              split_tokens=max(args.split, 0), dtype=wl.dtype)

    shape = shape_at(n_max)
    ws = torch.zeros(gva.gva_decode_step_workspace_bytes(shape) // 4 + 1, device=dev)

    def dec(i):
        v, k, M, sl = reps[i % R]
        gva.gva_decode(shape, q, qr, M, v, k, sl, tab, wl.scale, out, ws)

    def step(i):
        v, k, M, sl = reps[i % R]
        gva.gva_decode_step(shape, v_new, k_new, q, qr, M, v, k, sl, tab, wl.scale, wl.rope_base, out, ws)

    if args.profile_decode or args.profile_step:  # eager launches only, for counter runs
        for i in range(args.profile_decode):
            dec(i)
        for i in range(args.profile_step):
            step(i)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "ragged", "profile_decode": args.profile_decode,
                          "profile_step": args.profile_step, "replicas": R}))
        return
    res = {"mode": "ragged",
           "config": {"workload": f"ragged_paged: B={wl.B} lengths U[{wl.len_lo}, {wl.len_hi}] (seeded, "
                                  f"mean {lens.mean():.0f}) H={wl.H} G={wl.G} d_r={wl.d_r} bf16, 64-token pages "
                                  f"in a shuffled table, {R} cold replicas of the page pool", "steps": K,
                      "rounds": ROUNDS, "split_tokens": gva.gva_decode_split_tokens(shape_at(n_max))}}
    lens0 = torch.tensor(lens.astype(np.int32), device=dev)

    def reset_lengths():  # every round starts from the batch's own lengths
        for r in reps:
            r[3].copy_(lens0)
        torch.cuda.synchronize()

    graphs = {}
    for label, fn in (("decode", dec), ("fused_step", step)):
        for i in range(2 * R):
            fn(i)
        reset_lengths()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                fn(i)
        torch.cuda.synchronize()
        graphs[label] = g
    # the two graphs replayed in turn, ROUNDS times each: the comparison is not
    # at the mercy of one replay's clocks or of which graph runs first
    times = {"decode": [], "fused_step": []}
    tokens = {"decode": [], "fused_step": []}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(ROUNDS):
        for label in ("decode", "fused_step"):
            before = sum(int(r[3].sum()) for r in reps)
            e0.record()
            graphs[label].replay()
            e1.record()
            torch.cuda.synchronize()
            times[label].append(e0.elapsed_time(e1) / K * 1e3)
            # cache tokens read per launch: every replica's lengths (the step reads its new token too)
            after = sum(int(r[3].sum()) for r in reps)
            tokens[label].append((before + after) / 2 / R)
            reset_lengths()
    for label in ("decode", "fused_step"):
        us = statistics.median(times[label])
        nbytes = statistics.mean(tokens[label]) * bpt
        res[label] = {"us": round(us, 2), "us_each_round": [round(t, 2) for t in times[label]],
                      "cache_bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
                      "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)}
    pair = [s_ / d_ for s_, d_ in zip(times["fused_step"], times["decode"])]
    res["step_over_decode"] = {"median": round(statistics.median(pair), 4),
                               "each_round": [round(x, 4) for x in pair]}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_ragged(wl, lens, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def lifecycle_bench(args):
    """`--mode lifecycle`: paged-cache block copies (copy-on-write of 1024
    blocks of 64 tokens: every V row of 4 groups and the positional keys, read
    and written once), and the launch cost of fork (64 sequences) and rollback,
    each as K launches in one graph."""
    import numpy as np
    import torch

    import compact_kv_cache_amd as gva

    dev = torch.device("cuda:0")
    K = args.steps
    B, n_pairs, nblk = 64, 1024, 4096
    shape = gva.make_shape(B, 16, 4, 64, 64, 16, max_seq_len=64 * 64, block_size=64, num_blocks=nblk,
                           max_blocks_per_seq=64, dtype="bf16")
    v = torch.randn(nblk, 4, 64, 64, device=dev).bfloat16()
    k = torch.randn(nblk, 64, 16, device=dev).bfloat16()
    table = torch.arange(B * 64, dtype=torch.int32, device=dev).view(B, 64).contiguous()
    seq = torch.full((B,), 1000, dtype=torch.int32, device=dev)
    perm = np.random.Generator(np.random.PCG64(7)).permutation(nblk).astype(np.int32)
    pairs = [(torch.tensor(perm[i * 2 * n_pairs:(i * 2 + 1) * n_pairs], device=dev),
              torch.tensor(perm[(i * 2 + 1) * n_pairs:(i * 2 + 2) * n_pairs], device=dev)) for i in range(2)]
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    src_s = torch.arange(0, B // 2, dtype=torch.int32, device=dev)
    dst_s = torch.arange(B // 2, B, dtype=torch.int32, device=dev)

    def gtime(fn):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K * 1e3

    block_bytes = 4 * 64 * 64 * 2 + 64 * 16 * 2
    us_copy = gtime(lambda i: gva.gva_copy_blocks(shape, pairs[i % 2][0], pairs[i % 2][1], v, k))
    us_fork = gtime(lambda i: gva.gva_fork(shape, src_s, dst_s, seq, table))
    us_roll = gtime(lambda i: gva.gva_rollback(shape, seq, zero))
    moved = 2 * n_pairs * block_bytes  # read + write
    print(json.dumps({
        "mode": "lifecycle",
        "config": {"workload": f"paged bf16 cache, {nblk} blocks of 64 tokens (G=4, d_v=64, d_r=16, "
                               f"{block_bytes} B per block); copy {n_pairs} blocks; fork 32 of 64 sequences",
                   "steps": K},
        "copy_blocks_us": round(us_copy, 3), "copy_bytes_moved": moved,
        "copy_GBps": round(moved / us_copy / 1e3, 1), "copy_frac": round(moved / us_copy / 1e3 / HBM_PEAK_GBPS, 4),
        "fork_us": round(us_fork, 3), "rollback_us": round(us_roll, 3)}), flush=True)


def measure_gva_vs_gqa(wl, K: int) -> dict:
    """gva_decode and gva_gqa_ref_decode on the same B, S, G, H and d_v = d_h:
    the GVA cache (G value rows + one positional key per token) against the
    GQA cache (G key rows + G value rows per token). Each is timed as K
    back-to-back launches over cold replicas, queued behind a spin kernel."""
    import numpy as np
    import torch

    import compact_kv_cache_amd as gva

    dev = torch.device("cuda:0")
    out = {}
    for kind in ("gva", "gqa"):
        d_r = wl.d_r if kind == "gva" else 0
        bpt = gva.gva_cache_bytes_per_token(wl.G, wl.d_v, d_r, wl.dtype) * (1 if kind == "gva" else 2)
        nbytes = wl.B * wl.S * bpt
        R = max(2, math.ceil(512e6 / nbytes))
        rng = np.random.Generator(np.random.PCG64(wl.seed + (1 if kind == "gva" else 2)))
        # cache contents do not change the timing; seeded N(0,1) values, bf16
        base_v = torch.from_numpy(rng.standard_normal((wl.B, wl.G, wl.S, wl.d_v), dtype=np.float32)).to(dev).bfloat16()
        if kind == "gva":
            second = torch.from_numpy(rng.standard_normal((wl.B, wl.S, d_r), dtype=np.float32)).to(dev).bfloat16()
        else:
            second = torch.from_numpy(rng.standard_normal((wl.B, wl.G, wl.S, wl.d_v), dtype=np.float32)).to(dev).bfloat16()
        reps = [(base_v.clone(), second.clone()) for _ in range(R)]
        del base_v, second
        seq = torch.full((wl.B,), wl.S, dtype=torch.int32, device=dev)
        shape = gva.make_shape(wl.B, wl.H, wl.G, wl.d_n, wl.d_v, d_r, capacity=wl.S, max_seq_len=wl.S,
                               split_tokens=wl.split_tokens, dtype=wl.dtype)
        ws = torch.zeros(max(gva.gva_decode_workspace_bytes(shape), 4) // 4 + 1, dtype=torch.float32, device=dev)
        o = torch.empty(wl.B, wl.H, wl.d_v, dtype=torch.bfloat16, device=dev)
        q = torch.randn(wl.B, wl.H, wl.d_n, device=dev).bfloat16()
        qr = torch.randn(wl.B, wl.H, max(d_r, 1), device=dev).bfloat16()[:, :, :d_r].contiguous()
        M = (torch.randn(wl.H, wl.d_v, wl.d_n, device=dev) / 8).bfloat16()

        def call(i):
            a, b2 = reps[i % R]
            if kind == "gva":
                gva.gva_decode(shape, q, qr, M, a, b2, seq, None, wl.scale, o, ws)
            else:
                gva.gva_gqa_ref_decode(shape, q, b2, a, seq, None, 0.125, o, ws)

        host = []
        for i in range(2 * R):
            t0 = time.perf_counter()
            call(i)
            host.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        ci = [0]

        def next_call():
            call(ci[0])
            ci[0] += 1

        ms, _ = queued_time(next_call, R, K, 1e6 * float(np.median(host)))
        us = ms * 1e3
        out[kind] = {"us": round(us, 3), "bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
                     "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4), "replicas": R}
        del reps
        torch.cuda.empty_cache()
    return {"mode": "gqa_compare", "gva": out["gva"], "gqa": out["gqa"],
            "time_ratio_gqa_over_gva": round(out["gqa"]["us"] / out["gva"]["us"], 3),
            "byte_ratio_gqa_over_gva": round(out["gqa"]["bytes"] / out["gva"]["bytes"], 3)}


def _oracle_reps(fn, seconds: float, max_reps: int = 1000):
    """Call fn until `seconds` of wall time have passed (at least once)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= max_reps:
            return reps, el


def _oracle_threads() -> int:
    from threadpoolctl import threadpool_info
    return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))


def cpu_baseline(wl, seconds: float):
    """The CPU oracle as it stands, on a bounded sample of the same workload:
    full decode steps (all B sequences, n = S + 1) repeated until `seconds`
    of CPU time have passed."""
    import numpy as np

    import oracle as O
    import workloads as W

    inp = W.make_gva_inputs(wl, extra=1)
    n = np.full(wl.B, wl.S + 1)
    reps, el = _oracle_reps(lambda: O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, n, wl.scale,
                                                      wl.rope_base, wl.dtype), seconds)
    return {"value": round(reps / el, 4), "unit": "steps/s", "cores": _oracle_threads(),
            "kind": "oracle",
            "sample": f"{reps} full oracle decode steps of {wl.name} (B={wl.B}, n={wl.S + 1}) "
                      f"in {el:.1f} s, float64 numpy, {len(os.sched_getaffinity(0))} cpus visible"}


def cpu_baseline_gqa(wl, seconds: float, n_seq: int = 2):
    """Oracle GVA decode and oracle GQA decode on the first `n_seq` sequences
    of the workload (its full length S), each for about `seconds`, scaled to
    whole-batch decodes per second."""
    import dataclasses

    import numpy as np

    import oracle as O
    import workloads as W

    sub = dataclasses.replace(wl, B=n_seq)
    inp = W.make_gva_inputs(sub)
    n = np.full(n_seq, wl.S)
    kr_rot = [O.append_positional_keys(k, 0, wl.rope_base, wl.dtype) for k in inp.kr]
    q_rot = O.rope(inp.q_rope, (n - 1.0)[:, None], wl.rope_base)
    r_gva, el_gva = _oracle_reps(lambda: O.gva_decode(inp.V, kr_rot, inp.q_nope, q_rot, inp.M, n, wl.scale),
                                 seconds)
    q, K, V = W.make_gqa_inputs(sub)
    r_gqa, el_gqa = _oracle_reps(lambda: O.gqa_decode(q, K, V, n, wl.scale), seconds)
    frac = n_seq / wl.B
    return {"value": round(r_gva / el_gva * frac, 4), "unit": "decodes/s (whole batch)",
            "gqa_value": round(r_gqa / el_gqa * frac, 4), "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"oracle gva_decode x{r_gva} in {el_gva:.1f} s and oracle gqa_decode x{r_gqa} in "
                      f"{el_gqa:.1f} s on {n_seq} of the {wl.B} sequences (n={wl.S}), float64 numpy, "
                      f"scaled by {n_seq}/{wl.B}"}


def cpu_baseline_ragged(wl, lens, seconds: float, n_seq: int = 4):
    """Oracle fused decode steps on the first `n_seq` sequences of the ragged
    batch (their own lengths + the appended token), scaled to whole-batch
    steps per second by their share of the batch's cache tokens."""
    import dataclasses

    import numpy as np

    import oracle as O
    import workloads as W

    sub = dataclasses.replace(wl, B=n_seq)
    inp = W.make_gva_inputs(sub, extra=1, lens=np.asarray(lens[:n_seq]))
    n = np.asarray(lens[:n_seq]) + 1
    reps, el = _oracle_reps(lambda: O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, n, wl.scale,
                                                      wl.rope_base, wl.dtype), seconds)
    share = float(n.sum()) / float((np.asarray(lens) + 1).sum())
    return {"value": round(reps / el * share, 4), "unit": "steps/s (whole batch)", "cores": _oracle_threads(),
            "kind": "oracle",
            "sample": f"{reps} oracle fused steps of {n_seq} of the {wl.B} sequences (lengths "
                      f"{', '.join(str(int(x)) for x in n)}) in {el:.1f} s, float64 numpy, scaled by their "
                      f"share {share:.4f} of the batch's cache tokens"}


def cpu_baseline_prefill(wl, seconds: float):
    """Oracle causal prefill of one sequence's whole prompt (n = S queries over
    S tokens), in algorithmic TFLOP/s (the causal count the GPU line uses)."""
    import numpy as np

    import oracle as O
    import workloads as W

    rng = np.random.Generator(np.random.PCG64(wl.seed + 9))
    n = wl.S
    V = [W.round_storage(rng.standard_normal((wl.G, n, wl.d_v)), wl.dtype)]
    kr = [O.append_positional_keys(W.round_storage(rng.standard_normal((n, wl.d_r)), wl.dtype), 0, wl.rope_base,
                                   wl.dtype)]
    q = W.round_storage(rng.standard_normal((1, n, wl.H, wl.d_n)), wl.dtype)
    qr = W.round_storage(rng.standard_normal((1, n, wl.H, wl.d_r)), wl.dtype)
    M = W.round_storage(rng.standard_normal((wl.H, wl.d_v, wl.d_n)) / 8, wl.dtype)
    reps, el = _oracle_reps(lambda: O.gva_prefill(V, kr, q, qr, M, [n], wl.scale), seconds)
    fl = prefill_flops(1, wl.H, n, n, wl.d_v, wl.d_r, wl.d_n, True)
    return {"value": round(fl * reps / el / 1e12, 6), "unit": "TFLOP/s", "cores": _oracle_threads(),
            "kind": "oracle",
            "sample": f"{reps} oracle prefills of one {n}-token prompt (all {n} queries, H={wl.H}) in {el:.1f} s, "
                      f"float64 numpy; algorithmic causal flops as on the GPU line"}


if __name__ == "__main__":
    main()
