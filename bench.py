#!/usr/bin/env python3
"""Benchmark: packed-weight HBM GB/s of the M = 1 INT4 decode GEMVs of one
Qwen3-shaped decoder layer on one MI355X, with the prefill GEMM TFLOP/s, the
vocabulary-head GEMV and the INT3 QMoE layer reported alongside.

A step is one pass over the layer's projections (fused QKV 2048->4096, o_proj
2048->2048, gate and up 2048->6144, down 6144->2048, and the K-tail case
2050->1024) on the library's prepared INT4 weights: an mnb_gemv call each,
except gate and up, which read the same input vector (as in a SwiGLU MLP) and
go through one mnb_gemv_multi call (one launch for both).
Weights rotate over enough distinct copies (>= 1 GiB) that every step streams
them from HBM rather than from the 256 MB Infinity Cache.  The timed steps are
replayed from a HIP graph (launch overhead of the Python binding excluded) and
bracketed by torch.cuda.synchronize() on both sides.

The other workloads (vocabulary head, prefill GEMM, QMoE layers, quantizer)
are measured first, each from graph replays of its own launches (the median
per call over 20 back-to-back replays, with the 10th and 90th percentiles in
its `spread`); then the
headline's weight copies are prepared (host repack and upload) and its graphs
captured, and exactly `--warmup` untimed steps precede the `--steps` timed
ones.  The timed steps continue the weight rotation where the warm-up
stopped, so no timed step reads a copy that a warm-up step has just read.
For context, `extra` also times the vendor BLAS (torch.matmul) on the prefill
shapes with dense fp16 weights, after the headline region.  The roofline's average launch
duration comes from HIP events recorded on the launch stream around the same
timed graph replays (five GEMV kernel launches per step, back to back, so the
average includes the short gaps between kernels); its ceiling is a plain
16-byte streaming read of the same rotated buffers in the same five-launch
pattern.  The oracle is then timed on the host on the same workloads.

Prints one JSON line.  Everything is synthetic (seeded, synth.py).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense fp16 matrix, published (no sparsity)
ROTATE_BYTES = 1 << 30       # >= 4x the 256 MB MALL

LAYER = [  # name, K, N (M = 1, block 32, implicit zero point 8)
    ("qkv", 2048, 4096), ("o_proj", 2048, 2048), ("gate", 2048, 6144), ("up", 2048, 6144),
    ("down", 6144, 2048), ("tail", 2050, 1024)]


def gemv_bytes(K, N, bs=32, zp=False):
    """Algorithmic bytes of one GEMV: packed codes + scales (+ zero points)."""
    nb = -(-K // bs)
    return N * nb * bs // 2 + N * nb * 4 + (N * ((nb + 1) // 2) if zp else 0)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Graph:
    """A captured sequence of library calls, replayed on the current stream.
    With warm=False nothing runs before the capture (the library needs no lazy
    initialisation), so the captured steps execute only when replayed."""

    def __init__(self, torch, fn, warm=True):
        self.torch = torch
        if warm:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                fn()  # warm-up outside capture
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            fn()
        torch.cuda.synchronize()

    def replay(self):
        self.g.replay()


def graph_time(torch, calls, reps, min_calls=24, spread=None):
    """Captures `calls` (repeated to at least `min_calls` launches, so that the
    graph launch itself is amortised) in one graph and, after about 20 ms of
    warm-up replays, times `reps` back-to-back replays with one event between
    each two on the launch stream; returns the median per call in ms.  If
    `spread` is a dict it receives the 10th and 90th percentiles per call (us)
    and the replay count."""
    calls = list(calls) * max(1, -(-min_calls // len(calls)))
    g = Graph(torch, lambda: [c() for c in calls])
    # warm-up: about 20 ms of replays, so that clocks are at their sustained
    # level when the timed replays start
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.replay()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    for _ in range(max(2, int(20.0 / max(e0.elapsed_time(e1), 1e-3)))):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) / len(calls) for i in range(reps)])
    p10, p50, p90 = np.percentile(per, [10, 50, 90])
    if spread is not None:
        spread.update({"p10_us": round(1e3 * float(p10), 3), "p90_us": round(1e3 * float(p90), 3),
                       "replays": reps, "calls_per_replay": len(calls)})
    return float(p50)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_quantized_weight_03_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def host_info():
    """CPU model, logical CPUs visible, CPUs this process may run on, and the
    worker threads the oracle uses (the GPU machine grants 16 workers per GPU,
    whatever the machine reports)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count() or 1
    return {"cpu_model": model, "cpus_visible": os.cpu_count(), "cpus_allowed": allowed,
            "threads_used": max(1, min(16, allowed))}


def timed(fn, max_s=2.0):
    """Median wall time of 3 runs, or of 1 when the first run exceeds max_s."""
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
        if ts[0] > max_s:
            break
    return float(np.median(ts)), len(ts)


def cpu_baseline(layer_host, threads):
    """The oracle on the decoder layer's GEMVs (the headline workload), one
    pass per run, single-threaded and on `threads` threads."""
    import oracle

    def layer(nt):
        for (name, K, N), (B, s, a) in zip(LAYER, layer_host):
            oracle.mnb_gemm(a, B, s, None, K, N, bs=32, nthreads=nt)

    step_bytes = sum(gemv_bytes(K, N) for _, K, N in LAYER)
    t1, n1 = timed(lambda: layer(1))
    tn, nn = timed(lambda: layer(threads))
    return {"value": round(step_bytes / tn / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "single_thread_GB/s": round(step_bytes / t1 / 1e9, 3),
            "sample": f"one pass over the decoder-layer GEMVs (6 projections, {step_bytes} B of "
                      f"packed weights and scales), median of {nn} runs on {threads} threads "
                      f"({tn * 1e3:.1f} ms) and of {n1} single-threaded ({t1 * 1e3:.1f} ms)"}


def cpu_oracle_configs(threads):
    """The oracle's time on the other workloads, each single-threaded and on
    `threads` threads (median of 3, or 1 run past 2 s).  The 128-token QMoE
    layer is timed on 16 of its tokens and scaled (the oracle's cost is linear
    in the tokens: each token evaluates its own top-8 experts)."""
    import oracle
    res = {}

    def both(name, fn, units, unit_name, scale=1.0, note=None):
        t1, n1 = timed(lambda: fn(1))
        tn, nn = timed(lambda: fn(threads))
        r = {"single_thread_ms": round(t1 * scale * 1e3, 2), f"{threads}_threads_ms":
             round(tn * scale * 1e3, 2), "runs": [n1, nn],
             f"{unit_name}_single": round(units / (t1 * scale), 3),
             f"{unit_name}_{threads}_threads": round(units / (tn * scale), 3)}
        if note:
            r["sample"] = note
        res[name] = r

    K, N = 2048, 2048
    B = synth.int4_blocked_weights(synth.seed_for(1, 1), N, K, 32)
    s = synth.scales_f32(synth.seed_for(1, 2), (N, K // 32))
    a = synth.activations_f32(synth.seed_for(1, 3), 1, K)
    both("gemv_K2048_N2048", lambda nt: oracle.mnb_gemm(a, B, s, None, K, N, nthreads=nt),
         gemv_bytes(K, N) / 1e9, "GB/s")
    N = 151936
    B = synth.int4_blocked_weights(synth.seed_for(3, 1), N, K, 32)
    s = synth.scales_f32(synth.seed_for(3, 2), (N, K // 32))
    Z = synth.int4_zero_points(synth.seed_for(3, 3), N, K // 32)
    both("vocab_head_K2048_N151936", lambda nt: oracle.mnb_gemm(a, B, s, Z, K, N, nthreads=nt),
         gemv_bytes(K, N, zp=True) / 1e9, "GB/s")
    del B, s, Z
    K, N = 2048, 6144
    B = synth.int4_blocked_weights(synth.seed_for(4, K), N, K, 32)
    s = synth.scales_f32(synth.seed_for(4, K + 1), (N, K // 32))
    for M in (16, 128):
        A = synth.activations_f32(synth.seed_for(4, M), M, K)
        both(f"gemm_M{M}_K{K}_N{N}", lambda nt, A=A: oracle.mnb_gemm(A, B, s, None, K, N, nthreads=nt),
             2.0 * M * N * K / 1e9, "GFLOP/s")
    H, I, E, k, bs = 2048, 768, 128, 8, 64
    W1 = synth.packed_rows(synth.seed_for(5, 3), E * 2 * I, H, 3).reshape(E, 2 * I, -1)
    s1 = synth.scales_f16(synth.seed_for(5, 4), (E, 2 * I, H // bs))
    W2 = synth.packed_rows(synth.seed_for(5, 5), E * H, I, 3).reshape(E, H, -1)
    s2 = synth.scales_f16(synth.seed_for(5, 6), (E, H, I // bs))
    for T, Ts in ((1, 1), (128, 16)):
        x = synth.activations_f16(synth.seed_for(5, 1), T, H)[:Ts]
        lg = synth.router_logits(synth.seed_for(5, 2), T, E)[:Ts]
        both(f"qmoe_int3_T{T}", lambda nt, x=x, lg=lg: oracle.qmoe(x, lg, W1, s1, W2, s2, k=k, bs=bs,
                                                                   nthreads=nt),
             2.0 * T * k * (2 * I * H + H * I) / 1e9, "GFLOP/s", scale=T / Ts,
             note=None if T == Ts else f"{Ts} of {T} tokens timed, scaled by {T // Ts}")
    return res


def vendor_dense_gemm(torch, dev):
    """Context only (not this library): the vendor BLAS (torch.matmul) on the
    prefill shapes with the weights already dense fp16, fp16 A and fp16 output
    (no dequantization, no rounding pass, half the output bytes), graph-replayed
    like the library's calls.  Run after the headline region."""
    dense = {}
    for (K, N) in ((2048, 6144), (6144, 2048)):
        wd = (torch.rand(K, N, device=dev, generator=torch.Generator(device=dev).manual_seed(K)) * 2 - 1).half()
        for M in (512, 2048, 4096):
            ad = (torch.rand(M, K, device=dev, generator=torch.Generator(device=dev).manual_seed(M)) * 2 - 1).half()
            od = torch.empty((M, N), dtype=torch.float16, device=dev)
            us = 1e3 * graph_time(torch, [lambda ad=ad, wd=wd, od=od: torch.matmul(ad, wd, out=od)] * 4, 5)
            tf = 2.0 * M * N * K / us / 1e6
            dense[f"M{M}_K{K}_N{N}"] = {"us": round(us, 2), "TFLOP/s": round(tf, 1),
                                         "frac_of_fp16_peak": round(tf / PEAK_FP16_TFLOPS, 4)}
        del wd
    return dense


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1980)
    ap.add_argument("--warmup", type=int, default=660)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timings")
    args = ap.parse_args()
    if args.gpus != 1:
        sys.exit(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs are "
                 "not part of this build")

    import torch
    import block_quantized_weight_03_amd as mnb
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    # ---- the other workloads first, each from its own graphs ----------------
    extra = {}
    if not args.no_extras:
        extra.update(bench_extras(torch, mnb, dev))

    # ---- decoder-layer weights, rotated over >= 1 GiB ------------------------
    step_bytes = sum(gemv_bytes(K, N) for _, K, N in LAYER)
    copies = max(1, -(-ROTATE_BYTES // step_bytes))
    log(f"preparing {copies} copies of the layer ({step_bytes} B each)")
    acts = []
    for i, (name, K, N) in enumerate(LAYER):
        if name == "up":  # gate and up read the same input
            acts.append(acts[-1])
            continue
        a = synth.activations_f32(synth.seed_for(2, 100 + i), 1, K)
        acts.append((a, torch.from_numpy(a[0]).to(dev)))
    names = [n for n, _, _ in LAYER]
    gate, up = names.index("gate"), names.index("up")
    layers, layer_host = [], None
    for c in range(copies):
        ws = []
        host = []
        for i, (name, K, N) in enumerate(LAYER):
            nb = -(-K // 32)
            B = synth.int4_blocked_weights(synth.seed_for(2, 1000 * c + 10 * i + 1), N, K, 32)
            s = synth.scales_f32(synth.seed_for(2, 1000 * c + 10 * i + 2), (N, nb))
            ws.append(mnb.PreparedWeight(mnb.dense_desc(K, N), B, s, None))
            if c == 0:
                host.append((B, s, acts[i][0]))
        if c == 0:
            layer_host = host
        layers.append(ws)
    outs = [torch.empty(N, dtype=torch.float32, device=dev) for _, K, N in LAYER]
    gemv_ws = torch.empty(256, dtype=torch.uint8, device=dev)
    for ws in layers[0]:
        assert mnb.mnb_gemv_workspace_size(ws.plan) == 0

    def step(c):
        for i, w in enumerate(layers[c]):
            if i == up:
                continue
            if i == gate:
                mnb.mnb_gemv_multi([w.plan, layers[c][up].plan], acts[i][1], [outs[gate], outs[up]],
                                   gemv_ws, gemv_ws.numel())
            else:
                mnb.mnb_gemv(w.plan, acts[i][1], outs[i], gemv_ws, gemv_ws.numel())

    # captured without running: every step executes only as a warm-up or a
    # timed step.  The timed steps continue the rotation where the warm-up
    # stopped (copy W mod copies), so no timed step reads a copy that a warm-up
    # step has just read.
    wrem = args.warmup % copies
    rem = args.steps % copies
    wpart = Graph(torch, lambda: [step(c) for c in range(wrem)], warm=False) if wrem else None
    wfull = Graph(torch, lambda: [step(c) for c in range(copies)], warm=False)
    full = Graph(torch, lambda: [step((wrem + c) % copies) for c in range(copies)], warm=False)
    part = Graph(torch, lambda: [step((wrem + c) % copies) for c in range(rem)], warm=False) if rem else None

    # ---- exactly W warm-up steps, then exactly K timed steps ---------------
    for _ in range(args.warmup // copies):
        wfull.replay()
    if wpart:
        wpart.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps // copies):
        full.replay()
    if part:
        part.replay()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = step_bytes * args.steps / elapsed / 1e9
    us_per_step_event = e0.elapsed_time(e1) * 1e3 / args.steps

    # ---- roofline of the GEMV kernel over the same timed region --------------
    launches_per_step = len(LAYER) - 1  # gate and up share one launch
    launches = args.steps * launches_per_step
    avg_ms = e0.elapsed_time(e1) / launches
    avg_bytes = step_bytes / launches_per_step
    achieved = avg_bytes / (avg_ms * 1e-3) / 1e9
    gemv_hash = source_hash("gemv.hip")

    # the measured ceiling: a plain 16-byte streaming read of the same rotated
    # prepared buffers in the same five-launch pattern, steady state
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def rd(ws_list):
        return lambda: mnb.mnb_debug_stream_read(
            [(w.buffer, (w.plan.total_bytes // 16) * 16) for w in ws_list], sink)

    def read_step(c):
        return [rd([layers[c][i]]) if i != gate else rd([layers[c][gate], layers[c][up]])
                for i in range(len(LAYER)) if i != up]

    read_us = 1e3 * graph_time(torch, [f for c in range(copies) for f in read_step(c)], 10) \
        * launches_per_step
    gemv_steady_us = 1e3 * graph_time(torch, [lambda c=c: step(c) for c in range(copies)], 10)
    ceiling = step_bytes / read_us / 1e3
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": load_traffic("gemv_int4_f32/decoder_layer", gemv_hash),
                "kernel": "gemv_int4_f32", "launches": launches,
                "avg_launch_us": round(avg_ms * 1e3, 3),
                "algorithmic_bytes_per_launch": round(avg_bytes, 1),
                "ceiling_GBps": round(ceiling, 1),
                "frac_of_ceiling": round(achieved / ceiling, 4),
                "ceiling_note": "plain 16-byte nontemporal read of the same rotated buffers, five "
                                f"launches per step as the GEMVs ({read_us:.2f} us per step, steady "
                                f"state; the GEMV step in the same protocol: {gemv_steady_us:.2f} us)"}
    per_proj = {}
    for i, (name, K, N) in enumerate(LAYER):
        calls = [lambda w=layers[c][i], i=i: mnb.mnb_gemv(w.plan, acts[i][1], outs[i], gemv_ws,
                                                          gemv_ws.numel()) for c in range(copies)]
        us = 1e3 * graph_time(torch, calls, 10)
        rus = 1e3 * graph_time(torch, [rd([layers[c][i]]) for c in range(copies)], 10)
        per_proj[name] = {"us": round(us, 3), "GB/s": round(gemv_bytes(K, N) / us / 1e3, 1),
                          "read_us": round(rus, 3)}
    calls = [lambda c=c: mnb.mnb_gemv_multi([layers[c][gate].plan, layers[c][up].plan], acts[gate][1],
                                            [outs[gate], outs[up]], gemv_ws, gemv_ws.numel())
             for c in range(copies)]
    us = 1e3 * graph_time(torch, calls, 10)
    rus = 1e3 * graph_time(torch, [rd([layers[c][gate], layers[c][up]]) for c in range(copies)], 10)
    gu = gemv_bytes(LAYER[gate][1], LAYER[gate][2]) + gemv_bytes(LAYER[up][1], LAYER[up][2])
    per_proj["gate+up (one launch)"] = {"us": round(us, 3), "GB/s": round(gu / us / 1e3, 1),
                                        "read_us": round(rus, 3)}

    # ---- separately labelled extras: step-time spread over single replays,
    # one eager call with its launch, and a hot-cache figure (never the HBM one)
    reps = []
    for _ in range(30):
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record()
        full.replay()
        r1.record()
        torch.cuda.synchronize()
        reps.append(r0.elapsed_time(r1) * 1e3 / copies)
    q = np.percentile(reps, [10, 50, 90])
    spread = {"us_per_step_p10": round(float(q[0]), 3), "median": round(float(q[1]), 3),
              "p90": round(float(q[2]), 3), "replays": len(reps), "steps_per_replay": copies}
    o = names.index("o_proj")
    one = []
    for _ in range(50):
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        mnb.mnb_gemv(layers[0][o].plan, acts[o][1], outs[o], gemv_ws, gemv_ws.numel())
        torch.cuda.synchronize()
        one.append((time.perf_counter() - h0) * 1e6)
    single = {"projection": "o_proj", "us_median": round(float(np.median(one)), 2),
              "timing": "host wall clock around one eager call and a synchronize"}
    hot_us = 1e3 * graph_time(torch, [lambda: mnb.mnb_gemv(layers[0][o].plan, acts[o][1], outs[o],
                                                           gemv_ws, gemv_ws.numel())], 10)
    hot = {"projection": "o_proj", "us": round(hot_us, 3),
           "GB/s": round(gemv_bytes(LAYER[o][1], LAYER[o][2]) / hot_us / 1e3, 1),
           "note": "one weight copy replayed, cache-resident: not an HBM figure"}

    del full, part, wpart, wfull
    torch.cuda.synchronize()

    extra = {"per_projection": per_proj, "step_spread": spread, "single_call_latency": single,
             "hot_cache_gemv": hot, **extra}
    if not args.no_extras:
        extra["prefill_gemm_vendor_dense_fp16"] = vendor_dense_gemm(torch, dev)
    info = host_info()
    base = None
    if not args.no_cpu:
        log("timing the oracle on the host")
        base = cpu_baseline(layer_host, info["threads_used"])
        base.update(info)
        if not args.no_extras:
            extra["cpu_oracle"] = cpu_oracle_configs(info["threads_used"])

    rec = {"metric": "packed-weight HBM GB/s at M=1; prefill TFLOP/s; % of MI355X roofline",
           "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "us_per_step_event": round(us_per_step_event, 3),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": "Qwen3-shaped decoder layer of INT4 decode GEMVs, M=1, block 32, "
                                  "implicit zero point 8: QKV 2048->4096, o 2048->2048, gate and up "
                                  "2048->6144, down 6144->2048, tail 2050->1024",
                      "bytes_per_step": step_bytes, "rotation_copies": copies,
                      "timing": "HIP graph replay; value and ms_per_step from the host wall clock "
                                "between synchronizes, us_per_step_event from an event pair on "
                                "the launch stream over the same steps; exactly `warmup` untimed "
                                "steps before (the other workloads in extra ran earlier)"},
           "roofline": roofline, "cpu_baseline": base, "extra": extra}
    print(json.dumps(rec), flush=True)


def prepare_timed(torch, mnb, desc, B, s, Z=None):
    """mnb_prepare into a fresh device buffer; returns the prepared weight and
    the call's wall time (host validation and repack, upload, wait) in ms."""
    buf = torch.empty(max(mnb.mnb_prepacked_size(desc), 256), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    plan = mnb.mnb_prepare(desc, B, s, Z, buf, buf.numel())
    ms = (time.perf_counter() - t0) * 1e3
    w = mnb.PreparedWeight.__new__(mnb.PreparedWeight)
    w.desc, w.buffer, w.plan = desc, buf, plan
    return w, ms


def prep_record(ms, *arrays):
    mb = sum(a.nbytes for a in arrays if a is not None) / 1e6
    return {"ms": round(ms, 1), "contract_MB": round(mb, 1), "MB/s": round(mb / ms * 1e3, 1)}


def bench_extras(torch, mnb, dev):
    """Vocabulary head GEMV, prefill GEMM, the QMoE layer (INT3, INT4, bf16)
    and the INT3 RTN quantizer, each timed from graph replays of its own
    launches (weights rotated where the working set would fit in the
    Infinity Cache)."""
    out = {}
    # vocabulary head: K=2048, N=151936, explicit zero points
    K, N = 2048, 151936
    nb = K // 32
    copies = 6
    vw = []
    prep = {}
    for c in range(copies):
        B = synth.int4_blocked_weights(synth.seed_for(3, 10 * c + 1), N, K, 32)
        s = synth.scales_f32(synth.seed_for(3, 10 * c + 2), (N, nb))
        Z = synth.int4_zero_points(synth.seed_for(3, 10 * c + 3), N, nb)
        w, ms = prepare_timed(torch, mnb, mnb.dense_desc(K, N, 32, True), B, s, Z)
        vw.append(w)
        if c == 0:
            prep["vocab_head_K2048_N151936"] = prep_record(ms, B, s, Z)
    A = torch.from_numpy(synth.activations_f32(synth.seed_for(3, 0), 1, K)[0]).to(dev)
    Y = torch.empty(N, dtype=torch.float32, device=dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    calls = [lambda w=w: mnb.mnb_gemv(w.plan, A, Y, ws, 256) for w in vw]
    sp = {}
    us = 1e3 * graph_time(torch, calls, 20, spread=sp)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    reads = [lambda w=w: mnb.mnb_debug_stream_read([(w.buffer, (w.plan.total_bytes // 16) * 16)], sink)
             for w in vw]
    rus = 1e3 * graph_time(torch, reads, 10)
    vb = gemv_bytes(K, N, zp=True)
    out["vocab_head_gemv"] = {"K": K, "N": N, "zero_points": True, "us": round(us, 3),
                              "GB/s": round(vb / us / 1e3, 1),
                              "frac_of_hbm_peak": round(vb / us / 1e3 / PEAK_HBM_GBS, 4),
                              "read_ceiling_us": round(rus, 3),
                              "read_ceiling_GB/s": round(vb / rus / 1e3, 1),
                              "frac_of_ceiling": round(rus / us, 4), "spread": sp}
    del vw
    log("extras: vocabulary head done")
    # prefill GEMM at M = 16 .. 4096 on both shapes
    pre = {}
    for (K, N) in ((2048, 6144), (6144, 2048)):
        nb = K // 32
        w = mnb.PreparedWeight(mnb.dense_desc(K, N), synth.int4_blocked_weights(synth.seed_for(4, K), N, K, 32),
                               synth.scales_f32(synth.seed_for(4, K + 1), (N, nb)))
        for M in (16, 128, 512, 2048, 4096):
            a = torch.from_numpy(synth.activations_f32(synth.seed_for(4, M), M, K)).to(dev)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            need = mnb.mnb_gemm_workspace_size(w.plan, M)
            gws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
            call = lambda w=w, M=M, a=a, y=y, gws=gws: mnb.mnb_gemm(w.plan, M, a, y, gws, gws.numel())
            sp = {}
            us = 1e3 * graph_time(torch, [call] * 4, 20, spread=sp)
            tf = 2.0 * M * N * K / us / 1e6
            pre[f"M{M}_K{K}_N{N}"] = {"us": round(us, 2), "TFLOP/s": round(tf, 1),
                                       "frac_of_fp16_peak": round(tf / PEAK_FP16_TFLOPS, 4),
                                       "spread": sp}
        del w
    out["prefill_gemm"] = pre
    log("extras: prefill GEMM done")
    # QMoE layer: all-INT3 projections, and the all-INT4 layer the INT3 QMoE
    # page compares it with
    out["qmoe_int3_layer"] = qmoe_extra(torch, mnb, dev, 3, 3, prep=prep)
    log("extras: INT3 QMoE layer done")
    out["qmoe_int4_layer"] = qmoe_extra(torch, mnb, dev, 4, 4, prep=prep)
    log("extras: INT4 QMoE layer done")
    out["qmoe_int3_layer_bf16"] = qmoe_extra(torch, mnb, dev, 3, 3, bf16=True)
    log("extras: bf16 INT3 QMoE layer done")
    out["int3_rtn_quantizer"] = rtn_extra(torch, mnb, dev)
    log("extras: INT3 RTN quantizer done")
    out["prepare"] = prep
    return out


def qmoe_extra(torch, mnb, dev, bits1, bits2, bf16=False, prep=None):
    """QMoE layer (hidden 2048, 128 experts, intermediate 768, top-8, block 64)
    at T = 1, 128, 512 tokens, from graph replays over 4 weight copies; fp16
    or bfloat16 activations and scales.  At T >= 128 every call routes to all
    128 experts (about 1 GB over the copies); at T = 1 each copy is paired
    with 8 router-logit sets, so that the 32 calls route to 52 distinct experts
    per copy, 400 MB (INT3) to 520 MB (INT4), more than the 256 MB Infinity
    Cache (the same 8 experts per copy would be 60 / 80 MB, which the cache
    could hold across replays)."""
    H, I, E, k, bs = 2048, 768, 128, 8, 64
    scales = synth.scales_bf16 if bf16 else synth.scales_f16
    W1 = synth.packed_rows(synth.seed_for(5, 3), E * 2 * I, H, bits1)
    s1 = scales(synth.seed_for(5, 4), (E * 2 * I, H // bs))
    W2 = synth.packed_rows(synth.seed_for(5, 5), E * H, I, bits2)
    s2 = scales(synth.seed_for(5, 6), (E * H, I // bs))
    sd = mnb.MNB_DTYPE_BF16 if bf16 else mnb.MNB_DTYPE_F16
    copies = 4
    experts = []
    for c in range(copies):  # distinct device copies of the same expert bytes
        p1, ms1 = prepare_timed(torch, mnb, mnb.qmoe_proj_desc(H, 2 * I, E, bs, bits1, sd), W1, s1)
        p2, ms2 = prepare_timed(torch, mnb, mnb.qmoe_proj_desc(I, H, E, bs, bits2, sd), W2, s2)
        experts.append((p1, p2))
        if c == 0 and prep is not None:
            prep[f"qmoe_int{bits1}_fc1_E128_1536x2048"] = prep_record(ms1, W1, s1)
            prep[f"qmoe_int{bits2}_fc2_E128_2048x768"] = prep_record(ms2, W2, s2)
    q = mnb.make_qmoe_desc(k)
    per_expert = (2 * I * (bits1 * H // 8) + 2 * I * (H // bs) * 2 + H * (bits2 * I // 8)
                  + H * (I // bs) * 2)
    moe = {"bits": [bits1, bits2], "dtype": "bf16" if bf16 else "f16",
           "bytes_per_expert": per_expert}
    for T in (1, 128, 512):
        if bf16:  # bfloat16 patterns, carried as int16
            xa = synth.activations_bf16(synth.seed_for(5, 1), T, H).view(np.int16)
        else:
            xa = synth.activations_f16(synth.seed_for(5, 1), T, H)
        x = torch.from_numpy(xa).to(dev)
        nlg = 8 if T == 1 else 1
        lgs = [torch.from_numpy(synth.router_logits(synth.seed_for(5, 2 + 1000 * j), T, E)).to(dev)
               for j in range(nlg)]
        o = torch.empty((T, H), dtype=torch.int16 if bf16 else torch.float16, device=dev)
        need = mnb.qmoe_workspace_size(experts[0][0].plan, experts[0][1].plan, q, T)
        qws = torch.empty(need, dtype=torch.uint8, device=dev)
        calls = [lambda p=p, x=x, lg=lg, o=o, qws=qws, T=T: mnb.qmoe_forward(
            p[0].plan, p[1].plan, q, T, x, lg, o, qws, qws.numel()) for lg in lgs for p in experts]
        sp = {}
        us = 1e3 * graph_time(torch, calls, 20, spread=sp)
        # distinct experts routed per call (averaged over the logit sets)
        ids = sum(torch.topk(lg.float(), k, dim=1).indices.unique().numel() for lg in lgs) / nlg
        byts = ids * per_expert
        moe[f"T{T}"] = {"us": round(us, 2), "distinct_experts": ids,
                        "weight_GB/s": round(byts / us / 1e3, 1),
                        "frac_of_hbm_peak": round(byts / us / 1e3 / PEAK_HBM_GBS, 4),
                        "TFLOP/s": round(2.0 * T * k * (2 * I * H + H * I) / us / 1e6, 2),
                        "spread": sp}
    del experts
    return moe


def rtn_extra(torch, mnb, dev):
    """Producer-side INT3 RTN quantizer on the QMoE layer's FC1 stack (128
    experts x 1536 rows, K = 2048, block 64) from fp32 weights in HBM; bytes =
    fp32 weights read + codes, scales and status written."""
    rows, K, bs = 128 * 1536, 2048, 64
    gen = torch.Generator(device=dev).manual_seed(5)
    W = torch.randn((rows, K), generator=gen, device=dev, dtype=torch.float32) * 0.02
    B = torch.empty((rows, 3 * K // 8), dtype=torch.uint8, device=dev)
    s = torch.empty((rows, K // bs), dtype=torch.float16, device=dev)
    st = torch.empty((rows, K // bs), dtype=torch.uint8, device=dev)
    call = lambda: mnb.mnb_quantize_int3_rtn(W, rows, K, bs, B, s, st, None, mnb.MNB_DTYPE_F16)
    sp = {}
    us = 1e3 * graph_time(torch, [call], 20, min_calls=8, spread=sp)
    byts = rows * K * 4 + rows * 3 * K // 8 + rows * (K // bs) * 3
    res = {"rows": rows, "K": K, "block_size": bs, "us": round(us, 2),
           "GB/s": round(byts / us / 1e3, 1), "frac_of_hbm_peak": round(byts / us / 1e3 / PEAK_HBM_GBS, 4),
           "spread": sp}
    del W, B, s, st
    return res


if __name__ == "__main__":
    main()
