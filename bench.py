"""Throughput of the Q8_0 block-quantized linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  The default workload is the Qwen3-8B block linears (QKV 6144x4096,
fused gate_up 24576x4096 with SiLU(gate)*up, down 4096x12288, Q8_0 weights, float32
activations) at M = 1: a step is one decode token through 36 layers, each with its own
resident copy of the weights (6.7 GB in total, far above the 256 MB Infinity Cache, so
every step streams the weights from HBM).  `value` is the effective weight bandwidth:
algorithmic Q8_0 bytes per step / step time.  The same stack at M = 8 is reported in
"m8".  Other workloads (the other layer shapes) are selected with --workload.

Inputs are seeded synthetic data (workloads/); the timed region starts with everything
resident in HBM.  The CPU oracle is timed on a bounded sample of the same workload on
the host cores ("cpu_baseline").
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores
# float32 VALU lane operations per second without packed instructions (the build disables
# packed float32): 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_LANE_OPS_PER_S = 256 * 64 * 2.4e9
# dense float32 matrix cores (v_mfma_f32_4x4x1_16b_f32: 512 flops per 8 cycles per SIMD)
MFMA_FP32_PEAK_FLOPS = 157.3e12
METRIC = "effective weight GB/s & % of HBM peak for Q8_0 linear at M=1/8/16; decode tok/s"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def measured_traffic():
    """HBM bytes per launch of the M=1 fused gate_up kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, or None once the kernel sources (gemv_q8.hip, gemv_core.h,
    lds_dma.h, hashed in that order) differ from the ones the counters were taken with."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_gemv_q8_qwen3_8b_shapes.md")
    src = os.path.join(ROOT, "block_quantized_weight_linear_amd", "csrc")
    try:
        text = open(path).read()
        h = hashlib.sha256()
        for name in ("gemv_q8.hip", "gemv_core.h", "lds_dma.h"):
            with open(os.path.join(src, name), "rb") as f:
                h.update(f.read())
        want = re.search(r"sources_sha256: ([0-9a-f]{64})", text).group(1)
        if want != h.hexdigest():
            return None
        return int(re.search(r"gate_up_m1_traffic_bytes: (\d+)", text).group(1))
    except (OSError, AttributeError):
        return None


def measured_mfma():
    """Counter-based matrix-core utilisation of the prefill tiles from the committed
    rocprofv3 summary (SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs' cycles), or {} once
    gemm_q8_mfma.hip differs from the source the counters were taken with."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "mfma_prefill_qwen3_8b_gate_up_and_a3b_moe.md")
    src = os.path.join(ROOT, "block_quantized_weight_linear_amd", "csrc", "gemm_q8_mfma.hip")
    try:
        text = open(path).read()
        with open(src, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()
        if re.search(r"sources_sha256: ([0-9a-f]{64})", text).group(1) != h:
            return {}
        return {k: float(v) for k, v in re.findall(r"(\w+_mfma_busy_frac): ([0-9.]+)", text)}
    except (OSError, AttributeError):
        return {}


# --------------------------------------------------------------------- workloads


class Stack:
    """L layers of block linears, each layer with its own device copy of the weights."""

    def __init__(self, torch, dev, spec, layers, seed):
        import workloads as wl
        self.spec = spec
        self.layers = layers
        host = []
        for lin in spec.linears:
            wb, _, _ = wl.q8_weight(seed * 100 + len(host), lin.n, lin.k)
            host.append(wb)
        self.host = host
        base = [torch.from_numpy(h).to(dev) for h in host]
        self.w = [[b if i == 0 else b.clone() for b in base] for i in range(layers)]
        self.bytes_per_layer = sum(int(h.size) for h in host)

    def run(self, q8, x, bufs, m):
        """One decode step through every layer: QKV, gate_up(+SiLU), down (fed by gate_up)."""
        qkv, gu, dn = self.spec.linears
        for l in range(self.layers):
            wq, wg, wd = self.w[l]
            q8.q8_linear(wq, qkv.n, qkv.k, x, out=bufs["qkv"])
            q8.q8_linear_fused_gate_up_silu(wg, gu.n // 2, gu.k, x, out=bufs["h"])
            q8.q8_linear(wd, dn.n, dn.k, bufs["h"], out=bufs["y"])

    def run_q8act(self, q8, x, bufs, m):
        """The same step on the integer q8 x q8 path: each linear's input is quantized to
        int8 codes per 32-block on the device (QKV's and gate_up's separately, as their
        inputs differ in a real block), then multiplied with v_dot4 block dot products."""
        qkv, gu, dn = self.spec.linears
        for l in range(self.layers):
            wq, wg, wd = self.w[l]
            q8.q8_quantize_act(x, bufs["xq"], bufs["xd"])
            q8.q8_linear_q8act(wq, qkv.n, qkv.k, bufs["xq"], bufs["xd"], out=bufs["qkv"])
            q8.q8_quantize_act(x, bufs["xq"], bufs["xd"])
            q8.q8_linear_fused_gate_up_silu_q8act(wg, gu.n // 2, gu.k, bufs["xq"], bufs["xd"], out=bufs["h"])
            q8.q8_quantize_act(bufs["h"], bufs["hq"], bufs["hd"])
            q8.q8_linear_q8act(wd, dn.n, dn.k, bufs["hq"], bufs["hd"], out=bufs["y"])

    def run_gate_up_q8act(self, q8, bufs):
        gu = self.spec.linears[1]
        for l in range(self.layers):
            q8.q8_linear_fused_gate_up_silu_q8act(self.w[l][1], gu.n // 2, gu.k, bufs["xq"], bufs["xd"],
                                                  out=bufs["h"])

    def run_gate_up(self, q8, x, bufs):
        """The fused gate_up of every layer only (the dominant kernel)."""
        gu = self.spec.linears[1]
        for l in range(self.layers):
            q8.q8_linear_fused_gate_up_silu(self.w[l][1], gu.n // 2, gu.k, x, out=bufs["h"])


def time_steps(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per step


def host_cpu_info():
    """Logical and physical core counts and the CPU model of the host running the bench."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        import psutil
        physical = psutil.cpu_count(logical=False)
    except Exception:  # pragma: no cover
        physical = None
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"logical_cpus": os.cpu_count(), "physical_cores": physical, "usable_cpus": affinity, "model": model}


def cpu_baseline_block(spec, reps=5):
    """The oracle on one full layer of the stack (QKV, fused gate_up, down) at M = 1: one
    warm-up pass, then the best of `reps` timed passes (each includes the dequantization)."""
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    hosts = [wl.q8_weight(900 + i, lin.n, lin.k)[0] for i, lin in enumerate(spec.linears)]
    xs = [wl.activations(950 + i, 1, lin.k) for i, lin in enumerate(spec.linears)]
    nbytes = sum(int(h.size) for h in hosts)

    def one_layer():
        for lin, wb, x in zip(spec.linears, hosts, xs):
            if lin.fused_silu:
                oracle.fused_gate_up_silu_ref(wb, lin.n // 2, lin.k, x)
            else:
                oracle.q8_linear_ref(wb, lin.n, lin.k, x)

    one_layer()  # warm-up
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        one_layer()
        times.append(time.perf_counter() - t0)
    best = min(times)
    info = host_cpu_info()
    return {"value": round(nbytes / best / 1e9, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one full layer ({'+'.join(l.name for l in spec.linears)}, {nbytes} Q8_0 bytes) at M=1, "
                      f"float64 dequantize-then-matmul, one warm-up then best of {reps}",
            "tok_s_per_layer": round(1.0 / best, 3), "blas_threads": int(threads),
            "median_s": round(float(np.median(times)), 4), **info}


def bench_block(args, torch, dev, q8, spec, m_values):
    import workloads as wl
    layers = args.layers or spec.layers
    log(f"workload {spec.name}: {layers} layers, uploading weights")
    stack = Stack(torch, dev, spec, layers, spec.seed)
    qkv, gu, dn = spec.linears
    out = {}
    gate_up_bytes = gu.weight_bytes
    bytes_step = stack.bytes_per_layer * layers
    stream = torch.cuda.Stream()
    for m in m_values:
        x = torch.from_numpy(wl.activations(7 + m, m, spec.hidden)).to(dev)
        bufs = {"qkv": torch.empty((m, qkv.n), device=dev), "h": torch.empty((m, gu.n // 2), device=dev),
                "y": torch.empty((m, dn.n), device=dev)}
        with torch.cuda.stream(stream):
            # eager: one library call per linear from Python
            ms_eager = time_steps(torch, lambda: stack.run(q8, x, bufs, m), args.steps, args.warmup)
            eager_y = bufs["y"].clone()
            # the same step captured once as a HIP graph and replayed
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                stack.run(q8, x, bufs, m)
            graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(bufs["y"], eager_y):
                raise RuntimeError("graph replay differs from the eager step")
            ms = time_steps(torch, graph.replay, args.steps, args.warmup)
        # dominant kernel: the fused gate_up of every layer launched back to back (distinct
        # weights, so each launch streams from HBM), as a graph timed on its stream
        durs = [graph_launch_ms(torch, lambda: stack.run_gate_up(q8, x, bufs), layers,
                                replays=max(2, args.steps // 5))]
        res = {"ms_per_step": round(ms, 5), "gbps": round(bytes_step / (ms * 1e-3) / 1e9, 2),
               "tok_s": round(m * 1000.0 / ms, 2), "weight_bytes_per_step": bytes_step,
               "ms_per_step_eager": round(ms_eager, 5),
               "gbps_eager": round(bytes_step / (ms_eager * 1e-3) / 1e9, 2)}
        res["hbm_frac"] = round(res["gbps"] / HBM_PEAK_GBS, 4)
        avg_ms = float(np.mean(durs))
        res["gate_up_avg_us"] = round(avg_ms * 1e3, 3)
        res["gate_up_gbps"] = round(gate_up_bytes / (avg_ms * 1e-3) / 1e9, 2)
        if m > 1:
            # compute floor of the streaming rows form that runs this gate_up (K = 4096): on
            # the VALU one int8 -> float32 conversion per weight and, per 32-weight block and
            # lane, four scale broadcasts and one fma per group of four activation rows and
            # weight row (acc = fma(d, t, acc)); on the fp32 matrix cores the activation rows
            # rounded up to four; the two engines do not overlap, so the floor is the sum
            weights = gu.n * gu.k
            rows_mfma = 4 * ((m + 3) // 4)
            lane_ops = weights * (1.0 + (1 + rows_mfma // 4) / 8.0)
            floor_s = lane_ops / VALU_LANE_OPS_PER_S + 2.0 * weights * rows_mfma / MFMA_FP32_PEAK_FLOPS
            res["gate_up_compute_floor_us"] = round(floor_s * 1e6, 3)
            res["gate_up_compute_frac"] = round(floor_s / (avg_ms * 1e-3), 4)
        out[m] = res
        log(f"M={m}: {res}")
    return stack, out, gate_up_bytes


def bench_block_q8act(args, torch, dev, q8, stack, m_values):
    """The block step on the integer q8 x q8 path (quantize + int8-dot linears), captured
    as a HIP graph like the float32 step."""
    import workloads as wl
    qkv, gu, dn = stack.spec.linears
    out = {}
    bytes_step = stack.bytes_per_layer * stack.layers
    stream = torch.cuda.Stream()
    for m in m_values:
        x = torch.from_numpy(wl.activations(7 + m, m, stack.spec.hidden)).to(dev)
        f = gu.n // 2
        bufs = {"qkv": torch.empty((m, qkv.n), device=dev), "h": torch.empty((m, f), device=dev),
                "y": torch.empty((m, dn.n), device=dev),
                "xq": torch.empty((m, qkv.k), dtype=torch.int8, device=dev),
                "xd": torch.empty((m, qkv.k // 32), device=dev),
                "hq": torch.empty((m, f), dtype=torch.int8, device=dev),
                "hd": torch.empty((m, f // 32), device=dev)}
        with torch.cuda.stream(stream):
            stack.run_q8act(q8, x, bufs, m)
            torch.cuda.synchronize()
            eager_y = bufs["y"].clone()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                stack.run_q8act(q8, x, bufs, m)
            graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(bufs["y"], eager_y):
                raise RuntimeError("graph replay differs from the eager q8act step")
            ms = time_steps(torch, graph.replay, args.steps, args.warmup)
        gu_ms = graph_launch_ms(torch, lambda: stack.run_gate_up_q8act(q8, bufs), stack.layers,
                                replays=max(2, args.steps // 5))
        res = {"path": "q8 x q8 (int8 activation codes per 32-block, v_dot4)",
               "ms_per_step": round(ms, 5), "gbps": round(bytes_step / (ms * 1e-3) / 1e9, 2),
               "tok_s": round(m * 1000.0 / ms, 2), "weight_bytes_per_step": bytes_step,
               "hbm_frac": round(bytes_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "gate_up_avg_us": round(gu_ms * 1e3, 3),
               "gate_up_gbps": round(gu.weight_bytes / (gu_ms * 1e-3) / 1e9, 2)}
        out[m] = res
        log(f"q8act M={m}: {res}")
    return out


def graph_launch_ms(torch, seq, launches, replays=5):
    """Average ms per launch of a launch sequence: seq() (which makes `launches` library
    calls) is captured once as a HIP graph on a side stream and replayed back to back,
    timed with HIP events on that stream, so host call overhead does not hide short
    kernels."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        seq()  # warm (and the eager reference for the graph check below)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            seq()
        graph.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * launches)


def bench_linear(torch, dev, q8, name, n, k, m, fused, reps, min_bytes=600e6, fmt="q8_0"):
    """One linear launched back to back over distinct resident weight copies (enough of
    them to exceed the 256 MB Infinity Cache twice).  fmt: "q8_0", "q4_0", "q4_k" or
    "q6_k" weights."""
    import workloads as wl
    gen = {"q8_0": wl.q8_weight, "q4_0": wl.q4_0_weight, "q4_k": wl.q4_k_weight, "q5_k": wl.q5_k_weight,
           "q6_k": wl.q6_k_weight}[fmt]
    wb = gen(31, n, k)[0]
    plain = getattr(q8, "q8_linear" if fmt == "q8_0" else f"{fmt}_linear")
    fused_fn = getattr(q8, "q8_linear_fused_gate_up_silu" if fmt == "q8_0" else f"{fmt}_linear_fused_gate_up_silu")
    base = torch.from_numpy(wb).to(dev)
    copies = [base] + [base.clone() for _ in range(max(1, int(min_bytes // wb.size)))]
    x = torch.from_numpy(wl.activations(37, m, k)).to(dev)
    nout = n // 2 if fused else n
    y = torch.empty((m, nout), device=dev)
    launches = max(reps, len(copies))

    def seq():
        for i in range(launches):
            w = copies[i % len(copies)]
            if fused:
                fused_fn(w, nout, k, x, out=y)
            else:
                plain(w, n, k, x, out=y)

    ms = graph_launch_ms(torch, seq, launches)
    flops = 2.0 * m * n * k
    res = {"shape": [n, k], "m": m, "fused_silu": fused, "weights": fmt.upper(), "us_per_launch": round(ms * 1e3, 3),
           "weight_bytes": int(wb.size), "gbps": round(wb.size / (ms * 1e-3) / 1e9, 2),
           "hbm_frac": round(wb.size / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "distinct_weight_copies": len(copies)}
    if m >= 256:
        res["mfma_bf16_frac"] = round(res["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
    log(f"{name}: {res}")
    del copies
    return res


def bench_moe(torch, dev, q8, layers, steps, warmup, top_p=None):
    """Qwen3-30B-A3B MoE layers at 16 tokens: device router (softmax top-8, renormalized;
    with top_p, the adaptive expert top-p cut after it; the two-pass form) then the grouped
    SwiGLU expert mixture, each layer with its own resident experts."""
    import workloads as wl
    cfg = wl.QWEN3_30B_A3B_MOE
    e, f, hd, k, t = cfg.n_exp, cfg.ffn, cfg.hidden, cfg.k, cfg.tokens
    distinct = 8  # experts generated on the host; the device stacks repeat them (timing only)
    gu_h = np.concatenate([wl.q8_weight(cfg.seed * 100 + i, 2 * f, hd)[0] for i in range(distinct)])
    dn_h = np.concatenate([wl.q8_weight(cfg.seed * 100 + 50 + i, hd, f)[0] for i in range(distinct)])
    gu1, dn1 = torch.from_numpy(gu_h).to(dev), torch.from_numpy(dn_h).to(dev)
    gu_stack = torch.cat([gu1] * (e // distinct))
    dn_stack = torch.cat([dn1] * (e // distinct))
    gu = [gu_stack] + [gu_stack.clone() for _ in range(layers - 1)]
    dn = [dn_stack] + [dn_stack.clone() for _ in range(layers - 1)]
    del gu1, dn1
    wr = [torch.from_numpy(wl.router_weight(cfg.seed + 2 + l, e, hd, cfg.router_std)).to(dev) for l in range(layers)]
    x = torch.from_numpy(wl.activations(cfg.seed + 1, t, hd)).to(dev)
    idx = [torch.empty((t, k), dtype=torch.int32, device=dev) for _ in range(layers)]
    wts = [torch.empty((t, k), dtype=torch.float32, device=dev) for _ in range(layers)]
    y = torch.empty((t, hd), device=dev)
    ws = torch.empty(q8.q8_moe_workspace_bytes(t, k, e, f, hd), dtype=torch.uint8, device=dev)
    ws_route = torch.empty(q8.moe_route_workspace_bytes(t, e), dtype=torch.uint8, device=dev)
    per_expert = (gu_h.size + dn_h.size) // distinct

    def step():
        for l in range(layers):
            q8.moe_route_topk(x, wr[l], k, True, idx_out=idx[l], w_out=wts[l], top_p=top_p, workspace=ws_route)
            q8.q8_moe_grouped_linear(gu[l], dn[l], e, f, hd, x, idx[l], wts[l], out=y, workspace=ws)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        ms_eager = time_steps(torch, step, steps, warmup)
        y_eager = y.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(y, y_eager):
            raise RuntimeError("MoE graph replay differs from the eager step")
        ms = time_steps(torch, graph.replay, steps, warmup)
    used = [int(torch.unique(i[i >= 0]).numel()) for i in idx]
    slots = [int((i >= 0).sum()) for i in idx]
    expert_bytes = sum(used) * per_expert
    router_bytes = layers * e * hd * 4
    res = {"workload": cfg.name, "tokens": t, "layers": layers, "experts": e, "top_k": k,
           "ms_per_step": round(ms, 5), "ms_per_step_eager": round(ms_eager, 5),
           "us_per_layer": round(ms * 1e3 / layers, 3), "tok_s": round(t * 1000.0 / ms, 1),
           "experts_used_per_layer": used, "routed_slots_per_layer": slots, "bytes_per_expert": per_expert,
           "weight_bytes_per_step": expert_bytes + router_bytes,
           "gbps": round((expert_bytes + router_bytes) / (ms * 1e-3) / 1e9, 2)}
    res["hbm_frac"] = round(res["gbps"] / HBM_PEAK_GBS, 4)
    if top_p is not None:
        res["expert_top_p"] = top_p
    log(f"moe: {res}")
    return res


def bench_moe_prefill(torch, dev, q8, tokens, reps):
    """Qwen3-30B-A3B MoE layer at prefill size: device routing (two-pass) then the grouped
    mixture, which runs on the expert-grouped bf16 matrix-core tiles at this size.  Reports
    the mixture's time and the TFLOP/s of its expert products."""
    import workloads as wl
    cfg = wl.QWEN3_30B_A3B_MOE
    e, f, hd, k = cfg.n_exp, cfg.ffn, cfg.hidden, cfg.k
    distinct = 8
    gu_h = np.concatenate([wl.q8_weight(cfg.seed * 100 + i, 2 * f, hd)[0] for i in range(distinct)])
    dn_h = np.concatenate([wl.q8_weight(cfg.seed * 100 + 50 + i, hd, f)[0] for i in range(distinct)])
    gu = torch.cat([torch.from_numpy(gu_h).to(dev)] * (e // distinct))
    dn = torch.cat([torch.from_numpy(dn_h).to(dev)] * (e // distinct))
    x = torch.from_numpy(wl.activations(cfg.seed + 11, tokens, hd)).to(dev)
    wr = torch.from_numpy(wl.router_weight(cfg.seed + 12, e, hd, cfg.router_std)).to(dev)
    idx, wts = q8.moe_route_topk(x, wr, k, True, workspace=True)
    y = torch.empty((tokens, hd), device=dev)
    ws = torch.empty(q8.q8_moe_workspace_bytes(tokens, k, e, f, hd), dtype=torch.uint8, device=dev)
    ms = graph_launch_ms(torch, lambda: [q8.q8_moe_grouped_linear(gu, dn, e, f, hd, x, idx, wts, out=y, workspace=ws)
                                         for _ in range(reps)], reps)
    pairs = int((idx >= 0).sum())
    flops = 2.0 * pairs * (2 * f * hd + hd * f)
    res = {"workload": cfg.name + "-prefill", "tokens": tokens, "routed_pairs": pairs, "experts": e, "top_k": k,
           "path": "expert-grouped bf16 MFMA tiles", "us_per_layer": round(ms * 1e3, 2),
           "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "mfma_bf16_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "tok_s": round(tokens * 1000.0 / ms, 1)}
    log(f"moe prefill: {res}")
    return res


PROFILE_LINEARS = {"qkv": (6144, 4096, False), "gate_up": (24576, 4096, True), "down": (4096, 12288, False)}


def read_ceiling_us(torch, dev, q8, nbytes, min_bytes=600e6):
    """The time one launch of a plain streaming read of nbytes takes (best launch shape of
    the library's read probe), over distinct resident buffers back to back like
    bench_linear, so that every launch reads from HBM.  Returns (us, shape)."""
    nb = nbytes - nbytes % 4096
    copies = max(2, int(min_bytes // nb) + 1)
    pool = torch.randint(0, 256, (copies * nb,), dtype=torch.uint8, device=dev)
    views = [pool[i * nb:(i + 1) * nb] for i in range(copies)]
    best = None
    for shape in range(q8.probe_shape_count()):
        sink = q8.probe_stream_read(views[0], nb, shape)

        def seq():
            for v in views:
                q8.probe_stream_read(v, nb, shape, sink=sink)

        ms = graph_launch_ms(torch, seq, copies)
        if best is None or ms < best[0]:
            best = (ms, shape)
    del pool, views
    return best[0] * 1e3 * nbytes / nb, best[1]


def launch_floor_us(torch, dev, q8, blocks, launches=200):
    """Average time per launch of a kernel of `blocks` workgroups that does nothing,
    replayed back to back in a graph."""
    return graph_launch_ms(torch, lambda: [q8.probe_empty(blocks, dev) for _ in range(launches)], launches) * 1e3


def bench_bounds(torch, dev, q8, reps, known):
    """Each one-row linear against the two bounds of its launch on this GPU: a plain
    streaming read of its weight bytes in one launch, and an empty launch.  `known` maps
    names to bench_linear results already measured."""
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    floor = {"1_block": round(launch_floor_us(torch, dev, q8, 1), 3),
             f"{8 * cu}_blocks": round(launch_floor_us(torch, dev, q8, 8 * cu), 3)}
    log(f"launch floor: {floor}")
    linears = [("qwen3-8b-qkv-m1", 6144, 4096, False, "q8_0"), ("qwen3-8b-gate-up-m1", 24576, 4096, True, "q8_0"),
               ("qwen3-8b-down-m1", 4096, 12288, False, "q8_0"), ("qwen3-0.6b-qkv-m1", 4096, 1024, False, "q8_0"),
               ("qwen3-0.6b-gate-up-m1", 6144, 1024, True, "q8_0"), ("qwen3-0.6b-down-m1", 1024, 3072, False, "q8_0"),
               ("qwen3-8b-ffn-gate-up-q4_k-m1", 24576, 4096, True, "q4_k"),
               ("qwen3-8b-ffn-down-q6_k-m1", 4096, 12288, False, "q6_k")]
    out = {}
    for name, n, k, fused, fmt in linears:
        r = known.get(name) or bench_linear(torch, dev, q8, name, n, k, 1, fused, reps, fmt=fmt)
        read_us, shape = read_ceiling_us(torch, dev, q8, r["weight_bytes"])
        out[name] = {"weights": fmt.upper(), "bytes": r["weight_bytes"], "kernel_us": r["us_per_launch"],
                     "read_us": round(read_us, 3), "read_gbps": round(r["weight_bytes"] / read_us / 1e3, 1),
                     "kernel_over_read": round(read_us / r["us_per_launch"], 4),
                     "hbm_frac": round(r["weight_bytes"] / r["us_per_launch"] / 1e3 / HBM_PEAK_GBS, 4),
                     "read_hbm_frac": round(r["weight_bytes"] / read_us / 1e3 / HBM_PEAK_GBS, 4),
                     "read_probe_shape": shape}
        log(f"bounds {name}: {out[name]}")
    return {"launch_floor_us": floor, "one_row_linears": out,
            "note": "read_us: best of the library's plain streaming-read probe shapes over the same byte count in "
                    "one launch; kernel_over_read = read_us / kernel_us"}


def kernel_driver(which, m, q8act, fmt="q8_0"):
    """Short launch sequence for rocprofv3 counter and trace runs: a plain 256 MiB
    device-to-device copy (the calibration dispatch for FETCH_SIZE / WRITE_SIZE), then one
    Qwen3-8B linear at m rows with fmt weights ("q8_0", "q4_0", "q4_k", "q5_k", "q6_k") on
    12 distinct resident weight copies (each launch streams its weights from HBM), or with
    which = "moe" the Qwen3-30B-A3B MoE layer at m tokens."""
    import torch

    import block_quantized_weight_linear_amd as q8
    import workloads as wl

    dev = torch.device("cuda:0")
    src = torch.ones(64 << 20, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if which == "moe":
        # the Qwen3-30B-A3B MoE layer at m tokens: two-pass routing, then the grouped
        # mixture, four times over the same resident experts
        cfg = wl.QWEN3_30B_A3B_MOE
        e, f, hd, kk = cfg.n_exp, cfg.ffn, cfg.hidden, cfg.k
        gu_h = np.concatenate([wl.q8_weight(cfg.seed * 100 + i, 2 * f, hd)[0] for i in range(8)])
        dn_h = np.concatenate([wl.q8_weight(cfg.seed * 100 + 50 + i, hd, f)[0] for i in range(8)])
        gu = torch.cat([torch.from_numpy(gu_h).to(dev)] * (e // 8))
        dn = torch.cat([torch.from_numpy(dn_h).to(dev)] * (e // 8))
        x = torch.from_numpy(wl.activations(cfg.seed + 11, m, hd)).to(dev)
        wr = torch.from_numpy(wl.router_weight(cfg.seed + 12, e, hd, cfg.router_std)).to(dev)
        used = []
        for _ in range(4):
            idx, wts = q8.moe_route_topk(x, wr, kk, True, workspace=True)
            q8.q8_moe_grouped_linear(gu, dn, e, f, hd, x, idx, wts)
            used.append(int(torch.unique(idx).numel()))  # experts whose weights the call reads
        torch.cuda.synchronize()
        log(f"kernel driver: moe tokens={m} done; experts used per call: {used}; "
            f"gate_up / down bytes per expert: {2 * f * hd * 17 // 16} / {hd * f * 17 // 16}")
        return
    n, k, fused = PROFILE_LINEARS[which]
    gen = {"q8_0": wl.q8_weight, "q4_0": wl.q4_0_weight, "q4_k": wl.q4_k_weight, "q5_k": wl.q5_k_weight,
           "q6_k": wl.q6_k_weight}[fmt]
    if q8act and fmt != "q8_0":
        raise SystemExit("bench.py: --q8act takes Q8_0 weights")
    base = torch.from_numpy(gen(1, n, k)[0]).to(dev)
    ws = [base] + [base.clone() for _ in range(11)]
    x = torch.from_numpy(wl.activations(2, m, k)).to(dev)
    nout = n // 2 if fused else n
    if q8act:
        xq, xd = q8.q8_quantize_act(x)
    for w in ws:
        if q8act:
            fn = q8.q8_linear_fused_gate_up_silu_q8act if fused else q8.q8_linear_q8act
            fn(w, nout, k, xq, xd)
        else:
            pre = "q8" if fmt == "q8_0" else fmt
            fn = getattr(q8, f"{pre}_linear_fused_gate_up_silu" if fused else f"{pre}_linear")
            fn(w, nout, k, x)
    torch.cuda.synchronize()
    log(f"kernel driver: {which} m={m} fmt={fmt} q8act={q8act} done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3-8b-block-linears",
                    choices=["qwen3-8b-block-linears", "qwen3-0.6b-block-linears"])
    ap.add_argument("--layers", type=int, default=0, help="override the layer count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other workloads (q8 x q8 step, 0.6B, gate_up M=16/M=512, MoE layer)")
    ap.add_argument("--kernel-driver", nargs=2, metavar=("LINEAR", "M"),
                    help="profiling driver only: a 256 MiB copy, then the Qwen3-8B LINEAR "
                         "(qkv | gate_up | down) at M rows on 12 distinct weight copies")
    ap.add_argument("--q8act", action="store_true", help="with --kernel-driver: the q8 x q8 path")
    ap.add_argument("--fmt", default="q8_0", choices=["q8_0", "q4_0", "q4_k", "q5_k", "q6_k"],
                    help="with --kernel-driver: the weight format")
    args = ap.parse_args()
    if args.kernel_driver:
        kernel_driver(args.kernel_driver[0], int(args.kernel_driver[1]), args.q8act, args.fmt)
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported "
              "(the sharded path is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_quantized_weight_linear_amd as q8
    import workloads as wl

    dev = torch.device("cuda:0")
    if args.workload == "qwen3-8b-block-linears":
        spec = wl.QWEN3_8B_BLOCK
        m_values = (1, 8, 16)
    else:
        spec = wl.QWEN3_06B_BLOCK
        m_values = (1,)
    stack, res, gate_up_bytes = bench_block(args, torch, dev, q8, spec, m_values)
    r1 = res[1]
    line = {
        "metric": METRIC,
        "value": r1["gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r1["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "m": 1, "layers": stack.layers, "weights": "Q8_0",
                   "linears": {l.name: [l.n, l.k] for l in spec.linears},
                   "weight_bytes_per_step": r1["weight_bytes_per_step"]},
        "hbm_frac": r1["hbm_frac"],
        "decode_tok_s": r1["tok_s"],
        "execution": "HIP graph replay of the step (eager per-call timing in ms_per_step_eager)",
        "roofline": {"bound": "hbm", "kernel": "fused gate_up + SiLU, one activation row (gemv_one_row_kernel)",
                     "achieved": r1["gate_up_gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r1["gate_up_gbps"] / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE)",
                     "algorithmic_bytes_per_launch": gate_up_bytes, "avg_launch_us": r1["gate_up_avg_us"]},
    }
    for m, r in res.items():
        if m != 1:
            line[f"m{m}"] = r
    if not args.no_extras and args.workload == "qwen3-8b-block-linears":
        extras = {}
        reps = max(20, args.steps)
        for m, r in bench_block_q8act(args, torch, dev, q8, stack, m_values).items():
            extras[f"qwen3-8b-block-linears-q8act-m{m}"] = r
        extras["qwen3-0.6b-qkv-m1"] = bench_linear(torch, dev, q8, "0.6b qkv m1", 4096, 1024, 1, False, reps * 4)
        _, r06, _ = bench_block(args, torch, dev, q8, wl.QWEN3_06B_BLOCK, (1,))
        extras["qwen3-0.6b-block-linears-m1"] = r06[1]
        extras["qwen3-8b-gate-up-m16"] = bench_linear(torch, dev, q8, "8b gate_up m16", 24576, 4096, 16, True, reps)
        extras["qwen3-8b-gate-up-m512-prefill"] = bench_linear(torch, dev, q8, "8b gate_up m512", 24576, 4096, 512,
                                                               True, reps)
        mfma = measured_mfma()
        if "gate_up_m512_mfma_busy_frac" in mfma:
            extras["qwen3-8b-gate-up-m512-prefill"]["mfma_busy_frac_counters"] = mfma["gate_up_m512_mfma_busy_frac"]
        # GGUF Q4_K_M mix on the Qwen3-8B FFN: gate_up in Q4_K, down in Q6_K
        for m in (1, 8):
            extras[f"qwen3-8b-ffn-gate-up-q4_k-m{m}"] = bench_linear(torch, dev, q8, f"8b gate_up q4_k m{m}", 24576,
                                                                     4096, m, True, reps, fmt="q4_k")
            extras[f"qwen3-8b-ffn-down-q6_k-m{m}"] = bench_linear(torch, dev, q8, f"8b down q6_k m{m}", 4096, 12288,
                                                                  m, False, reps, fmt="q6_k")
        # GGUF Q4_0 weights: the Gemma 4 12B FFN (hidden 3840, intermediate 15360), one token
        extras["gemma-4-12b-ffn-gate-up-q4_0-m1"] = bench_linear(torch, dev, q8, "gemma4 12b gate_up q4_0 m1",
                                                                 30720, 3840, 1, True, reps, fmt="q4_0")
        extras["gemma-4-12b-ffn-down-q4_0-m1"] = bench_linear(torch, dev, q8, "gemma4 12b down q4_0 m1",
                                                              3840, 15360, 1, False, reps, fmt="q4_0")
        extras["qwen3-30b-a3b-moe-16tok"] = bench_moe(torch, dev, q8, 4, args.steps, args.warmup)
        extras["qwen3-30b-a3b-moe-2048tok-prefill"] = bench_moe_prefill(torch, dev, q8, 2048, 5)
        if "a3b_moe_2048_gate_up_mfma_busy_frac" in mfma:
            extras["qwen3-30b-a3b-moe-2048tok-prefill"]["mfma_busy_frac_counters"] = {
                "gate_up": mfma["a3b_moe_2048_gate_up_mfma_busy_frac"], "down": mfma["a3b_moe_2048_down_mfma_busy_frac"]}
        extras["qwen3-30b-a3b-moe-512tok"] = bench_moe_prefill(torch, dev, q8, 512, 5)
        extras["qwen3-30b-a3b-moe-16tok-expert-top-p-0.9"] = bench_moe(torch, dev, q8, 4, args.steps, args.warmup,
                                                                        top_p=0.9)
        line["configs"] = extras
        line["bounds"] = bench_bounds(torch, dev, q8, reps, {
            "qwen3-0.6b-qkv-m1": extras["qwen3-0.6b-qkv-m1"],
            "qwen3-8b-ffn-gate-up-q4_k-m1": extras["qwen3-8b-ffn-gate-up-q4_k-m1"],
            "qwen3-8b-ffn-down-q6_k-m1": extras["qwen3-8b-ffn-down-q6_k-m1"]})
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one layer")
        line["cpu_baseline"] = cpu_baseline_block(spec)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
