"""Benchmark of the fused Conv/MatMul -> BatchNorm -> activation operator on one MI355X.

A step is one fused forward of the layer over one batch of seeded synthetic input already
resident in HBM (the BN fold is load-time work and runs before timing; the layer build, fold
included, is reported separately as `layer_build_s`).  Each of the five workloads is timed
three ways, all with HIP events on the stream the kernels run on:

- graph: W warm-up launches, then exactly K launches captured back to back in one HIP graph
  and replayed between two events, torch.cuda.synchronize() on both sides.  The mean time per
  launch gives `value` / `ms_per_step` (workload 1, the bf16 3x3 conv N=32 56x56 64->64 + BN +
  ReLU) and each workload's `ms`.
- launches: single launches outside any graph, each between its own pair of events, enqueued
  while a spin kernel holds the GPU so that the host's launch gaps stay out of the figures;
  the median with p10 and p90 ("FlashRT 跨层融合深度解析" §5 times kernels one by one with
  events, outside graphs).
- cold (the two bf16 conv workloads): the graph rotates through enough distinct copies of
  the inputs and outputs (>= 300 MB) that every launch reads its inputs from HBM, not from the
  256 MB Infinity Cache.  The HBM roofline of an HBM-bound workload is taken from this time.

Every workload record carries its own roofline (bytes or FLOP per launch over the launch time,
against the MI355X peak of its bound, beside the rocprofv3 counter traffic when the counters
were taken on the current kernel sources) and its own CPU baseline: the oracle, as it stands,
on a bounded sample of the same workload on the host's cores.  The unfused chain (conv/GEMM,
BN or bias-add, residual add, activation, quantisation as separate kernels) is timed like the
graph figure for comparison.  A probe of the shader clock under MFMA load gives a clock-derived
peak beside the published one.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "fused Conv+BN+act TFLOP/s (% MFMA peak) + HBM bytes saved vs unfused chain"
# MI355X published peaks: dense matrix-core rates, the fp32 vector rate (the fp32 conv runs on
# FMA units, not the matrix cores) and HBM3E bandwidth
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "fp8": 5033.2}
PEAK_HBM_GBS = 8000.0
CUS = 256
FLOP_PER_CLK_CU = {"f32": 256, "bf16": 4096, "fp8": 8192}
DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
COLD_BYTES = 300 * 10 ** 6            # distinct bytes the cold rotation streams (> 256 MB MALL)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["mma_kernel.h", "mma_gemm.hip", "mma_bf16_dense.hip", "mma_bf16_gated.hip",
                  "mma_bf16_conv.hip", "mma_fp8_q.hip", "mma_fp8_b.hip", "mma_common.h", "conv_halo.hip",
                  "conv_f32.hip", "device_common.h", "kernels.h", "api.cpp"]   # api.cpp picks the route and tile


def flops(wl) -> int:
    m, n, k = wl.gemm_mnk
    return 2 * m * n * k


def bytes_model(wl):
    """Algorithmic HBM bytes: fused = each tensor once (x, W', per-channel params,
    [residual], out); unfused adds one write + one read per intermediate tensor."""
    m, n, k = wl.gemm_mnk
    if wl.kind == "conv":
        e = DTYPE_BYTES[wl.dtype]
        x = wl.n * wl.h * wl.w * wl.cin * e
        w = n * k * e
        out = m * n * e
        res = out if wl.residual else 0
        fused = x + w + 4 * n + res + out
        # conv (+conv bias) -> y; BN reads y + 4 vectors -> z; [add reads z, r -> u]; act reads -> out
        conv_bias = 4 * n if wl.conv_bias else 0
        hops = 2 + (1 if wl.residual else 0)           # intermediates written then read
        unfused = x + w + conv_bias + 16 * n + res + out + hops * 2 * out
        return fused, unfused
    if wl.kind == "gemm":
        x, w, out = m * k * 2, n * k * 2, m * n * 2
        bias = 4 * n if wl.bias else 0
        hops = 2 if wl.bias else 1                      # GEMM -> bias-add -> act
        return x + w + bias + out, x + w + bias + out + hops * 2 * out
    # fp8: codes in, codes out; fp32 intermediates y, z, u in the unfused chain
    x, w, out = m * k, n * k, m * n
    fused = x + w + 8 * n + out
    inter = m * n * 4
    unfused = x + w + 16 * n + out + 3 * 2 * inter
    return fused, unfused


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dl_fusion_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(wl_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on
    the current kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(wl_name)
    if not rec or rec.get("kernel_hash") != kernel_hash():
        return None
    return rec


# ---------------------------------------------------------------------------
# Timing
# ---------------------------------------------------------------------------
def time_graph(torch, fns, steps: int, warmup: int):
    """Warm up eagerly, capture `steps` calls (cycling through the list `fns`) in one graph,
    replay it once untimed and once between events.  Returns the mean milliseconds per call."""
    fns = fns if isinstance(fns, (list, tuple)) else [fns]
    for i in range(max(1, warmup)):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                fns[i % len(fns)]()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()                      # one untimed replay (graph upload; cold copies: a cold pass)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_eager(torch, fn, steps: int, warmup: int):
    for _ in range(max(1, warmup)):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


_SLEEP_CYCLES_PER_MS = None


def _hold_gpu(torch, ms: float):
    """Enqueue a spin kernel of about `ms` milliseconds (torch's clock-based sleep, calibrated
    once) so that the host can enqueue work behind it without the GPU waiting on the host."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 1_000_000 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(_SLEEP_CYCLES_PER_MS * ms))


def time_launches(torch, fn, n: int, warmup: int = 3):
    """Single launches outside a graph, each between its own two events, enqueued behind a spin
    kernel.  Returns {median, p10, p90, n} in milliseconds."""
    for _ in range(max(1, warmup)):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    _hold_gpu(torch, 0.1 * n + 5.0)       # well above the host's enqueue time of n launches
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)),
            "p90": float(np.percentile(t, 90)), "n": n}


def clock_probe(torch):
    """Shader clock (MHz) the chip holds with every SIMD issuing bf16 MFMAs back to back: the
    median over workgroups of the shader-counter ticks per 100 MHz constant-counter tick."""
    import dl_fusion_amd as d
    wgs, iters = 1024, 20000
    stamps = torch.zeros(4 * wgs, dtype=torch.int64, device="cuda")
    d.dlf_clock_probe(wgs, 200, stamps)           # warm-up
    torch.cuda.synchronize()
    d.dlf_clock_probe(wgs, iters, stamps)
    torch.cuda.synchronize()
    s = stamps.view(wgs, 4).cpu().numpy().astype(np.float64)
    dt, dr = s[:, 1] - s[:, 0], s[:, 3] - s[:, 2]
    ok = dr > 0
    mhz = float(np.median(dt[ok] / dr[ok] * 100.0))
    return {"sclk_mhz_under_mfma": mhz, "workgroups": wgs, "mfma_per_wave": 4 * iters,
            "peak_tflops_at_this_clock": {k: CUS * mhz * 1e6 * v / 1e12 for k, v in FLOP_PER_CLK_CU.items()}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------
# One workload
# ---------------------------------------------------------------------------
def roofline(wl, ms: float, fused_bytes: int, traffic, clock, timing: str):
    """The roofline of the workload's fused kernel at `ms` per launch: bound = the slower of
    its compute at peak and its algorithmic bytes at peak HBM bandwidth."""
    fl = flops(wl)
    peak_tf = PEAK_TFLOPS[wl.dtype]
    t_compute = fl / (peak_tf * 1e12)
    t_hbm = fused_bytes / (PEAK_HBM_GBS * 1e9)
    if t_hbm > t_compute:
        achieved = fused_bytes / (ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = fl / (ms * 1e-3) / 1e12
        r = {"bound": "alu" if wl.dtype == "f32" else "mfma", "achieved": achieved, "peak": peak_tf,
             "unit": "TFLOP/s", "frac": achieved / peak_tf}
        if clock:
            cp = clock["peak_tflops_at_this_clock"][wl.dtype]
            r["peak_at_measured_clock"] = cp
            r["frac_at_measured_clock"] = achieved / cp
    r["traffic"] = (traffic["fetch_bytes"] + traffic["write_bytes"]) if traffic else None
    r["algorithmic_bytes"] = fused_bytes
    r["flop"] = fl
    r["ms"] = ms
    r["timing"] = timing
    from dl_fusion_amd.rocprof import fused_kernel
    r["kernel"] = "dlf::" + fused_kernel(wl)
    return r


def cold_timing(torch, layer, wl, steps: int, warmup: int):
    """Graph time per launch over rotating copies of x (and the residual) and y: at least
    COLD_BYTES of distinct tensors, so every launch streams its inputs from HBM."""
    per_set = layer.x.numel() * layer.x.element_size() + layer.y.numel() * layer.y.element_size() \
        + (layer.res.numel() * layer.res.element_size() if layer.res is not None else 0)
    copies = max(2, -(-COLD_BYTES // per_set))
    xs = [layer.x.clone() for _ in range(copies)]
    rs = [layer.res.clone() for _ in range(copies)] if layer.res is not None else [None] * copies
    ys = [torch.empty_like(layer.y) for _ in range(copies)]
    fns = [lambda i=i: layer.forward(x=xs[i], residual=rs[i], y=ys[i]) for i in range(copies)]
    n = max(steps, copies)
    ms = time_graph(torch, fns, n, max(warmup, copies))
    del xs, rs, ys, fns
    torch.cuda.empty_cache()
    return ms, copies, per_set


def run_workload(torch, idx: int, args, clock, cpu_budget: float):
    from dl_fusion_amd.layers import make_layer
    wl = workloads.workload(idx)
    t0 = time.time()
    inp = workloads.generate(wl)
    gen_s = time.time() - t0
    t0 = time.perf_counter()
    layer = make_layer(inp, with_unfused=not args.no_unfused)   # includes the host BN fold + H2D copies
    build_s = time.perf_counter() - t0
    cold_ok = wl.kind == "conv" and wl.dtype == "bf16"
    fl = flops(wl)
    fused_b, unfused_b = bytes_model(wl)
    peak_tf = PEAK_TFLOPS[wl.dtype]
    rec = {"workload": wl.name, "dtype": wl.dtype, "gemm_mnk": list(wl.gemm_mnk)}
    ms = ms_cold = None
    if args.timing in ("all", "graph"):
        ms = (time_eager if args.eager else time_graph)(torch, layer.forward, args.steps, args.warmup)
        rec.update(ms=ms, tflops=fl / (ms * 1e-3) / 1e12)
        rec["frac_mfma_peak"] = rec["tflops"] / peak_tf
        rec["hbm_gbs_algorithmic"] = fused_b / (ms * 1e-3) / 1e9
        rec["frac_hbm_peak"] = rec["hbm_gbs_algorithmic"] / PEAK_HBM_GBS
    if args.timing == "all" and args.launches > 0:
        rec["launch_ms"] = time_launches(torch, layer.forward, args.launches)
    if cold_ok and args.timing in ("all", "cold"):
        ms_cold, copies, per_set = cold_timing(torch, layer, wl, args.steps, args.warmup)
        rec["cold"] = {"ms": ms_cold, "tflops": fl / (ms_cold * 1e-3) / 1e12,
                       "hbm_gbs_algorithmic": fused_b / (ms_cold * 1e-3) / 1e9,
                       "copies": copies, "bytes_rotated": copies * per_set}
    ms_unfused = None
    if not args.no_unfused and args.timing in ("all", "graph"):
        ms_unfused = time_graph(torch, layer.forward_unfused, args.steps, args.warmup)
    t_compute = fl / (peak_tf * 1e12)
    t_hbm = fused_b / (PEAK_HBM_GBS * 1e9)
    bound = "hbm" if t_hbm > t_compute else "mfma"
    rec.update({
        "bound": bound,
        "bytes_fused": fused_b,
        "bytes_unfused": unfused_b,
        "bytes_saved": unfused_b - fused_b,
        "ms_unfused_chain": ms_unfused,
        "speedup_vs_unfused": (ms_unfused / ms) if (ms_unfused and ms) else None,
        "gen_s": round(gen_s, 3),
        "layer_build_s": round(build_s, 4),
    })
    # the HBM roofline of an HBM-bound workload comes from its cold time; everything else from
    # the graph mean
    traffic = measured_traffic(wl.name)
    rec["traffic_measured"] = traffic
    if bound == "hbm" and ms_cold is not None:
        rec["roofline"] = roofline(wl, ms_cold, fused_b, traffic, clock, "cold graph mean")
        if ms is not None:
            rec["roofline_hot"] = roofline(wl, ms, fused_b, traffic, clock, "hot graph mean")
    elif ms is not None:
        rec["roofline"] = roofline(wl, ms, fused_b, traffic, clock, "graph mean")
    elif ms_cold is not None:
        rec["roofline"] = roofline(wl, ms_cold, fused_b, traffic, clock, "cold graph mean")
    if cpu_budget > 0:
        rec["cpu_baseline"] = cpu_baseline(inp, cpu_budget)
    del layer
    return wl, rec


def cpu_baseline(inp, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the workload, on this host's cores."""
    import oracle
    wl = inp["workload"]
    fl_total = flops(wl)
    m = wl.gemm_mnk[0]
    if wl.kind == "conv":
        # whole images: time one image first, then as many as fit the budget
        t0 = time.perf_counter()
        one = dict(inp)
        one["x"] = inp["x"][:1]
        if inp.get("residual") is not None:
            one["residual"] = inp["residual"][:1]
        one["workload"] = dataclasses.replace(wl, n=1)
        oracle.conv_bn_act(one)
        t1 = time.perf_counter() - t0
        imgs = int(max(1, min(wl.n, budget_s / max(t1, 1e-6))))
        sub = dict(inp)
        sub["x"] = inp["x"][:imgs]
        if inp.get("residual") is not None:
            sub["residual"] = inp["residual"][:imgs]
        sub["workload"] = dataclasses.replace(wl, n=imgs)
        # the whole workload can take well under the budget: then repeat it until the budget is
        # spent (at most 500 passes), so that the figure is not one short, noisy pass
        t0 = time.perf_counter()
        oracle.conv_bn_act(sub)
        first = time.perf_counter() - t0
        passes = 1 + int(max(0, min(499, (budget_s - t1 - first) / max(first, 1e-6))))
        for _ in range(passes - 1):
            oracle.conv_bn_act(sub)
        total_s = time.perf_counter() - t0
        dt = total_s / passes
        frac = imgs / wl.n
        sample = f"{imgs} of {wl.n} images (full conv+BN+act per image)" + (f", {passes} passes" if passes > 1 else "")
    else:
        fn = oracle.gemm_bias_act if wl.kind == "gemm" else oracle.fp8_gemm_bn_relu_quant
        t0 = time.perf_counter()
        fn(inp, rows=np.arange(4))
        t4 = time.perf_counter() - t0
        rows = int(max(4, min(m, 4 * budget_s / max(t4, 1e-6))))
        t0 = time.perf_counter()
        fn(inp, rows=np.arange(rows))
        dt = total_s = time.perf_counter() - t0
        frac = rows / m
        sample = f"{rows} of {m} rows (every output column of each row)"
    return {"value": fl_total * frac / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": sample, "seconds": round(total_s, 3), "cpu": cpu_model()}


def run_next_rows(torch, steps: int, warmup: int, eager: bool):
    """The widened rows, each against what it replaces:
    - the Q/K/V projections of a LLaMA-7B layer (4096 tokens, h = 4096) as one GEMM over the
      concatenated [3h, h] weights stored split into Q, K and V, vs three separate GEMMs;
    - the 4096 x 11008 x 4096 GEMM with the exact (erf) GELU epilogue, vs its unfused chain;
    - a ResNet stem (batch 32, 224x224x3, 7x7 stride 2, three input channels) and a two-block
      ResNet bottleneck stage (batch 32, 56x56x256 -> 28x28x512, strided downsample branch),
      each run under the host fusion pass's plan vs every op on its own;
    - BERT-base's feed-forward block (128, 8192 and 16384 tokens, 768 -> 3072 -> 768, GELU,
      residual) in one kernel vs two GEMMs with their epilogues and the intermediate in HBM."""
    import dl_fusion_amd as d
    from dl_fusion_amd.layers import make_layer
    timer = time_eager if eager else time_graph
    out = {}
    for tokens in (4096, 128):      # a prefill batch, and a small one where launches dominate
        wl = workloads.workload(3, m=tokens, n=3 * 4096, act="none", bias=True)
        inp = workloads.generate(wl)
        L = make_layer(inp, with_unfused=False)
        h = wl.n // 3
        parts = [torch.empty((wl.m, h), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        ms_split = timer(torch, lambda: d.dlf_gemm_fused_split(L.desc, L.x, L.w, None, L.bias, parts), steps,
                         warmup)
        desc1 = d.gemm_desc(wl.m, h, wl.k, "bf16", "bf16", "none")
        ws = [L.w[p * h:(p + 1) * h] for p in range(3)]
        bs = [L.bias[p * h:(p + 1) * h] for p in range(3)]

        def three():
            for p in range(3):
                d.dlf_gemm_fused(desc1, L.x, ws[p], None, bs[p], None, parts[p])
        ms_three = timer(torch, three, steps, warmup)
        tf = flops(wl) / (ms_split * 1e-3) / 1e12
        out[f"f1_qkv_split_store_{tokens}"] = {
            "workload": f"qkv_bf16_{wl.m}x{wl.n}x{wl.k}_bias_split3", "gemm_mnk": list(wl.gemm_mnk),
            "ms": ms_split, "tflops": tf, "frac_mfma_peak": tf / PEAK_TFLOPS["bf16"], "gemm_launches": 1,
            "ms_three_gemms": ms_three, "gemm_launches_three": 3, "speedup_vs_three_gemms": ms_three / ms_split}
        del L, inp, parts, ws, bs
        torch.cuda.empty_cache()
    wl = workloads.workload(3, act="gelu_erf")
    inp = workloads.generate(wl)
    L = make_layer(inp, with_unfused=True)
    ms = timer(torch, L.forward, steps, warmup)
    ms_u = timer(torch, L.forward_unfused, steps, warmup)
    fl = flops(wl)
    out["f2_gelu_erf_epilogue"] = {
        "workload": f"matmul_bf16_{wl.m}x{wl.n}x{wl.k}_bias_gelu_erf", "gemm_mnk": list(wl.gemm_mnk), "ms": ms,
        "tflops": fl / (ms * 1e-3) / 1e12, "frac_mfma_peak": fl / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
        "ms_unfused_chain": ms_u, "speedup_vs_unfused": ms_u / ms}
    del L, inp
    torch.cuda.empty_cache()
    for key, wl in (("f4_ffn_back_to_back", workloads.FFN_BERT_BASE),
                    ("f4_ffn_back_to_back_16k", dataclasses.replace(
                        workloads.FFN_BERT_BASE, name="ffn_bf16_16384x768x3072_bias_gelu_tanh_residual", m=16384)),
                    ("f4_ffn_back_to_back_128", dataclasses.replace(
                        workloads.FFN_BERT_BASE, name="ffn_bf16_128x768x3072_bias_gelu_tanh_residual", m=128))):
        inp = workloads.generate(wl)
        L = make_layer(inp, with_unfused=True)
        ms = timer(torch, L.forward, steps, warmup)
        ms_u = timer(torch, L.forward_unfused, steps, warmup)
        fl = 4 * wl.m * wl.d_model * wl.d_ff
        # HBM traffic of the intermediate h that the fusion avoids (one bf16 write and read), net
        # of the fp32 partial sums the d_ff split writes to its workspace and reads back
        h_bytes = 2 * wl.m * wl.d_ff * 2
        ws_traffic = 2 * L.ws_bytes
        out[key] = {
            "workload": wl.name, "m_dmodel_dff": [wl.m, wl.d_model, wl.d_ff], "ms": ms,
            "tflops": fl / (ms * 1e-3) / 1e12, "frac_mfma_peak": fl / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
            "dff_parts": (L.ws_bytes // (4 * wl.m * wl.d_model)) if L.ws_bytes else 1,
            "workspace_bytes": L.ws_bytes, "h_bytes_avoided": h_bytes, "workspace_traffic": ws_traffic,
            "hbm_bytes_saved": h_bytes - ws_traffic, "ms_two_gemms": ms_u, "speedup_vs_two_gemms": ms_u / ms}
        del L, inp
        torch.cuda.empty_cache()
    from dl_fusion_amd.layers import to_device
    from dl_fusion_amd.network import Network
    from workloads import graphs
    nets = (("f3_resnet_stem", "resnet_stem_bf16_n32_224x224x3_7x7s2_to_112x112x64_bn_relu", graphs.stem_graph(n=32)),
            ("f3_resnet_stage", "resnet_stage_bf16_n32_56x56x256_to_28x28x512_2_bottlenecks",
             graphs.resnet_stage_graph()))
    for key, name, g in nets:
        params = graphs.draw_params(g, seed=11)
        fused, plain = Network(g, params, fuse=True), Network(g, params, fuse=False)
        dev = {j: to_device(workloads.bf16_bits(params[j]["x"]), "bf16") for j in fused.inputs}
        ms = timer(torch, lambda: fused.forward(dev), steps, warmup)
        ms_u = timer(torch, lambda: plain.forward(dev), steps, warmup)
        fl = sum(nd["flops"] for nd in g if nd["op"] == "conv")
        out[key] = {"workload": name, "conv_gflop": fl / 1e9, "ms": ms, "tflops": fl / (ms * 1e-3) / 1e12,
                    "frac_mfma_peak": fl / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], "launches": fused.launches,
                    "hbm_bytes_saved_by_plan": fused.saved_bytes, "ms_unfused": ms_u,
                    "launches_unfused": plain.launches, "speedup_vs_unfused": ms_u / ms}
        del fused, plain, dev, params
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1, help="index of the headline workload (0-4)")
    ap.add_argument("--only", action="store_true", help="run only the headline workload")
    ap.add_argument("--no-unfused", action="store_true", help="skip the unfused-chain timing")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--no-next", action="store_true", help="skip the widened rows")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the headline's cpu_baseline (a quarter of it for the others)")
    ap.add_argument("--launches", type=int, default=100, help="single launches timed outside a graph")
    ap.add_argument("--timing", choices=("all", "graph", "cold"), default="all",
                    help="graph: hot graph timing only; cold: the rotating-copy graph only (conv workloads)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a captured graph")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration under rocprofv3)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this operator runs on one GPU; multi-GPU runs are not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import dl_fusion_amd  # noqa: F401  (fails loudly when the HIP library is missing)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.copy_calib_mb:
        n = args.copy_calib_mb * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy calibration: {n} bytes read, {n} bytes written", file=sys.stderr, flush=True)
        del src, dst

    clock = None
    if args.timing == "all" and not args.eager:
        clock = clock_probe(torch)
        print(f"# shader clock under MFMA load: {clock['sclk_mhz_under_mfma']:.0f} MHz", file=sys.stderr, flush=True)

    order = [args.workload] + ([] if args.only else [i for i in sorted(workloads.WORKLOADS) if i != args.workload])
    recs = {}
    for idx in order:
        print(f"# workload {idx}: {workloads.WORKLOADS[idx].name}", file=sys.stderr, flush=True)
        budget = 0.0 if args.no_cpu else (args.cpu_budget if idx == args.workload else args.cpu_budget / 4)
        wl, rec = run_workload(torch, idx, args, clock, budget)
        recs[idx] = rec
        msg = f"#   graph {rec['ms'] * 1e3:.2f} us" if rec.get("ms") else "#  "
        if rec.get("launch_ms"):
            lm = rec["launch_ms"]
            msg += f"  launches median {lm['median'] * 1e3:.2f} us (p10 {lm['p10'] * 1e3:.2f}, p90 {lm['p90'] * 1e3:.2f})"
        if rec.get("cold"):
            msg += f"  cold {rec['cold']['ms'] * 1e3:.2f} us"
        if rec.get("roofline"):
            r = rec["roofline"]
            msg += f"  roofline {r['bound']} {100 * r['frac']:.1f}%"
        print(msg, file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    head = recs[args.workload]
    wl = workloads.workload(args.workload)
    ms_head = head.get("ms") or head["cold"]["ms"]
    tflops_head = flops(wl) / (ms_head * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": tflops_head,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_head,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "gemm_mnk": list(wl.gemm_mnk),
                   "timing": "eager launches" if args.eager else (
                       "hipgraph of K launches on resident inputs" if head.get("ms") else
                       "hipgraph of launches over rotating input copies")},
        "frac_mfma_peak": tflops_head / PEAK_TFLOPS[wl.dtype],
        "hbm_bytes_saved_vs_unfused": head["bytes_saved"],
    }
    if head.get("roofline"):
        out["roofline"] = head["roofline"]
    if head.get("cpu_baseline"):
        out["cpu_baseline"] = head["cpu_baseline"]
    if clock:
        out["clock"] = clock
    out["workloads"] = {str(k): v for k, v in recs.items()}
    if not args.only and not args.no_next:
        print("# widened rows: split-store QKV GEMM, GELU-erf epilogue, FFN, ResNet stem and stage",
              file=sys.stderr, flush=True)
        out["next_rows"] = run_next_rows(torch, args.steps, args.warmup, args.eager)
        for k, v in out["next_rows"].items():
            print(f"#   {k}: {v['ms'] * 1e3:.1f} us  {v['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
