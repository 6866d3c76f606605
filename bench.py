"""Benchmark of the fused Conv/MatMul -> BatchNorm -> activation operator on one MI355X.

A step is one fused forward of the layer over one batch of seeded synthetic
input already resident in HBM (the BN fold is load-time work and runs before
timing; the layer build, fold included, is timed separately as `layer_build_s`).  W warm-up steps run first; then
exactly K steps, captured back to back in one HIP graph, are replayed between
two HIP events on the launch stream, with torch.cuda.synchronize() on both
sides.  The unfused chain (conv/GEMM, BN or bias-add, residual add, activation,
quantisation as separate kernels) is timed the same way for comparison.

Prints ONE JSON line.  `value` is the TFLOP/s of the default workload (the
bf16 3x3 conv, N=32 56x56 64->64, + BN + ReLU); the other four workloads are
reported under "workloads" with the same fields.
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
# MI355X published peaks (dense)
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "fp8": 5033.2}
PEAK_HBM_GBS = 8000.0
DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
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


def time_graph(torch, fn, steps: int, warmup: int):
    """Warm up eagerly, capture `steps` calls of fn in one graph, replay it between events.
    Returns the average milliseconds per call."""
    for _ in range(max(1, warmup)):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(steps):
                fn()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()                      # one untimed replay (graph upload)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
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


def run_workload(torch, idx: int, steps: int, warmup: int, eager: bool, unfused: bool):
    from dl_fusion_amd.layers import make_layer
    wl = workloads.workload(idx)
    t0 = time.time()
    inp = workloads.generate(wl)
    gen_s = time.time() - t0
    t0 = time.perf_counter()
    layer = make_layer(inp, with_unfused=unfused)        # includes the host BN fold + H2D copies
    build_s = time.perf_counter() - t0
    timer = time_eager if eager else time_graph
    ms = timer(torch, layer.forward, steps, warmup)
    ms_unfused = timer(torch, layer.forward_unfused, steps, warmup) if unfused else None
    fl = flops(wl)
    fused_b, unfused_b = bytes_model(wl)
    peak_tf = PEAK_TFLOPS[wl.dtype]
    tflops = fl / (ms * 1e-3) / 1e12
    gbs = fused_b / (ms * 1e-3) / 1e9
    t_mfma = fl / (peak_tf * 1e12)
    t_hbm = fused_b / (PEAK_HBM_GBS * 1e9)
    rec = {
        "workload": wl.name,
        "dtype": wl.dtype,
        "gemm_mnk": list(wl.gemm_mnk),
        "ms": ms,
        "tflops": tflops,
        "frac_mfma_peak": tflops / peak_tf,
        "hbm_gbs_algorithmic": gbs,
        "frac_hbm_peak": gbs / PEAK_HBM_GBS,
        "bound": "mfma" if t_mfma >= t_hbm else "hbm",
        "bytes_fused": fused_b,
        "bytes_unfused": unfused_b,
        "bytes_saved": unfused_b - fused_b,
        "ms_unfused_chain": ms_unfused,
        "speedup_vs_unfused": (ms_unfused / ms) if ms_unfused else None,
        "gen_s": round(gen_s, 3),
        "layer_build_s": round(build_s, 4),
    }
    return wl, inp, rec


def run_next_rows(torch, steps: int, warmup: int, eager: bool):
    """The widened rows, each against what it replaces:
    - the Q/K/V projections of a LLaMA-7B layer (4096 tokens, h = 4096) as one GEMM over the
      concatenated [3h, h] weights stored split into Q, K and V, vs three separate GEMMs;
    - the 4096 x 11008 x 4096 GEMM with the exact (erf) GELU epilogue, vs its unfused chain;
    - a ResNet stem (batch 32, 224x224x3, 7x7 stride 2, three input channels) and a two-block
      ResNet bottleneck stage (batch 32, 56x56x256 -> 28x28x512, strided downsample branch),
      each run under the host fusion pass's plan vs every op on its own;
    - BERT-base's feed-forward block (8192 and 16384 tokens, 768 -> 3072 -> 768, GELU,
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
        out[key] = {
            "workload": wl.name, "m_dmodel_dff": [wl.m, wl.d_model, wl.d_ff], "ms": ms,
            "tflops": fl / (ms * 1e-3) / 1e12, "frac_mfma_peak": fl / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
            "hbm_bytes_saved": 2 * wl.m * wl.d_ff * 2, "ms_two_gemms": ms_u, "speedup_vs_two_gemms": ms_u / ms}
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
        # the whole workload can take well under the budget: then repeat it (at most 20 passes
        # in all) so that the time is not one short, noisy pass
        t0 = time.perf_counter()
        oracle.conv_bn_act(sub)
        first = time.perf_counter() - t0
        passes = 1 + int(max(0, min(19, (budget_s - t1 - first) / max(first, 1e-6))))
        for _ in range(passes - 1):
            oracle.conv_bn_act(sub)
        total_s = time.perf_counter() - t0
        dt = total_s / passes
        frac = imgs / wl.n
        sample = f"{imgs} of {wl.n} images (full conv+BN+act per image)" + (f", {passes} passes" if passes > 1 else "")
    else:
        rows = max(1, min(m, 64))
        t0 = time.perf_counter()
        if wl.kind == "gemm":
            oracle.gemm_bias_act(inp, rows=np.arange(rows))
        else:
            oracle.fp8_gemm_bn_relu_quant(inp, rows=np.arange(rows))
        dt = time.perf_counter() - t0
        total_s = dt
        frac = rows / m
        sample = f"{rows} of {m} rows"
    return {"value": fl_total * frac / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": sample, "seconds": round(total_s, 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1, help="index of the headline workload (0-4)")
    ap.add_argument("--only", action="store_true", help="run only the headline workload")
    ap.add_argument("--no-unfused", action="store_true", help="skip the unfused-chain timing")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
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

    order = [args.workload] + ([] if args.only else [i for i in sorted(workloads.WORKLOADS) if i != args.workload])
    recs = {}
    head_inp = None
    for idx in order:
        print(f"# workload {idx}: {workloads.WORKLOADS[idx].name}", file=sys.stderr, flush=True)
        wl, inp, rec = run_workload(torch, idx, args.steps, args.warmup, args.eager, not args.no_unfused)
        tr = measured_traffic(wl.name)
        rec["traffic_measured"] = tr
        recs[idx] = rec
        print(f"#   {rec['ms'] * 1e3:.2f} us/step  {rec['tflops']:.1f} TFLOP/s  "
              f"({100 * rec['frac_mfma_peak']:.1f}% MFMA peak)  unfused {rec['ms_unfused_chain']}",
              file=sys.stderr, flush=True)
        if idx == args.workload:
            head_inp = inp
        else:
            del inp
        torch.cuda.empty_cache()

    head = recs[args.workload]
    wl = workloads.workload(args.workload)
    if head["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": head["tflops"], "peak": PEAK_TFLOPS[wl.dtype], "unit": "TFLOP/s",
                "frac": head["frac_mfma_peak"]}
    else:
        roof = {"bound": "hbm", "achieved": head["hbm_gbs_algorithmic"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": head["frac_hbm_peak"]}
    tr = head["traffic_measured"]
    roof["traffic"] = (tr["fetch_bytes"] + tr["write_bytes"]) if tr else None
    from dl_fusion_amd.rocprof import fused_kernel
    roof["kernel"] = "dlf::" + fused_kernel(wl)

    out = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "gemm_mnk": list(wl.gemm_mnk),
                   "timing": "eager" if args.eager else "hipgraph of K launches"},
        "frac_mfma_peak": head["frac_mfma_peak"],
        "hbm_bytes_saved_vs_unfused": head["bytes_saved"],
        "roofline": roof,
    }
    if not args.no_cpu and head_inp is not None:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(head_inp, args.cpu_budget)
    out["workloads"] = {str(k): v for k, v in recs.items()}
    if not args.only:
        print("# widened rows: split-store QKV GEMM, GELU-erf epilogue", file=sys.stderr, flush=True)
        out["next_rows"] = run_next_rows(torch, args.steps, args.warmup, args.eager)
        for k, v in out["next_rows"].items():
            print(f"#   {k}: {v['ms'] * 1e3:.1f} us  {v['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
