"""rocprofv3 harness: kernel durations, HBM bytes and MFMA busy time of the fused kernels.

Runs bench.py under rocprofv3 (the program directly after ``--``), reads the
rocpd SQLite databases it writes, and produces short text summaries plus
``traffic.json`` (measured bytes per launch of each workload's fused kernel,
keyed by workload, stamped with the hash of the kernel sources).

Passes (each its own rocprofv3 run; counters never share a run with tracing):
  trace  ``--kernel-trace --stats``: average duration of every kernel.
  fetch  ``--pmc FETCH_SIZE``  (KiB per dispatch, L2 <-> fabric reads)
  write  ``--pmc WRITE_SIZE``  (KiB per dispatch, L2 <-> fabric writes)
  mfma   ``--pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE``
The byte counters are calibrated on the same run: bench.py first copies a
buffer of known size on the device, and the ratio of known to counted bytes
for that copy scales the fused kernel's counts.

With --widened-rows it instead traces one whole bench.py run (headline workload and the
widened rows: QKV split store, GELU-erf epilogue, FFN, ResNet stem and stage, with their
unfused comparisons) and writes the per-kernel averages to kernels__widened_rows.md.

Usage (on a machine with the GPU):
  python -m dl_fusion_amd.rocprof --workloads 1 2 3 4 --out profiles --scratch /tmp/rocprof
  python -m dl_fusion_amd.rocprof --widened-rows --out profiles --scratch /tmp/rocprof
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import shutil
import sqlite3
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

COPY_MIB = 256
PYTHON = os.path.realpath(sys.executable)   # the interpreter itself, not a launcher
PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "mfma": ["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
}


def fused_kernel(wl) -> str:
    """Name fragment of the kernel the library runs for workload wl's fused layer."""
    if wl.kind == "conv":
        if wl.dtype == "f32":
            k = wl.kh * wl.kw * wl.cin
            return "conv_f32_regw_kernel" if wl.cin % 4 == 0 and 0 < k <= 256 else "conv_f32_kernel"
        # the routes of the library's halo plan, in its order
        if (wl.kh, wl.kw, wl.stride, wl.pad) != (3, 3, 1, 1) or wl.cout % 32 != 0:
            return "mma_kernel"
        if wl.cout % 64 == 0 and wl.cin == 64 and 32 % (wl.cout // 64) == 0 and wl.w <= 256 \
                and 3 * (wl.w + 2) * 128 <= 44 * 1024 and wl.h * wl.w * 128 < 2 ** 31:
            return "conv_halo_res_kernel"
        if wl.cin % 64 == 0 and wl.h * wl.w <= 256 and (wl.h + 2) * (wl.w + 2) * 128 <= 32 * 1024 \
                and wl.n * (wl.cout // 32) >= 128:
            return "conv_halo_img_kernel"
        if wl.cout % 64 == 0 and (wl.cin == 64 or wl.cin % 128 == 0) and wl.cin <= 1024 and wl.w <= 256:
            return "conv_halo_kernel"
    return "mma_kernel"


def shown(cmd: list[str]) -> str:
    """The command as a user re-runs it: repository paths under /root/repo, python3 by name."""
    out = []
    for c in cmd:
        if c == PYTHON:
            c = "python3"
        elif c.startswith(ROOT):
            c = "/root/repo" + c[len(ROOT):]
        out.append(c)
    return "cd /tmp && " + " ".join(out)


def timing_mode(wl) -> str:
    """The timing bench.py takes the workload's roofline from: the rotating-copy (cold) graph for
    an HBM-bound conv workload, the graph over resident inputs otherwise."""
    import bench  # noqa: E402
    fused, _ = bench.bytes_model(wl)
    hbm = fused / (bench.PEAK_HBM_GBS * 1e9) > bench.flops(wl) / (bench.PEAK_TFLOPS[wl.dtype] * 1e12)
    return "cold" if hbm and wl.kind == "conv" and wl.dtype == "bf16" else "graph"


def bench_cmd(idx: int, steps: int, extra: list[str], timing: str = "graph") -> list[str]:
    return [PYTHON, os.path.join(ROOT, "bench.py"), "--only", "--workload", str(idx),
            "--steps", str(steps), "--warmup", "2", "--no-cpu", "--no-unfused", "--timing", timing] + extra


def run(cmd: list[str], log: str, timeout: int) -> None:
    env = dict(os.environ, TMPDIR="/tmp")
    print("+ " + " ".join(cmd), flush=True)
    with open(log, "w") as f:
        p = subprocess.Popen(cmd, stdout=f, stderr=subprocess.STDOUT, cwd="/tmp", env=env,
                             start_new_session=True)
        try:
            rc = p.wait(timeout=timeout)
        except subprocess.TimeoutExpired:
            os.killpg(p.pid, 9)
            p.wait()
            raise RuntimeError(f"timed out after {timeout} s: {' '.join(cmd)} (log {log})")
    if rc != 0:
        # rocprofv3 may exit with a signal after the program finished and its results are
        # complete; accept that only if the profiled program printed its JSON line
        with open(log) as f:
            text = f.read()
        if '"metric"' not in text:
            raise RuntimeError(f"exit {rc}: {' '.join(cmd)} (log {log})")
        print(f"  (rocprofv3 exited {rc} after the program finished; results kept)", flush=True)


def bench_figure(log: str):
    """The roofline time (ms per launch, and how it was timed) that bench.py printed in its JSON
    line during a profiled run, or None if the log holds no such line."""
    with open(log) as f:
        for line in reversed(f.read().splitlines()):
            if line.startswith("{") and '"metric"' in line:
                r = json.loads(line).get("roofline") or {}
                return {"ms": r["ms"], "timing": r.get("timing", "")} if "ms" in r else None
    return None


def db_path(d: str) -> str:
    found = sorted(glob.glob(os.path.join(d, "**", "*results.db"), recursive=True))
    if not found:
        raise RuntimeError(f"no rocpd database under {d}")
    return found[-1]


def top_kernels(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, total_calls, average, total_duration, percentage from top_kernels "
                       "order by total_duration desc").fetchall()
    con.close()
    return rows


def counters(db: str):
    """{(dispatch_id, kernel_name): {counter: value summed over instances}}"""
    con = sqlite3.connect(db)
    out: dict = {}
    for disp, name, cn, val in con.execute(
            "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
        d = out.setdefault((disp, name), {})
        d[cn] = d.get(cn, 0.0) + float(val)
    con.close()
    return out


def per_kernel_avg(cnt, frag: str, name: str):
    vals = [v[name] for (disp, kn), v in cnt.items() if frag in kn and name in v]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def copy_dispatch(cnt, name: str):
    """Counter value of the calibration copy: the non-dlf dispatch with the largest count."""
    best = None
    for (disp, kn), v in cnt.items():
        if "dlf::" in kn or name not in v:
            continue
        if best is None or v[name] > best:
            best = v[name]
    return best


def kernel_hash() -> str:
    import bench  # noqa: E402  (same hash that bench.py checks)
    return bench.kernel_hash()


def widened_rows_trace(rocprof: str, out: str, scratch: str, steps: int) -> None:
    d = os.path.join(scratch, "widened_trace")
    shutil.rmtree(d, ignore_errors=True)
    prog = [PYTHON, os.path.join(ROOT, "bench.py"), "--steps", str(steps), "--warmup", "2", "--no-cpu",
            "--timing", "graph"]
    cmd = [rocprof, "--kernel-trace", "--stats", "-d", d, "-o", "t", "--"] + prog
    run(cmd, d + ".log", 600)
    rows = top_kernels(db_path(d))
    lines = ["# rocprofv3 summary: every kernel of a bench.py run (headline workload and widened rows)", "",
             f"command: `{shown(cmd)}`", "",
             "Each widened row is timed over the given steps as a captured graph, after its warmup, and "
             "so is its unfused comparison; the kernel names carry their template arguments (tile shape, "
             "column-block width and workgroups a CU of the streaming GEMM, activation, residual).", "",
             "| kernel | calls | avg us | total us | % |", "|---|---|---|---|---|"]
    for name, calls, avg, tot, pct in rows[:40]:
        lines.append(f"| `{name[:150]}` | {calls} | {avg:.3f} | {tot:.1f} | {pct:.1f} |")
    with open(os.path.join(out, "kernels__widened_rows.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote kernels__widened_rows.md", flush=True)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workloads", type=int, nargs="+", default=[1])
    ap.add_argument("--steps", type=int, default=20, help="timed launches in the trace pass")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--scratch", default="/tmp/rocprof")
    ap.add_argument("--passes", nargs="+", default=["trace", "fetch", "write", "mfma"])
    ap.add_argument("--widened-rows", action="store_true", help="trace a whole bench.py run instead")
    args = ap.parse_args()
    args.out = os.path.abspath(args.out)          # the profiler runs in /tmp
    args.scratch = os.path.abspath(args.scratch)
    rocprof = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    os.makedirs(args.out, exist_ok=True)
    os.makedirs(args.scratch, exist_ok=True)
    if args.widened_rows:
        widened_rows_trace(rocprof, args.out, args.scratch, args.steps)
        return
    traffic_file = os.path.join(args.out, "traffic.json")
    try:
        with open(traffic_file) as f:
            traffic = json.load(f)
    except (OSError, ValueError):
        traffic = {}
    khash = kernel_hash()

    for idx in args.workloads:
        wl = workloads.workload(idx)
        frag = fused_kernel(wl)
        lines = [f"# rocprofv3 summary: {frag} on {wl.name}", ""]
        res = {}
        for ps in args.passes:
            d = os.path.join(args.scratch, f"w{idx}_{ps}")
            shutil.rmtree(d, ignore_errors=True)
            if ps == "trace":
                prog = bench_cmd(idx, args.steps, [], timing_mode(wl))
                cmd = [rocprof, "--kernel-trace", "--stats", "-d", d, "-o", "t", "--"] + prog
                t0 = time.time()
                run(cmd, d + ".log", 300)
                rows = top_kernels(db_path(d))
                lines += ["## kernel trace (`--kernel-trace --stats`)", "", f"command: `{shown(cmd)}`", "",
                          "| kernel | calls | avg us | total us | % |", "|---|---|---|---|---|"]
                for name, calls, avg, tot, pct in rows[:8]:
                    lines.append(f"| `{name[:110]}` | {calls} | {avg:.3f} | {tot:.1f} | {pct:.1f} |")
                ours = [r for r in rows if "dlf::" in r[0]]
                if not ours or f"dlf::(anonymous namespace)::{frag}<" not in ours[0][0]:
                    raise SystemExit(f"workload {idx}: expected {frag} to dominate the trace, found "
                                     f"{ours[0][0] if ours else 'no library kernel'}")
                fused = [r for r in rows if frag in r[0]]
                if fused:
                    res["avg_us"] = fused[0][2]
                    res["kernel_name"] = fused[0][0]
                own = bench_figure(d + ".log")
                if own is not None and fused:
                    lines += ["", f"- bench.py's own figure in this run ({own['timing']}, HIP events on the "
                              f"launching stream): {own['ms'] * 1e3:.3f} us per launch; trace average / bench "
                              f"figure = {fused[0][2] / (own['ms'] * 1e3):.3f} (under the tracer a graph launch "
                              f"also pays the trace's own per-dispatch cost, which dominates a kernel of a few us)"]
                    res["bench_us"] = own["ms"] * 1e3
                lines.append("")
                print(f"  trace done in {time.time() - t0:.0f} s", flush=True)
            else:
                prog = bench_cmd(idx, 3, ["--eager", "--copy-calib-mb", str(COPY_MIB)])
                cmd = [rocprof, "--pmc"] + PASSES[ps] + ["-d", d, "-o", "p", "--"] + prog
                run(["timeout", "-s", "KILL", "120"] + cmd, d + ".log", 150)
                cnt = counters(db_path(d))
                res[ps + "_cmd"] = shown(["timeout", "-s", "KILL", "120"] + cmd)
                for cn in PASSES[ps]:
                    avg, n = per_kernel_avg(cnt, frag, cn)
                    res[cn] = avg
                    res[cn + "_n"] = n
                    if ps in ("fetch", "write"):
                        res[cn + "_copy"] = copy_dispatch(cnt, cn)
        # bytes per launch, calibrated on the copy (KiB counters)
        nbytes = COPY_MIB * (1 << 20)
        if res.get("FETCH_SIZE") and res.get("FETCH_SIZE_copy"):
            cal_f = nbytes / (res["FETCH_SIZE_copy"] * 1024.0)
            cal_w = nbytes / (res["WRITE_SIZE_copy"] * 1024.0) if res.get("WRITE_SIZE_copy") else None
            fetch_b = res["FETCH_SIZE"] * 1024.0 * cal_f
            write_b = res["WRITE_SIZE"] * 1024.0 * cal_w if (cal_w and res.get("WRITE_SIZE")) else None
            m, n, k = wl.gemm_mnk
            out_bytes = m * n * {"f32": 4, "bf16": 2, "fp8": 1}[wl.dtype]
            lines += ["## HBM bytes per launch (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`)", "",
                      f"fetch command: `{res['fetch_cmd']}`", f"write command: `{res['write_cmd']}`", "",
                      f"- calibration: a {COPY_MIB} MiB device copy counted {res['FETCH_SIZE_copy']:.0f} KiB fetched, "
                      f"{res.get('WRITE_SIZE_copy') or 0:.0f} KiB written -> factors {cal_f:.4f} / {cal_w or 0:.4f}",
                      f"- {frag}: FETCH_SIZE {res['FETCH_SIZE']:.0f} KiB, WRITE_SIZE {res.get('WRITE_SIZE') or 0:.0f} KiB "
                      f"per dispatch (average of {res['FETCH_SIZE_n']} dispatches)",
                      f"- calibrated: {fetch_b / 1e6:.3f} MB read, {(write_b or 0) / 1e6:.3f} MB written per launch",
                      f"- output tensor: {out_bytes / 1e6:.3f} MB -> writes / output = "
                      f"{(write_b or 0) / out_bytes:.3f}", ""]
            traffic[wl.name] = {"kernel": res.get("kernel_name", frag), "kernel_hash": khash,
                                "fetch_bytes": fetch_b, "write_bytes": write_b,
                                "fetch_kib_raw": res["FETCH_SIZE"], "write_kib_raw": res.get("WRITE_SIZE"),
                                "calib_fetch": cal_f, "calib_write": cal_w,
                                "write_over_output": (write_b or 0) / out_bytes,
                                "commands": [res["fetch_cmd"], res["write_cmd"]]}
        if res.get("SQ_VALU_MFMA_BUSY_CYCLES") and res.get("GRBM_GUI_ACTIVE"):
            # GRBM_GUI_ACTIVE counts on each of the 8 XCDs; MFMA busy cycles sum over 1024 SIMDs
            gui = res["GRBM_GUI_ACTIVE"] / 8.0
            util = res["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * 1024.0)
            lines += ["## MFMA busy (`--pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE`)", "",
                      f"command: `{res['mfma_cmd']}`", "",
                      f"- {frag}: SQ_VALU_MFMA_BUSY_CYCLES {res['SQ_VALU_MFMA_BUSY_CYCLES']:.4g}, GRBM_GUI_ACTIVE "
                      f"{res['GRBM_GUI_ACTIVE']:.4g} (8 XCDs) -> MFMA busy {100 * util:.1f}% of SIMD-cycles "
                      f"while the kernel ran (eager launches under counter collection)", ""]
            if wl.name in traffic:
                traffic[wl.name]["mfma_busy"] = util
        if "avg_us" in res and wl.name in traffic:
            traffic[wl.name]["trace_avg_us"] = res["avg_us"]
            if "bench_us" in res:
                traffic[wl.name]["bench_us_same_run"] = res["bench_us"]
        name = f"{frag}__{wl.name}.md"
        with open(os.path.join(args.out, name), "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"wrote {name}", flush=True)
    with open(traffic_file, "w") as f:
        json.dump(traffic, f, indent=1, sort_keys=True)
    print(f"wrote {traffic_file}", flush=True)


if __name__ == "__main__":
    main()
