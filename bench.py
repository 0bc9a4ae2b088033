#!/usr/bin/env python3
"""Benchmark of the NVFP4 + LoRA + AQN rollout hot path on one MI355X.

Workload (one "step"): a Qwen2.5-7B-shaped decode layer at token batches
M = 1, 8, 32 and 64. For each M: AQN RMSNorm (hidden 3584) -> qkv
(3584->4608); o (3584->3584); AQN RMSNorm -> gate and up (3584->18944);
down (18944->3584). Every linear is the fused W4A16 NVFP4 + LoRA forward
(r = 32, s = 2). Attention and SiLU are not part of this path, so o and down
read fresh synthetic activations. Weights are random N(0, 0.02) drawn on
the GPU, quantised by the library's own NVFP4 quantiser; 4 distinct layer
copies (4 x 131 MB) are rotated so that the 256 MB Infinity Cache cannot
serve a repeat and the weight stream comes from HBM.

Printed: one JSON line. ``value`` is decode weight GB/s over the whole step
(NVFP4 bytes of all linears / step time). ``roofline`` is for the dominant
kernel (the main linear kernel instantiation with the largest share of the
step), timed with HIP events around each of its launches on the stream it runs
on. ``cpu_baseline`` times the CPU oracle single-core on a fixed sample of the
same workload. Extra keys report the prefill GEMM (M = 8192) TFLOP/s, the
quantiser and the AQN RMSNorm bandwidth.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0         # MI355X dense fp8 MFMA, published
TOKENS = (1, 8, 32, 64)
RANK = 32
RANK_32B = 64
LORA_SCALE = 2.0
SIGMA, EPS = 1e-2, 1e-6
COPIES = 4
PREFILL_M = 8192
METRIC = "FP4+LoRA linear: decode weight GB/s, prefill TFLOP/s, % of roofline"


def nvfp4_bytes(n, k):
    return n * k // 2 + n * k // 16 + 4


def main_kernel_bytes(m, n, k, r):
    """Algorithmic bytes of one linear launch (up to 128 tokens one launch also makes t = s x A^T):
    weights, A, B, x in, y out."""
    return nvfp4_bytes(n, k) + 2 * r * k + 2 * n * r + 2 * m * k + 2 * m * n


def linear_flops(m, n, k, r):
    return 2 * m * n * k + 2 * m * r * (k + n)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip prefill / quantiser / AQN extra timings")
    p.add_argument("--backward-only", action="store_true",
                   help="time only the LoRA backward of the 7B layer at 8192 tokens (--steps passes)")
    p.add_argument("--gate-up-only", action="store_true", help="time only the gate/up + SiLU extra and exit")
    p.add_argument("--fp8-only", action="store_true",
                   help="time only the FP8 (E4M3) linears of the 7B layer: decode 1..64 tokens and the prefill")
    p.add_argument("--prefill-only", action="store_true",
                   help="time only the 7B layer's five linears at 8192 tokens (for counter runs)")
    p.add_argument("--decode32b-only", action="store_true",
                   help="time only the 32B decode pass at 128 tokens (for counter runs)")
    p.add_argument("--layers32b", type=int, default=64, help="layers of the 32B decode pass")
    p.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_DIR", "WORKLOAD"),
                   help="no GPU work: summarise a rocprofv3 --pmc run of the MFMA counters into "
                        "profiles/mfma_counters.json")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="first run a plain device-to-device copy of this many MiB three times (the reference "
                        "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script into "
                        "profiles/pmc_traffic.json")
    p.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT_MD"),
                   help="no GPU work: summarise a rocprofv3 --kernel-trace --stats run of this script")
    p.add_argument("--command", default="", help="command line recorded in a summary")
    return p.parse_args()


# --------------------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(target_s: float):
    """The oracle as it stands, one thread on one core, on a fixed row sample of the step."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import aqn, linear, nvfp4
    from workloads import QWEN25_7B, activations_bf16, lora_bf16, normal_f32

    frac = 16  # every linear keeps 1/16 of its output rows
    prep = []
    for name, (n, k) in QWEN25_7B.items():
        rows = n // frac
        w = normal_f32((rows, k), 0.02, 7000 + len(prep))
        codes, scales, st = nvfp4.quantize(w)
        a, b = lora_bf16(RANK, k, rows, 7100 + len(prep))
        prep.append((name, rows, k, codes, scales, st, a, b))
    xs = {m: activations_bf16(m, 3584, 7200 + m) for m in TOKENS}
    xd = {m: activations_bf16(m, 18944, 7300 + m) for m in TOKENS}
    wnorm = np.ones(3584, np.float32)

    def one_pass():
        wbytes = 0
        for m in TOKENS:
            h, _ = aqn.aqn_rmsnorm(xs[m], wnorm, SIGMA, 1, 0, 0, EPS)
            for name, rows, k, codes, scales, st, a, b in prep:
                x = xd[m] if name == "down" else xs[m]
                linear.lora_linear(x, codes, scales, st, a, b, LORA_SCALE)
                wbytes += nvfp4_bytes(rows, k)
        return wbytes

    affinity = os.sched_getaffinity(0)
    core = min(affinity)
    os.sched_setaffinity(0, {core})
    try:
        with threadpool_limits(limits=1):
            total_b, t0 = 0, time.perf_counter()
            passes = 0
            while True:
                total_b += one_pass()
                passes += 1
                el = time.perf_counter() - t0
                if el >= target_s or (passes >= 1 and el * (passes + 1) / passes > 2 * target_s):
                    break
    finally:
        os.sched_setaffinity(0, affinity)
    gbs = total_b / el / 1e9
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": 1, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"1/{frac} of every linear's output rows (qkv, o, gate, up, down), all of M = "
                      f"{list(TOKENS)}, AQN RMSNorm on the full token rows; {passes} pass(es) in {el:.1f} s "
                      f"on one core ({os.cpu_count()} visible)"}


# --------------------------------------------------------------------------- GPU workload

def build_layer(torch, fr, dev, shapes, seed):
    layer = {}
    fp32 = {}
    for i, (name, (n, k)) in enumerate(shapes.items()):
        g = torch.Generator(device=dev)
        g.manual_seed(seed * 100 + i)
        w = torch.randn((n, k), generator=g, device=dev, dtype=torch.float32).mul_(0.02)
        layer[name] = fr.nvfp4_quantize(w)
        fp32[name] = w
    return layer, fp32


PMC_TRAFFIC = os.path.join(ROOT, "profiles", "fp4_lora_linear_qwen25_7b_decode_pmc_traffic.json")
MFMA_COUNTERS = os.path.join(ROOT, "profiles", "mfma_counters.json")
KERNEL_SOURCES = ("linear.hip", "device.hpp", "launch.hpp")
MFMA_SOURCES = ("linear.hip", "device.hpp", "launch.hpp", "backward.hip", "gemm_nt.hpp")
MFMA_PMC = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA",
            "SQ_INSTS_VALU", "SQ_BUSY_CU_CYCLES")
SIMDS = 1024  # 256 CUs x 4 SIMDs
XCDS = 8      # GRBM_GUI_ACTIVE comes summed over the XCDs' graphics blocks (the busy time is the per-XCD value)


def kernel_source_sha(files=KERNEL_SOURCES):
    """Hash of the kernel sources: counter readings are void once these change."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "fp4_quantized_rl_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def mfma_roofline(achieved_tflops, kernels, workload=None):
    """The roofline block of an MFMA-bound extra: achieved vs the dense bf16 peak, with the MFMA busy
    fraction of its main kernels from the committed counter summary when that is current."""
    out = {"bound": "mfma", "achieved": round(achieved_tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": round(achieved_tflops / BF16_PEAK_TFLOPS, 4), "mfma_busy": None}
    if os.path.exists(MFMA_COUNTERS):
        with open(MFMA_COUNTERS) as fh:
            rec = json.load(fh)
        if rec.get("kernel_source_sha") == kernel_source_sha(MFMA_SOURCES):
            busy = {k: v["mfma_busy"] for k, v in rec.get("kernels", {}).items()
                    if any(same_kernel(v.get("kernel", k), name) for name in kernels)
                    and (workload is None or v.get("workload") == workload)}
            out["mfma_busy"] = busy or None
    return out


def summarize_mfma(pmc_dir, workload, command):
    """MFMA busy fraction and bf16 MFMA ops per dispatch of every library kernel in a rocprofv3 --pmc run."""
    import csv
    import glob
    rows = {}
    for f in sorted(glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id", "")))
                rows.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    if not rows:
        raise SystemExit(f"no counter rows under {pmc_dir}")
    per = {}
    for (kname, _), c in rows.items():
        if not all(n in c for n in MFMA_PMC):
            continue
        short = short_kernel_name(kname)
        if not any(t in short for t in ("prefill_kernel", "splitk_kernel", "mid_kernel", "nt_gemm_kernel",
                                          "skinny_kernel", "gemv_kernel", "fp8_decode_kernel",
                                          "e4m3_decode_kernel", "gate_up_kernel")):
            continue
        d = per.setdefault(short, {"dispatches": 0, "busy": 0.0, "gui": 0.0, "mops": 0.0, "mfma": 0.0,
                                   "valu": 0.0, "busy_cu": 0.0})
        d["dispatches"] += 1
        d["busy"] += c["SQ_VALU_MFMA_BUSY_CYCLES"]
        d["gui"] += c["GRBM_GUI_ACTIVE"]
        d["mops"] += c["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
        d["mfma"] += c["SQ_INSTS_MFMA"]
        d["valu"] += c["SQ_INSTS_VALU"]
        d["busy_cu"] += c["SQ_BUSY_CU_CYCLES"]
    kernels = {}
    for k, d in sorted(per.items()):
        n = d["dispatches"]
        kernels[f"{k} @ {workload}"] = {"kernel": k, "workload": workload, "dispatches": n,
                      "mfma_busy": round(d["busy"] * XCDS / (d["gui"] * SIMDS), 4) if d["gui"] else None,
                      "bf16_mfma_flops_per_dispatch": d["mops"] * 512 / n,
                      "mfma_instructions_per_dispatch": d["mfma"] / n,
                      "valu_per_mfma": round(d["valu"] / d["mfma"], 2) if d["mfma"] else None,
                      "gpu_active_cycles_per_dispatch": d["gui"] / n}
    rec = {"what": "rocprofv3 --pmc " + " ".join(MFMA_PMC) + ", per dispatch, summed over each kernel's "
                   "dispatches; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) "
                   "(the counter file sums GRBM_GUI_ACTIVE over the 8 XCDs: its eighth at ~2.3 GHz matches the "
                   "kernel-trace durations); bf16 MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512",
           "command": command, "kernel_source_sha": kernel_source_sha(MFMA_SOURCES), "kernels": kernels}
    old = {}
    if os.path.exists(MFMA_COUNTERS):
        with open(MFMA_COUNTERS) as fh:
            old = json.load(fh)
    if old.get("kernel_source_sha") == rec["kernel_source_sha"]:  # merge runs of the same sources
        merged = dict(old.get("kernels", {}))
        merged.update(kernels)
        rec["kernels"] = merged
        rec["command"] = old.get("command", "") + " ;\n" + command
    with open(MFMA_COUNTERS, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec, indent=1))


def short_kernel_name(full):
    """'void fp4rl::(anonymous namespace)::gemv_kernel<1, 8, 8>(...)' -> 'gemv_kernel<1, 8, 8>'."""
    full = full.replace("(anonymous namespace)::", "")
    depth, end = 0, len(full)
    for i, ch in enumerate(full):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            end = i
            break
    s = full[:end]
    if s.startswith("void "):
        s = s[5:]
    return s.rsplit("::", 1)[-1].strip()


def same_kernel(short, name):
    """A library kernel name may omit trailing defaulted template arguments."""
    return short == name or (name.endswith(">") and short.startswith(name[:-1] + ","))


def traffic_from_profile(kernel_name):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it is current."""
    if not os.path.exists(PMC_TRAFFIC):
        return None
    with open(PMC_TRAFFIC) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    ent = rec.get("kernels", {}).get(kernel_name)
    return None if not ent else ent.get("hbm_bytes_per_launch")


def _read_counters(d, counter):
    """Per-dispatch values of one counter from a rocprofv3 --pmc csv run: [(kernel, value)]."""
    import csv
    import glob
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not out:
        raise SystemExit(f"no {counter} rows under {d}")
    return out


def summarize_pmc(fetch_dir, write_dir, copy_mib, command):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of every library kernel, scaled by a plain copy's reading."""
    import fp4_quantized_rl_amd as fr
    fetch, write = _read_counters(fetch_dir, "FETCH_SIZE"), _read_counters(write_dir, "WRITE_SIZE")
    known = copy_mib * 2**20
    if known <= 0:
        raise SystemExit("--copy-calibration-mib must give the calibration copy size")

    def copy_kib(rows):
        vals = [v for k, v in rows if "copyBuffer" in k and v * 1024 > 0.5 * known]
        if not vals:
            raise SystemExit("calibration copy dispatches not found")
        return sum(vals) / len(vals)

    cf, cw = copy_kib(fetch), copy_kib(write)
    ff, wf = cf * 1024 / known, cw * 1024 / known
    from workloads import QWEN25_7B
    names = sorted({fr.fp4_linear_kernel_name(m, n, k, RANK) for m in TOKENS for n, k in QWEN25_7B.values()})
    kernels = {}
    for name in names:
        fv = [v for k, v in fetch if same_kernel(short_kernel_name(k), name)]
        wv = [v for k, v in write if same_kernel(short_kernel_name(k), name)]
        if not fv or not wv:
            continue
        fa, wa = sum(fv) / len(fv), sum(wv) / len(wv)
        kernels[name] = {"dispatches": len(fv), "fetch_kib_avg": round(fa, 1), "write_kib_avg": round(wa, 1),
                         "hbm_bytes_per_launch": int(fa * 1024 / ff + wa * 1024 / wf)}
    rec = {"what": "rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of bench.py, per dispatch of each main linear "
                   "kernel, averaged over that kernel's dispatches and divided by the factor a plain device copy "
                   "of known size reads (counter KiB x 1024 / true bytes)",
           "command": command, "kernel_source_sha": kernel_source_sha(),
           "copy_calibration": {"bytes": known, "fetch_kib": round(cf, 1), "write_kib": round(cw, 1),
                                "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "kernels": kernels}
    with open(PMC_TRAFFIC, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec, indent=1))


def summarize_trace(trace_dir, out_md, command):
    """Markdown table from a rocprofv3 --kernel-trace --stats run: library kernels and their durations."""
    import csv
    import glob
    stats = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True))
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = []
    with open(stats[0], newline="") as fh:
        for r in csv.DictReader(fh):
            rows.append((short_kernel_name(r["Name"]), int(r["Calls"]), float(r["TotalDurationNs"]),
                         float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]), float(r["Percentage"])))
    rows.sort(key=lambda t: -t[2])
    # dispatches in runs of at least RUN back-to-back dispatches of the same
    # kernel and grid: the per-kernel timing graphs (dozens of launches over
    # weight copies), which the events in the JSON line bracket; a layer pass
    # never repeats one kernel and grid that often
    RUN = 8
    b2b = {}
    traces = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
    if traces:
        with open(traces[0], newline="") as fh:
            tr = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))
        key = [(r["Kernel_Name"], r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"]) for r in tr]
        i = 0
        while i < len(tr):
            j = i
            while j + 1 < len(tr) and key[j + 1] == key[i]:
                j += 1
            if j - i + 1 >= RUN:
                lst = b2b.setdefault(short_kernel_name(tr[i]["Kernel_Name"]), [])
                lst.extend(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tr[i:j + 1])
            i = j + 1
    lines = ["# rocprofv3 kernel trace: " + os.path.basename(out_md).rsplit(".", 1)[0], "",
             "Command (from the repository root):", "", "```", command, "```", "",
             "'back to back' averages only the dispatches in runs of at least 8 consecutive dispatches of the "
             "same kernel and grid: the per-kernel timing graphs whose HIP-event average the JSON line reports.",
             "",
             "| kernel | calls | total ms | avg us | min us | max us | % of GPU time | back-to-back calls | "
             "back-to-back avg us |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for name, calls, tot, avg, mn, mx, pct in rows[:25]:
        bb = b2b.get(name, [])
        bbs = f"{len(bb)} | {sum(bb) / len(bb) / 1e3:.2f}" if bb else "0 | -"
        lines.append(f"| `{name}` | {calls} | {tot / 1e6:.3f} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} "
                     f"| {pct:.2f} | {bbs} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def median_time(torch, fn):
    """Median time of fn() over separate runs, each bracketed by HIP events on the current stream (every
    library call runs there): at least 50 runs, or 10 when one run takes over 10 ms. Returns (s, runs)."""
    import statistics
    fn()
    torch.cuda.synchronize()
    times = []
    while True:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
        need = 10 if statistics.median(times) > 10e-3 else 50
        if len(times) >= need:
            return statistics.median(times), len(times)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_calibration(torch, dev, mib):
    """A plain device-to-device copy of known size, the yardstick for the traffic counters."""
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    args = parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.copy_calibration_mib, args.command)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.command)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, args.command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline:
        progress("cpu oracle baseline")
        cpu = cpu_baseline(args.cpu_seconds)

    import torch

    import fp4_quantized_rl_amd as fr
    from workloads import QWEN25_7B

    fr.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration_mib > 0:
        copy_calibration(torch, dev, args.copy_calibration_mib)
    shapes = QWEN25_7B
    hidden = 3584
    inter = 18944

    progress("building weights")
    # weights: COPIES distinct NVFP4 layers, shared LoRA adapters, AQN weights
    layers = []
    for c in range(COPIES):
        layer, fp32 = build_layer(torch, fr, dev, shapes, seed=1 + c)
        layers.append(layer)
        del fp32
    torch.cuda.synchronize()
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    lora = {}
    for name, (n, k) in shapes.items():
        a = torch.randn((RANK, k), generator=g, device=dev).mul_(0.01).to(torch.bfloat16)
        b = torch.randn((n, RANK), generator=g, device=dev).mul_(0.01).to(torch.bfloat16)
        lora[name] = (a, b)
    wnorm = torch.ones(hidden, dtype=torch.float32, device=dev)
    if args.fp8_only:
        progress("FP8 linear timing")
        gb = torch.Generator(device=dev)
        gb.manual_seed(21)
        xs = {k: torch.randn((PREFILL_M, k), generator=gb, device=dev).to(torch.bfloat16)
              for k in sorted({k for _, k in shapes.values()})}
        print(json.dumps({"fp8_linear": run_fp8(torch, fr, dev, shapes, lora, xs, gb)}))
        return
    if args.gate_up_only:
        progress("gate/up + SiLU timing")
        gg = torch.Generator(device=dev).manual_seed(21)
        print(json.dumps({"gate_up_silu": run_gate_up(torch, fr, dev, shapes, layers, lora, gg),
                          "aqn_qkv_fold": run_qkv_fold(torch, fr, dev, shapes, layers, lora, gg)}))
        return
    if args.decode32b_only:
        progress(f"32B decode pass, {args.layers32b} layers")
        print(json.dumps({"decode_32b": run_decode_32b(torch, fr, dev, layers=args.layers32b)}))
        return
    if args.prefill_only:
        progress("prefill timing")
        print(json.dumps({"prefill": run_prefill(torch, fr, dev, shapes, layers[0], lora,
                                                 torch.Generator(device=dev).manual_seed(21))[0]}))
        return
    if args.backward_only:
        progress("LoRA backward timing")
        gb = torch.Generator(device=dev)
        gb.manual_seed(21)
        xs = {k: torch.randn((PREFILL_M, k), generator=gb, device=dev).to(torch.bfloat16)
              for k in sorted({k for _, k in shapes.values()})}
        print(json.dumps({"lora_backward": run_backward(torch, fr, dev, shapes, layers[0], lora, xs, gb)}))
        return

    # activations and preallocated outputs / workspaces per token count
    bufs = {}
    for m in TOKENS:
        xh = torch.randn((m, hidden), generator=g, device=dev).to(torch.bfloat16)
        xo = torch.randn((m, hidden), generator=g, device=dev).to(torch.bfloat16)
        xr = torch.randn((m, hidden), generator=g, device=dev).to(torch.bfloat16)
        xd = torch.randn((m, inter), generator=g, device=dev).to(torch.bfloat16)
        bufs[m] = {
            "xh": xh, "xo": xo, "xr": xr, "xd": xd,
            "h1": torch.empty_like(xh), "h2": torch.empty_like(xr),
            "ws": {name: fr.linear_workspace(fr.fp4_lora_linear_workspace_bytes(m, n, k, RANK), dev)
                   for name, (n, k) in shapes.items()},
            "y": {name: torch.empty((m, n), dtype=torch.bfloat16, device=dev) for name, (n, k) in shapes.items()},
        }
    weight_bytes_step = sum(nvfp4_bytes(n, k) for n, k in shapes.values()) * len(TOKENS)
    flops_step = sum(linear_flops(m, n, k, RANK) for m in TOKENS for n, k in shapes.values())
    total_bytes_step = 0
    for m in TOKENS:
        total_bytes_step += 2 * (4 * m * hidden + 4 * hidden)  # two norms: x in, y out (+ w)
        for n, k in shapes.values():
            total_bytes_step += nvfp4_bytes(n, k) + 2 * RANK * (k + n) + 2 * m * (k + n) + 8 * m * RANK

    def layer_input(B, name):
        return B["h1"] if name == "qkv" else B["xo"] if name == "o" else B["h2"] if name in ("gate", "up") else B["xd"]

    def step(s):
        """One pass of the hot path at every token count, on weight copy (s + i) % COPIES."""
        for mi, m in enumerate(TOKENS):
            L = layers[(s + mi) % COPIES]
            B = bufs[m]
            fr.aqn_rmsnorm(B["xh"], wnorm, SIGMA, 1, s, 0, EPS, out=B["h1"])
            fr.aqn_rmsnorm(B["xr"], wnorm, SIGMA, 1, s, 1, EPS, out=B["h2"])
            for name in ("qkv", "o", "gate", "up", "down"):
                a, b = lora[name]
                fr.fp4_lora_linear(layer_input(B, name), L[name], a, b, LORA_SCALE, out=B["y"][name],
                                   workspace=B["ws"][name])

    progress("warmup")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    # The step is launch-bound at small M, so it runs as HIP graphs: one per
    # weight-copy rotation phase, captured once, replayed in the timed region.
    graphs = []
    for p in range(COPIES):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step(p)
        graphs.append(gr)
    for s in range(args.warmup):
        graphs[s % COPIES].replay()
    torch.cuda.synchronize()

    progress("timed steps")
    t0 = time.perf_counter()
    for s in range(args.steps):
        graphs[s % COPIES].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = weight_bytes_step * args.steps / elapsed / 1e9
    del graphs

    # Per-kernel durations: for each (M, linear) a graph of back-to-back linear
    # launches (the fused launch the step runs) over distinct weight buffers
    # totalling >= 512 MB (twice the Infinity Cache), bracketed by HIP events
    # on the launch stream.
    clones = {}
    for name, (n, k) in shapes.items():
        lst = [layers[c][name] for c in range(COPIES)]
        while sum(w.nbytes for w in lst) < 512 * 2**20:
            src = lst[len(lst) % COPIES]
            lst.append(src.clone())
        clones[name] = lst
    progress("per-kernel timing")
    timing, timed_launches = {}, {}
    reps = 3
    for m in TOKENS:
        B = bufs[m]
        for name, (n, k) in shapes.items():
            x = layer_input(B, name)
            a, b = lora[name]
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for w in clones[name]:
                    fr.fp4_lora_linear(x, w, a, b, LORA_SCALE, out=B["y"][name], workspace=B["ws"][name])
            gr.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                gr.replay()
            e1.record()
            torch.cuda.synchronize()
            launches = reps * len(clones[name])
            total = e0.elapsed_time(e1) * 1e-3
            timing[(m, name)] = total / launches
            timed_launches[(m, name)] = (launches, total)
            del gr
    kname = {(m, name): fr.fp4_linear_kernel_name(m, n, k, RANK) for m in TOKENS for name, (n, k) in shapes.items()}
    # share of the step: one launch per (M, linear); launch-weighted averages
    # over the timed graphs (the way a kernel trace averages its dispatches)
    per_kernel = {}
    for (m, name), dt in timing.items():
        n, k = shapes[name]
        launches, total = timed_launches[(m, name)]
        d = per_kernel.setdefault(kname[(m, name)], {"step_time": 0.0, "per_step": 0, "time": 0.0, "launches": 0,
                                                     "bytes": 0})
        d["step_time"] += dt
        d["per_step"] += 1
        d["time"] += total
        d["launches"] += launches
        d["bytes"] += launches * main_kernel_bytes(m, n, k, RANK)
    dom = max(per_kernel, key=lambda kn: per_kernel[kn]["step_time"])
    dk = per_kernel[dom]
    achieved = dk["bytes"] / dk["time"] / 1e9
    traffic = traffic_from_profile(dom)
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom, "avg_launch_us": round(dk["time"] / dk["launches"] * 1e6, 3),
                "timed_launches": dk["launches"], "launches_per_step": dk["per_step"],
                "algorithmic_bytes_per_launch": int(dk["bytes"] / dk["launches"])}

    step_roof_s = max(total_bytes_step / (HBM_PEAK_GBS * 1e9), flops_step / (BF16_PEAK_TFLOPS * 1e12))
    breakdown = {
        "step_roofline_frac": round(step_roof_s / (ms_per_step * 1e-3), 4),
        "main_kernel_us": {f"M{m}/{name}": round(timing[(m, name)] * 1e6, 2) for m in TOKENS for name in shapes},
        "main_kernel_weight_gbs": {f"M{m}/{name}": round(nvfp4_bytes(*shapes[name]) / timing[(m, name)] / 1e9, 1)
                                   for m in TOKENS for name in shapes},
        "main_kernels_share_of_step": round(sum(timing.values()) / (ms_per_step * 1e-3), 4),
        "kernels": {kn: {"avg_us": round(v["time"] / v["launches"] * 1e6, 3), "launches_per_step": v["per_step"],
                         "GB/s": round(v["bytes"] / v["time"] / 1e9, 1)} for kn, v in sorted(per_kernel.items())},
    }
    del clones

    extras = {}
    if not args.no_extras:
        progress("prefill, quantiser and AQN timings")
        extras = run_extras(torch, fr, dev, shapes, layers, lora, None)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Qwen2.5-7B-shaped decode layer: AQN RMSNorm x2 + qkv 3584->4608, "
                               "o 3584->3584, gate/up 3584->18944, down 18944->3584 as NVFP4 W4A16 + LoRA",
                   "tokens_per_pass": list(TOKENS), "lora_rank": RANK, "lora_scale": LORA_SCALE,
                   "weight_copies_rotated": COPIES, "nvfp4_weight_bytes_per_step": weight_bytes_step,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "breakdown": breakdown,
    }
    out.update(extras)
    print(json.dumps(out))


def run_prefill(torch, fr, dev, shapes, layer, lora, g):
    """The 7B layer's five linears at M = 8192 tokens (16 x 512) with 0.1% outlier channels x20."""
    xs = {}
    for k in sorted({k for _, k in shapes.values()}):
        x = torch.randn((PREFILL_M, k), generator=g, device=dev)
        nout = round(0.001 * k)
        ch = torch.randperm(k, generator=g, device=dev)[:nout]
        x[:, ch] *= 20.0
        xs[k] = x.to(torch.bfloat16)
    ys = {name: torch.empty((PREFILL_M, n), dtype=torch.bfloat16, device=dev) for name, (n, k) in shapes.items()}
    pws = fr.linear_workspace(max(fr.fp4_lora_linear_workspace_bytes(PREFILL_M, n, k, RANK)
                                  for n, k in shapes.values()), dev)

    def prefill_pass():
        for name, (n, k) in shapes.items():
            a, b = lora[name]
            fr.fp4_lora_linear(xs[k], layer[name], a, b, LORA_SCALE, out=ys[name], workspace=pws)

    dt, runs = median_time(torch, prefill_pass)
    flops = sum(linear_flops(PREFILL_M, n, k, RANK) for n, k in shapes.values())
    del ys
    return ({"M": PREFILL_M, "tflops": round(flops / dt / 1e12, 2), "ms_per_layer": round(dt * 1e3, 3),
             "frac_of_bf16_peak": round(flops / dt / 1e12 / BF16_PEAK_TFLOPS, 4), "timing": f"median of {runs}",
             "roofline": mfma_roofline(flops / dt / 1e12, ("prefill_kernel<2>",), "7B prefill 8192 tokens")}, xs)


def run_extras(torch, fr, dev, shapes, layers, lora, fp32):
    layer = layers[0]
    res = {}
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    res["prefill"], xs = run_prefill(torch, fr, dev, shapes, layer, lora, g)
    res["lora_backward"] = run_backward(torch, fr, dev, shapes, layer, lora, xs, g)
    res["fp8_linear"] = run_fp8(torch, fr, dev, shapes, lora, xs, g)
    res["gate_up_silu"] = run_gate_up(torch, fr, dev, shapes, layers, lora, g)
    res["aqn_qkv_fold"] = run_qkv_fold(torch, fr, dev, shapes, layers, lora, g)
    del xs

    # quantiser on 14B shapes: one layer's five matrices, 0.02 t(3) weights with
    # 1e-4 outliers x50, fp32 (and bf16) input -> NVFP4; the 48 layers repeat
    # these shapes, so the 48-layer time is this layer's time x 48
    from workloads import QWEN25_14B, student_t3_weights_torch, tensor_seed
    del fp32
    w14 = {name: student_t3_weights_torch((n, k), tensor_seed(4, 0, name), dev) for name, (n, k) in QWEN25_14B.items()}
    params = sum(n * k for n, k in QWEN25_14B.values())
    for dt in ("fp32", "bf16"):
        ws = w14 if dt == "fp32" else {name: w.to(torch.bfloat16) for name, w in w14.items()}
        outs = {name: fr.nvfp4_quantize(w) for name, w in ws.items()}
        torch.cuda.synchronize()

        def quantize_layer():
            for name, w in ws.items():
                fr.nvfp4_quantize(w, out=outs[name])

        dt_s, runs = median_time(torch, quantize_layer)
        esz = 4 if dt == "fp32" else 2
        two_pass = params * (2 * esz + 0.5625)
        res[f"quantize_{dt}"] = {"shapes": "Qwen2.5-14B layer (qkv 7168x5120, o 5120x5120, gate/up 13824x5120, "
                                           "down 5120x13824), 0.02 t(3) + 1e-4 outliers x50",
                                 "params_per_layer": params, "ms_per_layer": round(dt_s * 1e3, 3),
                                 "ms_48_layers": round(dt_s * 48e3, 2),
                                 "GB/s_two_pass": round(two_pass / dt_s / 1e9, 1),
                                 "frac_of_hbm": round(two_pass / dt_s / 1e9 / HBM_PEAK_GBS, 4),
                                 "timing": f"median of {runs}"}
        if dt == "fp32":
            # the same pass also writing the rounding record (1 bit per weight)
            recs = {name: torch.empty((w.shape[0], w.shape[1] // 8), dtype=torch.uint8, device=dev)
                    for name, w in ws.items()}
            def quantize_layer_record():
                for name, w in ws.items():
                    fr.nvfp4_quantize(w, out=outs[name], round_up=recs[name])

            dt_r, _ = median_time(torch, quantize_layer_record)
            rec_bytes = two_pass + params / 8
            res["quantize_fp32_with_rounding_record"] = {
                "ms_per_layer": round(dt_r * 1e3, 3), "GB/s_two_pass": round(rec_bytes / dt_r / 1e9, 1),
                "frac_of_hbm": round(rec_bytes / dt_r / 1e9 / HBM_PEAK_GBS, 4),
                "record_bytes_per_layer": params // 8}
            del recs
        del outs
        if dt == "bf16":
            del ws
    del w14
    # AQN RMSNorm: 65536 x 5120 bf16 tokens
    m, d = 65536, 5120
    x = torch.randn((m, d), generator=g, device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    w = torch.ones(d, dtype=torch.float32, device=dev)
    sigmas = [fr.aqn_sigma(1e-2, 5e-4, kk, 10) for kk in range(10)]
    stage = [0]

    def aqn_call():  # the ten stages of the schedule in turn
        kk = stage[0] % 10
        stage[0] += 1
        fr.aqn_rmsnorm(x, w, sigmas[kk], 4, kk, 0, EPS, out=y)

    dt, runs = median_time(torch, aqn_call)
    res["aqn_rmsnorm"] = {"shape": [m, d], "us_per_call": round(dt * 1e6, 2), "timing": f"median of {runs}",
                          "GB/s": round(4 * m * d / dt / 1e9, 1), "frac_of_hbm": round(4 * m * d / dt / 1e9 / HBM_PEAK_GBS, 4)}
    del x, y
    res["decode_32b"] = run_decode_32b(torch, fr, dev)
    return res


def run_backward(torch, fr, dev, shapes, layer, lora, xs, g):
    """Backward through the frozen base (the training half of the step): the
    layer's five linears and adapters, M = 8192 tokens, dY ~ N(0, 0.05^2);
    dX, dA and dB of every linear per pass."""
    dys = {name: (torch.randn((PREFILL_M, n), generator=g, device=dev) * 0.05).to(torch.bfloat16)
           for name, (n, k) in shapes.items()}
    bws = torch.empty(max(fr.fp4_lora_linear_backward_workspace_bytes(PREFILL_M, n, k, RANK)
                          for n, k in shapes.values()), dtype=torch.uint8, device=dev)

    def backward_pass():
        for name, (n, k) in shapes.items():
            a, b = lora[name]
            fr.fp4_lora_linear_backward(dys[name], xs[k], layer[name], a, b, LORA_SCALE, workspace=bws)

    dt, runs = median_time(torch, backward_pass)
    # dX base 2MNK; LoRA: t and dA 2MrK each, h and dB 2MNr each, the dX LoRA term 2MrK
    bflops = sum(2 * PREFILL_M * n * k + 2 * PREFILL_M * RANK * (3 * k + 2 * n) for n, k in shapes.values())
    return {"M": PREFILL_M, "r": RANK, "tflops": round(bflops / dt / 1e12, 2), "ms_per_layer": round(dt * 1e3, 3),
            "frac_of_bf16_peak": round(bflops / dt / 1e12 / BF16_PEAK_TFLOPS, 4), "timing": f"median of {runs}",
            "workspace_GB": round(bws.numel() / 1e9, 3),
            "roofline": mfma_roofline(bflops / dt / 1e12, ("nt_gemm_kernel<true, 1, 0>",),
                                      "7B LoRA backward 8192 tokens")}


def run_fp8(torch, fr, dev, shapes, lora, xs, g):
    """FP8 (E4M3, per-row scale) rollout linears of the same 7B layer and
    adapters, W8A16 and W8A8 (tokens quantised per row inside the call):
    decode at 1, 8, 32, 64 tokens (FP8 weight GB/s; replays of one captured
    graph over two weight copies, like the other decode timings) and the 8192-token
    prefill (TFLOP/s; W8A8 against the dense FP8 peak, its base product
    running on the FP8 matrix cores)."""
    w8 = {name: fr.fp8_quantize(torch.randn((n, k), generator=g, device=dev).mul_(0.02))
          for name, (n, k) in shapes.items()}
    # decode: a second copy of the weights, so one graph replay over both streams 466 MB, more than the
    # Infinity Cache holds
    w8b = {name: fr.FP8Weight(q.codes.clone(), q.scales.clone()) for name, q in w8.items()}
    wbytes = sum(n * k + 4 * n for n, k in shapes.values())
    out = {}
    for m in TOKENS + (PREFILL_M,):
        xm = xs if m == PREFILL_M else {k: torch.randn((m, k), generator=g, device=dev).to(torch.bfloat16)
                                       for k in {k for _, k in shapes.values()}}
        ys = {name: torch.empty((m, n), dtype=torch.bfloat16, device=dev) for name, (n, k) in shapes.items()}
        for a8 in (False, True):
            wss = {name: torch.empty(max(fr.fp8_lora_linear_workspace_bytes(m, n, k, RANK, w8a8=a8), 256),
                                     dtype=torch.uint8, device=dev) for name, (n, k) in shapes.items()}

            def layer(ws8):
                def one():
                    for name, (n, k) in shapes.items():
                        a, b = lora[name]
                        fr.fp8_lora_linear(xm[k], ws8[name], a, b, LORA_SCALE, out=ys[name], workspace=wss[name],
                                           w8a8=a8)
                return one

            if m == PREFILL_M:
                dt, runs = median_time(torch, layer(w8))
            else:  # replays of one captured graph over both weight copies (no host gaps between launches)
                dt, runs = graph_call_time(torch, [layer(w8), layer(w8b)])
            flops = sum(linear_flops(m, n, k, RANK) for n, k in shapes.values())
            tag = "w8a8_" if a8 else ""
            if m == PREFILL_M:
                peak_key, peak = ("frac_of_fp8_peak", FP8_PEAK_TFLOPS) if a8 else ("frac_of_bf16_peak",
                                                                                   BF16_PEAK_TFLOPS)
                out[tag + "prefill"] = {"M": m, "ms_per_layer": round(dt * 1e3, 3),
                                        "tflops": round(flops / dt / 1e12, 2),
                                        peak_key: round(flops / dt / 1e12 / peak, 4), "timing": f"median of {runs}"}
            else:
                out[f"{tag}decode_M{m}"] = {"us_per_layer": round(dt * 1e6, 1),
                                            "weight_GB/s": round(wbytes / dt / 1e9, 1),
                                            "frac_of_hbm": round(wbytes / dt / 1e9 / HBM_PEAK_GBS, 4),
                                            "timing": f"median of {runs} replays of one graph over 2 weight copies"}
            del wss
        del ys
    return out


def graph_call_time(torch, calls):
    """Median time of one call among `calls` (closures over distinct weights), run back to back as one
    captured HIP graph: no host gaps between launches, and the weights rotate through more bytes than the
    Infinity Cache holds. Returns (s per call, replays)."""
    for c in calls:
        c()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for c in calls:
            c()
    dt, runs = median_time(torch, gr.replay)
    del gr
    return dt / len(calls), runs


def run_gate_up(torch, fr, dev, shapes, layers, lora, g):
    """The 7B layer's gate and up projections with the SiLU-gated product
    (fp4_gate_up_silu: one fused launch up to 16 tokens, two linears and the
    product above) at 1, 8, 32, 64 and 128 tokens, beside the two separate
    linears alone (which write gate and up and apply no SiLU), and the AQN
    RMSNorm folded into the fused launch beside the norm launch followed by
    fp4_gate_up_silu. Each variant runs over every weight copy as one graph;
    every call gets a preallocated workspace."""
    n, k = shapes["gate"]
    wbytes = 2 * nvfp4_bytes(n, k)
    lib = fr.load_library()
    out = {}
    for m in TOKENS + (128,):
        x = torch.randn((m, k), generator=g, device=dev).to(torch.bfloat16)
        h = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        need = fr.fp4_lora_linear_workspace_bytes(m, n, k, RANK)
        wsa, wsb = fr.linear_workspace(need, dev), fr.linear_workspace(need, dev)
        ya, yb = torch.empty_like(h), torch.empty_like(h)
        gws = torch.zeros(max(256, fr.fp4_gate_up_silu_workspace_bytes(m, n, k, RANK)), dtype=torch.uint8,
                          device=dev)
        wn = torch.ones(k, dtype=torch.float32, device=dev)
        xn = torch.empty_like(x)
        aws = torch.empty(max(256, lib.fp4rl_aqn_gate_up_silu_workspace(m, n, k, RANK)), dtype=torch.uint8,
                          device=dev)

        def entry(L):
            return lambda: fr.fp4_gate_up_silu(x, L["gate"], L["up"], lora["gate"], lora["up"], LORA_SCALE, out=h,
                                               workspace=gws)

        def separate(L):
            def f():
                fr.fp4_lora_linear(x, L["gate"], *lora["gate"], LORA_SCALE, out=ya, workspace=wsa)
                fr.fp4_lora_linear(x, L["up"], *lora["up"], LORA_SCALE, out=yb, workspace=wsb)
            return f

        # the AQN RMSNorm folded into the fused launch (raw x in, normalised
        # tokens never stored) against the norm launch followed by the entry point
        def folded(L):
            return lambda: fr.aqn_gate_up_silu(x, wn, SIGMA, 4, 0, 1, EPS, L["gate"], L["up"], lora["gate"],
                                               lora["up"], LORA_SCALE, out=h, workspace=aws)

        def norm_then_entry(L):
            def f():
                fr.aqn_rmsnorm(x, wn, SIGMA, 4, 0, 1, EPS, out=xn)
                fr.fp4_gate_up_silu(xn, L["gate"], L["up"], lora["gate"], lora["up"], LORA_SCALE, out=h,
                                    workspace=gws)
            return f

        res = {"path": "fused" if m <= 16 else "two linears + gated product"}
        for name, mk in (("entry_us", entry), ("two_linears_us", separate), ("aqn_folded_us", folded),
                         ("aqn_then_entry_us", norm_then_entry)):
            dt, runs = graph_call_time(torch, [mk(L) for L in layers])
            res[name] = round(dt * 1e6, 1)
        res["timing"] = f"median of {runs} replays of one graph over {len(layers)} weight copies"
        res["entry_weight_GB/s"] = round(wbytes / res["entry_us"] / 1e3, 1)
        res["entry_frac_of_hbm"] = round(wbytes / res["entry_us"] / 1e3 / HBM_PEAK_GBS, 4)
        out[f"M{m}"] = res
    return out


def run_qkv_fold(torch, fr, dev, shapes, layers, lora, g):
    """The 7B layer's qkv projection with the AQN RMSNorm folded in (fp4rl_aqn_lora_linear: raw x in, the
    normalised tokens never stored) beside the norm launch followed by the linear, at 1, 8, 32, 64 and 128
    tokens; each variant runs over every weight copy as one graph, with preallocated workspaces."""
    n, k = shapes["qkv"]
    out = {}
    for m in TOKENS + (128,):
        x = torch.randn((m, k), generator=g, device=dev).to(torch.bfloat16)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        xn = torch.empty_like(x)
        wn = torch.ones(k, dtype=torch.float32, device=dev)
        lws = fr.linear_workspace(fr.fp4_lora_linear_workspace_bytes(m, n, k, RANK), dev)
        fws = torch.empty(max(256, fr.load_library().fp4rl_aqn_lora_linear_workspace(m, n, k, RANK)),
                          dtype=torch.uint8, device=dev)

        def folded(L):
            return lambda: fr.aqn_lora_linear(x, wn, SIGMA, 4, 0, 0, EPS, L["qkv"], *lora["qkv"], LORA_SCALE, out=y,
                                              workspace=fws)

        def norm_then_linear(L):
            def f():
                fr.aqn_rmsnorm(x, wn, SIGMA, 4, 0, 0, EPS, out=xn)
                fr.fp4_lora_linear(xn, L["qkv"], *lora["qkv"], LORA_SCALE, out=y, workspace=lws)
            return f

        res = {}
        for name, mk in (("aqn_folded_us", folded), ("aqn_then_linear_us", norm_then_linear)):
            dt, runs = graph_call_time(torch, [mk(L) for L in layers])
            res[name] = round(dt * 1e6, 1)
        res["timing"] = f"median of {runs} replays of one graph over {len(layers)} weight copies"
        out[f"M{m}"] = res
    return out


def run_decode_32b(torch, fr, dev, layers=64, m=128, r=RANK_32B):
    """Qwen2.5-32B-shaped decode over all 64 layers' linears (NVFP4, ~17.5 GB resident), M = 128, r = 64,
    AQN RMSNorm before qkv and before gate/up in each layer. Attention and SiLU are not on this path, so
    o and down read fresh synthetic activations. One pass is captured as a HIP graph and replayed."""
    from workloads import QWEN25_32B, tensor_seed
    shapes = QWEN25_32B
    hidden, inter = 5120, 27648
    g = torch.Generator(device=dev)
    wts, lora = [], []
    for layer in range(layers):
        wl, ll = {}, {}
        for name, (n, k) in shapes.items():
            g.manual_seed(tensor_seed(3, layer, name))
            w = torch.randn((n, k), generator=g, device=dev, dtype=torch.float32).mul_(0.02)
            wl[name] = fr.nvfp4_quantize(w)
            del w
            ll[name] = (torch.randn((r, k), generator=g, device=dev).mul_(0.01).to(torch.bfloat16),
                        torch.randn((n, r), generator=g, device=dev).mul_(0.01).to(torch.bfloat16))
        wts.append(wl)
        lora.append(ll)
    g.manual_seed(3)
    xh, xo, xr = (torch.randn((m, hidden), generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
    xd = torch.randn((m, inter), generator=g, device=dev).to(torch.bfloat16)
    h1, h2 = torch.empty_like(xh), torch.empty_like(xr)
    wn = torch.ones(hidden, dtype=torch.float32, device=dev)
    ys = {name: torch.empty((m, n), dtype=torch.bfloat16, device=dev) for name, (n, k) in shapes.items()}
    wsb = max(fr.fp4_lora_linear_workspace_bytes(m, n, k, r) for n, k in shapes.values())
    ws = fr.linear_workspace(wsb, dev)
    inp = {"qkv": h1, "o": xo, "gate": h2, "up": h2, "down": xd}

    def one_pass():
        for layer in range(layers):
            fr.aqn_rmsnorm(xh, wn, SIGMA, 3, 0, 2 * layer, EPS, out=h1)
            fr.aqn_rmsnorm(xr, wn, SIGMA, 3, 0, 2 * layer + 1, EPS, out=h2)
            for name in ("qkv", "o", "gate", "up", "down"):
                a, b = lora[layer][name]
                fr.fp4_lora_linear(inp[name], wts[layer][name], a, b, LORA_SCALE, out=ys[name], workspace=ws)

    one_pass()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        one_pass()
    dt, runs = median_time(torch, gr.replay)
    wbytes = layers * sum(nvfp4_bytes(n, k) for n, k in shapes.values())
    flops = layers * sum(linear_flops(m, n, k, r) for n, k in shapes.values())
    total_bytes = layers * (sum(nvfp4_bytes(n, k) + 2 * r * (k + n) + 2 * m * (k + n) for n, k in shapes.values())
                            + 2 * 4 * m * hidden)
    roof_s = max(total_bytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
    del gr, wts, lora
    return {"layers": layers, "M": m, "lora_rank": r, "ms_per_pass": round(dt * 1e3, 3),
            "weight_GB/s": round(wbytes / dt / 1e9, 1), "tflops": round(flops / dt / 1e12, 1),
            "nvfp4_weight_bytes": wbytes, "roofline_ms": round(roof_s * 1e3, 3),
            "frac_of_roofline": round(roof_s / dt, 4), "timing": f"median of {runs} graph replays",
            "roofline": mfma_roofline(flops / dt / 1e12, (fr.fp4_linear_kernel_name(m, 27648, 5120, r),
                                                          fr.fp4_linear_kernel_name(m, 5120, 27648, r)),
                                      "32B decode 128 tokens")}


if __name__ == "__main__":
    main()
