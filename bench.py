#!/usr/bin/env python3
"""FP8 linear forward + backward throughput on one MI355X.

Workload: the isolated FP8 linears 512 -> 2048 and 2048 -> 512 at N = 131072
tokens with current tensorwise amax scaling (E4M3 X/W, E5M2 dY), the fused
cast emitting row and transposed layouts, and the three FP8 GEMMs with BF16
outputs -- all conversions included, as in the isolated-linear timings of
"Native FP8 MLP reconstruction".  One step = forward + backward of both
linears on seeded synthetic normal operands (X ~ N(0,1), W ~ N(0,0.02),
dY ~ N(0,1e-3)) resident in HBM.

Prints ONE JSON line: the metric (TFLOP/s = 6 N K M summed over the two
linears / step time), the quantize GB/s, per-stage times, the roofline of the
dominant stage and the oracle's throughput on host cores (cpu_baseline).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

Profile summaries (no GPU needed): walks a rocprofv3 kernel trace or counter
collection of a bench run, assigns each library dispatch of the timed steps to
its stage (the step's call order is fixed), and prints markdown tables.

    python bench.py --summarize DIR/PREFIX --steps K --warmup W
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 linear fwd+bwd TFLOP/s incl. quantize at N=131072; quantize GB/s"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
RIDGE = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)      # FLOP per byte
PEAK_CLOCK_GHZ = 2.4     # the clock the vendor peaks are quoted at
XCDS = 8                 # accelerator complex dies (one GRBM_GUI_ACTIVE instance each)
# RTX 4090 fused-layout FP8 medians of the pages (ms): context, not a target
PAGES_MS = {(512, 2048): 5.4075, (2048, 512): 5.4264}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tokens", type=int, default=131072)
    ap.add_argument("--reps", type=int, default=20, help="instrumented steps in the per-call breakdown")
    ap.add_argument("--cpu-tokens", type=int, default=131072, help="token sample of the oracle baseline (all threads)")
    ap.add_argument("--cpu-tokens-1core", type=int, default=8192, help="token sample of the one-thread oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-stage breakdown")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured ceilings (HBM probes, sustained GEMM clock)")
    ap.add_argument("--no-block", action="store_true", help="skip the block-scaling, stacked-linear (amax hand-off), BF16 comparator and delayed-scaling runs")
    ap.add_argument("--copy-reference", action="store_true",
                    help="after the steps, negate a 512 MiB fp16 tensor (counter calibration)")
    ap.add_argument("--summarize", metavar="PREFIX", help="summarize PREFIX_kernel_trace.csv / "
                    "PREFIX_counter_collection.csv of a profiled bench run and exit")
    ap.add_argument("--recipe", choices=("tensor", "block"), default="tensor",
                    help="with --summarize: which recipe's timed steps to summarize")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_PREFIX", "WRITE_PREFIX"),
                    help="per-stage HBM bytes per launch from a FETCH_SIZE and a WRITE_SIZE counter run "
                         "(each with --copy-reference), one line per stage, and exit")
    ap.add_argument("--mfma", metavar="PREFIX",
                    help="matrix-core utilisation of every GEMM launch of a counter run "
                         "(--pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_F8 GRBM_GUI_ACTIVE), grouped by kernel and shape, and exit")
    return ap.parse_args()


SHAPES = [(512, 2048), (2048, 512)]
KINDS = (("amax_partial_kernel", "amax"), ("amax_pair_kernel", "amax"), ("cast_kernel", "cast"),
         ("cast_pair_kernel", "cast"), ("gemm_block_kernel", "gemm"),
         ("gemm_block_wide_kernel", "gemm"), ("gemm_tensor_kernel", "gemm"), ("splitk_reduce_kernel", "reduce"))
COPY_BYTES = 2 * 512 * 1024 * 1024      # the --copy-reference kernel reads 512 MiB and writes 512 MiB


def step_sequence(shapes, recipe="tensor"):
    """Library kernels of one step, in launch order, grouped by stage (weight
    requantized every step; a tensorwise quantize runs the amax pass then the
    cast, a block-scaled one the cast alone).  Tensorwise, the forward pass
    quantizes X and W together: one amax launch and one cast launch for both
    (stage quant_xw)."""
    q = ("cast",) if recipe == "block" else ("amax", "cast")
    seq = []
    for K, M in shapes:
        tag = "%dx%d" % (K, M)
        if recipe == "block":
            seq += [("quant_w_" + tag, q), ("quant_x_" + tag, q)]
        else:
            seq += [("quant_xw_" + tag, q)]
        seq += [("gemm_fprop_" + tag, ("gemm",)), ("quant_dy_" + tag, q),
                ("gemm_dgrad_" + tag, ("gemm",)), ("gemm_wgrad_" + tag, ("gemm",))]
    return seq


def kernel_kind(name):
    if "fp8k::" not in name:
        return None
    for key, kind in KINDS:
        if "::" + key + "<" in name or "::" + key + "(" in name:
            return kind
    return None


def short_name(name):
    return (name.replace("void ", "").replace("fp8k::", "").replace("tensor::", "").replace("blockw::", "")
            .replace("block::", ""))


def _code_only(text):
    """C/C++ source without its comments and with runs of white space
    collapsed: edits to comments leave the digest unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest():
    """sha256 over the code (comments removed) of the library's HIP/C++
    sources and headers: the profiles record it, and counter figures are used
    only while it matches."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "fp8_mixed_precision_amax_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        if f.endswith((".hip", ".hpp", ".cpp", ".h")) and os.path.basename(f) != "ceilings.hip":
            h.update(os.path.basename(f).encode())
            with open(f, encoding="utf-8") as fh:
                h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def walk_steps(disp, steps, warmup, recipe="tensor"):
    """disp: [(kind, name, value)] of library dispatches in dispatch order.
    Returns the timed steps as lists of (stage, kind, name, value).  The
    block-scaled steps follow the tensorwise part of a run; they start at the
    first 128x128 weight cast (cast_kernel<0, 2>)."""
    seq = step_sequence(SHAPES, recipe)
    i, out = 0, []
    if recipe == "block":
        first = [k for k, d in enumerate(disp) if "cast_kernel<0, 2>" in d[1]]
        if not first:
            raise SystemExit("no block-scaled steps in this trace")
        i = first[0]
    for s in range(warmup + steps):
        cur = []
        for stage, kinds in seq:
            for kd in kinds:
                if i >= len(disp) or disp[i][0] != kd:
                    raise SystemExit("dispatch %d: expected a %s kernel for %s, found %s" %
                                     (i, kd, stage, disp[i][1] if i < len(disp) else "end of trace"))
                cur.append((stage,) + disp[i])
                i += 1
            if kinds == ("gemm",) and i < len(disp) and disp[i][0] == "reduce":
                cur.append((stage,) + disp[i])
                i += 1
        if s >= warmup:
            out.append(cur)
    return out


def counter_dispatches(prefix, counter):
    """[(kind, name, value)] of library dispatches and the calibration factor
    (bytes per counted KiB) of one counter run."""
    by = collections.OrderedDict()
    for r in csv.DictReader(open(prefix + "_counter_collection.csv")):
        if r["Counter_Name"] != counter:
            continue
        d = by.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "v": 0.0})
        d["v"] += float(r["Counter_Value"])
    items = [d for _, d in sorted(by.items())]
    cal = [d for d in items if "neg_kernel" in d["name"]]
    if not cal:
        raise SystemExit("%s: no calibration copy (run the bench with --copy-reference)" % prefix)
    # the copy moves COPY_BYTES / 2 each way
    factor = (COPY_BYTES / 2) / cal[-1]["v"]
    return [(kernel_kind(d["name"]), short_name(d["name"]), d["v"]) for d in items if kernel_kind(d["name"])], factor


def traffic(fetch_prefix, write_prefix, steps, warmup):
    rd, fr = counter_dispatches(fetch_prefix, "FETCH_SIZE")
    wr, fw = counter_dispatches(write_prefix, "WRITE_SIZE")
    tr, tw = walk_steps(rd, steps, warmup), walk_steps(wr, steps, warmup)
    per = collections.OrderedDict()
    for sr, sw in zip(tr, tw):
        stage_bytes = collections.OrderedDict()
        for (stage, _, _, vr), (_, _, _, vw) in zip(sr, sw):
            stage_bytes[stage] = stage_bytes.get(stage, 0.0) + vr * fr + vw * fw
        for stage, b in stage_bytes.items():
            per.setdefault(stage, []).append(b)
    print("# stage  HBM bytes per launch (FETCH_SIZE x %.4f + WRITE_SIZE x %.4f, bytes per counted KiB)  "
          "library code sha256 (comments stripped)" % (fr, fw))
    digest = source_digest()
    for stage, v in per.items():
        print("%s %d %s" % (stage, round(sum(v) / len(v)), digest))


# GEMM shapes (I, J, K) the bench launches: the headline step's, then the
# other workloads' (N x M x K forward, N x K x M data gradient, M x K x N
# weight gradient)
def _bench_gemm_shapes():
    lin = [(1024, 512, 512), (131072, 512, 2048), (131072, 2048, 512), (131072, 512, 8192), (16384, 8192, 8192),
           (262144, 512, 8192), (8192, 8192, 16384)]
    out = []
    for N, K, M in lin[:-1]:
        out += [(N, M, K), (N, K, M), (M, K, N)]
    out.append(lin[-1])
    return sorted(set(out))


def mfma_summary(prefix, steps, warmup):
    """Matrix-core utilisation of the GEMM launches of a counter run with
    MfmaUtil (100 x MFMA-busy SIMD cycles / (active GPU cycles x SIMDs)) and
    SQ_INSTS_VALU_MFMA_MOPS_F8 (FP8 matrix work in units of 512 FLOP): the
    GEMM calls of the timed tensorwise and block-scaled steps by stage, then
    every other GEMM launch grouped by kernel and FLOP count."""
    by = collections.OrderedDict()
    for r in csv.DictReader(open(prefix + "_counter_collection.csv")):
        d = by.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                  "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [(kernel_kind(d["name"]), short_name(d["name"]), d) for _, d in sorted(by.items())
            if kernel_kind(d["name"])]

    # GPU clock over a launch: GRBM_GUI_ACTIVE counts the active cycles of
    # each of the 8 XCDs (the run sums them) over the launch's duration; not
    # meaningful for launches of a few microseconds (dispatch overhead)
    def sclk(d):
        ok = "GRBM_GUI_ACTIVE" in d and d["ns"] >= 20000
        return d["GRBM_GUI_ACTIVE"] / XCDS / d["ns"] if ok else float("nan")

    def mean(v):
        return sum(v) / len(v)

    used = set()
    print("| recipe | stage | kernel | MFMA busy % (mean over the timed steps) | GPU clock GHz | "
          "busy x clock / 2.4 GHz % | FLOP per launch (counter) |")
    print("|---|---|---|---:|---:|---:|---:|")
    for recipe in ("tensor", "block"):
        per = collections.OrderedDict()
        for st in walk_steps(disp, steps, warmup, recipe):
            for stage, kind, name, d in st:
                if kind == "gemm":
                    per.setdefault((stage, name), []).append(d)
                    used.add(id(d))
        for (stage, name), ds in per.items():
            u, f = mean([x["MfmaUtil"] for x in ds]), mean([sclk(x) for x in ds])
            print("| %s | %s | %s | %.1f | %.2f | %.1f | %.4g |" % (recipe, stage, name, u, f, u * f / PEAK_CLOCK_GHZ,
                                                                  ds[0]["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512))
    shapes = _bench_gemm_shapes()
    groups = collections.OrderedDict()
    for kind, name, d in disp:
        if kind != "gemm" or id(d) in used:
            continue
        flops = d["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512
        match = [sh for sh in shapes if abs(2 * sh[0] * sh[1] * sh[2] - flops) <= 1e-6 * flops]
        tag = "%.4g (%s)" % (flops, ", ".join("%dx%dx%d" % sh for sh in match) if match else "?")
        groups.setdefault((name, tag), []).append(d)
    print()
    print("| kernel | FLOP per launch (GEMMs of the bench with that count, I x J x K) | launches | MFMA busy % mean | min | max "
          "| GPU clock GHz mean |")
    print("|---|---|---:|---:|---:|---:|---:|")
    for (name, tag), ds in groups.items():
        v = [x["MfmaUtil"] for x in ds]
        f = mean([sclk(x) for x in ds])
        print("| %s | %s | %d | %.1f | %.1f | %.1f | %s |" % (name, tag, len(v), mean(v), min(v), max(v),
                                                            "-" if math.isnan(f) else "%.2f" % f))


def summarize(prefix, steps, warmup, recipe="tensor"):
    out = []
    trace = prefix + "_kernel_trace.csv"
    stats = prefix + "_kernel_stats.csv"
    counters = prefix + "_counter_collection.csv"
    if os.path.exists(stats):
        out.append("## rocprofv3 --stats (whole run, all calls of each kernel)\n")
        out.append("| kernel | calls | average us | min us | max us | share % |")
        out.append("|---|---:|---:|---:|---:|---:|")
        for r in csv.DictReader(open(stats)):
            if kernel_kind(r["Name"]) is None:
                continue
            out.append("| %s | %s | %.1f | %.1f | %.1f | %.1f |" % (
                short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
        out.append("")
    if os.path.exists(trace):
        rows = sorted(csv.DictReader(open(trace)), key=lambda r: int(r["Dispatch_Id"]))
        disp = [(kernel_kind(r["Kernel_Name"]), short_name(r["Kernel_Name"]),
                 int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in rows
                if kernel_kind(r["Kernel_Name"])]
        timed = walk_steps(disp, steps, warmup, recipe)
        per = collections.OrderedDict()
        for st in timed:
            for stage, kind, name, ns in st:
                per.setdefault((stage, name), []).append(ns)
        out.append("## timed steps, per stage (%d steps after %d warmup)\n" % (steps, warmup))
        out.append("| stage | kernel | launches | average us | min us | max us |")
        out.append("|---|---|---:|---:|---:|---:|")
        for (stage, name), v in per.items():
            out.append("| %s | %s | %d | %.1f | %.1f | %.1f |" % (stage, name, len(v), sum(v) / len(v) / 1e3,
                                                                min(v) / 1e3, max(v) / 1e3))
        step_us = [sum(x[3] for x in st) / 1e3 for st in timed]
        out.append("\nsum of kernel durations per step: %.1f us (average over the timed steps)\n" %
                   (sum(step_us) / len(step_us)))
    if os.path.exists(counters):
        by = collections.OrderedDict()
        for r in csv.DictReader(open(counters)):
            d = by.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "c": collections.Counter()})
            d["c"][r["Counter_Name"]] += float(r["Counter_Value"])
        items = sorted(by.items())
        cal = [d for _, d in items if "neg_kernel" in d["name"]]
        disp = [(kernel_kind(d["name"]), short_name(d["name"]), d["c"]) for _, d in items if kernel_kind(d["name"])]
        timed = walk_steps(disp, steps, warmup)
        names = sorted({k for _, _, c in disp for k in c})
        out.append("## counters per dispatch (KiB for FETCH_SIZE / WRITE_SIZE), timed steps\n")
        if cal:
            c = cal[-1]["c"]
            out.append("calibration: 512 MiB fp16 negation (reads 512 MiB, writes 512 MiB): " +
                       ", ".join("%s = %.0f KiB -> factor %.4f" % (k, c[k], (COPY_BYTES / 2 / 1024) / c[k])
                                 for k in names if c[k] > 0) + "\n")
        out.append("| stage | kernel | " + " | ".join(names) + " |")
        out.append("|---|---|" + "---:|" * len(names))
        per = collections.OrderedDict()
        for st in timed:
            for stage, kind, name, c in st:
                per.setdefault((stage, name), []).append(c)
        for (stage, name), v in per.items():
            out.append("| %s | %s | " % (stage, name) + " | ".join(
                "%.0f" % (sum(x[k] for x in v) / len(v)) for k in names) + " |")
        out.append("")
    out.append("library code sha256 (comments stripped): %s" % source_digest())
    print("\n".join(out))


def stage_times(fp8, torch, layers, reps, recipe="tensor"):
    """Average duration of each kernel-level call of one step, in the step's
    own call order: `reps` instrumented steps made of the same library calls
    the linear launches (weight quantize, activation quantize, forward GEMM,
    gradient quantize, data-gradient GEMM, weight-gradient GEMM, per layer),
    with an event recorded between consecutive calls on the stream the kernels
    run on (torch's current stream).  Each call thus runs after the call that
    precedes it in a real step (e.g. a quantize reads while the previous
    GEMM's output drains to HBM).  One difference: the tensorwise forward
    quantizes X and W in shared launches, while here they are two calls, so
    each can be timed.  Returns (stages, ms per instrumented step)."""
    E4, E5 = fp8.E4M3, fp8.E5M2
    block = recipe == "block"
    act = fp8.SCALE_1x128 if block else fp8.SCALE_TENSOR
    wsc = fp8.SCALE_128x128 if block else fp8.SCALE_TENSOR
    # algorithmic bytes per element: tensorwise = amax read 2 + cast read 2 +
    # two 1-byte layouts; block = one read + two layouts + the fp32
    # dequantisation factor of each block of each layout (1x128: one per 128
    # elements per layout; 128x128: one per tile, shared by both layouts)
    act_b, w_b = (4 + 8 / 128, 4 + 4 / 16384) if block else (6, 6)
    seq = []
    for L in layers:
        lin, N, K, M = L["lin"], L["N"], L["K"], L["M"]
        wq = lin.w_q
        if block:
            sx = fp8.block_gemm_scale(lin.saved_x.scale_inv, 1)
            sw = fp8.block_gemm_scale(wq.scale_inv, 128)
            sdy = fp8.block_gemm_scale(lin.dy_q.scale_inv, 1)
            swt = fp8.block_gemm_scale(wq.scale_inv.t(), 128)
            sdyc = fp8.block_gemm_scale(lin.dy_q.scale_inv_col, 1)
            sxc = fp8.block_gemm_scale(lin.saved_x.scale_inv_col, 1)
        else:
            sx, sw, sdy = (fp8.gemm_scale(t.scale_inv) for t in (lin.saved_x, wq, lin.dy_q))
            swt, sdyc, sxc = sw, sdy, sx
        tag = "%dx%d" % (K, M)
        seq += [
            ("quant_w_" + tag, "quant", M * K * w_b, lambda L=L, wq=wq: fp8.quantize(L["w"], E4, wsc, out=wq)),
            ("quant_x_" + tag, "quant", N * K * act_b, lambda L=L, lin=lin: fp8.quantize(L["x"], E4, act, out=lin.saved_x)),
            ("gemm_fprop_" + tag, "gemm", (N, M, K),
             lambda L=L, lin=lin, wq=wq, sx=sx, sw=sw: fp8.gemm(lin.saved_x.q_row, E4, sx, wq.q_row, E4, sw, out=L["y"])),
            ("quant_dy_" + tag, "quant", N * M * act_b, lambda L=L, lin=lin: fp8.quantize(L["dy"], E5, act, out=lin.dy_q)),
            ("gemm_dgrad_" + tag, "gemm", (N, K, M),
             lambda L=L, lin=lin, wq=wq, sdy=sdy, swt=swt: fp8.gemm(lin.dy_q.q_row, E5, sdy, wq.q_col, E4, swt, out=L["dx"])),
            ("gemm_wgrad_" + tag, "gemm", (M, K, N),
             lambda L=L, lin=lin, sdyc=sdyc, sxc=sxc: fp8.gemm(lin.dy_q.q_col, E5, sdyc, lin.saved_x.q_col, E4, sxc,
                                                             out=L["dw"])),
        ]
    for _ in range(2):
        for _, _, _, fn in seq:
            fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 1)] for _ in range(reps)]
    for r in range(reps):
        for i, (_, _, _, fn) in enumerate(seq):
            ev[r][i].record()
            fn()
        ev[r][-1].record()
    torch.cuda.synchronize()
    res = []
    for i, (name, kind, size, _) in enumerate(seq):
        ms = sum(ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(reps)) / reps
        if kind == "quant":
            byts = int(size)
            res.append({"stage": name, "ms": ms, "bytes": byts, "gbs": byts / ms / 1e6})
        else:
            I, J, Kc = size
            flops = 2 * I * J * Kc
            byts = I * Kc + J * Kc + 2 * I * J
            res.append({"stage": name, "ms": ms, "flops": flops, "bytes": byts,
                        "tflops": flops / ms / 1e9, "gbs": byts / ms / 1e6, "ai": flops / byts})
    step_ms = sum(ev[r][0].elapsed_time(ev[r][-1]) for r in range(reps)) / reps
    return res, step_ms


def make_layers(fp8, torch, synth, N, recipe, dev):
    R = fp8.RECIPE_BLOCK if recipe == "block" else fp8.RECIPE_TENSOR
    layers = []
    for idx, (K, M) in enumerate(SHAPES):
        x, w, dy = synth.operands_on_device(N, K, M, seed=idx, device=dev)
        layers.append({"N": N, "K": K, "M": M, "x": x, "w": w, "dy": dy, "lin": fp8.Fp8Linear(N, K, M, R, device=dev),
                       "y": torch.empty((N, M), dtype=torch.bfloat16, device=dev),
                       "dx": torch.empty((N, K), dtype=torch.bfloat16, device=dev),
                       "dw": torch.empty((M, K), dtype=torch.bfloat16, device=dev)})
    return layers


def workload_layers(fp8, torch, synth, name, dev):
    """One linear of a named synthetic workload (its own distributions and
    recipe), in the form stage_times and time_steps take."""
    wl = synth.workload_on_device(name, seed=0, device=dev)
    N, K, M = wl["N"], wl["K"], wl["M"]
    R = fp8.RECIPE_BLOCK if wl["scaling"] == "block" else fp8.RECIPE_TENSOR
    return [{"N": N, "K": K, "M": M, "x": wl["x"], "w": wl["w"], "dy": wl["dy"],
             "lin": fp8.Fp8Linear(N, K, M, R, device=dev),
             "y": torch.empty((N, M), dtype=torch.bfloat16, device=dev),
             "dx": torch.empty((N, K), dtype=torch.bfloat16, device=dev),
             "dw": torch.empty((M, K), dtype=torch.bfloat16, device=dev)}], wl["scaling"]


MFMA_PEAK_TFLOPS = 5000.0   # dense FP8 matrix-core peak of the MI355X (vendor figure)


def config_times(fp8, torch, synth, steps, warmup, reps, dev):
    """The other linear workloads: the block-scaled 512->8192 at N=131072
    (1% outliers), the square 8192x8192 weight at N=16384 and 512->8192 at
    N=262144 under both recipes.  For each: forward + backward time (every
    quantization included) and each GEMM's rate against the dense FP8 peak."""
    names = ["linear_512x8192_n131072_block", "linear_8192x8192_n16384", "linear_8192x8192_n16384_block",
             "linear_512x8192_n262144", "linear_512x8192_n262144_block"]
    out = {}
    for name in names:
        layers, recipe = workload_layers(fp8, torch, synth, name, dev)
        L = layers[0]
        ms = time_steps(torch, layers, steps, warmup)
        st, _ = stage_times(fp8, torch, layers, reps, recipe)
        flops = 6 * L["N"] * L["K"] * L["M"]
        gemms = {}
        for s in st:
            if "flops" in s:
                gemms[s["stage"].split("_")[1]] = {"ms": round(s["ms"], 4), "tflops": round(s["tflops"], 1),
                                                   "mfma_frac": round(s["tflops"] / MFMA_PEAK_TFLOPS, 3)}
        quant = {s["stage"].split("_")[1]: {"ms": round(s["ms"], 4), "gbs": round(s["gbs"], 1)}
                 for s in st if "flops" not in s}
        out[name] = {"recipe": recipe, "N": L["N"], "K": L["K"], "M": L["M"], "ms_per_step": round(ms, 4),
                     "value": round(flops / (ms / 1e3) / 1e12, 2), "unit": "TFLOP/s", "gemms": gemms,
                     "quantize": quant}
        print("%s: %.4f ms/step, %.1f TFLOP/s; GEMMs %s" % (name, ms, out[name]["value"],
              ", ".join("%s %.0f" % (k, v["tflops"]) for k, v in gemms.items())), file=sys.stderr, flush=True)
        del layers, L
        torch.cuda.empty_cache()
    return out


def mlp_stack_times(fp8, torch, synth, N, cycles, dev, recipe="tensor", layers=8, mbs=4):
    """The MLP stack of the gradient-accumulation workload: `layers` blocks of
    512 -> 2048 (GELU) -> 512, `mbs` microbatches of N tokens per cycle, the
    GELU fused into the quantizers.  Timed over `cycles` cycles (one untimed
    first) with the weight cache (W quantized on microbatch 1, reused on the
    rest), without it (W requantized every microbatch), and, tensorwise, with
    the cache and the amax hand-off on the edges without a GELU between
    (block p's output is block p+1's input; block p+1's input gradient is
    block p's output gradient).  The weight gradients of the last cycle are
    compared bitwise across the runs.  The hand-off run also takes each
    block's forward in one call (fp8_mlp_fwd), whose up projection hands the
    GELU amax keys of its output to the down projection's input quantize."""
    d, h = 512, 2048
    R = fp8.RECIPE_BLOCK if recipe == "block" else fp8.RECIPE_TENSOR
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    weights = []
    for _ in range(layers):
        weights.append(synth.normal_bf16((h, d), 0.02, g, device=dev))
        weights.append(synth.normal_bf16((d, h), 0.02, g, device=dev))
    xs = [synth.normal_bf16((N, d), 1.0, g, device=dev) for _ in range(mbs)]
    dys = [synth.normal_bf16((N, d), 1e-3, g, device=dev) for _ in range(mbs)]
    shapes = [(d, h), (h, d)] * layers
    modes = [("cached", True, False), ("uncached", False, False)]
    if recipe == "tensor":
        modes.append(("cached_handoff", True, True))
    res, final = {}, {}
    for mode, cached, handoff in modes:
        lins = [fp8.Fp8Linear(N, K, M, R, device=dev, cache=cached) for K, M in shapes]
        pre = [torch.empty((N, h), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
        hid = [torch.empty((N, d), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
        dws = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for K, M in shapes]
        dg = torch.empty((N, h), dtype=torch.bfloat16, device=dev)
        dh = [torch.empty((N, d), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        pa, pb = (fp8.amax_partials(dev), fp8.amax_partials(dev)) if handoff else (None, None)
        mlps = [fp8.Fp8Mlp(N, d, h, R, dev, up=lins[2 * p], down=lins[2 * p + 1]) for p in range(layers)] \
            if handoff else None

        def cycle():
            for mb in range(mbs):
                flag = (mb == 0) if cached else None
                x = xs[mb]
                for p in range(layers):
                    if handoff:
                        mlps[p].forward(x, weights[2 * p], weights[2 * p + 1], y=hid[p], a=pre[p],
                                        is_first_microbatch=flag, x_amax=pa if p > 0 else None,
                                        y_amax=pa if p + 1 < layers else None)
                    else:
                        lins[2 * p].forward(x, weights[2 * p], y=pre[p], is_first_microbatch=flag)
                        lins[2 * p + 1].forward(pre[p], weights[2 * p + 1], y=hid[p], is_first_microbatch=flag,
                                                gelu=True)
                    x = hid[p]
                g_in = dys[mb]
                for p in reversed(range(layers)):
                    lins[2 * p + 1].backward(g_in, dx=dg, dw=dws[2 * p + 1],
                                             dy_amax=pb if (handoff and p + 1 < layers) else None)
                    out = dh[p & 1]
                    lins[2 * p].backward(dg, dx=out, dw=dws[2 * p], gelu_input=pre[p],
                                         dx_amax=pb if (handoff and p > 0) else None)
                    g_in = out
        cycle()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(cycles):
            cycle()
        e1.record()
        torch.cuda.synchronize()
        res[mode] = e0.elapsed_time(e1) / cycles
        final[mode] = [w.clone() for w in dws]
        del lins, mlps, pre, hid, dws, dg, dh, pa, pb
        torch.cuda.empty_cache()
    flops = mbs * sum(6 * N * K * M for K, M in shapes)
    out = {"workload": "%d x (512->2048, GELU, 2048->512), N=%d per microbatch, %d microbatches per cycle, %s"
                       % (layers, N, mbs, "tensorwise" if recipe == "tensor" else "1x128 / 128x128 blocks"),
           "ms_per_cycle_cached": round(res["cached"], 3), "ms_per_cycle_uncached": round(res["uncached"], 3),
           "value_cached": round(flops / (res["cached"] / 1e3) / 1e12, 2),
           "value_uncached": round(flops / (res["uncached"] / 1e3) / 1e12, 2), "unit": "TFLOP/s",
           "cache_speedup": round(res["uncached"] / res["cached"], 4),
           "dw_cached_equals_uncached": all(torch.equal(a, b) for a, b in zip(final["cached"], final["uncached"]))}
    if "cached_handoff" in res:
        out["ms_per_cycle_cached_handoff"] = round(res["cached_handoff"], 3)
        out["value_cached_handoff"] = round(flops / (res["cached_handoff"] / 1e3) / 1e12, 2)
        out["dw_handoff_equals_cached"] = all(torch.equal(a, b)
                                              for a, b in zip(final["cached_handoff"], final["cached"]))
    return out


def _amd_smi_sample():
    """GFX clocks (MHz, one per XCD) and socket power (W) from `amd-smi
    metric`, or None where the tool is missing or prints no such fields."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-c", "-p"], capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    txt = r.stdout
    clocks = []
    for blk in re.split(r"\n\s*GFX_\d+:", txt)[1:]:
        m = re.search(r"^\s*CLK:\s*(\d+)\s*MHz", blk, re.M)
        if m:
            clocks.append(int(m.group(1)))
    pw = re.search(r"SOCKET_POWER:\s*(\d+)\s*W", txt)
    if not clocks:
        return None
    return {"gfx_mhz": clocks, "socket_power_w": int(pw.group(1)) if pw else None}


def ceilings(fp8, torch, synth, dev):
    """What this GPU reaches with plain kernels (libfp8ceilings.so): HBM
    read, write and copy bandwidth on a 2 GiB buffer (eight times the
    memory-side cache; best launch of a few), the rate of back-to-back FP8
    matrix-core instructions with the shader clock they ran at, and the GFX
    clock and socket power while 8192 x 8192 x 16384 FP8 GEMMs of the library
    run back to back for about two seconds."""
    import ctypes
    import threading
    path = os.path.join(ROOT, "fp8_mixed_precision_amax_amd", "libfp8ceilings.so")
    if not os.path.exists(path):
        return None
    cl = ctypes.CDLL(path)
    cl.fp8c_hbm_read.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_void_p]
    cl.fp8c_hbm_write.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    cl.fp8c_hbm_copy.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    cl.fp8c_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 2 << 30
    n16 = nbytes // 16
    x = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    y = torch.empty_like(x)
    o = torch.zeros(4, dtype=torch.int32, device=dev)

    def best(fn, moved):
        rates = []
        for grid in (1024, 2048, 4096, 8192):
            if fn(grid) != 0:
                raise RuntimeError("ceiling probe launch failed")
            ms = _ms(torch, lambda: fn(grid), 10)
            rates.append(moved / ms / 1e6)
        return round(max(rates), 1)

    res = {"hbm_buffer_bytes": nbytes}
    res["hbm_read_gbs"] = max(best(lambda g, v=v: cl.fp8c_hbm_read(v, g, x.data_ptr(), n16, o.data_ptr(), st), nbytes)
                              for v in (0, 1, 2))
    res["hbm_write_gbs"] = max(best(lambda g, v=v: cl.fp8c_hbm_write(v, g, y.data_ptr(), n16, st), nbytes)
                               for v in (0, 1))
    res["hbm_copy_gbs"] = best(lambda g: cl.fp8c_hbm_copy(g, x.data_ptr(), y.data_ptr(), n16, st), 2 * nbytes)
    res["hbm_copy_gbs_torch"] = round(2 * nbytes / _ms(torch, lambda: y.copy_(x), 10) / 1e6, 1)
    del x, y

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    grid, block, iters = 2 * cus, 512, 20000
    out = torch.empty(grid * block, dtype=torch.float32, device=dev)
    clk = torch.zeros(2 * grid, dtype=torch.int64, device=dev)
    run = lambda: cl.fp8c_mfma(grid, block, iters, out.data_ptr(), clk.data_ptr(), st)
    if run() != 0:
        raise RuntimeError("ceiling probe launch failed")
    ms = _ms(torch, run, 3)
    c = clk.view(grid, 2).double().cpu()
    res["mfma_only_tflops"] = round(grid * (block // 64) * iters * 4 * (2 * 32 * 32 * 64) / ms / 1e9, 1)
    res["mfma_only_shader_ghz"] = round(float((c[:, 0] / (c[:, 1] / 100e6)).mean()) / 1e9, 3)

    # sustained GEMM: clock and power as the power limit sees them
    I = J = 8192
    K = 16384
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    qa = fp8.quantize(synth.normal_bf16((I, K), 1.0, g, device=dev), fp8.E4M3, layouts=fp8.LAYOUT_ROW)
    qb = fp8.quantize(synth.normal_bf16((J, K), 1.0, g, device=dev), fp8.E4M3, layouts=fp8.LAYOUT_ROW)
    cout = torch.empty((I, J), dtype=torch.bfloat16, device=dev)
    sa, sb = fp8.gemm_scale(qa.scale_inv), fp8.gemm_scale(qb.scale_inv)
    gemm = lambda: fp8.gemm(qa.q_row, fp8.E4M3, sa, qb.q_row, fp8.E4M3, sb, out=cout)
    samples = []
    stop = threading.Event()

    def sampler():
        time.sleep(0.5)
        while not stop.is_set():
            s = _amd_smi_sample()
            if s is None:
                return
            samples.append(s)
            time.sleep(0.2)

    for _ in range(3):
        gemm()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler)
    th.start()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < 2.5:
        for _ in range(16):
            gemm()
        n += 16
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    ms = e0.elapsed_time(e1) / n
    gt = {"workload": "%dx%dx%d tensorwise FP8 GEMM, back to back for %.1f s" % (I, J, K, time.perf_counter() - t0),
          "tflops": round(2 * I * J * K / ms / 1e9, 1), "samples": len(samples)}
    if samples:
        mhz = [sum(s["gfx_mhz"]) / len(s["gfx_mhz"]) for s in samples]
        gt["gfx_mhz_mean"] = round(sum(mhz) / len(mhz))
        pw = [s["socket_power_w"] for s in samples if s["socket_power_w"] is not None]
        gt["socket_power_w_mean"] = round(sum(pw) / len(pw)) if pw else None
        # the dense FP8 peak scales with the clock: 256 CUs x 8192 FLOP per clock
        gt["mfma_peak_at_that_clock_tflops"] = round(256 * 8192 * gt["gfx_mhz_mean"] * 1e6 / 1e12, 1)
        gt["frac_of_clock_peak"] = round(gt["tflops"] / gt["mfma_peak_at_that_clock_tflops"], 3)
    res["sustained_gemm"] = gt
    return res


def timing_groups(torch, step, steps, warmup, groups=5):
    """The timing protocol: `warmup` untimed steps, then exactly `steps` steps
    split into `groups` consecutive groups (as equal as possible), an event
    pair around each group on torch's current stream (the stream the library
    launches on), a device synchronisation on both sides of the timed region.
    Returns the median group's ms per step, the mean over all steps and the
    per-group figures (the pages report medians of five timing groups)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    g = max(1, min(groups, steps))
    sizes = [steps // g + (1 if i < steps % g else 0) for i in range(g)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in sizes]
    for (e0, e1), n in zip(ev, sizes):
        e0.record()
        for _ in range(n):
            step()
        e1.record()
    torch.cuda.synchronize()
    per = [e0.elapsed_time(e1) / n for (e0, e1), n in zip(ev, sizes)]
    total = sum(e0.elapsed_time(e1) for e0, e1 in ev)
    med = sorted(per)[len(per) // 2] if len(per) % 2 else sum(sorted(per)[len(per) // 2 - 1:len(per) // 2 + 1]) / 2
    return {"ms": med, "mean_ms": total / steps, "group_steps": sizes, "group_ms": per}


def linear_step(layers):
    def step():
        for L in layers:
            L["lin"].forward(L["x"], L["w"], y=L["y"])
            L["lin"].backward(L["dy"], dx=L["dx"], dw=L["dw"])
    return step


def time_steps(torch, layers, steps, warmup):
    """ms per step (median of five timing groups over `steps` steps after
    `warmup` untimed ones)."""
    return timing_groups(torch, linear_step(layers), steps, warmup)["ms"]


def latency_small(fp8, torch, synth, dev, steps=500, warmup=50):
    """The small linear 512 -> 512 at N = 1024 (tensorwise, X ~ N(0,1),
    W ~ N(0,0.02), dY ~ N(0,1e-3), seed 0): forward + backward latency in
    microseconds, median of five timing groups."""
    layers, _ = workload_layers(fp8, torch, synth, "linear_512x512_n1024", dev)
    L = layers[0]
    step = linear_step(layers)
    t = timing_groups(torch, step, steps, warmup)
    # the same step captured once into a HIP graph (the library allocates
    # nothing and records no memset, so its launches capture as they are)
    # and replayed: what launch overhead the eager step pays
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    tg = timing_groups(torch, graph.replay, steps, warmup)
    flops = 6 * L["N"] * L["K"] * L["M"]
    return {"workload": "fp8 linear 512->512 fwd+bwd, N=1024, tensorwise current scaling",
            "us_per_step": round(t["ms"] * 1e3, 2), "us_per_step_mean": round(t["mean_ms"] * 1e3, 2),
            "us_per_step_graph": round(tg["ms"] * 1e3, 2),
            "steps": steps, "value": round(flops / (t["ms"] / 1e3) / 1e12, 2),
            "value_graph": round(flops / (tg["ms"] / 1e3) / 1e12, 2), "unit": "TFLOP/s"}


def chain_times(fp8, torch, synth, N, steps, warmup, dev):
    """The two linears stacked (512 -> 2048 -> 512: Y1 is X2, dX2 is dY1),
    tensorwise, timed without and with the amax hand-off: with it the
    forward GEMM of layer 1 emits Y1's amax partials and layer 2 quantizes X2
    in one pass; the data-gradient GEMM of layer 2 does the same for dY1."""
    (K1, M1), (K2, M2) = SHAPES
    x1, w1, _ = synth.operands_on_device(N, K1, M1, seed=0, device=dev)
    _, w2, dy2 = synth.operands_on_device(N, K2, M2, seed=1, device=dev)
    l1 = fp8.Fp8Linear(N, K1, M1, device=dev)
    l2 = fp8.Fp8Linear(N, K2, M2, device=dev)
    y1 = torch.empty((N, M1), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty((N, M2), dtype=torch.bfloat16, device=dev)
    dx2 = torch.empty((N, K2), dtype=torch.bfloat16, device=dev)
    dx1 = torch.empty((N, K1), dtype=torch.bfloat16, device=dev)
    dw1 = torch.empty((M1, K1), dtype=torch.bfloat16, device=dev)
    dw2 = torch.empty((M2, K2), dtype=torch.bfloat16, device=dev)
    pa, pb = fp8.amax_partials(dev), fp8.amax_partials(dev)

    def step(h):
        l1.forward(x1, w1, y=y1, y_amax=pa if h else None)
        l2.forward(y1, w2, y=y2, x_amax=pa if h else None)
        l2.backward(dy2, dx=dx2, dw=dw2, dx_amax=pb if h else None)
        l1.backward(dx2, dx=dx1, dw=dw1, dy_amax=pb if h else None)

    res = {}
    for h in (False, True):
        for _ in range(warmup):
            step(h)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step(h)
        e1.record()
        torch.cuda.synchronize()
        res[h] = e0.elapsed_time(e1) / steps
    flops = sum(6 * N * K * M for K, M in SHAPES)
    return {"workload": "512->2048->512 stack (Y1 = X2, dX2 = dY1), N=%d, tensorwise" % N,
            "ms_per_step": round(res[False], 4), "ms_per_step_handoff": round(res[True], 4),
            "value": round(flops / (res[False] / 1e3) / 1e12, 2),
            "value_handoff": round(flops / (res[True] / 1e3) / 1e12, 2), "unit": "TFLOP/s"}


BF16_PEAK_TFLOPS = 2500.0   # dense BF16 matrix-core peak of the MI355X (vendor figure)


def bf16_comparator(fp8, torch, synth, N, steps, warmup, reps, dev):
    """The pages' baseline: the same two linears' forward + backward in BF16
    (no quantization), timed two ways: this library's hand-written BF16
    matrix-core GEMMs (fp8_bf16_linear_fwd / _bwd; W and the gradients' left
    operands read output-major, no transposed copies) and hipBLASLt through
    torch.mm (right-hand operands contiguous).  Per GEMM of the hand-written
    path: time and fraction of the dense BF16 peak."""
    ops = []
    for idx, (K, M) in enumerate(SHAPES):
        x, w, dy = synth.operands_on_device(N, K, M, seed=idx, device=dev)
        ops.append((x, w, w.t().contiguous(), dy, fp8.Bf16Linear(N, K, M, device=dev),
                    torch.empty((N, M), dtype=torch.bfloat16, device=dev),
                    torch.empty((N, K), dtype=torch.bfloat16, device=dev),
                    torch.empty((M, K), dtype=torch.bfloat16, device=dev)))

    def step_lib():
        for x, w, wt, dy, lin, y, dx, dw in ops:
            torch.mm(x, wt)            # Y = X W^T
            torch.mm(dy, w)            # dX = dY W
            torch.mm(dy.t(), x)        # dW = dY^T X

    def step_own():
        for x, w, wt, dy, lin, y, dx, dw in ops:
            lin.forward(x, w, y=y)
            lin.backward(dy, x, w, dx=dx, dw=dw)

    flops = sum(6 * N * K * M for K, M in SHAPES)
    t_lib = timing_groups(torch, step_lib, steps, warmup)["ms"]
    t_own = timing_groups(torch, step_own, steps, warmup)["ms"]
    gemms = {}
    for x, w, wt, dy, lin, y, dx, dw in ops:
        K, M = lin.K, lin.M
        tag = "%dx%d" % (K, M)
        for name, fn, fl in (("fprop", lambda: fp8.bf16_gemm(x, w, 0, 0, out=y), 2 * N * K * M),
                             ("dgrad", lambda: fp8.bf16_gemm(dy, w, 0, 1, out=dx), 2 * N * K * M),
                             ("wgrad", lambda: fp8.bf16_gemm(dy, x, 1, 1, out=dw), 2 * N * K * M)):
            ms = _ms(torch, fn, reps)
            gemms["%s_%s" % (name, tag)] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                                            "bf16_peak_frac": round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 3)}
    del ops
    torch.cuda.empty_cache()
    return {"workload": "the same two linears in BF16, N=%d: hand-written BF16 matrix-core GEMMs, and hipBLASLt "
                        "via torch.mm (bf16 out)" % N,
            "ms_per_step": round(t_own, 4), "value": round(flops / (t_own / 1e3) / 1e12, 2),
            "ms_per_step_hipblaslt": round(t_lib, 4), "value_hipblaslt": round(flops / (t_lib / 1e3) / 1e12, 2),
            "unit": "TFLOP/s", "gemms": gemms}


def delayed_quant_times(fp8, torch, synth, N, reps, dev):
    """Quantize of a dY-sized tensor (N x 2048, E5M2, both layouts): delayed
    scaling (scale from a 1024-entry amax history, one pass: 2 B read + 2 B
    written per element) against current scaling (amax pass + cast: 6 B)."""
    M = SHAPES[0][1]
    _, _, dy = synth.operands_on_device(N, SHAPES[0][0], M, seed=0, device=dev)
    hist = torch.zeros(1024, dtype=torch.float32, device=dev)
    qd = fp8.QTensor(N, M, fp8.SCALE_TENSOR, dev)
    qc = fp8.QTensor(N, M, fp8.SCALE_TENSOR, dev)
    res = {}
    for name, fn in (("delayed", lambda: fp8.quantize_delayed(dy, fp8.E5M2, hist, out=qd)),
                     ("current", lambda: fp8.quantize(dy, fp8.E5M2, out=qc))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / reps
    n = N * M
    return {"workload": "dY %dx%d E5M2, both layouts; delayed: 1024-entry amax history" % (N, M),
            "ms_delayed": round(res["delayed"], 4), "gbs_delayed": round(4 * n / res["delayed"] / 1e6, 1),
            "ms_current": round(res["current"], 4), "gbs_current": round(6 * n / res["current"] / 1e6, 1)}


def _ms(torch, fn, reps, warm=3):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def mlp_gelu_times(fp8, torch, synth, N, steps, warmup, reps, dev):
    """GELU between the two linears (the MLP block 512 -> 2048 -> 512).
    Quantize level, on the hidden activation [N, 2048]: GELU fused into the
    second linear's X quantize against GELU written out in bf16 and then
    quantized, and dGELU fused into the first linear's dY quantize against
    the same two steps unfused.  Algorithmic bytes per element, tensorwise:
    fused GELU 6 (x read twice, two codes), unfused 10 (+ the bf16
    activation written and read); fused dGELU 10 (both inputs read twice),
    unfused 12; 1x128 (one pass): fused 4 and 6.  Block level: one forward +
    backward of the MLP block, fused entry points against unfused ones."""
    (K1, M1), (K2, M2) = SHAPES
    g = torch.Generator(device=dev).manual_seed(77)
    a = synth.normal_bf16((N, M1), 0.45, g, device=dev)          # pre-activation, sigma 0.02 * sqrt(512)
    dh = synth.normal_bf16((N, M1), 1e-3, g, device=dev)
    n = N * M1
    res = {"workload": "MLP block 512->2048 (GELU) ->512, N=%d; hidden activation %dx%d" % (N, N, M1)}
    hbuf = torch.empty_like(a)
    for scaling, sname in ((fp8.SCALE_TENSOR, "tensor"), (fp8.SCALE_1x128, "1x128")):
        qx = fp8.QTensor(N, M1, scaling, dev)
        qd = fp8.QTensor(N, M1, scaling, dev)
        t = {
            "gelu_fused": _ms(torch, lambda: fp8.quantize_gelu(a, fp8.E4M3, scaling, out=qx), reps),
            "gelu_unfused": _ms(torch, lambda: fp8.quantize(fp8.gelu(a, out=hbuf), fp8.E4M3, scaling, out=qx), reps),
            "dgelu_fused": _ms(torch, lambda: fp8.quantize_dgelu(dh, a, fp8.E5M2, scaling, out=qd), reps),
            "dgelu_unfused": _ms(torch, lambda: fp8.quantize(fp8.dgelu(dh, a, out=hbuf), fp8.E5M2, scaling, out=qd),
                                 reps),
        }
        one = sname == "1x128"
        algo = {"gelu_fused": 4 if one else 6, "gelu_unfused": 8 if one else 10,
                "dgelu_fused": 6 if one else 10, "dgelu_unfused": 10 if one else 12}
        res[sname] = {k: {"ms": round(v, 4), "algorithmic_gbs": round(algo[k] * n / v / 1e6, 1),
                          "hbm_frac": round(algo[k] * n / v / 1e6 / HBM_PEAK_GBS, 3)} for k, v in t.items()}
        del qx, qd
    del hbuf
    # one forward + backward of the block, tensorwise
    x, w1, _ = synth.operands_on_device(N, K1, M1, seed=0, device=dev)
    _, w2, dy = synth.operands_on_device(N, K2, M2, seed=1, device=dev)
    l1, l2 = fp8.Fp8Linear(N, K1, M1, device=dev), fp8.Fp8Linear(N, K2, M2, device=dev)
    ya = torch.empty((N, M1), dtype=torch.bfloat16, device=dev)
    h = torch.empty_like(ya)
    dhid = torch.empty_like(ya)
    y2 = torch.empty((N, M2), dtype=torch.bfloat16, device=dev)
    dx1 = torch.empty((N, K1), dtype=torch.bfloat16, device=dev)
    dw1 = torch.empty((M1, K1), dtype=torch.bfloat16, device=dev)
    dw2 = torch.empty((M2, K2), dtype=torch.bfloat16, device=dev)

    def fused():
        l1.forward(x, w1, y=ya)
        l2.forward(ya, w2, y=y2, gelu=True)
        l2.backward(dy, dx=dhid, dw=dw2)
        l1.backward(dhid, dx=dx1, dw=dw1, gelu_input=ya)

    def unfused():
        l1.forward(x, w1, y=ya)
        l2.forward(fp8.gelu(ya, out=h), w2, y=y2)
        l2.backward(dy, dx=dhid, dw=dw2)
        l1.backward(fp8.dgelu(dhid, ya, out=h), dx=dx1, dw=dw1)

    mlp = fp8.Fp8Mlp(N, K1, M1, device=dev)

    def handoff():
        # forward in one call: the up projection's GEMM hands the GELU amax
        # keys of its output to the down projection's input quantize
        mlp.forward(x, w1, w2, y=y2, a=ya)
        dh_, _ = mlp.down.backward(dy, dx=dhid, dw=dw2)
        mlp.up.backward(dhid, dx=dx1, dw=dw1, gelu_input=ya)

    flops = sum(6 * N * K * M for K, M in SHAPES)
    bf, bu, bh = _ms(torch, fused, steps, warmup), _ms(torch, unfused, steps, warmup), _ms(torch, handoff, steps, warmup)
    # the down projection's input quantize alone: two passes, or the cast pass
    # fed by the keys the up projection's GEMM wrote
    keys = fp8.gelu_amax_partials(dev)
    qx = fp8.QTensor(N, M1, fp8.SCALE_TENSOR, dev)
    sx, sw = fp8.gemm_scale(l1.saved_x.scale_inv), fp8.gemm_scale(l1.w_q.scale_inv)
    fp8.gemm(l1.saved_x.q_row, fp8.E4M3, sx, l1.w_q.q_row, fp8.E4M3, sw, out=ya, gelu_amax_out=keys)
    q_two = _ms(torch, lambda: fp8.quantize_gelu(ya, fp8.E4M3, out=qx), reps)
    q_one = _ms(torch, lambda: fp8.quantize_gelu(ya, fp8.E4M3, out=qx, gelu_amax_partials=keys), reps)
    res["block"] = {"ms_fused": round(bf, 4), "ms_unfused": round(bu, 4), "ms_fused_gelu_handoff": round(bh, 4),
                    "tflops_fused": round(flops / (bf / 1e3) / 1e12, 2),
                    "tflops_unfused": round(flops / (bu / 1e3) / 1e12, 2),
                    "tflops_fused_gelu_handoff": round(flops / (bh / 1e3) / 1e12, 2), "unit": "TFLOP/s",
                    "gelu_quantize_two_pass_ms": round(q_two, 4), "gelu_quantize_from_keys_ms": round(q_one, 4),
                    "gelu_quantize_from_keys_gbs": round(4 * n / q_one / 1e6, 1)}
    return res


def measured_traffic(stage):
    """HBM bytes per launch of `stage` from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by the copy calibration), or None when
    there is none for this stage or the library sources changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    digest = source_digest()
    for line in open(path):
        f = line.split()
        if line.startswith("#"):
            continue
        if len(f) == 3 and f[0] == stage and f[2] == digest:
            return int(f[1])
    return None


def roofline_of(stage):
    r = {"stage": stage["stage"], "launch_ms": round(stage["ms"], 4)}
    if "flops" in stage and stage["ai"] >= RIDGE:
        r.update({"bound": "mfma", "achieved": round(stage["tflops"], 1), "peak": FP8_PEAK_TFLOPS,
                  "unit": "TFLOP/s", "frac": round(stage["tflops"] / FP8_PEAK_TFLOPS, 4)})
    else:
        r.update({"bound": "hbm", "achieved": round(stage["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(stage["gbs"] / HBM_PEAK_GBS, 4)})
    r["traffic"] = measured_traffic(stage["stage"])
    return r


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_step(oracle, xb, wb, dyb, stage_s):
    """The oracle's linear forward + backward (tensorwise), the same calls
    oracle.linear_fwd / linear_bwd make, timed per stage."""
    def timed(name, fn, *a):
        t0 = time.perf_counter()
        r = fn(*a)
        stage_s[name] = stage_s.get(name, 0.0) + time.perf_counter() - t0
        return r
    N, K = xb.shape
    M = wb.shape[0]
    xq = timed("quantize_x", oracle.quant_tensor, xb, "e4m3")
    wq = timed("quantize_w", oracle.quant_tensor, wb, "e4m3")
    a, sa, b, sb = oracle.fprop_operands(xq, wq, "tensor", N, K, M)
    timed("gemm_fprop", oracle.gemm_tensor, a, "e4m3", b, "e4m3", sa.s[0], sb.s[0])
    dyq = timed("quantize_dy", oracle.quant_tensor, dyb, "e5m2")
    a, sa, b, sb = oracle.dgrad_operands(dyq, wq, "tensor", N, K, M)
    timed("gemm_dgrad", oracle.gemm_tensor, a, "e5m2", b, "e4m3", sa.s[0], sb.s[0])
    a, sa, b, sb = oracle.wgrad_operands(dyq, xq, "tensor", N, K, M)
    timed("gemm_wgrad", oracle.gemm_tensor, a, "e5m2", b, "e4m3", sa.s[0], sb.s[0])


def cpu_baseline(shapes, tokens, tokens_1core):
    """The oracle as it stands (plain C, OpenMP) on a token sample of the same
    two linears, forward + backward, on this host: once on all its threads
    (N = `tokens`), once on one thread (N = `tokens_1core`), each timed per
    stage (quantize of X, W, dY; the three GEMMs)."""
    import oracle
    import synth
    legs = {}
    all_threads = oracle.num_threads()
    for leg, n_tok, threads in (("all_cores", tokens, all_threads), ("one_core", tokens_1core, 1)):
        oracle.set_num_threads(threads)
        stage_s = {}
        flops = 0
        for idx, (K, M) in enumerate(shapes):
            x, w, dy = synth.operands(n_tok, K, M, seed=100 + idx)
            _oracle_step(oracle, synth.bits(x), synth.bits(w), synth.bits(dy), stage_s)
            flops += 6 * n_tok * K * M
        t = sum(stage_s.values())
        legs[leg] = {"tokens": n_tok, "threads": threads, "s": round(t, 3),
                     "value": round(flops / t / 1e12, 6), "unit": "TFLOP/s",
                     "stage_s": {k: round(v, 3) for k, v in stage_s.items()}}
    oracle.set_num_threads(all_threads)
    a = legs["all_cores"]
    return {"value": a["value"], "unit": "TFLOP/s", "cores": all_threads, "kind": "oracle",
            "cpu_model": _cpu_model(), "one_core": legs["one_core"], "all_cores": legs["all_cores"],
            "sample": "fwd+bwd of 512->2048 and 2048->512 at N=%d tokens (of 131072) on %d threads, %.1f s; "
                      "and at N=%d on 1 thread, %.1f s" % (tokens, all_threads, a["s"], tokens_1core,
                                                           legs["one_core"]["s"])}


def targets(stages, configs):
    """The goals next to what this run measured: >= 80% of the HBM peak on
    the quantize kernels, >= 70% of the dense FP8 matrix-core peak on the
    large GEMMs (the 8192 x 8192 weight at N = 16384, and the gradient GEMMs
    of 512 -> 8192 at N = 262144)."""
    q = [s["gbs"] / HBM_PEAK_GBS for s in stages if s["stage"].startswith("quant_x") or
         s["stage"].startswith("quant_dy")]
    out = {"quantize_hbm_frac": {"target": 0.80, "measured_min": round(min(q), 3), "measured_max": round(max(q), 3),
                                 "over": "activation and gradient quantizes of the headline step"}}
    if configs:
        fr = []
        for name in ("linear_8192x8192_n16384", "linear_8192x8192_n16384_block"):
            if name in configs:
                fr += [v["mfma_frac"] for v in configs[name]["gemms"].values()]
        for name in ("linear_512x8192_n262144", "linear_512x8192_n262144_block"):
            if name in configs:
                fr += [v["mfma_frac"] for k, v in configs[name]["gemms"].items() if k in ("dgrad", "wgrad")]
        if fr:
            out["large_gemm_mfma_frac"] = {"target": 0.70, "measured_min": round(min(fr), 3),
                                           "measured_max": round(max(fr), 3),
                                           "over": "GEMMs of the 8192x8192 weight at N=16384 and gradient GEMMs of "
                                                   "512->8192 at N=262144, both recipes"}
    return out


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.steps, args.warmup, args.recipe)
        return
    if args.traffic:
        traffic(args.traffic[0], args.traffic[1], args.steps, args.warmup)
        return
    if args.mfma:
        mfma_summary(args.mfma, args.steps, args.warmup)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch

    import fp8_mixed_precision_amax_amd as fp8
    import synth
    fp8.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    N = args.tokens
    shapes = SHAPES
    layers = make_layers(fp8, torch, synth, N, "tensor", dev)
    t0 = time.perf_counter()
    timing = timing_groups(torch, linear_step(layers), args.steps, args.warmup)
    wall = time.perf_counter() - t0
    ms = timing["ms"]
    flops = sum(6 * N * K * M for K, M in shapes)
    value = flops / (ms / 1e3) / 1e12
    print("timed %d steps in %d groups: median group %.4f ms/step, mean %.4f ms/step (wall %.3f s)" %
          (args.steps, len(timing["group_steps"]), ms, timing["mean_ms"], wall), file=sys.stderr, flush=True)

    if args.copy_reference:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.no_breakdown:
        print(json.dumps({"ms_per_step": round(ms, 4), "value": round(value, 2)}), flush=True)
        return
    stages, inst_ms = stage_times(fp8, torch, layers, args.reps)
    print("instrumented steps: %.4f ms/step (events between calls)" % inst_ms, file=sys.stderr, flush=True)
    for s in stages:
        print("  %-24s %8.4f ms  %s" % (s["stage"], s["ms"],
                                        ("%.1f TFLOP/s %.0f GB/s" % (s["tflops"], s["gbs"])) if "flops" in s
                                        else "%.0f GB/s" % s["gbs"]), file=sys.stderr, flush=True)
    q = [s for s in stages if s["stage"].startswith("quant")]
    quant_gbs = sum(s["bytes"] for s in q) / sum(s["ms"] for s in q) / 1e6
    dom = max(stages, key=lambda s: s["ms"])     # the stage (one library call) that takes longest
    lat = latency_small(fp8, torch, synth, dev)
    print("512->512 at N=1024: %.2f us/step eager, %.2f us/step replayed from a HIP graph" %
          (lat["us_per_step"], lat["us_per_step_graph"]), file=sys.stderr, flush=True)
    block = None
    if not args.no_block:
        # the same two linears under block scaling (X, dY 1x128; W 128x128)
        del layers
        torch.cuda.empty_cache()
        blayers = make_layers(fp8, torch, synth, N, "block", dev)
        bms = time_steps(torch, blayers, args.steps, args.warmup)
        bst, binst_ms = stage_times(fp8, torch, blayers, args.reps, "block")
        print("block scaling: %.4f ms/step" % bms, file=sys.stderr, flush=True)
        for st in bst:
            print("  %-24s %8.4f ms  %s" % (st["stage"], st["ms"],
                                            ("%.1f TFLOP/s %.0f GB/s" % (st["tflops"], st["gbs"])) if "flops" in st
                                            else "%.0f GB/s" % st["gbs"]), file=sys.stderr, flush=True)
        bq = [st for st in bst if st["stage"].startswith("quant")]
        block = {"recipe": "X, dY 1x128 blocks; W 128x128 blocks", "value": round(flops / (bms / 1e3) / 1e12, 2),
                 "unit": "TFLOP/s", "ms_per_step": round(bms, 4),
                 "quantize_gbs": round(sum(st["bytes"] for st in bq) / sum(st["ms"] for st in bq) / 1e6, 1),
                 "instrumented_ms_per_step": round(binst_ms, 4),
                 "stages": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in st.items()} for st in bst],
                 "roofline": roofline_of(max(bst, key=lambda st: st["ms"]))}
        block["roofline"]["traffic"] = None
        del blayers
        torch.cuda.empty_cache()
    chain = None
    if not args.no_block:
        chain = chain_times(fp8, torch, synth, N, args.steps, args.warmup, dev)
        print("stacked linears: %.4f ms/step, with the amax hand-off %.4f ms/step" %
              (chain["ms_per_step"], chain["ms_per_step_handoff"]), file=sys.stderr, flush=True)
    bf16 = None
    if not args.no_block:
        bf16 = bf16_comparator(fp8, torch, synth, N, args.steps, args.warmup, args.reps, dev)
        bf16["fp8_speedup"] = round(bf16["ms_per_step"] / ms, 3)
        bf16["fp8_speedup_vs_hipblaslt"] = round(bf16["ms_per_step_hipblaslt"] / ms, 3)
        print("bf16 comparator: hand-written %.4f ms/step, hipBLASLt %.4f ms/step (FP8 step %.2fx / %.2fx faster); "
              "GEMMs %s" % (bf16["ms_per_step"], bf16["ms_per_step_hipblaslt"], bf16["fp8_speedup"],
                            bf16["fp8_speedup_vs_hipblaslt"],
                            ", ".join("%s %.0f" % (k, v["tflops"]) for k, v in bf16["gemms"].items())),
              file=sys.stderr, flush=True)
    delayed = None
    if not args.no_block:
        delayed = delayed_quant_times(fp8, torch, synth, N, args.reps, dev)
        print("delayed-scaling quantize %.4f ms (%.0f GB/s), current scaling %.4f ms" %
              (delayed["ms_delayed"], delayed["gbs_delayed"], delayed["ms_current"]), file=sys.stderr, flush=True)
    mlp = None
    if not args.no_block:
        mlp = mlp_gelu_times(fp8, torch, synth, N, args.steps, args.warmup, args.reps, dev)
        print("MLP block with GELU: fused %.4f ms, unfused %.4f ms, fused with the GELU amax hand-off %.4f ms; "
              "GELU quantize fused %.4f ms, unfused %.4f ms, from the keys %.4f ms" %
              (mlp["block"]["ms_fused"], mlp["block"]["ms_unfused"], mlp["block"]["ms_fused_gelu_handoff"],
               mlp["tensor"]["gelu_fused"]["ms"], mlp["tensor"]["gelu_unfused"]["ms"],
               mlp["block"]["gelu_quantize_from_keys_ms"]), file=sys.stderr, flush=True)
    configs = None
    stack = None
    if not args.no_block:
        configs = config_times(fp8, torch, synth, args.steps, args.warmup, args.reps, dev)
        stack = {r: mlp_stack_times(fp8, torch, synth, N, 2, dev, r) for r in ("tensor", "block")}
        for r, v in stack.items():
            print("MLP stack (%s): %.3f ms/cycle cached, %.3f uncached%s" %
                  (r, v["ms_per_cycle_cached"], v["ms_per_cycle_uncached"],
                   ", %.3f cached with the amax hand-off" % v["ms_per_cycle_cached_handoff"]
                   if "ms_per_cycle_cached_handoff" in v else ""), file=sys.stderr, flush=True)
    ceil = None
    if not args.no_block and not args.no_ceilings:
        ceil = ceilings(fp8, torch, synth, dev)
        if ceil:
            print("ceilings: HBM read %.0f, write %.0f, copy %.0f GB/s; MFMA-only %.0f TFLOP/s at %.2f GHz; "
                  "sustained GEMM %s" % (ceil["hbm_read_gbs"], ceil["hbm_write_gbs"], ceil["hbm_copy_gbs"],
                                         ceil["mfma_only_tflops"], ceil["mfma_only_shader_ghz"],
                                         ceil["sustained_gemm"]), file=sys.stderr, flush=True)
    pages_tflops = sum(6 * 131072 * K * M for K, M in shapes) / (sum(PAGES_MS[s] for s in shapes) / 1e3) / 1e12

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "timing": {"protocol": "median of %d timing groups of %s steps (events on the launch stream)" %
                   (len(timing["group_steps"]), "/".join(str(n) for n in timing["group_steps"])),
                   "ms_per_step_mean": round(timing["mean_ms"], 4),
                   "group_ms_per_step": [round(v, 4) for v in timing["group_ms"]]},
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": round(value / pages_tflops, 3) if N == 131072 else None,
        "baseline_note": "pages' RTX 4090 fused-layout FP8 medians (5.4075 + 5.4264 ms = %.1f TFLOP/s): context" % pages_tflops,
        "dtype": "fp8(e4m3,e5m2)->fp32 accum->bf16", "data": "synthetic",
        "config": {"workload": "fp8 linear 512->2048 + 2048->512 fwd+bwd, N=%d, tensorwise current scaling" % N,
                   "tokens": N, "shapes": ["512x2048", "2048x512"], "recipe": "tensor"},
        "quantize_gbs": round(quant_gbs, 1),
        "instrumented_ms_per_step": round(inst_ms, 4),
        "stages": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()} for s in stages],
        "roofline": roofline_of(dom),
        "cpu_baseline": None,
        "latency_512x512_n1024": lat,
        "targets": targets(stages, configs),
        "block_scaling": block,
        "amax_handoff": chain,
        "bf16_comparator": bf16,
        "delayed_scaling_quantize": delayed,
        "mlp_gelu": mlp,
        "other_configs": configs,
        "mlp_stack_weight_cache": stack,
        "ceilings": ceil,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shapes, args.cpu_tokens, args.cpu_tokens_1core)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
