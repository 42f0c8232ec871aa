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
dominant kernel and the oracle's throughput on host cores (cpu_baseline).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 linear fwd+bwd TFLOP/s incl. quantize at N=131072; quantize GB/s"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
RIDGE = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)      # FLOP per byte
# RTX 4090 fused-layout FP8 medians of the pages (ms): context, not a target
PAGES_MS = {(512, 2048): 5.4075, (2048, 512): 5.4264}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tokens", type=int, default=131072)
    ap.add_argument("--reps", type=int, default=20, help="repetitions per stage in the breakdown")
    ap.add_argument("--cpu-tokens", type=int, default=65536, help="token sample of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def stage_times(fp8, torch, layers, reps):
    """Average duration of each kernel-level call of one step, timed with
    events on the stream the kernels run on (torch's current stream)."""
    res = []
    for L in layers:
        lin, N, K, M = L["lin"], L["N"], L["K"], L["M"]
        wq = lin.w_q
        E4, E5, T = fp8.E4M3, fp8.E5M2, fp8.SCALE_TENSOR
        sx, sw, sdy = (fp8.gemm_scale(t.scale_inv) for t in (lin.saved_x, wq, lin.dy_q))
        tag = "%dx%d" % (K, M)
        calls = [
            ("quant_x_" + tag, "quant", N * K, lambda: fp8.quantize(L["x"], E4, T, out=lin.saved_x)),
            ("quant_w_" + tag, "quant", M * K, lambda: fp8.quantize(L["w"], E4, T, out=wq)),
            ("gemm_fprop_" + tag, "gemm", (N, M, K), lambda: fp8.gemm(lin.saved_x.q_row, E4, sx, wq.q_row, E4, sw, out=L["y"])),
            ("quant_dy_" + tag, "quant", N * M, lambda: fp8.quantize(L["dy"], E5, T, out=lin.dy_q)),
            ("gemm_dgrad_" + tag, "gemm", (N, K, M), lambda: fp8.gemm(lin.dy_q.q_row, E5, sdy, wq.q_col, E4, sw, out=L["dx"])),
            ("gemm_wgrad_" + tag, "gemm", (M, K, N), lambda: fp8.gemm(lin.dy_q.q_col, E5, sdy, lin.saved_x.q_col, E4, sx, out=L["dw"])),
        ]
        for name, kind, size, fn in calls:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            if kind == "quant":
                byts = 6 * size            # amax read 2 + cast read 2 + two 1-byte layouts
                res.append({"stage": name, "ms": ms, "bytes": byts, "gbs": byts / ms / 1e6})
            else:
                I, J, Kc = size
                flops = 2 * I * J * Kc
                byts = I * Kc + J * Kc + 2 * I * J
                res.append({"stage": name, "ms": ms, "flops": flops, "bytes": byts,
                            "tflops": flops / ms / 1e9, "gbs": byts / ms / 1e6, "ai": flops / byts})
    return res


def roofline_of(stage):
    if "flops" in stage and stage["ai"] >= RIDGE:
        return {"bound": "mfma", "achieved": round(stage["tflops"], 1), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(stage["tflops"] / FP8_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": stage["stage"]}
    return {"bound": "hbm", "achieved": round(stage["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(stage["gbs"] / HBM_PEAK_GBS, 4), "traffic": None, "kernel": stage["stage"]}


def cpu_baseline(shapes, tokens):
    """The oracle as it stands (plain C, OpenMP) on a token sample of the same
    two linears, forward + backward, on this host's cores."""
    import oracle
    import synth
    t_total = 0.0
    flops = 0
    for idx, (K, M) in enumerate(shapes):
        x, w, dy = synth.operands(tokens, K, M, seed=100 + idx)
        xb, wb, dyb = synth.bits(x), synth.bits(w), synth.bits(dy)
        t0 = time.perf_counter()
        _, ctx = oracle.linear_fwd(xb, wb, "tensor")
        oracle.linear_bwd(dyb, ctx)
        t_total += time.perf_counter() - t0
        flops += 6 * tokens * K * M
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "fwd+bwd of 512->2048 and 2048->512 at N=%d tokens (of 131072), %.1f s" % (tokens, t_total)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch

    import fp8_mixed_precision_amax_amd as fp8
    import synth
    fp8.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    N = args.tokens
    shapes = [(512, 2048), (2048, 512)]
    layers = []
    for idx, (K, M) in enumerate(shapes):
        x, w, dy = synth.operands_on_device(N, K, M, seed=idx, device=dev)
        lin = fp8.Fp8Linear(N, K, M, fp8.RECIPE_TENSOR, device=dev)
        layers.append({"N": N, "K": K, "M": M, "x": x, "w": w, "dy": dy, "lin": lin,
                       "y": torch.empty((N, M), dtype=torch.bfloat16, device=dev),
                       "dx": torch.empty((N, K), dtype=torch.bfloat16, device=dev),
                       "dw": torch.empty((M, K), dtype=torch.bfloat16, device=dev)})

    def step():
        for L in layers:
            L["lin"].forward(L["x"], L["w"], y=L["y"])
            L["lin"].backward(L["dy"], dx=L["dx"], dw=L["dw"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    flops = sum(6 * N * K * M for K, M in shapes)
    value = flops / (ms / 1e3) / 1e12
    print("timed %d steps: %.4f ms/step (wall %.3f s)" % (args.steps, ms, wall), file=sys.stderr, flush=True)

    stages = stage_times(fp8, torch, layers, args.reps)
    for s in stages:
        print("  %-24s %8.4f ms  %s" % (s["stage"], s["ms"],
                                        ("%.1f TFLOP/s %.0f GB/s" % (s["tflops"], s["gbs"])) if "flops" in s
                                        else "%.0f GB/s" % s["gbs"]), file=sys.stderr, flush=True)
    q = [s for s in stages if s["stage"].startswith("quant")]
    quant_gbs = sum(s["bytes"] for s in q) / sum(s["ms"] for s in q) / 1e6
    dom = max(stages, key=lambda s: s["ms"])
    pages_tflops = sum(6 * 131072 * K * M for K, M in shapes) / (sum(PAGES_MS[s] for s in shapes) / 1e3) / 1e12

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": round(value / pages_tflops, 3) if N == 131072 else None,
        "baseline_note": "pages' RTX 4090 fused-layout FP8 medians (5.4075 + 5.4264 ms = %.1f TFLOP/s): context" % pages_tflops,
        "dtype": "fp8(e4m3,e5m2)->fp32 accum->bf16", "data": "synthetic",
        "config": {"workload": "fp8 linear 512->2048 + 2048->512 fwd+bwd, N=%d, tensorwise current scaling" % N,
                   "tokens": N, "shapes": ["512x2048", "2048x512"], "recipe": "tensor"},
        "quantize_gbs": round(quant_gbs, 1),
        "stages": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()} for s in stages],
        "roofline": roofline_of(dom),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shapes, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
