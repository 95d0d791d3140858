#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 linear-layer path on one MI355X.

One step = the whole hot path of a training-step linear layer (Qwen3-8B
down_proj shape, X [8192 x 12288], W [4096 x 12288], dY [8192 x 4096], all
bf16, seeded synthetic data) on the GPU:
    128x128 weight quantization (+ transposed codes)
    dual 1x128 quantization of X  (row-wise + token-axis)
    FProp  Y  = X W^T
    dual 1x128 quantization of dY (row-wise + token-axis)
    DGrad  dX = dY W
    WGrad  dW = dY^T X
value = 3 * 2*N*D*C FLOP / step time (TFLOP/s), inputs resident in HBM.
Three copies of every input (1.1 GB) rotate between steps so nothing is
reused from the 256 MB Infinity Cache across steps.

The K timed steps carry no timing events; a second pass of K steps with an
event around every launch gives the per-kernel figures.

Printed JSON line: the contract fields, a per-kernel breakdown (HIP-event
time per launch on the launch stream, TFLOP/s or GB/s, fraction of the
MI355X peak), the roofline of the dominant kernel, a bf16 hipBLASLt
baseline on the same GEMM shapes, and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

METRIC = "block-scaled FP8 GEMM TFLOPS (FProp/DGrad/WGrad) + quantize GB/s, % of peak"
N, C, D = 8192, 12288, 4096
NCOPIES = 3                   # input copies rotated between timed steps (1.1 GB)
REPS = 50                     # timed launches per kernel in the side sections


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first (after only 5 the timed steps still ran ~5%% slow)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the decode / MXFP8 / MoE kernel timings")
    ap.add_argument("--only-section", choices=["fused", "other"],
                    help="time one side section alone and print its JSON (no training step)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="minimum duration of the timed oracle baseline sample (seconds)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn two rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE, WRITE_SIZE) of this benchmark into profiles/traffic_gemm_train.json")
    ap.add_argument("--counters", nargs=2, metavar=("SQ1_CSV", "SQ2_CSV"),
                    help="no GPU work: turn the two rocprofv3 --pmc SQ counter passes of this benchmark "
                         "(SQ_PASS1, SQ_PASS2) into profiles/counters_train_layer.md")
    return ap.parse_args()


def src_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_scaled_fp8_02_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes():
    """Bytes each kernel must move at minimum (inputs once, outputs once)."""
    g = (C + 127) // 128
    gd = (D + 127) // 128
    gn = (N + 127) // 128
    return {
        "quant_weight": D * C * 2 + D * C * 2 + gd * g * 4,            # bf16 in, q + qT, scales
        "quant_dual_X": N * C * 2 + 2 * N * C + N * g * 4 + C * gn * 4,
        "quant_dual_dY": N * D * 2 + 2 * N * D + N * gd * 4 + D * gn * 4,
        "fprop": N * C + D * C + N * g * 4 + gd * g * 4 + N * D * 2,
        "dgrad": N * D + C * D + N * gd * 4 + gd * g * 4 + N * C * 2,
        "wgrad": D * N + C * N + D * gn * 4 + C * gn * 4 + D * C * 2,
    }


KERNEL_ORDER = ["quant_weight", "quant_dual_X", "fprop", "quant_dual_dY", "dgrad", "wgrad"]
CALIB_BYTES = 256 << 20       # the copy kernel reads and writes this many bytes


def calibrate_copy(torch, dev):
    """A plain copy kernel of known size (torch's elementwise neg over 256 MiB
    of fp32), run once before the timed region; its FETCH_SIZE / WRITE_SIZE
    readings calibrate the counters of the library's kernels."""
    a = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    out = torch.empty_like(a)
    torch.neg(a, out=out)
    torch.cuda.synchronize()
    del a, out


def traffic_summary(fetch_csv, write_csv):
    """Per-launch HBM-side bytes of every library kernel from two --pmc runs.
    Counter values are KiB per dispatch, summed over the dispatch's instances;
    each is scaled by copy_bytes / counter reading of the calibration copy."""
    import csv

    def load(path, counter):
        per = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            e = per.setdefault(d, [r["Kernel_Name"], 0.0])
            e[1] += float(r["Counter_Value"]) * 1024.0
        return [per[d] for d in sorted(per)]

    out = {"src_sha": src_sha("gemm.hip", "gemm_common.hpp", "device_common.hpp"),
           "src_sha_quant": src_sha("quant.hip", "device_common.hpp"),
           "copy_bytes": CALIB_BYTES, "kernels": {}}
    for counter, path, key in (("FETCH_SIZE", fetch_csv, "fetch"), ("WRITE_SIZE", write_csv, "write")):
        rows = load(path, counter)
        calib = [v for n, v in rows if "neg" in n.lower()]
        if not calib:
            raise SystemExit(f"{path}: no calibration copy dispatch found")
        factor = CALIB_BYTES / calib[0]
        out[f"{key}_factor"] = round(factor, 5)
        lib = [(n, v) for n, v in rows if "k_quant" in n or "k_gemm" in n]
        for k, (n, v) in enumerate(lib):
            name = KERNEL_ORDER[k % len(KERNEL_ORDER)]
            e = out["kernels"].setdefault(name, {"kernel": n.split("(")[0], "fetch": [], "write": []})
            e[key].append(v * factor)
    for name, e in out["kernels"].items():
        e["fetch_bytes"] = round(float(np.median(e.pop("fetch"))))
        e["write_bytes"] = round(float(np.median(e.pop("write"))))
        e["bytes_per_launch"] = e["fetch_bytes"] + e["write_bytes"]
        e["alg_bytes"] = algorithmic_bytes()[name]
    path = os.path.join(ROOT, "profiles", "traffic_gemm_train.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


# The two SQ counter passes summarised by --counters (at most 8 SQ and 2
# GRBM counters per pass).
SQ_PASS1 = ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_VALU_MFMA_BUSY_CYCLES",
            "SQ_INSTS_MFMA", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"]
SQ_PASS2 = ["SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_LDS_BANK_CONFLICT",
            "SQ_INSTS_VALU", "SQ_ACTIVE_INST_MISC", "SQ_INST_LEVEL_LDS", "SQ_CYCLES"]


def counters_summary(sq1_csv, sq2_csv):
    """Per-kernel SQ counter figures of the training-layer step from two
    --pmc passes (values summed over a dispatch's instances; medians over the
    step's launches), written to profiles/counters_train_layer.md with the
    hashes of the kernel sources they were taken on."""
    import csv

    def load(path):
        per = {}
        for r in csv.DictReader(open(path)):
            d = int(r["Dispatch_Id"])
            e = per.setdefault(d, {"name": r["Kernel_Name"], "t": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return [per[d] for d in sorted(per) if "k_quant" in per[d]["name"] or "k_gemm" in per[d]["name"]]

    a, b = load(sq1_csv), load(sq2_csv)
    if len(a) != len(b) or len(a) % len(KERNEL_ORDER):
        raise SystemExit(f"counter passes disagree: {len(a)} and {len(b)} library dispatches")
    rows = []
    for k, step in enumerate(KERNEL_ORDER):
        ds = [{**a[i], **{c: v for c, v in b[i].items() if c not in ("name", "t")}}
              for i in range(k, len(a), len(KERNEL_ORDER))]
        med = lambda f: float(np.median([f(d) for d in ds]))
        t = med(lambda d: d["t"])
        clock = med(lambda d: d["GRBM_GUI_ACTIVE"] / 8 / d["t"])
        ent = {"step": step, "kernel": ds[0]["name"].split("(")[0].replace("void ", ""), "us": t * 1e6,
               "ghz": clock / 1e9}
        if med(lambda d: d["SQ_INSTS_MFMA"]) > 0:
            ent["mfma_busy"] = med(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * d["t"] * d["GRBM_GUI_ACTIVE"] / 8 / d["t"]))
            ent["busy_per_mfma"] = med(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / d["SQ_INSTS_MFMA"])
            ent["valu_per_mfma"] = med(lambda d: d["SQ_INSTS_VALU"] / d["SQ_INSTS_MFMA"])
        for key, c in (("wait", "SQ_WAIT_ANY"), ("issue_wait", "SQ_WAIT_INST_ANY"), ("active", "SQ_ACTIVE_INST_ANY"),
                       ("lds_active", "SQ_ACTIVE_INST_LDS")):
            ent[key] = med(lambda d: d[c] / d["SQ_WAVE_CYCLES"])
        ent["lds_bank_conflict_per_lds"] = med(lambda d: d["SQ_LDS_BANK_CONFLICT"] / max(d["SQ_INSTS_LDS"], 1.0))
        rows.append(ent)
    pct = lambda v: f"{100 * v:.0f}%"
    lines = [
        "# SQ counters: training-step linear layer GEMMs and tile quantizers (X 8192x12288, W 4096x12288, dY 8192x4096)",
        "",
        "Commands (from the repository root, on one MI355X; two counter passes over the same launches):",
        "",
        "```",
        "timeout -s KILL 120 rocprofv3 --pmc " + " ".join(SQ_PASS1) + " --output-format csv -d $PWD/gpurun_out/gsq1 -o b "
        "-- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-other",
        "timeout -s KILL 120 rocprofv3 --pmc " + " ".join(SQ_PASS2) + " --output-format csv -d $PWD/gpurun_out/gsq2 -o b "
        "-- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-other",
        "python3 bench.py --counters gpurun_out/gsq1/b_counter_collection.csv gpurun_out/gsq2/b_counter_collection.csv",
        "```",
        "",
        f"Kernel sources hashed as gemm {src_sha('gemm.hip', 'gemm_common.hpp', 'device_common.hpp')}, "
        f"quant {src_sha('quant.hip', 'device_common.hpp')}.",
        "",
        "Derived per kernel (median over the step's launches; the counter runs serialize launches, so durations are",
        "those of the profiled runs): clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /",
        "(1024 SIMDs x cycles); VALU per MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA (the MFMAs included); wait, issue-wait,",
        "active and LDS-active = SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_ANY, SQ_ACTIVE_INST_LDS over SQ_WAVE_CYCLES.",
        "",
        "| Step | Kernel | Duration (us) | Clock (GHz) | MFMA busy | Busy cycles per MFMA | VALU per MFMA | Wait | Issue-wait | Active | LDS active | Bank conflicts per LDS instr. |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    for e in rows:
        if "mfma_busy" in e:
            mf = f"{pct(e['mfma_busy'])} | {e['busy_per_mfma']:.1f} | {e['valu_per_mfma']:.2f}"
        else:
            mf = "- | - | -"
        lines.append(f"| {e['step']} | `{e['kernel']}` | {e['us']:.1f} | {e['ghz']:.2f} | {mf} | {pct(e['wait'])} | "
                     f"{pct(e['issue_wait'])} | {pct(e['active'])} | {pct(e['lds_active'])} | "
                     f"{e['lds_bank_conflict_per_lds']:.2f} |")
    path = os.path.join(ROOT, "profiles", "counters_train_layer.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    args = parse()
    if args.traffic:
        traffic_summary(*args.traffic)
        return
    if args.counters:
        counters_summary(*args.counters)
        return
    if args.gpus != 1:
        print(f"bench.py times one GPU's share of the work; --gpus {args.gpus} is not supported "
              f"(run it with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_fp8_02_amd as fb
    from block_scaled_fp8_02_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only_section:                        # one side section alone (for kernel traces)
        fn = {"fused": fused_producers, "other": other_workloads}[args.only_section]
        print(json.dumps({"section": args.only_section, "result": fn(torch, fb, wl, dev, args.seed)}), flush=True)
        return
    t0 = time.time()
    w = wl.train(args.seed)
    print(f"[bench] inputs drawn in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def to_dev(bits):
        return torch.from_numpy(bits).view(torch.bfloat16).to(dev)

    # three copies of every input (3 x 368 MB = 1.1 GB) rotate between steps:
    # more than the 256 MB Infinity Cache and the L2s can hold, so every step
    # reads its bf16 inputs from HBM
    copies = []
    for k in range(NCOPIES):
        Xd, Wd, Gd = to_dev(w["X"]), to_dev(w["W"]), to_dev(w["dY"])
        copies.append((Xd, Wd, Gd))
    # preallocated outputs (allocation is outside the timed region)
    cdiv = lambda a, b: (a + b - 1) // b
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    bufs = dict(
        wq=torch.empty((D, C), **u8), ws=torch.empty((cdiv(D, 128), cdiv(C, 128)), **f32),
        wqT=torch.empty((C, D), **u8),
        xq=torch.empty((N, C), **u8), xs=torch.empty((N, cdiv(C, 128)), **f32),
        xqT=torch.empty((C, N), **u8), xsT=torch.empty((C, cdiv(N, 128)), **f32),
        gq=torch.empty((N, D), **u8), gs=torch.empty((N, cdiv(D, 128)), **f32),
        gqT=torch.empty((D, N), **u8), gsT=torch.empty((D, cdiv(N, 128)), **f32),
        y=torch.empty((N, D), dtype=torch.bfloat16, device=dev),
        dx=torch.empty((N, C), dtype=torch.bfloat16, device=dev),
        dw=torch.empty((D, C), dtype=torch.bfloat16, device=dev),
    )
    b = bufs
    names = KERNEL_ORDER
    calibrate_copy(torch, dev)
    events = {n: [] for n in names}

    def step(i, record):
        Xd, Wd, Gd = copies[i % NCOPIES]
        ev = []

        def mark():
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                ev.append(e)
        mark()
        fb.fp8_quantize_weight_128x128(Wd, transpose=True, q=b["wq"], s=b["ws"], qT=b["wqT"])
        mark()
        fb.fp8_quantize_transposed(Xd, rowwise=True, qT=b["xqT"], sT=b["xsT"], q=b["xq"], s=b["xs"])
        mark()
        fb.fp8_gemm_fprop(b["xq"], b["xs"], b["wq"], b["ws"], N, D, C, y=b["y"])
        mark()
        fb.fp8_quantize_transposed(Gd, rowwise=True, qT=b["gqT"], sT=b["gsT"], q=b["gq"], s=b["gs"])
        mark()
        fb.fp8_gemm_dgrad(b["gq"], b["gs"], b["wqT"], b["ws"], N, D, C, dx=b["dx"])
        mark()
        fb.fp8_gemm_wgrad(b["gqT"], b["gsT"], b["xqT"], b["xsT"], N, D, C, dw=b["dw"])
        mark()
        return ev

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    # the timed steps carry no instrumentation: a timing event between two
    # dependent kernels costs the GPU several microseconds of its own
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i, False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    # then the same steps again with an event around every kernel, for the
    # per-kernel figures (their sum exceeds the clean step by the events' cost)
    all_ev = []
    t_start = time.perf_counter()
    for i in range(args.steps):
        all_ev.append(step(i, True))
    torch.cuda.synchronize()
    elapsed_instrumented = time.perf_counter() - t_start
    for ev in all_ev:
        for k, n in enumerate(names):
            events[n].append(ev[k].elapsed_time(ev[k + 1]) * 1e-3)   # seconds

    flops_gemm = 2.0 * N * D * C
    abytes = algorithmic_bytes()
    kernels = {}
    for n in names:
        t = float(np.mean(events[n]))
        p10, p50, p90 = np.percentile(events[n], [10, 50, 90])
        ent = {"us": round(t * 1e6, 2), "us_p10": round(p10 * 1e6, 2), "us_median": round(p50 * 1e6, 2),
               "us_p90": round(p90 * 1e6, 2)}
        if n in ("fprop", "dgrad", "wgrad"):
            tf = flops_gemm / t / 1e12
            ent.update(tflops=round(tf, 1), frac_fp8_peak=round(tf / PEAK_FP8_TFLOPS, 4))
        gbs = abytes[n] / t / 1e9
        ent.update(alg_bytes=abytes[n], gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
        kernels[n] = ent
    step_s = elapsed / args.steps
    value = 3 * flops_gemm / step_s / 1e12

    # warm, after the timed steps: each kernel 20 times back-to-back on one
    # set of inputs, which then stays in the Infinity Cache between launches
    # (the cold figures above are the headline)
    Xd, Wd, Gd = copies[0]
    warm_fns = {
        "quant_weight": lambda: fb.fp8_quantize_weight_128x128(Wd, transpose=True, q=b["wq"], s=b["ws"], qT=b["wqT"]),
        "quant_dual_X": lambda: fb.fp8_quantize_transposed(Xd, rowwise=True, qT=b["xqT"], sT=b["xsT"], q=b["xq"],
                                                           s=b["xs"]),
        "fprop": lambda: fb.fp8_gemm_fprop(b["xq"], b["xs"], b["wq"], b["ws"], N, D, C, y=b["y"]),
        "quant_dual_dY": lambda: fb.fp8_quantize_transposed(Gd, rowwise=True, qT=b["gqT"], sT=b["gsT"], q=b["gq"],
                                                            s=b["gs"]),
        "dgrad": lambda: fb.fp8_gemm_dgrad(b["gq"], b["gs"], b["wqT"], b["ws"], N, D, C, dx=b["dx"]),
        "wgrad": lambda: fb.fp8_gemm_wgrad(b["gqT"], b["gsT"], b["xqT"], b["xsT"], N, D, C, dw=b["dw"]),
    }
    if not args.no_other:                        # a side measurement, like the other sections
        for n, fn in warm_fns.items():
            kernels[n]["us_warm"] = round(time_warm(torch, fn) * 1e6, 2)

    dom = max(("fprop", "dgrad", "wgrad"), key=lambda n: kernels[n]["us"])
    t_dom = kernels[dom]["us"] * 1e-6
    achieved = flops_gemm / t_dom / 1e12
    # HBM-side bytes per launch from the committed counter runs, used only
    # while the kernel sources are the ones the counters were taken on
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic_gemm_train.json")
    if os.path.exists(tfile):
        tj = json.load(open(tfile))
        fresh = {"gemm": tj.get("src_sha") == src_sha("gemm.hip", "gemm_common.hpp", "device_common.hpp"),
                 "quant": tj.get("src_sha_quant") == src_sha("quant.hip", "device_common.hpp")}
        for n, e in tj.get("kernels", {}).items():
            if n in kernels and fresh["quant" if n.startswith("quant") else "gemm"]:
                kernels[n]["traffic_bytes"] = e["bytes_per_launch"]
        traffic = kernels[dom].get("traffic_bytes")
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                "traffic": traffic, "alg_bytes": abytes[dom]}

    # bf16 hipBLASLt baseline on the same three GEMM shapes
    Xd, Wd, Gd = copies[0]
    bf = {}
    for name, fn in (("fprop", lambda: torch.matmul(Xd, Wd.t())),
                     ("dgrad", lambda: torch.matmul(Gd, Wd)),
                     ("wgrad", lambda: torch.matmul(Gd.t(), Xd))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        tf = flops_gemm / t / 1e12
        bf[name] = {"us": round(t * 1e6, 1), "tflops": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}

    # measured ceilings on this GPU, same process: a streaming copy (1 GiB
    # read + 1 GiB written) and the per-tensor-scaled fp8 GEMM of hipBLASLt
    # on the same codes (no per-block scales: an upper reference for the
    # block-scaled kernels, which also pay the per-block promotion)
    ceil = {}
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(REPS):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 / (e0.elapsed_time(e1) * 1e-3 / REPS) / 1e9
    ceil["hbm_copy_gbs"] = round(copy_gbs, 1)
    del src, dst
    for n in ("quant_weight", "quant_dual_X", "quant_dual_dY"):
        kernels[n]["frac_measured_copy"] = round(kernels[n]["gbs"] / copy_gbs, 4)
    # the same copy at each quantizer's own size (half its algorithmic bytes
    # read, half written), rotating over six sources so that none is in the
    # Infinity Cache: the ceiling a kernel of that size meets, ramp included
    same = {}
    for n in ("quant_weight", "quant_dual_X", "quant_dual_dY"):
        nel = kernels[n]["alg_bytes"] // 8
        srcs = [torch.empty(nel, dtype=torch.float32, device=dev).fill_(1.0) for _ in range(6)]
        dst = torch.empty(nel, dtype=torch.float32, device=dev)
        for i in range(6):
            dst.copy_(srcs[i])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(30):
            dst.copy_(srcs[i % 6])
        e1.record()
        torch.cuda.synchronize()
        gbs = 2 * nel * 4 / (e0.elapsed_time(e1) * 1e-3 / 30) / 1e9
        same[n] = round(gbs, 1)
        kernels[n]["frac_same_size_copy"] = round(kernels[n]["gbs"] / gbs, 4)
        del srcs, dst
    ceil["hbm_copy_gbs_same_size"] = same
    one = torch.ones((), device=dev)
    f8 = lambda t: t.view(torch.float8_e4m3fn)
    tw = {}
    for name, (a_, b_) in (("fprop", (b["xq"], b["wq"])), ("dgrad", (b["gq"], b["wqT"])),
                           ("wgrad", (b["gqT"], b["xqT"]))):
        try:
            fn = lambda: torch._scaled_mm(f8(a_), f8(b_).t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(REPS):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / REPS
            tw[name] = {"us": round(t * 1e6, 1), "tflops": round(flops_gemm / t / 1e12, 1)}
        except Exception as ex:                                     # no fp8 GEMM in this torch build
            tw[name] = {"error": str(ex)[:120]}
    ceil["fp8_tensorwise_hipblaslt"] = tw
    # matrix-core throughput on random register operands, all compute units
    ceil["mfma_random_operands"] = mfma_peaks(torch, fb, dev)
    pk8 = ceil["mfma_random_operands"]["fp8_16x16x128"]["tflops"]
    pk16 = ceil["mfma_random_operands"]["bf16_16x16x32"]["tflops"]
    fmt = {"fprop": "fp8_with_block_scale_promotion", "dgrad": "fp8_with_block_scale_promotion",
           "wgrad": "fp8_with_row_scale_promotion"}
    for n in ("fprop", "dgrad", "wgrad"):
        kernels[n]["frac_measured_fp8_mfma"] = round(kernels[n]["tflops"] / pk8, 4)
        kernels[n]["frac_measured_format_ceiling"] = round(
            kernels[n]["tflops"] / ceil["mfma_random_operands"][fmt[n]]["tflops"], 4)
    roofline["frac_measured_peak"] = round(roofline["achieved"] / pk8, 4)
    roofline["measured_peak"] = pk8
    # the same kernel against the measured ceiling of its scale format (MFMAs
    # plus the FP32 promotion, no memory traffic)
    roofline["format_ceiling"] = ceil["mfma_random_operands"][fmt[dom]]["tflops"]
    roofline["frac_format_ceiling"] = round(roofline["achieved"] / roofline["format_ceiling"], 4)
    for n, e in bf.items():
        e["frac_measured_bf16_mfma"] = round(e["tflops"] / pk16, 4)

    pow2 = requant = deqbwd = None
    if not args.no_other:
        pow2 = pow2_layer(torch, fb, copies, flops_gemm)
        requant = requant_layer(torch, fb, copies)
        deqbwd = dequant_backward(torch, fb, copies, flops_gemm)
        pk16 = ceil["mfma_random_operands"]["bf16_16x16x32"]["tflops"]
        for n in ("dgrad", "wgrad"):
            deqbwd[n]["frac_measured_bf16_mfma"] = round(deqbwd[n]["tflops"] / pk16, 4)
            deqbwd[n]["speedup_vs_torch_bf16"] = round(bf[n]["us"] / deqbwd[n]["us"], 3)

    other = fused = None
    if not args.no_other:
        del copies, bufs, b
        torch.cuda.empty_cache()
        other = other_workloads(torch, fb, wl, dev, args.seed)
        fused = fused_producers(torch, fb, wl, dev, args.seed)

    tiny = None
    if not args.no_other:
        tiny = tiny_layer(torch, fb, wl, dev, args.seed)

    cpu = cpu_cfg = qerr = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)
        del w
        cpu_cfg = cpu_oracle_configs(args.seed, cpu)
        qerr = quant_error_mx_vs_blockscaled(args.seed)
        if other is not None:
            for op in ("fprop", "dgrad", "wgrad"):
                qerr[op]["tflops_blockscaled"] = other["decode_1x128"][op].get("tflops")
                qerr[op]["tflops_mxfp8"] = other["decode_mxfp8"][op].get("tflops")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "ms_per_step_with_kernel_events": round(elapsed_instrumented / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "training-step linear layer, Qwen3-8B down_proj shape: X bf16 [8192x12288] "
                               "(1% outlier channels x50), W bf16 [4096x12288], dY bf16 [8192x4096]; "
                               "1x128 act/grad + 128x128 weight FP8 path, FProp+DGrad+WGrad",
                   "N": N, "C": C, "D": D, "seed": args.seed, "inputs_resident_in_hbm": True},
        "kernels": kernels, "roofline": roofline, "bf16_baseline": bf, "cpu_baseline": cpu,
        "cpu_oracle_by_config": cpu_cfg,
        "quant_error_mx_vs_blockscaled": qerr,
        "tiny_layer": tiny,
        "measured_ceilings": ceil,
        "pow2_scales_layer": pow2,
        "requant_from_fp8_X": requant,
        "fused_producers": fused,
        "dequantized_backward": deqbwd,
        "other_workloads": other,
    }
    print(json.dumps(out), flush=True)


def time_cold(torch, fn, flush, reps=REPS, warmup=2):
    """Median seconds of fn() on the current stream, each launch preceded
    (outside the events) by a 1 GiB read so that L2 and the Infinity Cache
    hold none of its operands."""
    for _ in range(warmup):
        fn()
    ts = []
    for _ in range(reps):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    return float(np.median(ts))


def time_warm(torch, fn, reps=20, warmup=3):
    """Mean seconds of fn() over reps back-to-back launches on the same
    inputs (warm: whatever fits stays in L2 and the Infinity Cache)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def report(t, alg_bytes, flops=None):
    """Time, rates and the fraction of the kernel's own roofline,
    t_min / t with t_min = max(flops / FP8 peak, bytes / HBM peak)."""
    t_min = max(alg_bytes / (PEAK_HBM_GBS * 1e9), (flops or 0.0) / (PEAK_FP8_TFLOPS * 1e12))
    e = {"us": round(t * 1e6, 2), "alg_bytes": int(alg_bytes), "gbs": round(alg_bytes / t / 1e9, 1),
         "bound": "hbm" if alg_bytes / (PEAK_HBM_GBS * 1e9) >= (flops or 0.0) / (PEAK_FP8_TFLOPS * 1e12) else "mfma",
         "frac_roofline": round(t_min / t, 4)}
    if flops:
        e["tflops"] = round(flops / t / 1e12, 1)
        e["frac_fp8_peak"] = round(flops / t / 1e12 / PEAK_FP8_TFLOPS, 4)
    return e


def pow2_layer(torch, fb, copies, flops_gemm):
    """The same training layer with power-of-two block scales: the quantizers
    also emit E8M0 bytes, and the three GEMMs run on the scaled MFMA (MXFP8
    kernels), with no per-block promotion.  Warm operands like the main
    step; each kernel timed alone over 10 launches."""
    Xd, Wd, Gd = copies[0]
    N, C = Xd.shape
    D = Wd.shape[0]
    xqT, xsT, xeT, xq, xs, xe = fb.fp8_quantize_transposed_pow2(Xd, rowwise=True)
    gqT, gsT, geT, gq, gs, ge = fb.fp8_quantize_transposed_pow2(Gd, rowwise=True)
    wq, ws, wqT, we, weT = fb.fp8_quantize_weight_128x128_pow2(Wd)
    y = torch.empty((N, D), dtype=torch.bfloat16, device=Xd.device)
    dx = torch.empty((N, C), dtype=torch.bfloat16, device=Xd.device)
    dw = torch.empty((D, C), dtype=torch.bfloat16, device=Xd.device)
    runs = {
        "quant_weight": lambda: fb.fp8_quantize_weight_128x128_pow2(Wd),
        "quant_dual_X": lambda: fb.fp8_quantize_transposed_pow2(Xd, rowwise=True),
        "quant_dual_dY": lambda: fb.fp8_quantize_transposed_pow2(Gd, rowwise=True),
        "fprop": lambda: fb.fp8_mx_gemm_fprop(xq, xe, wq, we, N, D, C, y=y),
        "dgrad": lambda: fb.fp8_mx_gemm_dgrad(gq, ge, wqT, weT, N, D, C, dx=dx),
        "wgrad": lambda: fb.fp8_mx_gemm_wgrad(gqT, geT, xqT, xeT, N, D, C, dw=dw),
    }
    out = {}
    for name, fn in runs.items():
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(REPS):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / REPS
        ent = {"us": round(t * 1e6, 2)}
        if name in ("fprop", "dgrad", "wgrad"):
            ent["tflops"] = round(flops_gemm / t / 1e12, 1)
            ent["frac_fp8_peak"] = round(flops_gemm / t / 1e12 / PEAK_FP8_TFLOPS, 4)
        out[name] = ent
    gemm_us = sum(out[n]["us"] for n in ("fprop", "dgrad", "wgrad"))
    out["gemm_tflops"] = round(3 * flops_gemm / (gemm_us * 1e-6) / 1e12, 1)
    return out


def requant_layer(torch, fb, copies):
    """X's two FP8 forms for the training layer made from the saved FP8
    copy: the 1x128 quantizer alone in the forward pass, then the token-axis
    requantizer in the backward pass, against the dual quantizer reading
    bf16 X once for both.  Each kernel timed cold against its own HBM
    roofline; `kept_bytes` is what stays resident between the passes."""
    Xd = copies[0][0]
    N, C = Xd.shape
    cd = lambda a, b: (a + b - 1) // b
    flush = torch.empty(1 << 28, dtype=torch.float32, device=Xd.device).fill_(1.0)
    q, s = fb.fp8_quantize_act_1x128(Xd)
    qT, sT = fb.fp8_requantize_transposed(q, s, C)
    d = fb.fp8_quantize_transposed(Xd, rowwise=True)
    rs, ts = N * cd(C, 128) * 4, C * cd(N, 128) * 4               # row-wise / token-axis scale bytes
    out = {
        "quant_act_1x128_X": report(time_cold(torch, lambda: fb.fp8_quantize_act_1x128(Xd, q, s), flush),
                                    2 * N * C + N * C + rs),
        "requant_X": report(time_cold(torch, lambda: fb.fp8_requantize_transposed(q, s, C, qT, sT), flush),
                            N * C + rs + N * C + ts),
        "quant_dual_X": report(time_cold(torch, lambda: fb.fp8_quantize_transposed(
            Xd, rowwise=True, qT=d[0], sT=d[1], q=d[2], s=d[3]), flush), 2 * N * C + 2 * N * C + rs + ts),
        "kept_bytes": {"bf16_X": 2 * N * C, "fp8_X": N * C + rs},
    }
    del flush
    return out


def dequant_backward(torch, fb, copies, flops_gemm):
    """The training layer's backward in the dequantized mode: DGrad and
    WGrad as bf16 GEMMs (the library's bf16 MFMA kernel) on the forward's
    FP8 W and X codes dequantized to bf16; each entry point's time includes
    the transposing copies that give the GEMM its K-contiguous operands (W^T
    dequantized for DGrad; X^T dequantized and dY^T for WGrad).  Also the
    plain dequantization kernels alone, and the bytes each mode keeps between
    the forward and the backward pass.  Warm operands, REPS launches."""
    Xd, Wd, Gd = copies[0]
    N, C = Xd.shape
    D = Wd.shape[0]
    cd = lambda a, b: (a + b - 1) // b
    xq, xs = fb.fp8_quantize_act_1x128(Xd)
    wq, ws, _ = fb.fp8_quantize_weight_128x128(Wd, transpose=False)
    bf = dict(dtype=torch.bfloat16, device=Xd.device)
    workW, workX = torch.empty((C, D), **bf), torch.empty((C + D, N), **bf)
    plainW, plainX = torch.empty((D, C), **bf), torch.empty((N, C), **bf)
    dx, dw = torch.empty((N, C), **bf), torch.empty((D, C), **bf)
    runs = {
        "dequant_W": (lambda: fb.fp8_dequantize_bf16(wq, ws, fb.FP8B_SCALE_BLOCKS_128X128, C, out=plainW),
                      D * C + cd(D, 128) * cd(C, 128) * 4 + 2 * D * C, None),
        "dequant_X": (lambda: fb.fp8_dequantize_bf16(xq, xs, fb.FP8B_SCALE_ROWS_1X128, C, out=plainX),
                      N * C + N * cd(C, 128) * 4 + 2 * N * C, None),
        "dgrad": (lambda: fb.fp8_dequant_gemm_dgrad(Gd, wq, ws, fb.FP8B_SCALE_BLOCKS_128X128, N, D, C,
                                                    dx=dx, work=workW), None, flops_gemm),
        "wgrad": (lambda: fb.fp8_dequant_gemm_wgrad(Gd, xq, xs, fb.FP8B_SCALE_ROWS_1X128, N, D, C,
                                                    dw=dw, work=workX), None, flops_gemm),
    }
    out = {}
    for name, (fn, nbytes, flops) in runs.items():
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(REPS):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / REPS
        ent = {"us": round(t * 1e6, 2)}
        if nbytes:
            ent["gbs"] = round(nbytes / t / 1e9, 1)
            ent["frac_hbm"] = round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)
        if flops:
            ent["tflops"] = round(flops / t / 1e12, 1)
            ent["frac_bf16_peak"] = round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        out[name] = ent
    fp8_x = N * C + N * cd(C, 128) * 4
    out["kept_bytes"] = {"fp8_backward": 2 * fp8_x, "dequantized_backward": fp8_x,
                         "dequantized_transient_workspace": 2 * (C + D) * N}
    del workW, workX, plainW, plainX, dx, dw
    return out


def fused_producers(torch, fb, wl, dev, seed):
    """The fused producers of the 1x128 quantizer at the training shape
    (Qwen3-8B: hidden 4096, intermediate 12288, 8192 tokens), each timed cold
    against its HBM roofline, beside the unfused pair (torch's bf16 operator
    writing the activation, then the 1x128 quantizer reading it back)."""
    N, H, I = 8192, 4096, 12288
    cd = lambda a, b: (a + b - 1) // b
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    rng = wl.rng_for(seed + 11)
    to = lambda bits: torch.from_numpy(bits).view(torch.bfloat16).to(dev)
    x = to(wl.normal_bf16(rng, (N, H), 1.0))
    w = to(wl.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32)))
    gu = to(wl.normal_bf16(rng, (N, 2 * I), 1.0))
    g, u = gu[:, :I], gu[:, I:]
    out = {}
    q, s, r, _ = fb.fp8_rmsnorm_quantize_1x128(x, w, 1e-6, rstd=True)
    rn_bytes = 2 * N * H + 2 * H + N * H + N * cd(H, 128) * 4 + 4 * N
    out["rmsnorm_quant"] = report(time_cold(torch, lambda: fb.fp8_rmsnorm_quantize_1x128(
        x, w, 1e-6, rstd=r, q=q, s=s), flush), rn_bytes)

    def unfused_rn():
        y = torch.nn.functional.rms_norm(x, (H,), w, eps=1e-6)
        fb.fp8_quantize_act_1x128(y, q, s)
    out["rmsnorm_then_quant_unfused"] = report(time_cold(torch, unfused_rn, flush), rn_bytes)
    qa, sa, _ = fb.fp8_silu_mul_quantize_1x128(g, u)
    sm_bytes = 2 * 2 * N * I + N * I + N * cd(I, 128) * 4
    out["silu_mul_quant"] = report(time_cold(torch, lambda: fb.fp8_silu_mul_quantize_1x128(
        g, u, q=qa, s=sa), flush), sm_bytes)

    def unfused_sm():
        a = torch.nn.functional.silu(g) * u
        fb.fp8_quantize_act_1x128(a, qa, sa)
    out["silu_mul_then_quant_unfused"] = report(time_cold(torch, unfused_sm, flush), sm_bytes)
    del x, gu, flush
    torch.cuda.synchronize()
    return out


def other_workloads(torch, fb, wl, dev, seed):
    """The decode (1x128 and MXFP8) and MoE layers: every kernel timed cold,
    reported against its own roofline (these shapes are HBM-bound)."""
    out = {}
    cd = lambda a, b: (a + b - 1) // b
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    to = lambda bits: torch.from_numpy(bits).view(torch.bfloat16).to(dev)

    # decode FProp: X [64 x 4096] against the fused gate+up W [24576 x 4096]
    w = wl.mx(seed)
    N, C, D = w["N"], w["C"], w["D"]
    X, W, dY = to(w["X"]), to(w["W"]), to(w["dY"])
    xq, xs = fb.fp8_quantize_act_1x128(X)
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(W, transpose=True)
    y = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    dec = {}
    dec["quant_act_1x128"] = report(time_cold(torch, lambda: fb.fp8_quantize_act_1x128(X, xq, xs), flush),
                                    N * C * 3 + N * cd(C, 128) * 4)
    dec["quant_weight"] = report(time_cold(torch, lambda: fb.fp8_quantize_weight_128x128(
        W, transpose=False, q=wq, s=ws), flush), D * C * 3 + cd(D, 128) * cd(C, 128) * 4)
    dec["fprop"] = report(time_cold(torch, lambda: fb.fp8_gemm_fprop(xq, xs, wq, ws, N, D, C, y=y), flush),
                          N * C + D * C + N * cd(C, 128) * 4 + cd(D, 128) * cd(C, 128) * 4 + N * D * 2,
                          2.0 * N * D * C)
    # the decode layout of the weight (written once per weight update) and
    # FProp on it: the rollout path, bit for bit the row-major FProp
    wp, _ = fb.fp8_pack_decode_weight(wq, D, C)
    dec["pack_decode_layout"] = report(time_cold(torch, lambda: fb.fp8_pack_decode_weight(wq, D, C, wp=wp), flush),
                                       2 * D * C)
    dec["fprop_packed"] = report(time_cold(torch, lambda: fb.fp8_gemm_fprop_decode(xq, xs, wp, ws, N, D, C, y=y),
                                           flush),
                                 N * C + D * C + N * cd(C, 128) * 4 + cd(D, 128) * cd(C, 128) * 4 + N * D * 2,
                                 2.0 * N * D * C)
    # the rollout step (quantize the activation, then FProp on the packed
    # weight) as two eager launches and as one HIP graph replay of the same
    # two kernels
    def step():
        fb.fp8_quantize_act_1x128(X, xq, xs)
        fb.fp8_gemm_fprop_decode(xq, xs, wp, ws, N, D, C, y=y)
    step_bytes = (N * C * 2 + 2 * (N * C + N * cd(C, 128) * 4) + D * C + cd(D, 128) * cd(C, 128) * 4
                  + N * D * 2)
    dec["step_eager"] = report(time_cold(torch, step, flush), step_bytes, 2.0 * N * D * C)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    dec["step_graph"] = report(time_cold(torch, graph.replay, flush), step_bytes, 2.0 * N * D * C)
    del graph
    # a chain of 16 rollout steps over four copies of the packed weight (403 MB,
    # more than the Infinity Cache holds, so each step reads its weight from
    # HBM): eager launches, one HIP graph replay of all 32 kernels, and the
    # packed FProp alone back-to-back; times per step
    nch = 16
    wps = [wp] + [wp.clone() for _ in range(3)]

    def chain():
        for i in range(nch):
            fb.fp8_quantize_act_1x128(X, xq, xs)
            fb.fp8_gemm_fprop_decode(xq, xs, wps[i % 4], ws, N, D, C, y=y)

    def fprops():
        for i in range(nch):
            fb.fp8_gemm_fprop_decode(xq, xs, wps[i % 4], ws, N, D, C, y=y)
    dec["step_chain16_eager"] = report(time_cold(torch, chain, flush, reps=20) / nch, step_bytes, 2.0 * N * D * C)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    dec["step_chain16_graph"] = report(time_cold(torch, graph.replay, flush, reps=20) / nch, step_bytes,
                                       2.0 * N * D * C)
    del graph
    dec["fprop_packed_back_to_back"] = report(
        time_cold(torch, fprops, flush, reps=20) / nch,
        N * C + D * C + N * cd(C, 128) * 4 + cd(D, 128) * cd(C, 128) * 4 + N * D * 2, 2.0 * N * D * C)
    del wps
    # warm: the same weight back-to-back (its 100 MB of codes stay in the
    # Infinity Cache)
    dbytes = N * C + D * C + N * cd(C, 128) * 4 + cd(D, 128) * cd(C, 128) * 4 + N * D * 2
    dec["fprop_warm"] = report(time_warm(torch, lambda: fb.fp8_gemm_fprop(xq, xs, wq, ws, N, D, C, y=y)), dbytes,
                               2.0 * N * D * C)
    dec["fprop_packed_warm"] = report(time_warm(torch, lambda: fb.fp8_gemm_fprop_decode(xq, xs, wp, ws, N, D, C, y=y)),
                                      dbytes, 2.0 * N * D * C)
    # the backward GEMMs of the same 64-token layer on the 1x128 / 128x128
    # path (the MXFP8 section below times the same three GEMMs): DGrad with
    # dY [64 x 24576] quantized along D (split along K, 64 rows), WGrad with
    # both operands quantized along the 64-token axis (one partial group)
    gq, gs = fb.fp8_quantize_act_1x128(dY)
    gqT, gsT, _, _ = fb.fp8_quantize_transposed(dY)
    xqT, xsT, _, _ = fb.fp8_quantize_transposed(X)
    dx1 = torch.empty((N, C), dtype=torch.bfloat16, device=dev)
    dw1 = torch.empty((D, C), dtype=torch.bfloat16, device=dev)
    dec["dgrad"] = report(time_cold(torch, lambda: fb.fp8_gemm_dgrad(gq, gs, wqT, ws, N, D, C, dx=dx1), flush),
                          N * D + D * C + N * cd(D, 128) * 4 + cd(D, 128) * cd(C, 128) * 4 + N * C * 2,
                          2.0 * N * D * C)
    dec["wgrad"] = report(time_cold(torch, lambda: fb.fp8_gemm_wgrad(gqT, gsT, xqT, xsT, N, D, C, dw=dw1), flush),
                          (D + C) * 128 + (D + C) * 4 + D * C * 2, 2.0 * N * D * C)
    del gq, gqT, xqT, dx1, dw1, wqT, wp
    out["decode_1x128"] = dec

    # the same tensors through the MXFP8 path (plus dY [64 x 24576])
    mx = {}
    q_x = fb.fp8_mx_quantize_1x32(X)
    q_w = fb.fp8_mx_quantize_1x32(W)
    q_g = fb.fp8_mx_quantize_1x32(dY)
    both = lambda r, c: r * c * 2 + 2 * (r * c + r * c // 32)
    mx["quant_X"] = report(time_cold(torch, lambda: fb.fp8_mx_quantize_1x32(X), flush), both(N, C))
    mx["quant_W"] = report(time_cold(torch, lambda: fb.fp8_mx_quantize_1x32(W), flush), both(D, C))
    mx["quant_dY"] = report(time_cold(torch, lambda: fb.fp8_mx_quantize_1x32(dY), flush), both(N, D))
    dx = torch.empty((N, C), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((D, C), dtype=torch.bfloat16, device=dev)
    mx["fprop"] = report(time_cold(torch, lambda: fb.fp8_mx_gemm_fprop(q_x[0], q_x[1], q_w[0], q_w[1], N, D, C, y=y),
                                   flush), N * C * 33 // 32 + D * C * 33 // 32 + N * D * 2, 2.0 * N * D * C)
    mp = fb.fp8_pack_decode_weight(q_w[0], D, C, we=q_w[1])
    mx["pack_decode_layout"] = report(time_cold(torch, lambda: fb.fp8_pack_decode_weight(
        q_w[0], D, C, we=q_w[1], wp=mp[0], wep=mp[1]), flush), 2 * D * C * 33 // 32)
    mx["fprop_packed"] = report(time_cold(torch, lambda: fb.fp8_mx_gemm_fprop_decode(
        q_x[0], q_x[1], mp[0], mp[1], N, D, C, y=y), flush),
        N * C * 33 // 32 + D * C * 33 // 32 + N * D * 2, 2.0 * N * D * C)

    # the MXFP8 rollout step, as decode_1x128's step_eager: the activation's
    # row-wise copy (all FProp needs) and the FProp on the packed weight
    xr = fb.fp8_mx_quantize_1x32(X, colwise=False)

    def mx_step():
        fb.fp8_mx_quantize_1x32(X, colwise=False, q=xr[0], e=xr[1])
        fb.fp8_mx_gemm_fprop_decode(xr[0], xr[1], mp[0], mp[1], N, D, C, y=y)
    mx["quant_X_rowwise"] = report(time_cold(torch, lambda: fb.fp8_mx_quantize_1x32(
        X, colwise=False, q=xr[0], e=xr[1]), flush), N * C * 2 + N * C + N * C // 32)
    mx["step_eager"] = report(time_cold(torch, mx_step, flush),
                              N * C * 2 + 2 * (N * C + N * C // 32) + D * C * 33 // 32 + N * D * 2, 2.0 * N * D * C)
    del mp, xr
    mx["dgrad"] = report(time_cold(torch, lambda: fb.fp8_mx_gemm_dgrad(q_g[0], q_g[1], q_w[2], q_w[3], N, D, C, dx=dx),
                                   flush), N * D * 33 // 32 + D * C * 33 // 32 + N * C * 2, 2.0 * N * D * C)
    Kp = 128   # the token axis (64) padded to one 128-wide block
    mx["wgrad"] = report(time_cold(torch, lambda: fb.fp8_mx_gemm_wgrad(q_g[2], q_g[3], q_x[2], q_x[3], N, D, C, dw=dw),
                                   flush), (D + C) * Kp * 33 // 32 + D * C * 2, 2.0 * N * D * C)
    out["decode_mxfp8"] = mx
    del X, W, dY, q_x, q_w, q_g, wq, xq, dx, dw, y

    # MoE layer: 4096 tokens, top-8 of 128 experts, hidden 2048, intermediate 768
    m = wl.moe(seed)
    offs = m["offsets"]
    E, I2, H = m["W_gu"].shape
    I = m["inter"]
    R = int(offs[-1])
    od = torch.from_numpy(offs.astype(np.int32)).to(dev)
    Wgu, Wd = to(m["W_gu"].reshape(E * I2, H)), to(m["W_d"].reshape(E * H, I))
    Xp, A, dH, dYd = to(m["X_perm"]), to(m["A"]), to(m["dH"]), to(m["dY_d"])
    moe = {}
    gu = fb.fp8_quantize_weight_128x128(Wgu)
    dn = fb.fp8_quantize_weight_128x128(Wd)
    moe["quant_W_gu"] = report(time_cold(torch, lambda: fb.fp8_quantize_weight_128x128(Wgu, q=gu[0], s=gu[1], qT=gu[2]),
                                         flush), E * I2 * H * 4)
    qx = fb.fp8_quantize_transposed_grouped(Xp, od, rowwise=True)
    qa = fb.fp8_quantize_transposed_grouped(A, od, rowwise=True)
    qh = fb.fp8_quantize_transposed_grouped(dH, od, rowwise=True)
    qy = fb.fp8_quantize_transposed_grouped(dYd, od, rowwise=True)
    moe["quant_dual_X"] = report(time_cold(torch, lambda: fb.fp8_quantize_transposed_grouped(
        Xp, od, rowwise=True, qT=qx[0], sT=qx[1], q=qx[2], s=qx[3]), flush), R * H * 4)
    fl_gu, fl_d = 2.0 * R * I2 * H, 2.0 * R * H * I
    y_gu = torch.empty((R, I2), dtype=torch.bfloat16, device=dev)
    y_d = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    dx_gu = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    dx_d = torch.empty((R, I), dtype=torch.bfloat16, device=dev)
    dw_gu = torch.empty((E, I2, H), dtype=torch.bfloat16, device=dev)
    dw_d = torch.empty((E, H, I), dtype=torch.bfloat16, device=dev)
    moe["gu_fprop"] = report(time_cold(torch, lambda: fb.fp8_gemm_fprop_grouped(
        qx[2], qx[3], gu[0], I2 * gu[0].stride(0), gu[1], (I2 // 128) * gu[1].stride(0), od, R, I2, H, y=y_gu),
        flush), R * H + E * I2 * H + R * I2 * 2, fl_gu)
    moe["gu_dgrad"] = report(time_cold(torch, lambda: fb.fp8_gemm_dgrad_grouped(
        qh[2], qh[3], gu[2], I2, gu[1], (I2 // 128) * gu[1].stride(0), od, R, I2, H, dx=dx_gu),
        flush), R * I2 + E * I2 * H + R * H * 2, fl_gu)
    moe["gu_wgrad"] = report(time_cold(torch, lambda: fb.fp8_gemm_wgrad_grouped(
        qh[0], qh[1], qx[0], qx[1], od, R, I2, H, dw=dw_gu), flush), R * (I2 + H) + E * I2 * H * 2, fl_gu)
    moe["d_fprop"] = report(time_cold(torch, lambda: fb.fp8_gemm_fprop_grouped(
        qa[2], qa[3], dn[0], H * dn[0].stride(0), dn[1], (H // 128) * dn[1].stride(0), od, R, H, I, y=y_d),
        flush), R * I + E * H * I + R * H * 2, fl_d)
    moe["d_dgrad"] = report(time_cold(torch, lambda: fb.fp8_gemm_dgrad_grouped(
        qy[2], qy[3], dn[2], H, dn[1], (H // 128) * dn[1].stride(0), od, R, H, I, dx=dx_d),
        flush), R * H + E * H * I + R * I * 2, fl_d)
    moe["d_wgrad"] = report(time_cold(torch, lambda: fb.fp8_gemm_wgrad_grouped(
        qy[0], qy[1], qa[0], qa[1], od, R, H, I, dw=dw_d), flush), R * (H + I) + E * H * I * 2, fl_d)
    out["moe_layer"] = moe
    torch.cuda.synchronize()
    return out


def cpu_baseline(w, budget_s: float):
    """The oracle as it stands (plain C, fp32 quantizers, fp64 GEMMs) on a
    bounded sample of the same workload: all of W quantized 128x128, then
    `rows` sampled token rows through the 1x128 quantizer and FProp/DGrad,
    and `rows` sampled dW rows through the token-axis quantizer and WGrad.
    Reported in TFLOP/s of GEMM work per second of the sampled pipeline."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    rng = np.random.default_rng(99)
    rows = 256
    t0 = time.perf_counter()
    while True:
        ridx = np.sort(rng.choice(N, rows, replace=False))
        didx = np.sort(rng.choice(D, rows, replace=False))
        ts = time.perf_counter()
        wq, ws, _ = oracle.quant_128x128(w["W"], with_transpose=False)
        xq, xs = oracle.quant_1x128(w["X"][ridx])
        oracle.fprop(xq, xs, wq, ws, C)
        gq, gs = oracle.quant_1x128(w["dY"][ridx])
        oracle.dgrad(gq, gs, wq, ws, D, C)
        gqT, gsT = oracle.quant_colwise(np.ascontiguousarray(w["dY"][:, didx]))
        xqT, xsT = oracle.quant_colwise(w["X"])
        oracle.wgrad(gqT, gsT, xqT, xsT, N)
        dt = time.perf_counter() - ts
        # one timed sample of at least budget_s seconds of CPU work, doubling
        # the sampled rows; at most 4 x budget_s in all
        if dt >= budget_s or time.perf_counter() - t0 > 4 * budget_s or rows >= 4096:
            break
        rows *= 2
    flops = 2.0 * rows * D * C + 2.0 * rows * C * D + 2.0 * rows * C * N
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"W quantized 128x128 in full; {rows} token rows of X and dY through 1x128 "
                      f"quantization and FProp/DGrad; X and {rows} columns of dY through token-axis "
                      f"quantization and {rows} rows of WGrad (fp64 GEMMs)"}


def mfma_peaks(torch, fb, dev):
    """Matrix-core throughput on random operands held in registers (the
    library's measurement kernel fp8b_mfma_peak): fp8 16x16x128 and bf16
    16x16x32 MFMAs on every compute unit with 2 and 4 waves per SIMD, and the
    fp8 loop with the FP32-scale recipe's per-block promotion (one FMA per
    result for the 1x128 x 128x128 GEMMs; a multiply and an FMA per result
    for the token-axis WGrad): the ceiling the format itself leaves on this
    chip.  The faster setting is the measured ceiling.  Median of REPS
    launches."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {}
    for kind, name, iters, spec in ((0, "fp8_16x16x128", 2000, PEAK_FP8_TFLOPS),
                                    (1, "bf16_16x16x32", 4000, PEAK_BF16_TFLOPS),
                                    (2, "fp8_with_block_scale_promotion", 2000, PEAK_FP8_TFLOPS),
                                    (3, "fp8_with_row_scale_promotion", 2000, PEAK_FP8_TFLOPS)):
        runs = {}
        for wps in (2, 4):
            blocks = cus * wps                      # a block is one wave per SIMD of a CU
            buf, flops = fb.fp8b_mfma_peak(kind, blocks, iters, seed=1)
            for _ in range(2):
                fb.fp8b_mfma_peak(kind, blocks, iters, seed=1, out=buf)
            torch.cuda.synchronize()
            ts = []
            for _ in range(REPS):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fb.fp8b_mfma_peak(kind, blocks, iters, seed=1, out=buf)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3)
            t = float(np.median(ts))
            runs[f"{wps}_waves_per_simd"] = {"us": round(t * 1e6, 1), "tflops": round(flops / t / 1e12, 1)}
        best = max(r["tflops"] for r in runs.values())
        out[name] = {"tflops": best, "frac_spec": round(best / spec, 4), "spec_tflops": spec, "runs": runs}
    return out


def tiny_layer(torch, fb, wl, dev, seed):
    """The tiny plumbing layer (X fp32 [256 x 512], W [384 x 512], dY [256 x
    384]): every kernel of the path, warm, the mean of REPS back-to-back
    launches (launch-latency bound: time only)."""
    w = wl.tiny(seed)
    X, W, dY = (torch.from_numpy(w[k]).to(dev) for k in ("X", "W", "dY"))
    Nt, Ct, Dt = w["N"], w["C"], w["D"]
    xq, xs = fb.fp8_quantize_act_1x128(X)
    gq, gs = fb.fp8_quantize_act_1x128(dY)
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(W)
    xd = fb.fp8_quantize_transposed(X, rowwise=True)
    gd = fb.fp8_quantize_transposed(dY, rowwise=True)
    y = torch.empty((Nt, Dt), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((Nt, Ct), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((Dt, Ct), dtype=torch.bfloat16, device=dev)
    runs = {
        "quant_act_X": lambda: fb.fp8_quantize_act_1x128(X, xq, xs),
        "quant_act_dY": lambda: fb.fp8_quantize_act_1x128(dY, gq, gs),
        "quant_weight": lambda: fb.fp8_quantize_weight_128x128(W, q=wq, s=ws, qT=wqT),
        "quant_dual_X": lambda: fb.fp8_quantize_transposed(X, rowwise=True, qT=xd[0], sT=xd[1], q=xd[2], s=xd[3]),
        "quant_dual_dY": lambda: fb.fp8_quantize_transposed(dY, rowwise=True, qT=gd[0], sT=gd[1], q=gd[2], s=gd[3]),
        "fprop": lambda: fb.fp8_gemm_fprop(xq, xs, wq, ws, Nt, Dt, Ct, y=y),
        "dgrad": lambda: fb.fp8_gemm_dgrad(gq, gs, wqT, ws, Nt, Dt, Ct, dx=dx),
        "wgrad": lambda: fb.fp8_gemm_wgrad(gd[0], gd[1], xd[0], xd[1], Nt, Dt, Ct, dw=dw),
    }
    out = {}
    for name, fn in runs.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(REPS):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = {"us": round(e0.elapsed_time(e1) * 1e3 / REPS, 2)}
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def quant_error_mx_vs_blockscaled(seed):
    """Quantization error of the two recipes on the MXFP8 workload's tensors
    (X [64 x 4096], W [24576 x 4096], dY [64 x 24576], bf16): for each
    GEMM, max |y_recipe - y_exact| / ||y_exact row||, with y_recipe the
    oracle's GEMM on the recipe's dequantized operands (1x128 / 128x128 FP32
    scales, or MXFP8 1x32 E8M0) and y_exact the fp64 GEMM of the unquantized
    bf16 inputs."""
    import oracle
    from block_scaled_fp8_02_amd import workloads as wl
    w = wl.mx(seed)
    X, W, dY = w["X"], w["W"], w["dY"]
    Nm, Cm, Dm = w["N"], w["C"], w["D"]
    Xf, Wf, Gf = (oracle.as_f32(t).astype(np.float64) for t in (X, W, dY))
    xq, xs = oracle.quant_1x128(X)
    wq, ws, _ = oracle.quant_128x128(W, with_transpose=False)
    gq, gs = oracle.quant_1x128(dY)
    gqT, gsT = oracle.quant_colwise(dY)
    xqT, xsT = oracle.quant_colwise(X)
    mxq, mxe = oracle.mx_quant_rows(X)
    mxqT, mxeT = oracle.mx_quant_cols(X)
    mwq, mwe = oracle.mx_quant_rows(W)
    mwqT, mweT = oracle.mx_quant_cols(W)
    mgq, mge = oracle.mx_quant_rows(dY)
    mgqT, mgeT = oracle.mx_quant_cols(dY)
    ops = {
        "fprop": (lambda: oracle.matmul_f64(Xf, Wf.T), lambda: oracle.fprop(xq, xs, wq, ws, Cm),
                  lambda: oracle.mx_gemm(mxq, mxe, mwq, mwe, Cm)),
        "dgrad": (lambda: oracle.matmul_f64(Gf, Wf), lambda: oracle.dgrad(gq, gs, wq, ws, Dm, Cm),
                  lambda: oracle.mx_gemm(mgq, mge, mwqT, mweT, Dm)),
        "wgrad": (lambda: oracle.matmul_f64(Gf.T, Xf), lambda: oracle.wgrad(gqT, gsT, xqT, xsT, Nm),
                  lambda: oracle.mx_gemm(mgqT, mgeT, mxqT, mxeT, Nm)),
    }
    out = {}
    for op, (exact, blk, mx) in ops.items():
        ye = exact()
        out[op] = {"blockscaled_1x128_128x128": float(f"{oracle.rel_row_error(blk(), ye):.4e}"),
                   "mxfp8_1x32": float(f"{oracle.rel_row_error(mx(), ye):.4e}")}
    out["metric"] = ("max |y_q - y_exact| / ||y_exact row||_2, y_q the oracle GEMM on one recipe's "
                     "dequantized operands, y_exact the fp64 GEMM of the unquantized bf16 inputs")
    return out


def cpu_oracle_configs(seed, c3_sample):
    """The oracle as it stands, on the host's cores, on every workload:
    quantizers at full size everywhere, GEMMs at full size on the tiny,
    decode, MXFP8 and MoE workloads; the training GEMMs are extrapolated
    from the timed row sample of cpu_baseline (flagged).  Bytes are the
    algorithmic bytes of the same operation on the GPU."""
    import oracle
    from block_scaled_fp8_02_amd import workloads as wl
    cd = lambda a, b: (a + b - 1) // b
    rup = lambda a: cd(a, 128) * 128

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return time.perf_counter() - t0, r

    def qent(fn, nbytes):
        t, r = timed(fn)
        return {"s": round(t, 4), "gbs": round(nbytes / t / 1e9, 3)}, r

    def gent(fn, flops):
        t, r = timed(fn)
        return {"s": round(t, 4), "gflops": round(flops / t / 1e9, 3)}, r

    def b_act(rows, cols, esz):                         # 1x128 quantizer: in + codes + scales
        return rows * cols * esz + rows * rup(cols) + rows * cd(cols, 128) * 4

    def b_dual(rows, cols, esz):                        # row-wise + token-axis copies
        return rows * cols * esz + rows * rup(cols) + cols * rup(rows) + (rows * cd(cols, 128) + cols * cd(rows, 128)) * 4

    def b_w(Dw, Cw, esz, qT=True):
        return Dw * Cw * esz + Dw * rup(Cw) * (2 if qT else 1) + cd(Dw, 128) * cd(Cw, 128) * 4

    res = {"threads": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), "cpu_model": cpu_model()}

    # tiny (fp32 inputs)
    w = wl.tiny(seed)
    X, W, dY = w["X"], w["W"], w["dY"]
    n, c, d = w["N"], w["C"], w["D"]
    e = {}
    e["quant_weight"], (wq, ws, _) = qent(lambda: oracle.quant_128x128(W), b_w(d, c, 4))
    e["quant_dual_X"], (xq, xs, xqT, xsT) = qent(lambda: oracle.quant_1x128(X) + oracle.quant_colwise(X),
                                                 b_dual(n, c, 4))
    e["quant_dual_dY"], (gq, gs, gqT, gsT) = qent(lambda: oracle.quant_1x128(dY) + oracle.quant_colwise(dY),
                                                  b_dual(n, d, 4))
    e["fprop"], _ = gent(lambda: oracle.fprop(xq, xs, wq, ws, c), 2.0 * n * d * c)
    e["dgrad"], _ = gent(lambda: oracle.dgrad(gq, gs, wq, ws, d, c), 2.0 * n * d * c)
    e["wgrad"], _ = gent(lambda: oracle.wgrad(gqT, gsT, xqT, xsT, n), 2.0 * n * d * c)
    res["tiny"] = e

    # decode (bf16)
    w = wl.decode(seed)
    X, W = w["X"], w["W"]
    n, c, d = w["N"], w["C"], w["D"]
    e = {}
    e["quant_act_X"], (xq, xs) = qent(lambda: oracle.quant_1x128(X), b_act(n, c, 2))
    e["quant_weight"], (wq, ws, _) = qent(lambda: oracle.quant_128x128(W, with_transpose=False), b_w(d, c, 2, False))
    e["fprop"], _ = gent(lambda: oracle.fprop(xq, xs, wq, ws, c), 2.0 * n * d * c)
    res["decode"] = e
    del w, X, W, wq

    # training layer: quantizers at full size, GEMMs from the row sample
    w = wl.train(seed)
    X, W, dY = w["X"], w["W"], w["dY"]
    n, c, d = w["N"], w["C"], w["D"]
    e = {}
    e["quant_weight"], _ = qent(lambda: oracle.quant_128x128(W), b_w(d, c, 2))
    e["quant_dual_X"], _ = qent(lambda: oracle.quant_1x128(X) + oracle.quant_colwise(X), b_dual(n, c, 2))
    e["quant_dual_dY"], _ = qent(lambda: oracle.quant_1x128(dY) + oracle.quant_colwise(dY), b_dual(n, d, 2))
    if c3_sample:
        rate = c3_sample["value"] * 1e12
        for op in ("fprop", "dgrad", "wgrad"):
            e[op] = {"s_extrapolated": round(2.0 * n * d * c / rate, 2), "gflops": round(rate / 1e9, 3),
                     "flag": "extrapolated linearly from the timed row sample (cpu_baseline)"}
    res["train"] = e
    del w, X, W, dY

    # MXFP8 workload: MX quantizers (both orientations) and GEMMs, and the
    # 1x128 / 128x128 path on the same tensors, all at full size
    w = wl.mx(seed)
    X, W, dY = w["X"], w["W"], w["dY"]
    n, c, d = w["N"], w["C"], w["D"]
    mxb = lambda r, k: r * k * 2 + 2 * (r * rup(k) + r * rup(k) // 32)
    e = {}
    e["mx_quant_X"], (mxq, mxe, mxqT, mxeT) = qent(lambda: oracle.mx_quant_rows(X) + oracle.mx_quant_cols(X), mxb(n, c))
    e["mx_quant_W"], (mwq, mwe, mwqT, mweT) = qent(lambda: oracle.mx_quant_rows(W) + oracle.mx_quant_cols(W), mxb(d, c))
    e["mx_quant_dY"], (mgq, mge, mgqT, mgeT) = qent(lambda: oracle.mx_quant_rows(dY) + oracle.mx_quant_cols(dY),
                                                    mxb(n, d))
    e["mx_fprop"], _ = gent(lambda: oracle.mx_gemm(mxq, mxe, mwq, mwe, c), 2.0 * n * d * c)
    e["mx_dgrad"], _ = gent(lambda: oracle.mx_gemm(mgq, mge, mwqT, mweT, d), 2.0 * n * d * c)
    e["mx_wgrad"], _ = gent(lambda: oracle.mx_gemm(mgqT, mgeT, mxqT, mxeT, n), 2.0 * n * d * c)
    del mwq, mwqT
    e["quant_weight"], (wq, ws, _) = qent(lambda: oracle.quant_128x128(W), b_w(d, c, 2))
    e["quant_dual_X"], (xq, xs, xqT, xsT) = qent(lambda: oracle.quant_1x128(X) + oracle.quant_colwise(X),
                                                 b_dual(n, c, 2))
    e["quant_dual_dY"], (gq, gs, gqT, gsT) = qent(lambda: oracle.quant_1x128(dY) + oracle.quant_colwise(dY),
                                                  b_dual(n, d, 2))
    e["fprop"], _ = gent(lambda: oracle.fprop(xq, xs, wq, ws, c), 2.0 * n * d * c)
    e["dgrad"], _ = gent(lambda: oracle.dgrad(gq, gs, wq, ws, d, c), 2.0 * n * d * c)
    e["wgrad"], _ = gent(lambda: oracle.wgrad(gqT, gsT, xqT, xsT, n), 2.0 * n * d * c)
    res["mx"] = e
    del w, X, W, dY, wq

    # MoE layer: stacked expert weights, grouped token-axis quantizers, and
    # all six GEMMs expert by expert
    m = wl.moe(seed)
    offs = m["offsets"]
    E, I2, H = m["W_gu"].shape
    I = m["inter"]
    R = int(offs[-1])
    P = oracle.padded_offsets(offs)
    e = {}
    e["quant_W_gu"], (guq, gus, _) = qent(lambda: oracle.quant_128x128(m["W_gu"].reshape(E * I2, H)),
                                          b_w(E * I2, H, 2))
    e["quant_W_d"], (dnq, dns, _) = qent(lambda: oracle.quant_128x128(m["W_d"].reshape(E * H, I)), b_w(E * H, I, 2))
    q = {}
    for name, t, k in (("X", m["X_perm"], H), ("A", m["A"], I), ("dH", m["dH"], I2), ("dY", m["dY_d"], H)):
        e[f"quant_dual_{name}"], q[name] = qent(lambda: oracle.quant_1x128(t) + oracle.quant_colwise(t, offs),
                                                b_dual(R, k, 2) + 128 * E * k)
    tg = {k: 0.0 for k in ("gu_fprop", "gu_dgrad", "gu_wgrad", "d_fprop", "d_dgrad", "d_wgrad")}
    for x in range(E):
        a, b = int(offs[x]), int(offs[x + 1])
        p0, p1 = int(P[x]), int(P[x + 1])
        for pre, wq_, ws_, Dn, Cn, xin, gin in (("gu", guq, gus, I2, H, q["X"], q["dH"]),
                                                 ("d", dnq, dns, H, I, q["A"], q["dY"])):
            wq_e = wq_[x * Dn:(x + 1) * Dn]
            ws_e = ws_[x * Dn // 128:(x + 1) * Dn // 128]
            t, _ = timed(lambda: oracle.fprop(xin[0][a:b], xin[1][a:b], wq_e, ws_e, Cn))
            tg[f"{pre}_fprop"] += t
            t, _ = timed(lambda: oracle.dgrad(gin[0][a:b], gin[1][a:b], wq_e, ws_e, Dn, Cn))
            tg[f"{pre}_dgrad"] += t
            t, _ = timed(lambda: oracle.wgrad(gin[2][:, p0:p1], gin[3][:, p0 // 128:p1 // 128],
                                              xin[2][:, p0:p1], xin[3][:, p0 // 128:p1 // 128], p1 - p0))
            tg[f"{pre}_wgrad"] += t
    for k, t in tg.items():
        fl = 2.0 * R * I2 * H if k.startswith("gu") else 2.0 * R * H * I
        e[k] = {"s": round(t, 4), "gflops": round(fl / t / 1e9, 3)}
    res["moe"] = e
    return res


if __name__ == "__main__":
    main()
