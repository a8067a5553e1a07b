#!/usr/bin/env python3
"""Throughput of the rotated W4A4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload flux]

One step is the whole hot path over one batch: for each layer of the
workload, rq_rotate_quant (rotate + per-token 4-bit quantize) followed by
rq_w4a4_linear (low-bit GEMM + rescale), back to back on one stream.  The
default workload "flux" is the FLUX-scale MLP pair: the up-projection
9216 x 3072 -> 12288 (RPBH block 256) and the down-projection
9216 x 12288 -> 3072 (RPBH block 512), 2 x 4608 tokens (two guidance
branches), bf16 activations and outputs.  Inputs are seeded synthetic
tensors resident in HBM; a ring of two independent layer instances keeps the
timed steps from reading what the previous step left in the 256 MB
Infinity Cache.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value          TOPS = 2 * T * Kq * N summed over the step's layers / time
  ms_per_step    wall time per step (host clock around K synchronized steps)
  roofline       the dominant kernel (the GEMM), from HIP events on the
                 launch stream: algorithmic ops per launch / mean duration,
                 against the int8 MFMA peak
  cpu_baseline   the CPU oracle on a bounded sample of the same workload
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

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
PEAK_FP6_TOPS = 10100.0      # MI355X dense fp6/fp4 MFMA, TOP/s (the INT4 GEMM's matrix cores)
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E

WORKLOADS = {
    "flux": ["flux_up", "flux_down"],
    "flux_asym": ["flux_up_asym", "flux_down_asym"],
    "flux_up": ["flux_up"],
    "flux_down": ["flux_down"],
    "tiny": ["tiny"],
    "pixart": ["pixart"],
    "video": ["video"],
    "video_w4": ["video_w4"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(name: str) -> str:
    p = os.path.join(ROOT, "rotated_w4a4_quantized_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def profiled_traffic(kernel_file: str, summary: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when the summary is missing or was taken on a different kernel
    source (the summary stores a hash of the source file)."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (ValueError, OSError):
        return None
    if data.get("source_sha256_16") != source_hash(kernel_file):
        return None
    return data.get("hbm_bytes_per_launch")


# kernels summarized from rocprofv3 runs: (summary file, kernel source, name match)
PMC_KERNELS = {
    "gemm": ("rq_gemm_fp6.hip", "gemm_fp6_mma_kernel"),
    "gemm_int8": ("rq_gemm_w4a4.hip", "gemm_w4a4_kernel"),
    "gemm_codebook": ("rq_gemm_codebook.hip", "gemm_codebook_kernel"),
    "rotate": ("rq_rpbh.hip", "rpbh_quant_kernel"),
    "dense": ("rq_dense.hip", "dense_rotate_kernel"),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _read_pmc(d):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        rows += list(csv.DictReader(open(f)))
    return rows


def summarize_pmc(fetch_dir, write_dir, workload, copy_bytes, command):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) into per-launch HBM bytes, each counter scaled by what it reads
    for the plain device-to-device copy of copy_bytes in the same run."""
    out = {}
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = {}
        for r in _read_pmc(d):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        copy = [v for k, v in vals.items() if COPY_KERNEL in k]
        big = max((x for lst in copy for x in lst), default=0.0)
        factor = copy_bytes / (big * 1024.0) if big > 0 else None
        per[counter] = (vals, factor, big)
    for key, (src, match) in PMC_KERNELS.items():
        fetch_vals = [x for k, lst in per["FETCH_SIZE"][0].items() if match in k for x in lst]
        write_vals = [x for k, lst in per["WRITE_SIZE"][0].items() if match in k for x in lst]
        if not fetch_vals or not write_vals:
            continue
        ff, wf = per["FETCH_SIZE"][1], per["WRITE_SIZE"][1]
        fetch = sum(fetch_vals) / len(fetch_vals) * 1024.0 * (ff or 1.0)
        write = sum(write_vals) / len(write_vals) * 1024.0 * (wf or 1.0)
        data = {
            "kernel": match, "workload": workload, "dispatches": len(fetch_vals),
            "fetch_kib_per_dispatch_raw": round(sum(fetch_vals) / len(fetch_vals), 1),
            "write_kib_per_dispatch_raw": round(sum(write_vals) / len(write_vals), 1),
            "copy_calibration": {"bytes": copy_bytes,
                                 "fetch_kib_raw": per["FETCH_SIZE"][2],
                                 "write_kib_raw": per["WRITE_SIZE"][2],
                                 "fetch_factor": ff, "write_factor": wf},
            "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
            "hbm_bytes_per_launch": round(fetch + write),
            "source_sha256_16": source_hash(src),
            "command": command,
        }
        name = f"{key}_{workload}_counters.json"
        json.dump(data, open(os.path.join(ROOT, "profiles", name), "w"), indent=1)
        out[name] = data
    return out


def summarize_stats(stats_csv, workload, command):
    """Short text summary of a rocprofv3 --kernel-trace --stats csv."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics, workload {workload}", "",
             "Command (from the repository root on the GPU host):", "", "    " + command, "",
             "| kernel | calls | average (us) | min (us) | max (us) | share (%) |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("rq::(anonymous namespace)::", "").replace("|", "/")
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                     f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    path = os.path.join(ROOT, "profiles", f"kernel_stats_{workload}.md")
    open(path, "w").write("\n".join(lines) + "\n")
    return path


def rotate_bytes(w) -> int:
    """Algorithmic HBM bytes of one rotate+quant launch: X read, codes,
    scales (and top) written."""
    xb = 4 if w.xdtype == "f32" else 2
    b = w.T * w.K * xb + w.T * (w.Kq // 2) + 4 * w.T
    if w.quant == "int4_asym":
        b += 4 * w.T   # zero points
    if w.r:
        b += 2 * w.T * w.r
    return b


def cpu_baseline(names, budget_s: float):
    """Oracle layer (rotate + quantize + integer GEMM + fp64 output) on a
    bounded token sample of each layer, scaled to TOPS."""
    from oracle import oracle as orc
    from rotated_w4a4_quantized_amd import datagen
    from tests import _layer as H

    threads = orc.num_threads()
    total_ops, total_t, parts = 0, 0.0, []
    for name in names:
        w = datagen.WORKLOADS[name]
        inp = datagen.make_inputs(w)
        t0 = time.perf_counter()
        wts = H.oracle_weights(w, inp)        # offline fold, not part of the rate
        log(f"[cpu_baseline] {name}: oracle weight fold {time.perf_counter() - t0:.1f}s")
        ntok = 8
        while True:
            rows = np.arange(ntok)
            t0 = time.perf_counter()
            act = H.oracle_act(w, inp, rows)
            ta = np.repeat(rows, w.N)
            nw = np.tile(np.arange(w.N), ntok)
            H.oracle_yhat_pairs(w, act, wts, ta, nw, act_rows=rows)
            dt = time.perf_counter() - t0
            if dt > budget_s / (4 * len(names)) or ntok >= w.T:
                break
            ntok = min(w.T, ntok * 4)
        ops = 2 * ntok * w.Kq * w.N
        total_ops += ops
        total_t += dt
        parts.append(f"{name}: first {ntok} tokens x all {w.N} outputs ({dt:.1f}s)")
        log(f"[cpu_baseline] {parts[-1]}")
    return {"value": total_ops / total_t / 1e12, "unit": "TOPS", "cores": threads,
            "kind": "oracle", "sample": "; ".join(parts)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="flux", choices=sorted(WORKLOADS))
    ap.add_argument("--ring", type=int, default=2, help="independent layer instances cycled")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after timing, run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="offline: summarize two rocprofv3 --pmc runs into profiles/")
    ap.add_argument("--summarize-stats", metavar="STATS_CSV",
                    help="offline: summarize a rocprofv3 --stats csv into profiles/")
    ap.add_argument("--command", default="", help="command recorded in the summaries")
    args = ap.parse_args()

    if args.summarize_pmc or args.summarize_stats:
        if args.summarize_pmc:
            res = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                                args.copy_calibration, args.command)
            print(json.dumps({k: v["hbm_bytes_per_launch"] for k, v in res.items()}))
        if args.summarize_stats:
            print(summarize_stats(args.summarize_stats, args.workload, args.command))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(token-parallel sharding is described in the design notes); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from rotated_w4a4_quantized_amd import datagen, rq
    from rotated_w4a4_quantized_amd.layer import QuantLinear

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rq.load()
    int8_gemm = os.environ.get("RQ_W4A4_MFMA") == "int8"
    names = WORKLOADS[args.workload]
    wls = [datagen.WORKLOADS[n] for n in names]

    # ring of independent instances (distinct seeds), all resident in HBM
    ring = []
    for i in range(args.ring):
        layers = []
        for w in wls:
            inp = datagen.make_inputs(w, seed_offset=100 * i)
            # RPBH INT4 layers hand the GEMM its codes in the matrix-core layout
            mode = ("mma" if (w.rot == "rpbh" and w.quant in ("int4", "int4_asym") and not int8_gemm)
                    else "canonical")
            layers.append(QuantLinear(w, inp, codes=mode))
            log(f"[bench] instance {i} layer {w.name}: T={w.T} K={w.K} N={w.N} ready")
        ring.append(layers)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    nl = len(wls)

    def step(i, ev=None):
        for j, L in enumerate(ring[i % args.ring]):
            if ev is not None:
                ev[j][0].record(stream)
            L.rotate_quant()
            if ev is not None:
                ev[j][1].record(stream)
            L.linear()
            if ev is not None:
                ev[j][2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps, host clock, synchronized on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # per-kernel durations: a second pass of K steps bracketed by HIP events
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nl)]
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    rot_ms = np.array([[evs[i][j][0].elapsed_time(evs[i][j][1]) for j in range(nl)]
                       for i in range(args.steps)])
    gemm_ms = np.array([[evs[i][j][1].elapsed_time(evs[i][j][2]) for j in range(nl)]
                        for i in range(args.steps)])

    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ops = [w.ops() for w in wls]
    value = sum(ops) / (ms_step * 1e-3) / 1e12
    layers = []
    for j, w in enumerate(wls):
        rm, gm = float(np.mean(rot_ms[:, j])), float(np.mean(gemm_ms[:, j]))
        layers.append({
            "layer": w.name, "T": w.T, "K": w.K, "N": w.N, "rotation": w.rot,
            "block": w.block, "quant": w.quant,
            "rotate_quant_us": round(rm * 1e3, 2),
            "rotate_quant_GBps": round(rotate_bytes(w) / (rm * 1e-3) / 1e9, 1),
            "gemm_us": round(gm * 1e3, 2),
            "gemm_TOPS": round(w.ops() / (gm * 1e-3) / 1e12, 1),
            "layer_ms": round(rm + gm, 4),
            "layer_TOPS": round(w.ops() / ((rm + gm) * 1e-3) / 1e12, 1),
        })
        log(f"[bench] {json.dumps(layers[-1])}")

    is_codebook = all(w.quant == "lloydmax" for w in wls)
    if is_codebook:
        peak, gsrc, gkey, gname = PEAK_BF16_TFLOPS, "rq_gemm_codebook.hip", "gemm_codebook", "gemm_codebook_kernel"
    elif int8_gemm:
        peak, gsrc, gkey, gname = PEAK_INT8_TOPS, "rq_gemm_w4a4.hip", "gemm_int8", "gemm_w4a4_kernel"
    else:
        # the INT4 GEMM computes on the FP6 matrix cores: its own dtype's peak
        peak, gsrc, gkey, gname = PEAK_FP6_TOPS, "rq_gemm_fp6.hip", "gemm", "gemm_fp6_mma_kernel"
    gemm_mean_ms = float(np.mean(gemm_ms))
    achieved = float(np.mean(ops)) / (gemm_mean_ms * 1e-3) / 1e12
    traffic = profiled_traffic(gsrc, f"{gkey}_{args.workload}_counters.json")
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s" if is_codebook else "TOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": gname}
    rot_mean_ms = float(np.mean(rot_ms))
    rot_bytes = float(np.mean([rotate_bytes(w) for w in wls]))
    rot_gbs = rot_bytes / (rot_mean_ms * 1e-3) / 1e9
    roofline_rot = {"bound": "hbm", "achieved": round(rot_gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(rot_gbs / PEAK_HBM_GBS, 4),
                    "traffic": profiled_traffic("rq_rpbh.hip",
                                                f"rotate_{args.workload}_counters.json"),
                    "kernel": "rotate_quant"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(names, args.cpu_budget)

    out = {
        "metric": "fused rotate+quant+W4A4 linear TOPS & ms/layer at FLUX-scale; % int8 MFMA peak",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_layer": round(ms_step / nl, 4),
        "pct_int8_peak": round(100 * value / PEAK_INT8_TOPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if is_codebook else ("i8" if int8_gemm else "fp6"),
        "data": "synthetic",
        "config": {"workload": args.workload, "layers": [
            {"name": w.name, "T": w.T, "K": w.K, "N": w.N, "rotation": w.rot, "block": w.block,
             "r": w.r, "quant": w.quant, "x": w.xdtype, "y": w.ydtype} for w in wls],
            "ring_instances": args.ring},
        "layers": layers,
        "roofline": roofline,
        "roofline_rotate_quant": roofline_rot,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
