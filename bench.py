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
Infinity Cache.  Before the W warmup steps the step runs for --settle-ms
(40 ms) so that the GPU has left its idle clock state (the line's `settle`
field); nothing of it is timed.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value          TOPS = 2 * T * Kq * N summed over the step's layers / time
  ms_per_step    wall time per step (host clock around K synchronized steps)
  roofline       the dominant kernel (the GEMM), from HIP events on the
                 launch stream: algorithmic ops per launch / mean duration,
                 against the peak of the matrix cores it runs on (FP6 / FP4:
                 10.1 POP/s, int8: 5.0, bf16: 2.5 PFLOP/s)
  roofline_rotate_quant  the activation kernel: algorithmic bytes / time
                 against HBM (RPBH), or fp32 FMA flops against the
                 non-packed fp32 rate (dense and TR-DQ rotations)
  sclk_mhz       shader clock sampled with rocm-smi while the steps run
  cpu_baseline   the CPU oracle on a bounded sample of the same workload,
                 on all host threads and on one

Other workloads (--workload): tiny, pixart, video, video_w4, flux_asym,
flux_mxfp4 (the FP4 variant), flux_up_w4a8 / flux_up_w8a8 (8-bit
activations), flux_up_trdq (TR-DQ's rotation, W4A8).
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
    "flux_mxfp4": ["flux_up_mxfp4", "flux_down_mxfp4"],
    "flux_up": ["flux_up"],
    "flux_down": ["flux_down"],
    "flux_up_w4a8": ["flux_up_w4a8"],
    "flux_up_w8a8": ["flux_up_w8a8"],
    "flux_up_trdq": ["flux_up_trdq"],
    "flux_up_trdq_w6a6": ["flux_up_trdq_w6a6"],
    "flux_up_w6a6": ["flux_up_w6a6"],
    "tiny": ["tiny"],
    "pixart": ["pixart"],
    "video": ["video"],
    "video_w4": ["video_w4"],
}
# non-packed fp32 fused multiply-add rate: 256 CUs x 64 lanes x 2 flops x 2.4 GHz
# (the chip's 157.3 TFLOP/s counts packed fp32, which this build does not emit)
PEAK_FP32_FMA_TFLOPS = 78.6


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
    "gemm_conv": ("rq_gemm_fp6.hip", "gemm_fp6_kernel"),
    "gemm_int8": ("rq_gemm_w4a4.hip", "gemm_w4a4_kernel"),
    "gemm_i8": ("rq_gemm_i8.hip", "gemm_i8_kernel"),
    "gemm_codebook": ("rq_gemm_codebook.hip", "gemm_cb_kernel"),
    "gemm_mx": ("rq_gemm_mx.hip", "gemm_mx_kernel"),
    "rotate": ("rq_rpbh.hip", "rpbh_quant_kernel"),
    "trdq": ("rq_trdq.hip", "trdq_tile_kernel"),
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


def summarize_stats(stats_csv, workload, command, bench_json=None):
    """Short text summary of a rocprofv3 --kernel-trace --stats csv; with
    the JSON line that the profiled bench run printed, also the two timings
    of the dominant kernel side by side."""
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
    if bench_json:
        line = json.loads(open(bench_json).read().strip().splitlines()[-1])
        rf = line["roofline"]
        kern = rf["kernel"]
        prof = [r for r in rows if kern + "<" in r["Name"]]
        calls = sum(int(r["Calls"]) for r in prof)
        avg = sum(float(r["AverageNs"]) * int(r["Calls"]) for r in prof) / max(calls, 1) / 1e3
        ev = [l["gemm_us"]["mean"] for l in line["layers"]]
        lines += ["", f"The bench line this run printed: {line['ms_per_step']} ms per step, "
                  f"{line['value']} {line['unit']}; `{kern}` {rf['achieved']} {rf['unit']} = "
                  f"{rf['frac']} of peak from its HIP-event means "
                  f"({', '.join(f'{x:.2f}' for x in ev)} us per layer, {np.mean(ev):.2f} us on average "
                  f"over its {len(line['layers']) * line['steps']} timed launches). The profile's "
                  f"average over all {calls} launches of the kernel (settle, warmup, timed, event-timed "
                  f"and clock-sampling steps) is {avg:.2f} us, "
                  f"{100.0 * (avg / np.mean(ev) - 1.0):+.1f}% from the event mean."]
    path = os.path.join(ROOT, "profiles", f"kernel_stats_{workload}.md")
    open(path, "w").write("\n".join(lines) + "\n")
    return path


def summarize_trace(trace_csv, workload, command, warmup=3):
    """Where a step's time goes, from a rocprofv3 --kernel-trace csv of a
    bench run: per kernel and grid, the mean duration of all launches and of
    those after the warmup steps; and the idle time between consecutive
    kernels of this library that follow each other within 100 us (gaps
    above that are the bench's host synchronizations between its phases)."""
    import csv
    rows = [r for r in csv.DictReader(open(trace_csv)) if "rq::" in r["Kernel_Name"]]

    def short(name):
        name = name.replace("void rq::(anonymous namespace)::", "").replace("rq::(anonymous namespace)::", "")
        return name.split("(")[0]

    ks = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short(r["Kernel_Name"]),
                 int(r["Grid_Size_X"])) for r in rows)
    per = {}
    for b, e, n, g in ks:
        per.setdefault((n, g), []).append(e - b)
    lines = [f"# Kernel timeline, workload {workload}", "",
             "Command (from the repository root on the GPU host):", "", "    " + command, "",
             f"Durations per kernel and grid (the first {warmup} launches of each are the warmup steps):", "",
             "| kernel | grid | launches | mean, all (us) | mean after warmup (us) | min (us) |",
             "|---|---|---|---|---|---|"]
    for (n, g), d in sorted(per.items()):
        d = np.array(d) / 1e3
        lines.append(f"| `{n}` | {g} | {d.size} | {d.mean():.2f} | {d[warmup:].mean() if d.size > warmup else d.mean():.2f} | {d.min():.2f} |")
    gaps = [b1 - e0 for (b0, e0, _, _), (b1, e1, _, _) in zip(ks, ks[1:]) if b1 - e0 < 100_000]
    busy = sum(e - b for b, e, _, _ in ks)
    lines += ["", f"Idle gaps between back-to-back kernels (under 100 us): {len(gaps)} gaps, mean "
              f"{np.mean(gaps) / 1e3:.2f} us, median {np.median(gaps) / 1e3:.2f} us, max "
              f"{np.max(gaps) / 1e3:.2f} us; kernels busy {busy / 1e3:.1f} us in all."]
    path = os.path.join(ROOT, "profiles", f"kernel_timeline_{workload}.md")
    open(path, "w").write("\n".join(lines) + "\n")
    return path


def rotate_bytes(w) -> int:
    """Algorithmic HBM bytes of one rotate+quant launch: X read, codes,
    scales (and top) written, in the method's minimal encoding."""
    xb = 4 if w.xdtype == "f32" else 2
    b = w.T * w.K * xb
    if w.quant == "mxfp4":
        return b + w.T * (w.K // 2) + w.T * (w.K // 32)     # E2M1 codes, E8M0 per 32
    if w.quant == "lloydmax":
        return b + w.T * (w.K // 2) + 4 * w.T
    b += w.T * w.code_bytes + 4 * w.T
    if w.quant == "int4_asym":
        b += 4 * w.T   # zero points
    if w.r:
        b += 2 * w.T * w.r
    return b


def rotate_flops(w) -> int:
    """Algorithmic fp32 flops of a rotation that runs as fused multiply-add
    chains (dense: 2 T K^2; TR-DQ: two block rotations, 4 T K b)."""
    if w.rot == "dense":
        return 2 * w.T * w.K * w.K
    if w.rot == "trdq":
        return 4 * w.T * w.K * w.block
    return 0


def pct(a, q):
    return float(np.percentile(a, q))


def sample_sclk():
    """Current shader clock (MHz) as rocm-smi reports it, or None."""
    import re
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                             timeout=20).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    m = re.search(r"sclk[^\n]*?\((\d+)\s*Mhz\)", out, re.I)
    return int(m.group(1)) if m else None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(names, budget_s: float, threads=None):
    """Oracle layer (rotate + quantize + integer GEMM + fp64 output) on a
    bounded token sample of each layer, scaled to TOPS.  threads: OpenMP
    threads (None: all)."""
    from oracle import oracle as orc
    from rotated_w4a4_quantized_amd import datagen
    from tests import _layer as H

    prev = orc.num_threads()
    if threads:
        orc.set_threads(threads)
    used = orc.num_threads()
    try:
        total_ops, total_t, parts = 0, 0.0, []
        for name in names:
            w = datagen.WORKLOADS[name]
            inp = datagen.make_inputs(w)
            wts = H.oracle_weights(w, inp)        # offline fold, not part of the rate
            ntok = 2
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
            log(f"[cpu_baseline] {used} threads, {parts[-1]}")
    finally:
        orc.set_threads(prev)
    return {"value": total_ops / total_t / 1e12, "unit": "TOPS", "cores": used,
            "kind": "oracle", "sample": "; ".join(parts)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="flux", choices=sorted(WORKLOADS))
    ap.add_argument("--engine", default="auto", choices=["auto", "fp6", "int8"],
                    help="matrix cores of the INT4 GEMM (int8: the int8-MFMA engine on canonical codes)")
    ap.add_argument("--ring", type=int, default=2, help="independent layer instances cycled")
    ap.add_argument("--settle-ms", type=float, default=40.0,
                    help="before the warmup steps, run the step this long (ms) so the GPU "
                         "leaves its idle clock state")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sclk", action="store_true", help="skip the rocm-smi clock sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after timing, run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="offline: summarize two rocprofv3 --pmc runs into profiles/")
    ap.add_argument("--summarize-stats", metavar="STATS_CSV",
                    help="offline: summarize a rocprofv3 --stats csv into profiles/")
    ap.add_argument("--summarize-trace", metavar="TRACE_CSV",
                    help="offline: kernel gaps from a rocprofv3 --kernel-trace csv into profiles/")
    ap.add_argument("--command", default="", help="command recorded in the summaries")
    ap.add_argument("--bench-json", default=None,
                    help="with --summarize-stats: the JSON line the profiled run printed")
    args = ap.parse_args()

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.workload, args.command, warmup=args.warmup))
    if args.summarize_pmc or args.summarize_stats:
        if args.summarize_pmc:
            res = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                                args.copy_calibration, args.command)
            print(json.dumps({k: v["hbm_bytes_per_launch"] for k, v in res.items()}))
        if args.summarize_stats:
            print(summarize_stats(args.summarize_stats, args.workload, args.command, args.bench_json))
        return
    if args.summarize_trace:
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(token-parallel sharding is described in the design notes); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from rotated_w4a4_quantized_amd import datagen, rq
    from rotated_w4a4_quantized_amd.layer import QuantLinear, mma_capable

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rq.load()
    names = WORKLOADS[args.workload]
    wls = [datagen.WORKLOADS[n] for n in names]
    int8_gemm = args.engine == "int8" or any(w.a_bits != 4 for w in wls)

    # Code layout per layer: 4-bit integer codes (RPBH, DENSE) and MXFP4
    # reach the GEMM in the matrix-core fragment layout, except a 4-bit
    # integer layer with fewer 256 x 256 output tiles than a quarter of the
    # CUs, which takes the canonical codes: their GEMM runs 128 x 128 tiles.
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def use_mma(w):
        if not mma_capable(w) or (args.engine == "int8" and w.quant != "mxfp4"):
            return False
        small = -(-w.T // 256) * -(-w.N // 256) < cus // 4
        return not (w.quant in ("int4", "int4_asym") and w.a_bits == 4 and w.r == 0 and small)

    # ring of independent instances (distinct seeds), all resident in HBM
    ring = []
    for i in range(args.ring):
        layers = []
        for w in wls:
            inp = datagen.make_inputs(w, seed_offset=100 * i)
            layers.append(QuantLinear(w, inp, codes="mma" if use_mma(w) else "canonical"))
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
            L.linear(engine=args.engine)
            if ev is not None:
                ev[j][2].record(stream)

    # Settle.  After idle the shader clock climbs over the first ~20 ms of
    # sustained work: a kernel trace of this bench shows the FLUX step at
    # 1.54, 0.63, 0.56, 0.52, 0.50 ms ... every five steps, steady at
    # ~0.46 ms after ~25 ms.  Running the step for settle_ms first puts the
    # W warmup and the K timed steps at the steady clock; the line reports it.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(4):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3

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
    # on the launch stream
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nl)]
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    rot_ms = np.array([[evs[i][j][0].elapsed_time(evs[i][j][1]) for j in range(nl)]
                       for i in range(args.steps)])
    gemm_ms = np.array([[evs[i][j][1].elapsed_time(evs[i][j][2]) for j in range(nl)]
                        for i in range(args.steps)])

    # shader clock under this load: the step loop keeps running while
    # rocm-smi is sampled
    sclk = None
    if not args.no_sclk:
        import threading
        samples = []
        stop = threading.Event()

        def sampler():
            while not stop.is_set() and len(samples) < 3:
                v = sample_sclk()
                if v is None:
                    break
                samples.append(v)

        th = threading.Thread(target=sampler)
        th.start()
        t_end = time.perf_counter() + 3.0
        i = 0
        while th.is_alive() and time.perf_counter() < t_end:
            step(i)
            i += 1
            if i % 20 == 0:
                torch.cuda.synchronize()
        stop.set()
        torch.cuda.synchronize()
        th.join()
        sclk = int(np.median(samples)) if samples else None

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
        r, g = rot_ms[:, j] * 1e3, gemm_ms[:, j] * 1e3       # us
        entry = {
            "layer": w.name, "T": w.T, "K": w.K, "N": w.N, "rotation": w.rot,
            "block": w.block, "quant": w.quant, "a_bits": w.a_bits, "w_bits": w.w_bits,
            "codes": "mma" if use_mma(w) else "canonical",
            "rotate_quant_us": {"mean": round(float(r.mean()), 2), "median": round(pct(r, 50), 2),
                                "p10": round(pct(r, 10), 2), "p90": round(pct(r, 90), 2)},
            "rotate_quant_GBps": round(rotate_bytes(w) / (r.mean() * 1e-6) / 1e9, 1),
            "gemm_us": {"mean": round(float(g.mean()), 2), "median": round(pct(g, 50), 2),
                        "p10": round(pct(g, 10), 2), "p90": round(pct(g, 90), 2)},
            "gemm_TOPS": round(w.ops() / (g.mean() * 1e-6) / 1e12, 1),
            "layer_us": round(float((r + g).mean()), 2),
        }
        if rotate_flops(w):
            entry["rotate_TFLOPs"] = round(rotate_flops(w) / (r.mean() * 1e-6) / 1e12, 2)
        layers.append(entry)
        log(f"[bench] {json.dumps(entry)}")

    w0 = wls[0]
    if w0.quant == "lloydmax":
        peak, gsrc, gkey, gname, dtype = PEAK_BF16_TFLOPS, "rq_gemm_codebook.hip", "gemm_codebook", \
            "gemm_cb_kernel", "bf16"
    elif w0.quant == "mxfp4":
        peak, gsrc, gkey, gname, dtype = PEAK_FP6_TOPS, "rq_gemm_mx.hip", "gemm_mx", "gemm_mx_kernel", "fp4"
    elif w0.a_bits != 4:
        peak, gsrc, gkey, gname, dtype = PEAK_INT8_TOPS, "rq_gemm_i8.hip", "gemm_i8", \
            "gemm_i8_kernel", "i8"
    elif int8_gemm:
        peak, gsrc, gkey, gname, dtype = PEAK_INT8_TOPS, "rq_gemm_w4a4.hip", "gemm_int8", \
            "gemm_w4a4_kernel", "i8"
    else:
        # the INT4 GEMM computes on the FP6 matrix cores: its own dtype's peak
        peak, gsrc, gkey, gname, dtype = (PEAK_FP6_TOPS, "rq_gemm_fp6.hip", "gemm", "gemm_fp6_mma_kernel", "fp6")
        if not use_mma(w0):
            gkey, gname = "gemm_conv", "gemm_fp6_kernel"
    gemm_mean_ms = float(np.mean(gemm_ms))
    achieved = float(np.mean(ops)) / (gemm_mean_ms * 1e-3) / 1e12
    traffic = profiled_traffic(gsrc, f"{gkey}_{args.workload}_counters.json")
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s" if w0.quant == "lloydmax" else "TOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": gname,
                "timing": "mean of per-launch HIP-event durations on the launch stream"}
    if sclk:
        roofline["frac_at_measured_sclk"] = round(achieved / (peak * sclk / 2400.0), 4)
    rot_mean_ms = float(np.mean(rot_ms))
    if w0.rot == "rpbh":
        rot_bytes = float(np.mean([rotate_bytes(w) for w in wls]))
        rot_gbs = rot_bytes / (rot_mean_ms * 1e-3) / 1e9
        roofline_rot = {"bound": "hbm", "achieved": round(rot_gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(rot_gbs / PEAK_HBM_GBS, 4),
                        "traffic": profiled_traffic("rq_rpbh.hip", f"rotate_{args.workload}_counters.json"),
                        "kernel": "rpbh_quant_kernel"}
    else:
        fl = float(np.mean([rotate_flops(w) for w in wls])) / (rot_mean_ms * 1e-3) / 1e12
        roofline_rot = {"bound": "alu", "achieved": round(fl, 2), "peak": PEAK_FP32_FMA_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(fl / PEAK_FP32_FMA_TFLOPS, 4), "traffic": None,
                        "kernel": "dense_rotate_kernel" if w0.rot == "dense" else "trdq_tile_kernel"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(names, args.cpu_budget)
        cpu["cpu_model"] = cpu_model()
        one = cpu_baseline(names, args.cpu_budget / 4, threads=1)
        cpu["one_thread"] = {"value": one["value"], "unit": one["unit"], "sample": one["sample"]}

    out = {
        "metric": "fused rotate+quant+W4A4 linear TOPS & ms/layer at FLUX-scale; % int8 MFMA peak",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"steps": settle_steps, "ms": round(settle_ms, 1)},
        "ms_per_step": round(ms_step, 4),
        "ms_per_layer": round(ms_step / nl, 4),
        "pct_int8_peak": round(100 * value / PEAK_INT8_TOPS, 2),
        "pct_fp6_peak": round(100 * value / PEAK_FP6_TOPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "layers": [
            {"name": w.name, "T": w.T, "K": w.K, "N": w.N, "rotation": w.rot, "block": w.block,
             "r": w.r, "quant": w.quant, "a_bits": w.a_bits, "w_bits": w.w_bits, "x": w.xdtype,
             "y": w.ydtype} for w in wls],
            "ring_instances": args.ring, "engine": args.engine},
        "sclk_mhz": sclk,
        "layers": layers,
        "roofline": roofline,
        "roofline_rotate_quant": roofline_rot,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
