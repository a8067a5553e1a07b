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
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E

WORKLOADS = {
    "flux": ["flux_up", "flux_down"],
    "flux_up": ["flux_up"],
    "flux_down": ["flux_down"],
    "tiny": ["tiny"],
    "pixart": ["pixart"],
    "video": ["video"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(name: str) -> str:
    p = os.path.join(ROOT, "rotated_w4a4_quantized_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def profiled_traffic(kernel_file: str, summary: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when that summary is missing or was taken on a different kernel
    source."""
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


def rotate_bytes(w) -> int:
    """Algorithmic HBM bytes of one rotate+quant launch: X read, codes,
    scales (and top) written."""
    xb = 4 if w.xdtype == "f32" else 2
    b = w.T * w.K * xb + w.T * (w.Kq // 2) + 4 * w.T
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
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(token-parallel sharding is described in the design notes); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from rotated_w4a4_quantized_amd import datagen, rq
    from tests import _layer as H

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rq.load()
    names = WORKLOADS[args.workload]
    wls = [datagen.WORKLOADS[n] for n in names]

    # ring of independent instances (distinct seeds), all resident in HBM
    ring = []
    for i in range(args.ring):
        layers = []
        for w in wls:
            inp = datagen.make_inputs(w, seed_offset=100 * i)
            layers.append(H.GpuLayer(w, inp))
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
    peak = PEAK_BF16_TFLOPS if is_codebook else PEAK_INT8_TOPS
    gemm_mean_ms = float(np.mean(gemm_ms))
    achieved = float(np.mean(ops)) / (gemm_mean_ms * 1e-3) / 1e12
    traffic = profiled_traffic("rq_gemm.hip", f"gemm_{args.workload}_counters.json")
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s" if is_codebook else "TOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": "gemm_codebook_kernel" if is_codebook else "gemm_w4a4_kernel"}
    rot_mean_ms = float(np.mean(rot_ms))
    rot_bytes = float(np.mean([rotate_bytes(w) for w in wls]))
    rot_gbs = rot_bytes / (rot_mean_ms * 1e-3) / 1e9
    roofline_rot = {"bound": "hbm", "achieved": round(rot_gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(rot_gbs / PEAK_HBM_GBS, 4),
                    "traffic": profiled_traffic("rq_rotate.hip",
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
        "dtype": "bf16" if is_codebook else "i8",
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
