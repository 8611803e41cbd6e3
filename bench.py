"""HLWQ Q5 quantize + dequantize throughput on one MI355X.

One step = HLWQ Q5 quantize of a whole MoE layer's expert banks followed by the
dequantize of the result, each as one grouped launch over the two banks: the
Qwen3.6-35B-A3B-shaped layer, 256 experts, gate_up [256, 1024, 2048] and down
[256, 2048, 512] bf16 (805,306,368 weights, 2.13 GB of algorithmic traffic per
direction).  Inputs are seeded synthetic N(0, 0.02^2) values with 0.1 % of each
expert's entries scaled by 20, resident in HBM before timing starts.

Prints one JSON line: weights/s of quantize + dequantize, with the per-kernel
HBM roofline (algorithmic bytes / kernel time from HIP events on the launch
stream) and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 50] [--warmup 1000] [--config NAME]
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

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "weights/s and achieved HBM GB/s (% of peak) for Q5 quantize+dequantize"

WORKLOADS = {
    "qwen36_moe_bank": ("Qwen3.6-35B-A3B-shaped MoE layer, Q5 quantize+dequantize of gate_up "
                        "[256,1024,2048] + down [256,2048,512] bf16, N(0,0.02^2) with 0.1% x20 outliers"),
    "gemma4_moe_bank": ("Gemma-4-26B-A4B-shaped MoE layer, Q5 quantize+dequantize of gate_up "
                        "[128,1408,2816] + down [128,2816,704] bf16, N(0,0.02^2)"),
}


def algorithmic_bytes(shapes, bits=5):
    """bf16 weights + packed codes + fp16 norms moved by one direction."""
    w = p = n = 0
    for E, out, n_in in shapes:
        nb = -(-n_in // 128)
        w += E * out * n_in * 2
        p += E * out * nb * 16 * bits
        n += E * out * nb * 2
    return w + p + n


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in ("weight_quantization_amd/csrc/hlwq.hip", "weight_quantization_amd/csrc/gen_tables.cpp"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(config):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{config}_q5.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return {k: float(vals[k]) for k in ("quantize_bytes_per_launch", "dequantize_bytes_per_launch")}
    except (KeyError, ValueError):
        return None


def copy_ceiling(torch, dev, nbytes, reps=10):
    """Device-to-device copy moving the same number of bytes (half read, half
    written) as one quantize or dequantize launch: the practical HBM ceiling."""
    n = nbytes // 4  # bytes read = bytes written = nbytes / 2
    src = torch.empty(n // 2, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    moved = 2 * src.numel() * 4
    del src, dst
    return {"gbs": round(moved / (ms * 1e-3) / 1e9, 1), "bytes": moved, "ms": round(ms, 4),
            "kernel": "torch copy_ (float32 device-to-device)"}


def cpu_baseline(config, budget_s=12.0):
    """The oracle (fp32 canonical tier) on whole expert matrices until the budget is used."""
    from oracle import hlwq_ref as ref
    tensors = list(synth.CONFIGS[config])
    done_w = 0
    mats = 0
    t0 = time.perf_counter()
    e = 0
    while time.perf_counter() - t0 < budget_s and e < 256:
        for t in tensors:
            w = synth.expert_matrix(config, t, e)
            packed, n16 = ref.quantize_c(w, 5)
            ref.dequantize_c(packed, n16, w.shape[1], 5)
            done_w += w.size
            mats += 1
        e += 1
    dt = time.perf_counter() - t0
    return {
        "value": done_w / dt,
        "unit": "weights/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{mats} expert matrices ({e} experts x {len(tensors)} banks) of {config}, "
                  f"Q5 quantize+dequantize, one process, {dt:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the card needs a few hundred milliseconds of sustained load to reach its
    # steady clocks; 1000 untimed steps is about 0.8 s
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", default="qwen36_moe_bank", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the HLWQ path shards by expert / row with no exchange, "
              "and multi-GPU runs are not part of this build; use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_quantization_amd as wq

    wq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    config = args.config
    tensors = list(synth.CONFIGS[config])
    shapes = [synth.CONFIGS[config][t][1] for t in tensors]
    weights = sum(E * o * i for E, o, i in shapes)
    bytes_dir = algorithmic_bytes(shapes)

    print(f"[bench] generating {config} ({weights} weights)", file=sys.stderr, flush=True)
    qitems, ditems = [], []
    for t, (E, out, n_in) in zip(tensors, shapes):
        host = synth.weight(config, t)
        w = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).to(dev)
        del host
        nb = -(-n_in // 128)
        p = torch.empty((E, out, nb, 80), dtype=torch.uint8, device=dev)
        n = torch.empty((E, out, nb), dtype=torch.float16, device=dev)
        qitems.append((w, p, n))
        ditems.append((torch.empty_like(w), p, n))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        wq.hlwq_quantize_grouped(qitems, 5)
        wq.hlwq_dequantize_grouped(ditems, 5)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        wq.hlwq_quantize_grouped(qitems, 5)
        ev[s][1].record(stream)
        wq.hlwq_dequantize_grouped(ditems, 5)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q_ms = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in range(args.steps)])
    d_ms = np.array([ev[s][1].elapsed_time(ev[s][2]) for s in range(args.steps)])
    ms_per_step = wall * 1e3 / args.steps

    q_gbs = bytes_dir / (q_ms.mean() * 1e-3) / 1e9
    d_gbs = bytes_dir / (d_ms.mean() * 1e-3) / 1e9
    dominant = "quantize" if q_ms.mean() >= d_ms.mean() else "dequantize"
    dom_ms = max(q_ms.mean(), d_ms.mean())
    achieved = bytes_dir / (dom_ms * 1e-3) / 1e9
    traffic = stored_traffic(config)
    roofline = {
        "bound": "hbm",
        "kernel": f"hlwq_{dominant}_kernel<5> (grouped launch over both banks)",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": (None if traffic is None else traffic[f"{dominant}_bytes_per_launch"]),
        "algorithmic_bytes_per_launch": bytes_dir,
        "avg_launch_ms": round(dom_ms, 4),
    }
    result = {
        "metric": METRIC,
        "value": weights / (ms_per_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[config], "weights": weights, "bits": 5, "block": 128,
                   "experts": shapes[0][0]},
        "hbm_gbs": round(2 * bytes_dir / (ms_per_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(2 * bytes_dir / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "quantize": {"ms": round(float(q_ms.mean()), 4), "ms_min": round(float(q_ms.min()), 4),
                     "gbs": round(q_gbs, 1), "weights_per_s": weights / (q_ms.mean() * 1e-3)},
        "dequantize": {"ms": round(float(d_ms.mean()), 4), "ms_min": round(float(d_ms.min()), 4),
                       "gbs": round(d_gbs, 1), "weights_per_s": weights / (d_ms.mean() * 1e-3)},
        "roofline": roofline,
    }
    result["copy_ceiling"] = copy_ceiling(torch, dev, bytes_dir)
    result["copy_frac"] = round(2 * bytes_dir / (ms_per_step * 1e-3) / 1e9 / result["copy_ceiling"]["gbs"], 4)
    del qitems, ditems
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(config)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
