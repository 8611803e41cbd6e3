"""HLWQ quantize + dequantize throughput on one MI355X.

Default workload (the headline): HLWQ Q5 of one Qwen3.6-35B-A3B-shaped MoE
layer, 256 experts, gate_up [256, 1024, 2048] and down [256, 2048, 512] bf16
(805,306,368 weights, 2.13 GB of algorithmic traffic per direction).  One step
= quantize of both banks (one grouped launch) followed by the dequantize of the
result (one grouped launch).  Inputs are seeded synthetic N(0, 0.02^2) values
with 0.1 % of each expert's entries scaled by 20, resident in HBM before timing
starts; the step's working set (5.8 GB) is far larger than the 256 MB
Infinity Cache, so every step streams from HBM.  The same run then times the
Gemma-4-26B-A4B-shaped bank (gate_up [128, 1408, 2816], down [128, 2816, 704])
the same way and reports it under "gemma4_moe_bank".

Other workloads (--config) use the same procedure: the Gemma-4-26B-A4B-shaped
bank alone, the dense hidden-5120 Linears (Q5 or --bits 3; dense_5120_int4
follows the quantize with the fused dequantize -> INT4), the H256 KV cache (Q3
or --bits 2; three independent caches rotate so the working set exceeds the
cache), the whole prompt appended to an empty streaming cache in one call
(kv_h256_prefill), the streaming KV decode step (kv_h256_decode,
latency-bound), and TQ3 on the Qwen3.6-shaped bank (qwen36_moe_bank_tq3).
--layout codes8 stores one code per byte.

Before any warm-up step, the run measures the streaming ceiling of each
kernel's own read:write mix (libhlwq_stream, include/hlwq_stream.h: the same
1 KB-contiguous loads and stores with no arithmetic, best of a few wave and
unit shapes), then runs the workload's own steps for 0.3 s ("settle" in the
output: from idle the card needs ~20 ms of these kernels to reach its steady
clocks), so the W warm-up steps and the K timed steps run at the clocks a
long quantization job sees.

Prints one JSON line: weights/s of quantize + dequantize, with the per-kernel
HBM roofline (algorithmic bytes / kernel time from HIP events on the launch
stream), each kernel's fraction of its mix's streaming ceiling, and the CPU
oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 50] [--warmup 1000] [--config NAME] [--bits 5|3|2] [--layout packed|codes8]
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
# VALU issue peak for unpacked fp32 / integer ops: 256 CUs x 4 SIMDs x 16 lanes
# x 2.4 GHz = 39.3 T lane-ops/s (a wave64 instruction takes 4 cycles on a SIMD)
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
METRIC = "weights/s and achieved HBM GB/s (% of peak) for Q5 quantize+dequantize"

DESCRIPTIONS = {
    "qwen36_moe_bank": ("Qwen3.6-35B-A3B-shaped MoE layer, quantize+dequantize of gate_up "
                        "[256,1024,2048] + down [256,2048,512] bf16, N(0,0.02^2) with 0.1% x20 outliers"),
    "gemma4_moe_bank": ("Gemma-4-26B-A4B-shaped MoE layer, quantize+dequantize of gate_up "
                        "[128,1408,2816] + down [128,2816,704] bf16, N(0,0.02^2)"),
    "dense_5120": ("dense hidden-5120 Linears, quantize+dequantize of [5120,5120] + [17408,5120] + "
                   "[5120,17408] bf16, Student-t(5)*0.02"),
    "kv_h256": ("KV cache K and V [1,4,32768,256] bf16 N(0,1), per-head H256, 8 centroids, 3-bit "
                "(4 centroids, 2-bit with --bits 2), newest 128 tokens kept bf16; quantize+dequantize"),
    "linear_64x256": "single Linear W[64,256] bf16 N(0,0.02^2), quantize+dequantize (launch-bound)",
    "dense_5120_int4": ("dense hidden-5120 Linears [5120,5120] + [17408,5120] + [5120,17408] bf16, "
                        "Student-t(5)*0.02: HLWQ quantize, then dequantize straight to INT4 with a scale and "
                        "zero point per 128-column group"),
    "qwen36_moe_bank_tq3": ("Qwen3.6-35B-A3B-shaped MoE layer (the model of the TQ3 checkpoint), TQ3 "
                            "quantize+dequantize of gate_up [256,1024,2048] + down [256,2048,512] bf16, "
                            "N(0,0.02^2) with 0.1% x20 outliers: random-sign H128 (seed 42), 8 Lloyd-Max "
                            "centroids, 3-bit codes, fp32 shape-gain norms"),
    "kv_h256_prefill": ("streaming KV cache K and V [1,4,32768,256] bf16 N(0,1) with a 128-token bf16 window: "
                        "the whole 32768-token prompt appended to empty caches in one hlwq_kv_append call "
                        "(KV quantize kernel for the tokens that leave the window, a copy into the ring for the rest), "
                        "then dequantized"),
    "kv_h256_decode": ("streaming KV cache K and V [1,4,32768,256] bf16 N(0,1) with a 128-token bf16 window: "
                       "one decode step appends one token to each of the 8 head caches (one launch), encoding "
                       "the 8 tokens that leave the window (latency-bound)"),
}


def algorithmic_bytes(shapes, bits=5, norm_bytes=2):
    """bf16 weights + packed codes + norms (fp16, or TQ3's fp32) moved by one direction."""
    w = p = n = 0
    for E, out, n_in in shapes:
        nb = -(-n_in // 128)
        w += E * out * n_in * 2
        p += E * out * nb * 16 * bits
        n += E * out * nb * norm_bytes
    return w + p + n


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in ("weight_quantization_amd/csrc/hlwq.hip", "weight_quantization_amd/csrc/gen_tables.cpp"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(config, bits):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{config}_q{bits}.txt")
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


def stored_valu(config, bits):
    """VALU instructions per weight (SQ_INSTS_VALU x 64 lanes / weights) of
    the quantize and dequantize kernels from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"counters_{config}_q{bits}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        for key in ("kernel_source_sha256_16", "valu_ops_per_value_quantize", "valu_ops_per_value_dequantize"):
            if line.startswith(key + ":"):
                vals[key] = line.split(":", 1)[1].strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return {"quantize": float(vals["valu_ops_per_value_quantize"]),
                "dequantize": float(vals["valu_ops_per_value_dequantize"]),
                "source": os.path.relpath(path, ROOT)}
    except (KeyError, ValueError):
        return None


# Working sets below this many bytes are held in two copies, and dequantize
# reads the copy that quantize did not just write, so its input comes from HBM
# and not from the 256 MB memory-side cache.
_CACHE_SAFE_BYTES = 1 << 30


# (variant, 4-wave workgroups per CU, bytes of the larger side of a unit):
# the kernels' own shape first (load 16 KB, wait, store; two workgroups per
# CU), then the shapes a sweep found fastest on MI355X (one or two workgroups
# per CU, larger units or double-buffered smaller ones)
CEILING_SHAPES = [(0, 2, 16384), (1, 1, 16384), (1, 1, 32768), (2, 1, 16384), (2, 1, 8192), (3, 1, 4096),
                  (3, 2, 4096)]
_STREAM_MAX_READ = {0: 16384, 1: 32768, 2: 16384, 3: 4096}


class StreamCeiling:
    """Streaming ceilings of a read:write mix on the current device."""

    def __init__(self, torch, dev, read_max, write_max):
        import ctypes
        from weight_quantization_amd import build as wqb
        if not os.path.exists(wqb.STREAM_LIB):
            raise RuntimeError(f"{wqb.STREAM_LIB} is missing: build it with __graft_entry__.build()")
        self.lib = ctypes.CDLL(wqb.STREAM_LIB)
        f = self.lib.hlwq_stream_mix
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        self.torch = torch
        # at least 1 GiB each, and consecutive launches start at rotating
        # offsets, so a small mix streams from HBM and not from the 256 MB
        # memory-side cache (as the kernels' rotating input sets do)
        self.src = torch.empty(max(read_max, _CACHE_SAFE_BYTES) + 65536, dtype=torch.uint8, device=dev)
        self.dst = torch.empty(max(write_max, _CACHE_SAFE_BYTES) + 65536, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()
        self.k = 0

    def _launch(self, r, w, units, variant, wpc):
        import ctypes
        rspan, wspan = self.src.numel() - units * r, self.dst.numel() - units * w
        ro = (self.k * units * r) % rspan // 256 * 256 if rspan > 0 else 0
        wo = (self.k * units * w) % wspan // 256 * 256 if wspan > 0 else 0
        self.k += 1
        st = self.lib.hlwq_stream_mix(self.src.data_ptr() + ro, self.dst.data_ptr() + wo, r, w, units, variant, wpc,
                                      ctypes.c_void_p(self.stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"hlwq_stream_mix failed with status {st}")

    def warm(self, seconds=1.0):
        """Stream for about `seconds` (the kernels' own shape, quantize mix)."""
        units = min(self.src.numel() // 16384, self.dst.numel() // 5248)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(50):
                self._launch(16384, 5248, units, 0, 2)
            self.torch.cuda.synchronize()

    def measure(self, read_total, write_total, reps=10):
        """Best GB/s over CEILING_SHAPES for a launch reading `read_total` and
        writing `write_total` bytes (units scaled to the same mix)."""
        torch = self.torch
        big_is_read = read_total >= write_total
        ratio = min(read_total, write_total) / max(read_total, write_total)
        rows = []
        for variant, wpc, big in CEILING_SHAPES:
            small = max(16, int(round(big * ratio / 16.0)) * 16)
            r, w = (big, small) if big_is_read else (small, big)
            if r > _STREAM_MAX_READ[variant] or w > 32768:
                continue
            units = int(min(read_total // r, write_total // w, self.src.numel() // r, self.dst.numel() // w))
            for _ in range(2):
                self._launch(r, w, units, variant, wpc)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ms = []
            for _ in range(reps):
                e0.record(self.stream)
                self._launch(r, w, units, variant, wpc)
                e1.record(self.stream)
                e1.synchronize()
                ms.append(e0.elapsed_time(e1))
            t = float(np.median(ms))
            rows.append({"variant": variant, "workgroups_per_cu": wpc, "unit_read": r, "unit_write": w,
                         "ms": round(t, 4), "gbs": round(units * (r + w) / (t * 1e-3) / 1e9, 1)})
        best = max(rows, key=lambda x: x["gbs"])
        return {"gbs": best["gbs"], "best": best, "shapes": rows}


def to_device(torch, dev, bits_u16):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).view(torch.bfloat16).to(dev)


def weight_workload(torch, wq, dev, config, bits, layout="packed"):
    tq3 = config.endswith("_tq3")
    if tq3:
        config = config[:-len("_tq3")]
    tensors = list(synth.CONFIGS[config])
    shapes = []
    for t in tensors:
        shape = synth.CONFIGS[config][t][1]
        shapes.append((shape if len(shape) == 3 else (1, *shape)))
    field = 8 if layout == "codes8" else bits   # bits per stored code
    nbytes = algorithmic_bytes(shapes, field, 4 if tq3 else 2)
    w_bytes = sum(E * o * i * 2 for E, o, i in shapes)   # bf16 of the real columns
    c_bytes = nbytes - w_bytes                           # codes + norms
    copies = 1 if nbytes >= _CACHE_SAFE_BYTES else 2
    sets = []
    for c in range(copies):
        qitems, ditems = [], []
        for t, (E, out, n_in) in zip(tensors, shapes):
            shape = synth.CONFIGS[config][t][1]
            w = to_device(torch, dev, synth.weight(config, t, seed=synth.DEFAULT_SEED + c))
            nb = -(-n_in // 128)
            lead = (E, out) if len(shape) == 3 else (out,)
            p = torch.empty(lead + (nb, 16 * field), dtype=torch.uint8, device=dev)
            n = torch.empty(lead + (nb,), dtype=torch.float32 if tq3 else torch.float16, device=dev)
            qitems.append((w, p, n))
            ditems.append((torch.empty_like(w), p, n))
        sets.append((qitems, ditems))
    state = {"i": 0}

    if layout == "codes8":   # one code per byte: one launch per tensor
        def quant():
            for w, p, n in sets[state["i"] % copies][0]:
                wq.hlwq_quantize_codes8(w, bits, codes=p, norms=n)

        def dequant():
            for o, p, n in sets[(state["i"] + 1) % copies][1]:
                wq.hlwq_dequantize_codes8(p, n, o.shape[-1], bits, out=o)
            state["i"] += 1
    elif tq3:
        def quant():
            wq.hlwq_tq3_quantize_grouped(sets[state["i"] % copies][0], 42)

        def dequant():
            wq.hlwq_tq3_dequantize_grouped(sets[(state["i"] + 1) % copies][1], 42)
            state["i"] += 1
    else:
        def quant():
            wq.hlwq_quantize_grouped(sets[state["i"] % copies][0], bits)

        def dequant():
            wq.hlwq_dequantize_grouped(sets[(state["i"] + 1) % copies][1], bits)
            state["i"] += 1

    for c in range(copies):
        state["i"] = c
        quant()
    state["i"] = 0

    return {
        "quantize": quant,
        "dequantize": dequant,
        "weights": sum(E * o * i for E, o, i in shapes),
        "bytes": nbytes,
        "rw": (w_bytes, c_bytes),      # quantize: read, write
        "rw_d": (c_bytes, w_bytes),    # dequantize: read, write
        "kernels": ((f"hlwq_quantize_kernel<3, 3, 2>", f"hlwq_dequantize_kernel<3, 3, 2>") if tq3 else
                    (f"hlwq_quantize_kernel<{bits}, {field}>", f"hlwq_dequantize_kernel<{bits}, {field}>")),
        "launches": len(shapes) if layout == "codes8" else 1,
        "copies": copies,
        "keep": sets,
    }


def int4_workload(torch, wq, dev, bits, config="dense_5120", copies=2):
    """HLWQ quantize of the dense Linears (one grouped launch), then the
    dequantize to INT4 of all of them (one grouped launch); two rotating sets,
    as for the other small working sets."""
    tensors = list(synth.CONFIGS[config])
    shapes = [tuple(synth.CONFIGS[config][t][1]) for t in tensors]
    sets = []
    for c in range(copies):
        items, outs = [], []
        for t, (out, n_in) in zip(tensors, shapes):
            w = to_device(torch, dev, synth.weight(config, t, seed=synth.DEFAULT_SEED + c))
            p, n = wq.hlwq_quantize(w, bits)
            items.append((w, p, n))
            outs.append((torch.empty((out, n_in // 2), dtype=torch.uint8, device=dev),
                         torch.empty((out, n_in // 128), dtype=torch.float32, device=dev),
                         torch.empty((out, n_in // 128), dtype=torch.uint8, device=dev)))
        sets.append((items, outs))
    state = {"i": 0}

    def quant():
        wq.hlwq_quantize_grouped(sets[state["i"] % copies][0], bits)

    def to_int4():
        items, outs = sets[(state["i"] + 1) % copies]
        wq.hlwq_dequantize_int4_grouped([(p, n, q4, sc, z) for (w, p, n), (q4, sc, z) in zip(items, outs)], bits)
        state["i"] += 1

    weights = sum(o * i for o, i in shapes)
    blocks = weights // 128
    return {
        "quantize": quant,
        "dequantize": to_int4,
        "weights": weights,
        "bytes": algorithmic_bytes([(1, o, i) for o, i in shapes], bits),
        # codes + norm in; 64 B of nibbles + fp32 scale + u8 zero point out, per 128 weights
        "bytes_d": blocks * (16 * bits + 2 + 64 + 4 + 1),
        "rw": (weights * 2, blocks * (16 * bits + 2)),
        "rw_d": (blocks * (16 * bits + 2), blocks * (64 + 4 + 1)),
        "kernels": (f"hlwq_quantize_kernel<{bits}>", f"hlwq_dequantize_int4_kernel<{bits}>"),
        "launches": 1,
        "launches_d": 1,
        "copies": copies,
        "keep": sets,
    }


def kv_workload(torch, wq, dev, copies=3, n_residual=128, bits=3):
    """K and V of the cache held as one tensor [2 * batch, heads, tokens, 256]
    (K first), so one launch encodes (or decodes) both; three rotating copies
    (0.9 GB, well past the 256 MB memory-side cache), and dequantize reads a
    copy that quantize did not just write."""
    sets = []
    for c in range(copies):
        host = np.concatenate([synth.kv_cache("kv_h256", t, seed=synth.DEFAULT_SEED + c) for t in ("K", "V")], axis=0)
        kv = to_device(torch, dev, host)
        p, n = wq.hlwq_kv_quantize(kv, n_residual=n_residual, bits=bits)
        out = kv.clone()
        sets.append((kv, p, n, out))
    state = {"i": 0}
    B, H, T, D = synth.CONFIGS["kv_h256"]["K"][1]
    tq = T - n_residual
    elems = 2 * B * H * tq * D

    def quant():
        kv, p, n, _ = sets[state["i"] % copies]
        wq.hlwq_kv_quantize(kv, n_residual=n_residual, bits=bits, packed=p, norms=n)

    def dequant():
        _, p, n, out = sets[(state["i"] + 1) % copies]
        wq.hlwq_kv_dequantize(p, n, out, n_residual=n_residual, bits=bits)
        state["i"] += 1

    return {
        "quantize": quant,
        "dequantize": dequant,
        "weights": elems,
        "bytes": elems * 2 + 2 * B * H * tq * (32 * bits + 2),
        "rw": (elems * 2, 2 * B * H * tq * (32 * bits + 2)),
        "rw_d": (2 * B * H * tq * (32 * bits + 2), elems * 2),
        "kernels": ("hlwq_kv_quantize_kernel", "hlwq_kv_dequantize_kernel"),
        "launches": 1,
        "copies": copies,
        "keep": sets,
    }


def prefill_workload(torch, wq, dev, copies=3, n_residual=128, bits=3):
    """The K and V prompts ([2, 4, 32768, 256]) appended to empty streaming
    caches in one hlwq_kv_append call each step, then the encoded tokens
    dequantized; three rotating sets, as for kv_h256."""
    sets = []
    B, H, T, D = synth.CONFIGS["kv_h256"]["K"][1]
    cap = T - n_residual
    for c in range(copies):
        host = np.concatenate([synth.kv_cache("kv_h256", t, seed=synth.DEFAULT_SEED + c) for t in ("K", "V")], axis=0)
        kv = to_device(torch, dev, host)
        window = torch.empty((2 * B, H, n_residual, D), dtype=torch.bfloat16, device=dev)
        p = torch.empty((2 * B, H, cap, 32 * bits), dtype=torch.uint8, device=dev)
        n = torch.empty((2 * B, H, cap), dtype=torch.float16, device=dev)
        wq.hlwq_kv_append(kv, window, p, n, 0, n_residual=n_residual, bits=bits)
        sets.append((kv, window, p, n, kv.clone()))
    state = {"i": 0}
    elems = 2 * B * H * T * D

    def append():
        kv, window, p, n, _ = sets[state["i"] % copies]
        wq.hlwq_kv_append(kv, window, p, n, 0, n_residual=n_residual, bits=bits)

    def dequant():
        _, _, p, n, out = sets[(state["i"] + 1) % copies]
        wq.hlwq_kv_dequantize(p, n, out, n_residual=n_residual, bits=bits)
        state["i"] += 1

    vec_out = 2 * B * H * cap * (32 * bits + 2)
    return {
        "quantize": append,
        "dequantize": dequant,
        "weights": elems,
        # the prompt in; codes and norms of the tokens that leave, and the window, out
        "bytes": elems * 2 + vec_out + 2 * B * H * n_residual * D * 2,
        # codes and norms in, bf16 of the encoded tokens out
        "bytes_d": vec_out + 2 * B * H * cap * D * 2,
        "rw": (elems * 2, vec_out + 2 * B * H * n_residual * D * 2),
        "rw_d": (vec_out, 2 * B * H * cap * D * 2),
        "kernels": ("hlwq_kv_append (hlwq_kv_quantize_kernel, then hlwq_kv_ring_fill_kernel for the window)",
                    "hlwq_kv_dequantize_kernel"),
        "launches": 2,
        "launches_d": 1,
        "copies": copies,
        "keep": sets,
    }


def decode_workload(torch, wq, dev, bits, steps_total, n_residual=128, pool=64):
    """K and V caches (stacked, [2, 4, ...]) prefilled with 32768 tokens; each
    step appends one token per head through hlwq_kv_append."""
    host = np.concatenate([synth.kv_cache("kv_h256", t) for t in ("K", "V")], axis=0)
    B, H, T, D = host.shape
    kv = to_device(torch, dev, host)
    cap = T - n_residual + steps_total + 1
    packed = torch.empty((B, H, cap, 32 * bits), dtype=torch.uint8, device=dev)
    norms = torch.empty((B, H, cap), dtype=torch.float16, device=dev)
    p0, n0 = wq.hlwq_kv_quantize(kv, n_residual=n_residual, bits=bits)
    packed[:, :, :T - n_residual] = p0
    norms[:, :, :T - n_residual] = n0
    window = torch.empty((B, H, n_residual, D), dtype=torch.bfloat16, device=dev)
    for t in range(T - n_residual, T):
        window[:, :, t % n_residual] = kv[:, :, t]
    del kv, p0, n0
    new = to_device(torch, dev, synth.random_bf16((pool, B, H, 1, D), seed=5, sigma=1.0))
    state = {"tokens": T, "i": 0}

    def step():
        state["tokens"] = wq.hlwq_kv_append(new[state["i"] % pool], window, packed, norms, state["tokens"],
                                            n_residual=n_residual, bits=bits)
        state["i"] += 1

    return step, B * H, B * H * (2 * D + 2 * D + 32 * bits + 2)


def decode_main(args, bits):
    import torch
    import weight_quantization_amd as wq

    wq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    step, vectors, nbytes = decode_workload(torch, wq, dev, bits, args.warmup + 2 * args.steps)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        step()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in range(args.steps)])
    ms_per_step = wall * 1e3 / args.steps
    # the same steps captured in one HIP graph, as a serving loop issues them:
    # replays repeat the captured appends (same cost, positions and sizes), so
    # this is a timing of the launches without host overhead
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            step()
    graph.replay()
    torch.cuda.synchronize()
    replays = 5
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(replays):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / (replays * args.steps)
    result = {
        "metric": "KV decode-step append: vectors encoded per second (latency-bound)",
        "value": vectors / (ms_per_step * 1e-3),
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS["kv_h256_decode"], "name": "kv_h256_decode", "bits": bits,
                   "vectors_per_step": vectors},
        "append": {"ms": round(float(ms.mean()), 4), "ms_median": round(float(np.median(ms)), 4),
                   "ms_min": round(float(ms.min()), 4), "ms_max": round(float(ms.max()), 4)},
        "graph": {"ms_per_step": round(graph_ms, 5), "vectors_per_s": vectors / (graph_ms * 1e-3),
                  "steps_per_graph": args.steps, "replays": replays},
        "roofline": {"bound": "hbm", "kernel": "hlwq_kv_append_small_kernel (one wave per head)", "achieved":
                     round(nbytes / (ms.mean() * 1e-3) / 1e9, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (ms.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS, 6), "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": round(float(ms.mean()), 4),
                     "note": "one launch moves a few KB: launch latency, not bandwidth, sets the time"},
    }
    print(json.dumps(result), flush=True)


def _oracle_samples(config, bits, worker):
    """Inputs for one CPU worker: one expert matrix (or 256 rows) of every
    tensor of the workload, or 1024 tokens of one KV head."""
    if config in ("kv_h256", "kv_h256_prefill"):
        kv = synth.kv_cache("kv_h256", "K", tokens=1024 + 128)
        return [kv[:, worker % kv.shape[1]:][:, :1]]
    source = {"dense_5120_int4": "dense_5120", "qwen36_moe_bank_tq3": "qwen36_moe_bank"}.get(config, config)
    samples = []
    for t in synth.CONFIGS[source]:
        tid, shape, dist, sigma, ofrac, omult = synth.CONFIGS[source][t]
        if len(shape) == 3:
            samples.append(synth.expert_matrix(source, t, worker % shape[0]))
        else:
            rng = synth.stream(synth.DEFAULT_SEED, synth.CONFIG_IDS[source], 90 + tid, worker)
            samples.append(synth.draw(dist, rng, (min(shape[0], 256), shape[1]), sigma, ofrac, omult))
    return samples


def _oracle_worker(args):
    config, bits, worker, budget_s = args
    from oracle import hlwq_ref as ref
    from oracle import lloyd_max
    from oracle import tq3_ref
    lloyd_max.table(bits)  # the codebook is computed once, outside the timing
    tq3_ref.sign_vectors(42)
    samples = _oracle_samples(config, bits, worker)
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        for w in samples:
            if config == "kv_h256_prefill":
                p, n, _ = ref.kv_stream_c([w], n_residual=128, bits=bits)
                ref.kv_dequantize_c(p, n, bits=bits)
                done += p.shape[2] * 256
            elif config == "kv_h256":
                p, n = ref.kv_quantize_c(w, n_residual=128, bits=bits)
                ref.kv_dequantize_c(p, n, bits=bits)
                done += p.shape[2] * 256
            elif config == "qwen36_moe_bank_tq3":
                packed, g = tq3_ref.quantize_c(w, 42)
                tq3_ref.dequantize_c(packed, g, w.shape[1], 42)
                done += w.size
            elif config == "dense_5120_int4":
                packed, n16 = ref.quantize_c(w, bits)
                ref.dequantize_to_int4_c(packed, n16, w.shape[1], bits)
                done += w.size
            else:
                packed, n16 = ref.quantize_c(w, bits)
                ref.dequantize_c(packed, n16, w.shape[1], bits)
                done += w.size
    return done, time.perf_counter() - t0


def _pool_map(n, args):
    """Run _oracle_worker over `args` on n forked processes; the pool is
    closed and joined, so no worker outlives the call."""
    import multiprocessing as mp
    pool = mp.get_context("fork").Pool(n)
    try:
        return pool.map(_oracle_worker, args)
    finally:
        pool.close()
        pool.join()


# One GPU's share of an 8-GPU MI355X host's CPU cores is 16, whatever the
# affinity mask shows; the pool uses every core of the mask up to that share.
HOST_SHARE_CORES = 16


def cpu_baseline(config, bits, budget_s=10.0):
    """The oracle (fp32 canonical tier, plain numpy, untouched) on the host
    cores: one forked process per core (every core of the affinity mask, at
    most one GPU's share of the host), each quantizing and dequantizing its own
    slice of the workload for `budget_s` seconds.  Inputs are drawn before each
    worker's clock starts; only oracle calls are timed."""
    mask = len(os.sched_getaffinity(0))
    cores = max(1, min(HOST_SHARE_CORES, mask))
    single = _pool_map(1, [(config, bits, 0, budget_s / 2)])[0]  # one process alone on the host
    res = _pool_map(cores, [(config, bits, k, budget_s) for k in range(cores)])
    done = sum(r[0] for r in res)
    wall = max(r[1] for r in res)
    what = ("1024 tokens of one KV head" if config in ("kv_h256", "kv_h256_prefill")
            else "one expert matrix (or 256 rows) of each tensor")
    return {
        "value": done / wall,
        "unit": "weights/s",
        "cores": cores,
        "affinity_cores": mask,
        "kind": "oracle",
        "single_process": {"value": single[0] / single[1], "seconds": round(single[1], 2)},
        "sample": f"{cores} processes x {budget_s:.0f} s (every core of the {mask}-core affinity mask, "
                  f"at most {HOST_SHARE_CORES}: one GPU's share of the host), each on {what} of {config} "
                  f"({'TQ3' if config.endswith('_tq3') else f'Q{bits}'} quantize+"
                  f"{'dequantize to INT4' if config == 'dense_5120_int4' else 'dequantize'}, repeated): "
                  f"{done} weights in {wall:.1f} s; "
                  f"{done / wall / cores:.3g} weights/s per core",
    }


def make_workload(torch, wq, dev, config, bits, layout):
    if config == "kv_h256":
        return kv_workload(torch, wq, dev, bits=bits)
    if config == "kv_h256_prefill":
        return prefill_workload(torch, wq, dev, bits=bits)
    if config == "dense_5120_int4":
        return int4_workload(torch, wq, dev, bits)
    return weight_workload(torch, wq, dev, config, bits, layout=layout)


SETTLE_S = 0.3


def settle(torch, wl, seconds=SETTLE_S):
    """Run the workload's steps for `seconds` before the warm-up steps.  From
    idle, the card takes about 25 steps (~20 ms) of these kernels to reach its
    steady clocks, and pure streaming does not bring it there; a
    quantization job of a whole model runs for seconds at the steady rate,
    which is what the K timed steps measure.  Returns the steps run."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            wl["quantize"]()
            wl["dequantize"]()
        n += 20
        torch.cuda.synchronize()
    return n


def time_workload(torch, wl, steps, warmup):
    """W untimed steps, then K timed steps between two synchronisations; HIP
    events on the launch stream around each kernel.  Returns per-step quantize
    and dequantize ms and the wall time of the K steps."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        wl["quantize"]()
        wl["dequantize"]()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        wl["quantize"]()
        ev[s][1].record(stream)
        wl["dequantize"]()
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q_ms = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in range(steps)])
    d_ms = np.array([ev[s][1].elapsed_time(ev[s][2]) for s in range(steps)])
    return q_ms, d_ms, wall


def valu_rate(ops_per_value, values, ms):
    """VALU lane-ops per second of a leg (the committed per-value instruction
    count x 64 lanes, over the live kernel time) against the VALU issue peak."""
    if ops_per_value is None:
        return None
    tops = ops_per_value * values / (ms * 1e-3) / 1e12
    return {"achieved": round(tops, 2), "peak": round(VALU_PEAK_TOPS, 2), "unit": "T VALU lane-ops/s",
            "frac": round(tops / VALU_PEAK_TOPS, 4)}


def roofline_of(kernel, gbs, ceiling_gbs, valu):
    """The roofline of the dominant kernel.  It is HBM-bound ("hbm": algorithmic
    GB/s against 8 TB/s) unless it uses more of the VALU issue peak than of the
    measured streaming rate of its own read:write mix; then it is bound by
    VALU issue ("alu": lane-ops/s against the peak), and the HBM figures are
    kept under "hbm".  Without a committed VALU count it is "hbm"."""
    hbm = {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
           "frac_of_ceiling": round(gbs / ceiling_gbs, 4)}
    if valu is not None and valu["frac"] > gbs / ceiling_gbs:
        return {"bound": "alu", "kernel": kernel, **{k: valu[k] for k in ("achieved", "peak", "unit", "frac")},
                "hbm": hbm}
    return {"bound": "hbm", "kernel": kernel, **hbm, "valu": valu}


def leg(ms, nbytes, weights, ceiling, ops_per_value=None):
    """Timing summary of one kernel (leg of the step): GB/s are algorithmic
    bytes over the mean time; fractions of the 8 TB/s peak and of the
    streaming ceiling of the same read:write mix; with the committed VALU
    count per value, the fraction of the VALU issue peak."""
    gbs = nbytes / (ms.mean() * 1e-3) / 1e9
    out = {"ms": round(float(ms.mean()), 4), "ms_median": round(float(np.median(ms)), 4),
           "ms_min": round(float(ms.min()), 4), "ms_max": round(float(ms.max()), 4),
           "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4), "weights_per_s": weights / (ms.mean() * 1e-3)}
    if ceiling is not None:
        out["ceiling_gbs"] = ceiling["gbs"]
        out["frac_of_ceiling"] = round(gbs / ceiling["gbs"], 4)
    if ops_per_value is not None:
        out["valu"] = valu_rate(ops_per_value, weights, float(ms.mean()))
    return out


def ceilings(ceil, wl):
    q = ceil.measure(*wl["rw"])
    d = ceil.measure(*wl["rw_d"])
    return {"kernel": "hlwq_stream_mix (libhlwq_stream.so): the kernels' loads and stores without arithmetic",
            "quantize_mix": {"read_bytes": wl["rw"][0], "write_bytes": wl["rw"][1], **q},
            "dequantize_mix": {"read_bytes": wl["rw_d"][0], "write_bytes": wl["rw_d"][1], **d}}


def extra_bank(torch, wq, dev, ceil, config, bits, steps, warmup):
    """Time a second MoE-bank workload the same way (its own ceilings too)."""
    print(f"[bench] generating {config}", file=sys.stderr, flush=True)
    wl = make_workload(torch, wq, dev, config, bits, "packed")
    torch.cuda.synchronize()
    ceil.warm(1.0)
    c = ceilings(ceil, wl)
    n_settle = settle(torch, wl)
    print(f"[bench] timing {steps} steps of {config}", file=sys.stderr, flush=True)
    q_ms, d_ms, wall = time_workload(torch, wl, steps, warmup)
    weights, nbytes = wl["weights"], wl["bytes"]
    step_gbs = 2 * nbytes / (wall / steps) / 1e9
    valu = stored_valu(config, bits)
    out = {"workload": DESCRIPTIONS[config], "weights": weights, "bits": bits, "steps": steps, "warmup": warmup,
           "algorithmic_bytes_per_launch": nbytes, "ms_per_step": round(wall * 1e3 / steps, 4),
           "weights_per_s": weights / (wall / steps), "hbm_gbs": round(step_gbs, 1),
           "hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
           "settle": {"seconds": SETTLE_S, "steps": n_settle},
           "quantize": leg(q_ms, nbytes, weights, c["quantize_mix"], (valu or {}).get("quantize")),
           "dequantize": leg(d_ms, nbytes, weights, c["dequantize_mix"], (valu or {}).get("dequantize")),
           "traffic": stored_traffic(config, bits),
           "valu_ops_per_value": valu,
           "ceiling": c}
    del wl
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", default="qwen36_moe_bank", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--bits", type=int, default=None, choices=(5, 3, 2))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-bank", action="store_true",
                    help="skip the Gemma-4-shaped bank the default run also times")
    ap.add_argument("--layout", default="packed", choices=("packed", "codes8"),
                    help="weight codes packed (bits per code) or one code per byte")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the HLWQ path shards by expert, row or head with no "
              "exchange step, so one GPU's throughput is the per-GPU figure; use --gpus 1", file=sys.stderr)
        sys.exit(2)
    config = args.config
    kv = config.startswith("kv_")
    bits = args.bits if args.bits is not None else (3 if kv or config.endswith("_tq3") else 5)
    if config.endswith("_tq3") and (bits != 3 or args.layout != "packed"):
        ap.error("TQ3 is 3-bit with packed codes")
    if kv and bits not in (3, 2):
        ap.error("the KV-cache path is 3- or 2-bit")
    if not kv and bits not in (5, 3):
        ap.error("weights are 5- or 3-bit")
    if config == "kv_h256_decode":
        decode_main(args, bits)
        return
    print(f"[bench] timing the CPU oracle ({config}, Q{bits})", file=sys.stderr, flush=True)

    # the CPU oracle runs first, in forked processes, before this process
    # touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(config, bits)

    import torch
    import weight_quantization_amd as wq

    wq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    print(f"[bench] generating {config}", file=sys.stderr, flush=True)
    wl = make_workload(torch, wq, dev, config, bits, args.layout)
    weights, bytes_dir, launches = wl["weights"], wl["bytes"], wl["launches"]
    bytes_d = wl.get("bytes_d", bytes_dir)  # the second leg may move other bytes (INT4 output)
    launches_d = wl.get("launches_d", launches)
    torch.cuda.synchronize()

    # the headline bank's run also times the other MoE bank
    extra = None
    if config == "qwen36_moe_bank" and bits == 5 and args.layout == "packed" and not args.no_extra_bank:
        extra = "gemma4_moe_bank"

    # streaming ceilings of both kernels' mixes; about a second of streaming
    # first, which also brings the card to its steady clocks
    rmax = max(wl["rw"][0], wl["rw_d"][0])
    wmax = max(wl["rw"][1], wl["rw_d"][1])
    if extra is not None:
        gb = sum(E * o * i * 2 for E, o, i in (synth.CONFIGS[extra][t][1] for t in synth.CONFIGS[extra]))
        rmax, wmax = max(rmax, gb), max(wmax, gb)
    print("[bench] measuring the streaming ceilings", file=sys.stderr, flush=True)
    ceil = StreamCeiling(torch, dev, rmax, wmax)
    ceil.warm(1.0)
    ceiling = ceilings(ceil, wl)
    n_settle = settle(torch, wl)

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    q_ms, d_ms, wall = time_workload(torch, wl, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps

    dom = 0 if q_ms.mean() >= d_ms.mean() else 1
    dom_ms = max(q_ms.mean(), d_ms.mean())
    dom_bytes, dom_launches = (bytes_dir, launches) if dom == 0 else (bytes_d, launches_d)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = stored_traffic(config, bits) if args.layout == "packed" else None
    valu = stored_valu(config, bits) if args.layout == "packed" else None
    roofline = roofline_of(wl["kernels"][dom] + ("" if dom_launches == 1 else f" ({dom_launches} launches per step)"),
                           achieved, ceiling["quantize_mix" if dom == 0 else "dequantize_mix"]["gbs"],
                           valu_rate(None if valu is None else valu["quantize" if dom == 0 else "dequantize"],
                                     weights, float(dom_ms)))
    roofline.update({
        "traffic": (None if traffic is None else
                    traffic["quantize_bytes_per_launch" if dom == 0 else "dequantize_bytes_per_launch"]),
        "algorithmic_bytes_per_launch": dom_bytes // dom_launches,
        "avg_launch_ms": round(dom_ms / dom_launches, 4),
    })
    step_gbs = (bytes_dir + bytes_d) / (ms_per_step * 1e-3) / 1e9
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
        # the arithmetic is fp32 (norms, butterflies, compares); weights are
        # read and written as bf16
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[config], "name": config, "weights": weights, "bits": bits,
                   "block": 256 if config.startswith("kv_") else 128, "input_sets": wl["copies"],
                   "layout": "packed" if config.startswith("kv_") else args.layout},
        "hbm_gbs": round(step_gbs, 1),
        "hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        # untimed steps run before the W warm-up steps, until the card's
        # clocks have settled (see settle())
        "settle": {"seconds": SETTLE_S, "steps": n_settle},
        "quantize": leg(q_ms, bytes_dir, weights, ceiling["quantize_mix"], (valu or {}).get("quantize")),
        "dequantize": leg(d_ms, bytes_d, weights, ceiling["dequantize_mix"], (valu or {}).get("dequantize")),
        "roofline": roofline,
        # VALU instructions per quantised value from the committed counters
        # (null when they were taken on other kernel source)
        "valu_ops_per_value": valu,
        "ceiling": ceiling,
    }
    del wl
    torch.cuda.empty_cache()
    if extra is not None:
        result[extra] = extra_bank(torch, wq, dev, ceil, extra, bits, args.steps, args.warmup)
    del ceil
    torch.cuda.empty_cache()
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
