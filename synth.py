"""Seeded synthetic inputs for the HLWQ quantize / dequantize workloads.

This module is shared by the tests, the benchmark and the CPU oracle checks.
It holds no quantization arithmetic: only random draws and the rounding of the
drawn float32 values to the bf16 storage format the weights arrive in.

Every tensor comes from its own PCG64 stream keyed by
``(seed, config_id, tensor_id, expert_id)``, so one expert matrix of a bank can
be regenerated on its own and checked in isolation.

Workloads (shapes follow the model cards):

* ``linear_64x256``   one Linear W[64, 256], N(0, 0.02^2), seed 0.
* ``qwen36_moe_bank`` a Qwen3.6-35B-A3B-shaped MoE layer: 256 experts,
  gate_up [256, 1024, 2048] and down [256, 2048, 512], N(0, 0.02^2) with 0.1 %
  of the entries of every expert matrix (chosen without replacement) scaled by
  20 before rounding.  (Model card "Qwen3.6-35B-A3B — HLWQ Q5", table
  "Architecture": hidden 2048, expert intermediate 512, 256 experts.)
* ``gemma4_moe_bank`` a Gemma-4-26B-A4B-shaped MoE layer: gate_up
  [128, 1408, 2816] and down [128, 2816, 704], N(0, 0.02^2).  (Model card
  "Gemma-4-26B-A4B-it-HLWQ-Q5", section "Technical Details".)  in = 704 is not a
  multiple of 128, so every down row ends in a zero-padded block.
* ``dense_5120``      dense Linears of a hidden-5120 model: [5120, 5120],
  [17408, 5120], [5120, 17408], Student-t(5) * 0.02.  (Model card
  "Qwopus3.6-27B-v2 · HLWQ Q5", section "Architecture": hidden_size 5120.)
* ``kv_h256``         K and V caches [1, 4, 32768, 256], N(0, 1).  (Same card:
  4 KV heads, head_dim 256.)

Trained weights are not available; these seeded tensors stand in for them.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

CONFIG_IDS = {
    "linear_64x256": 0,
    "qwen36_moe_bank": 1,
    "gemma4_moe_bank": 2,
    "dense_5120": 3,
    "kv_h256": 4,
}

# tensor name -> (tensor_id, shape, distribution, sigma, outlier_frac, outlier_mult)
# shape is (experts, out, in) for weight banks, (out, in) for single Linears,
# (batch, heads, tokens, head_dim) for KV caches.
CONFIGS = {
    "linear_64x256": {
        "W": (0, (64, 256), "normal", 0.02, 0.0, 1.0),
    },
    "qwen36_moe_bank": {
        "gate_up": (0, (256, 1024, 2048), "normal", 0.02, 0.001, 20.0),
        "down": (1, (256, 2048, 512), "normal", 0.02, 0.001, 20.0),
    },
    "gemma4_moe_bank": {
        "gate_up": (0, (128, 1408, 2816), "normal", 0.02, 0.0, 1.0),
        "down": (1, (128, 2816, 704), "normal", 0.02, 0.0, 1.0),
    },
    "dense_5120": {
        "qo": (0, (5120, 5120), "student_t5", 0.02, 0.0, 1.0),
        "mlp_up": (1, (17408, 5120), "student_t5", 0.02, 0.0, 1.0),
        "mlp_down": (2, (5120, 17408), "student_t5", 0.02, 0.0, 1.0),
    },
    "kv_h256": {
        "K": (0, (1, 4, 32768, 256), "normal", 1.0, 0.0, 1.0),
        "V": (1, (1, 4, 32768, 256), "normal", 1.0, 0.0, 1.0),
    },
}

DEFAULT_SEED = 0


def stream(seed: int, config_id: int, tensor_id: int, expert_id: int) -> np.random.Generator:
    """The PCG64 stream for one (config, tensor, expert) triple."""
    return np.random.default_rng([seed, config_id, tensor_id, expert_id])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw(dist: str, rng: np.random.Generator, shape, sigma: float,
         outlier_frac: float = 0.0, outlier_mult: float = 1.0) -> np.ndarray:
    """Draw one matrix in float32 and round it to bf16 bits."""
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "student_t5":
        x = rng.standard_t(5, size=shape).astype(np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    x *= np.float32(sigma)
    if outlier_frac > 0.0:
        n = int(np.prod(shape))
        k = int(round(outlier_frac * n))
        idx = rng.choice(n, size=k, replace=False)
        flat = x.reshape(-1)
        flat[idx] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def tensor_spec(config: str, tensor: str):
    return CONFIGS[config][tensor]


def expert_matrix(config: str, tensor: str, expert: int, seed: int = DEFAULT_SEED) -> np.ndarray:
    """One [out, in] matrix of a bank (expert index ignored for 2-D tensors)."""
    tid, shape, dist, sigma, ofrac, omult = CONFIGS[config][tensor]
    mat_shape = shape[-2:]
    r = stream(seed, CONFIG_IDS[config], tid, expert)
    return draw(dist, r, mat_shape, sigma, ofrac, omult)


def weight(config: str, tensor: str, seed: int = DEFAULT_SEED, workers: int = 8) -> np.ndarray:
    """A whole weight tensor as bf16 bits: [E, out, in] for banks, [out, in] otherwise.

    Experts are drawn on a thread pool (numpy's generators release the GIL);
    each expert has its own stream, so the result does not depend on `workers`.
    """
    tid, shape, dist, sigma, ofrac, omult = CONFIGS[config][tensor]
    if len(shape) == 2:
        return expert_matrix(config, tensor, 0, seed)
    out = np.empty(shape, dtype=np.uint16)

    def fill(e):
        out[e] = expert_matrix(config, tensor, e, seed)

    if workers > 1:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(shape[0])))
    else:
        for e in range(shape[0]):
            fill(e)
    return out


def kv_cache(config: str, tensor: str, seed: int = DEFAULT_SEED, tokens: int | None = None) -> np.ndarray:
    """A KV cache [batch, heads, tokens, head_dim] as bf16 bits, one stream per head."""
    tid, shape, dist, sigma, ofrac, omult = CONFIGS[config][tensor]
    b, h, t, d = shape
    if tokens is not None:
        t = tokens
    out = np.empty((b, h, t, d), dtype=np.uint16)
    for bi in range(b):
        for hi in range(h):
            r = stream(seed, CONFIG_IDS[config], tid, bi * h + hi)
            out[bi, hi] = draw(dist, r, (t, d), sigma, ofrac, omult)
    return out


def random_bf16(shape, seed: int, key: int = 0, dist: str = "normal", sigma: float = 0.02,
                outlier_frac: float = 0.0, outlier_mult: float = 1.0) -> np.ndarray:
    """Ad-hoc seeded tensor for tests (config id 99)."""
    r = stream(seed, 99, key, 0)
    return draw(dist, r, tuple(shape), sigma, outlier_frac, outlier_mult)
