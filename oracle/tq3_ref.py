"""TQ3 (scalar HIGGS) quantize / dequantize, plain CPU reference (oracle).

TEST INFRASTRUCTURE ONLY: see the package docstring of ``oracle``.

The method ("Qwen3.6-35B-A3B-TQ3-native", section "What TQ3 actually does";
section "Files" for the stored tensors and ``tq_config.json``):

* a weight row is cut into groups of 128 consecutive values;
* every group is rotated by a Walsh-Hadamard transform wrapped in two random
  +-1 sign vectors;
* every rotated value is replaced by the index of the nearest of 8 Lloyd-Max
  centroids for N(0, 1) (3 bits);
* every group keeps one fp32 "shape-gain" norm, the original norm divided by
  the norm of the reconstruction;
* stored tensors: packed codes (uint8) and the norms (float32); the quantizer
  state is bits = 3, group size = 128, seed = 42.

Readings (the page leaves these open; the plainest reading is taken):

R1  rotation.  R = D2 H D1 / sqrt(128): D1 multiplies the group before the
    unnormalised Sylvester transform H, D2 multiplies its output.  R is
    orthogonal, so the inverse is R^T = D1 H D2 / sqrt(128).
R2  sign generator.  The page names a seed but no generator.  Both vectors come
    from SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014; the generator of Java's
    SplittableRandom): output i (i = 0, 1, 2, ...) for a seed s is
    mix64(s + (i + 1) * 0x9E3779B97F4A7C15 mod 2^64).  Entry i of D1 is -1 when
    bit 63 of output i is set, entry i of D2 likewise with output 128 + i.
    Parity with checkpoints made by the page's own tool is therefore unpinned;
    the generator itself is pinned to its published outputs.
R3  scale.  Like HLWQ, the rotated unit vector is multiplied by sqrt(128) so its
    coordinates follow the codebook's N(0, 1): y = sqrt(128) R x / ||x||; a zero
    group gives y = 0.
R4  shape-gain.  The reconstruction of the unit vector u = x / ||x|| is
    R^T c[codes] / sqrt(128), of norm ||c[codes]|| / sqrt(128); the stored norm
    is g = ||x|| / that, and dequantisation returns g R^T c[codes] / sqrt(128),
    whose norm is ||x|| exactly (in real arithmetic).
R5  packing.  The page fixes only "uint8"; codes use the HLWQ 3-bit packing
    (8 codes -> 3 bytes, first code in the low bits), 48 bytes per group, the
    last group of a row zero-padded.

Tier D (fp64) is the definition; tier C (fp32) fixes one operation order:

  quantize:  n = norm tree of the squares (as HLWQ), correctly rounded sqrt;
             r = RN(1 / n), 0 when n is below the smallest normal fp32;
             z = butterflies (strides 1, 2, ..., 64) of D1 x (exact sign flips);
             y = D2 RN(z r)  (exact sign flips);
             code = number of fp32 thresholds strictly below y;
             e = RN(c[code]^2); rho2 = the exact sum of the 128 e values,
             rounded once to fp32 (the sum of squares has no order of its
             own; this one does not depend on any); rho = correctly rounded
             sqrt;
             t = RN(rho * RN(1 / sqrt(128))); g = RN(n / t).
  dequant :  v = D2 c[code]; z = butterflies of v; s = RN(g * 2^-7);
             out = bf16_RNE(D1 RN(z s)).
"""
from __future__ import annotations

import math

import numpy as np

from . import hlwq_ref, lloyd_max

GROUP = 128
BITS = 3
SEED = 42  # "Qwen3.6-35B-A3B-TQ3-native", section "Files": tq_config.json
_M64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


# --------------------------------------------------------------------------
# R2: SplitMix64 and the two sign vectors
# --------------------------------------------------------------------------

def splitmix64(seed: int, count: int) -> list[int]:
    """The first `count` outputs of SplitMix64 for `seed` (Steele, Lea & Flood 2014).

    State s_i = seed + i * gamma (mod 2^64); output i = mix64(s_{i+1}) with
    mix64(z): z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
    z *= 0x94D049BB133111EB; z ^= z >> 31 (all mod 2^64).
    """
    out = []
    s = seed & _M64
    for _ in range(count):
        s = (s + _GAMMA) & _M64
        z = s
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        out.append(z ^ (z >> 31))
    return out


def sign_vectors(seed: int = SEED, n: int = GROUP) -> tuple[np.ndarray, np.ndarray]:
    """(D1, D2) as int8 arrays of +-1 (reading R2)."""
    draws = splitmix64(seed, 2 * n)
    s = np.array([-1 if (v >> 63) else 1 for v in draws], dtype=np.int8)
    return s[:n].copy(), s[n:].copy()


# --------------------------------------------------------------------------
# Tier D: definition in fp64
# --------------------------------------------------------------------------

def rotation_matrix(d1: np.ndarray, d2: np.ndarray) -> np.ndarray:
    """R = D2 H D1 / sqrt(L) as a dense fp64 matrix (reading R1); y = R @ x."""
    L = len(d1)
    h = hlwq_ref.sylvester_hadamard(L)
    return (np.asarray(d2, np.float64)[:, None] * h * np.asarray(d1, np.float64)[None, :]) / math.sqrt(L)


def quantize_def(x_groups: np.ndarray, d1: np.ndarray, d2: np.ndarray):
    """Tier D on (..., 128) groups: returns (codes, g fp64, y fp64, n fp64)."""
    x = np.asarray(x_groups, dtype=np.float64)
    L = x.shape[-1]
    c32, _ = lloyd_max.table(BITS)
    n = np.sqrt(np.sum(x * x, axis=-1))
    safe = np.where(n > 0.0, n, 1.0)
    u = np.where((n > 0.0)[..., None], x / safe[..., None], 0.0)
    y = (u @ rotation_matrix(d1, d2).T) * math.sqrt(L)
    codes = hlwq_ref.nearest_code(y, c32)
    yhat = c32.astype(np.float64)[codes]
    recon_norm = np.sqrt(np.sum(yhat * yhat, axis=-1)) / math.sqrt(L)
    return codes, n / recon_norm, y, n


def dequantize_def(codes: np.ndarray, g: np.ndarray, d1: np.ndarray, d2: np.ndarray) -> np.ndarray:
    """Tier D inverse: g * R^T c[codes] / sqrt(L), fp64, unrounded (reading R4)."""
    c32, _ = lloyd_max.table(BITS)
    yhat = c32.astype(np.float64)[np.asarray(codes)]
    L = yhat.shape[-1]
    return np.asarray(g, np.float64)[..., None] * (yhat @ rotation_matrix(d1, d2)) / math.sqrt(L)


# --------------------------------------------------------------------------
# Tier C: canonical fp32 operation order
# --------------------------------------------------------------------------

def recon_sumsq_f32(codes: np.ndarray, c32: np.ndarray) -> np.ndarray:
    """rho^2 of tier C: the squares e = RN(c^2), summed exactly, rounded once.

    Every e is an fp32 value in [c_min^2, c_max^2] ~ [0.06, 4.64], a multiple of
    2^-28, and 128 of them sum to less than 2^10, so every partial sum is a
    multiple of 2^-28 below 2^10: 38 significant bits, exact in fp64.  The fp64
    sum is therefore the exact sum, and its conversion the one rounding.
    """
    e = (c32 * c32).astype(np.float32)[np.asarray(codes)]
    return np.sum(e.astype(np.float64), axis=-1).astype(np.float32)


def quantize_groups_c(x: np.ndarray, d1: np.ndarray, d2: np.ndarray):
    """Tier C on (..., 128) float32 groups: returns (codes, g float32, y float32)."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle inputs must be finite")
    c32, b32 = lloyd_max.table(BITS)
    f = np.float32
    n = hlwq_ref.norm_tree_f32(x)
    with np.errstate(divide="ignore"):
        r = np.where(n >= hlwq_ref.FLT_MIN, f(1.0) / n, f(0.0)).astype(f)
    z = hlwq_ref.fwht_f32(x * np.asarray(d1, dtype=f))
    y = ((z * r[..., None]).astype(f) * np.asarray(d2, dtype=f)).astype(f)
    codes = hlwq_ref.codes_from_y(y, b32)
    rho = np.sqrt(recon_sumsq_f32(codes, c32)).astype(f)
    t = (rho * f(1.0 / math.sqrt(GROUP))).astype(f)
    g = (n / t).astype(f)
    return codes, g, y


def dequantize_groups_c(codes: np.ndarray, g: np.ndarray, d1: np.ndarray, d2: np.ndarray) -> np.ndarray:
    """Tier C inverse on (..., 128) codes: float32 before the bf16 rounding."""
    c32, _ = lloyd_max.table(BITS)
    f = np.float32
    v = (c32[np.asarray(codes)] * np.asarray(d2, dtype=f)).astype(f)
    z = hlwq_ref.fwht_f32(v)
    s = (np.asarray(g, dtype=f) * f(2.0 ** -7)).astype(f)
    return ((z * s[..., None]).astype(f) * np.asarray(d1, dtype=f)).astype(f)


def quantize_c(w_bits: np.ndarray, seed: int = SEED):
    """Tier C TQ3 quantize of one bf16 matrix (rows, in): returns packed uint8
    (rows, n_groups, 48) and float32 norms (rows, n_groups)."""
    d1, d2 = sign_vectors(seed)
    x, _ = hlwq_ref.blocks_from_rows(w_bits, GROUP)
    codes, g, _ = quantize_groups_c(x, d1, d2)
    return hlwq_ref.pack_codes(codes, BITS), g


def dequantize_c(packed: np.ndarray, g: np.ndarray, n_in: int, seed: int = SEED) -> np.ndarray:
    """Tier C TQ3 dequantize: packed (rows, nb, 48), norms (rows, nb) -> bf16 bits (rows, in)."""
    d1, d2 = sign_vectors(seed)
    codes = hlwq_ref.unpack_codes(packed, BITS)
    w = dequantize_groups_c(codes, g, d1, d2)
    return hlwq_ref.f32_to_bf16_rne(w.reshape(w.shape[0], -1)[:, :n_in])
