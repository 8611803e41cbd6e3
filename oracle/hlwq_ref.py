"""HLWQ quantize / dequantize, plain CPU reference (oracle).

TEST INFRASTRUCTURE ONLY: see the package docstring of ``oracle``.

The method ("Qwen3.6-35B-A3B — HLWQ Q5", section "Method", steps [1]-[5]):

[1] view W (out x in) as (out, n_blocks, 128), zero-padding the last block;
[2] L2-normalise every block and keep its norm (fp16, "Gemma-4-26B-A4B-it-HLWQ-Q5",
    "Technical Details");
[3] rotate: blocks @ H128 * sqrt(128), H128 the orthonormal Walsh-Hadamard
    matrix, deterministic ("Qwen3.5-9B — HLWQ INT4", naming notice);
[4] snap each value to the nearest of 32 Lloyd-Max centroids for N(0, 1);
[5] pack 8 five-bit codes into 5 bytes (0.625 byte/weight, "Qwopus3.6-27B-v2 ·
    HLWQ Q5", "Methodology notes").

Dequantisation is the inverse: unpack, look up centroids, rotate back, scale by
the stored norm, round to bf16 ("Qwopus3.6-27B-v2 · HLWQ Q5", "Pipeline":
dequantize per Linear to BF16).  The Q3 variant uses 8 centroids and packs
8 codes into 3 bytes.  The KV-cache path ("Qwopus3.6-27B-v2 · HLWQ Q5",
"Methodology notes", KV bullet) rotates every 256-wide head vector by H256, uses
8 centroids and 3-bit codes, and leaves the newest 128 tokens unquantised; the
2-bit variant uses 4 centroids ("Qwen3.6-35B-A3B — HLWQ Q5", "Speed
Benchmarks": Q3 and Q2 KV).  During generation the cache is streamed: each new
token enters the unquantised window and the token it pushes out is encoded
(``kv_stream_c``).

Two tiers:

* Tier D ("definition", fp64): the steps as printed, in the printed order, with
  a dense Sylvester Hadamard matrix and fp64 arithmetic; code = nearest fp32
  centroid.  It is the mathematical authority for the quality pins and the
  "distance to a decision boundary" of every value.
* Tier C ("canonical", fp32): one fixed IEEE-fp32 operation sequence for the
  same map.  Every operation is a single correctly rounded numpy float32 op, so
  the rounding of every intermediate is defined.  Readings taken here:
    - the norm is an adjacent-pair tree over the squares: level 0 forms each
      pair x_2i^2 + x_2i+1^2 with one rounding of x_2i^2 + RN(x_2i+1^2) (a
      fused multiply-add), level l adds the partial sums 2i and 2i+1; then a
      correctly rounded sqrt; fp16 by round-to-nearest-even from that fp32
      value;
    - normalise-then-rotate is carried out as rotate-then-scale (the map is
      linear, one rounding fewer): the unnormalised +-1 butterflies
      (a, b) -> (a + b, a - b) at strides 1, 2, 4, ..., then y = z * (1/n) with
      1/n correctly rounded, and 1/n := 0 when n is below the smallest normal
      fp32 value (zero blocks);
    - the code is the number of fp32 thresholds strictly below y;
    - dequant multiplies the same butterflies of the centroids by n16 / L
      (2^-7 for 128-blocks, 2^-8 for 256-wide KV vectors; exact in fp32) and
      rounds to bf16, nearest-even.
  Tier C is what a kernel must reproduce bit for bit.

Bit order of a packed group: code i of a group of 8 occupies bits
[bits*i, bits*i + bits) of a little-endian integer, i.e. the first code sits in
the low bits of the first byte.
"""
from __future__ import annotations

import collections
import math

import numpy as np

from . import lloyd_max

BLOCK = 128
KV_DIM = 256
FLT_MIN = np.float32(np.finfo(np.float32).tiny)


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even; NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def blocks_from_rows(w_bits: np.ndarray, block: int = BLOCK) -> tuple[np.ndarray, int]:
    """Step [1]: (rows, in) bf16 bits -> (rows, n_blocks, block) float32, zero padded."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    rows, n_in = w_bits.shape
    nb = -(-n_in // block)
    x = np.zeros((rows, nb * block), dtype=np.float32)
    x[:, :n_in] = bf16_to_f32(w_bits)
    return x.reshape(rows, nb, block), nb


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Step [5]: (..., n) codes, n % 8 == 0 -> (..., n // 8 * bits) bytes."""
    codes = np.asarray(codes)
    assert codes.shape[-1] % 8 == 0
    if codes.size and (codes.min() < 0 or codes.max() >= (1 << bits)):
        raise ValueError("code out of range")
    g = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // 8, 8)).astype(np.uint64)
    v = np.zeros(g.shape[:-1], dtype=np.uint64)
    for i in range(8):
        v |= g[..., i] << np.uint64(bits * i)
    out = np.empty(g.shape[:-1] + (bits,), dtype=np.uint8)
    for m in range(bits):
        out[..., m] = ((v >> np.uint64(8 * m)) & np.uint64(0xFF)).astype(np.uint8)
    return out.reshape(codes.shape[:-1] + (codes.shape[-1] // 8 * bits,))


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_codes: (..., m * bits) bytes -> (..., m * 8) codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    assert packed.shape[-1] % bits == 0
    g = packed.reshape(packed.shape[:-1] + (packed.shape[-1] // bits, bits)).astype(np.uint64)
    v = np.zeros(g.shape[:-1], dtype=np.uint64)
    for m in range(bits):
        v |= g[..., m] << np.uint64(8 * m)
    mask = np.uint64((1 << bits) - 1)
    codes = np.empty(g.shape[:-1] + (8,), dtype=np.int64)
    for i in range(8):
        codes[..., i] = ((v >> np.uint64(bits * i)) & mask).astype(np.int64)
    return codes.reshape(packed.shape[:-1] + (packed.shape[-1] // bits * 8,))


# --------------------------------------------------------------------------
# Tier D: definition in fp64
# --------------------------------------------------------------------------

def sylvester_hadamard(n: int) -> np.ndarray:
    """The +-1 Walsh-Hadamard matrix of order n (power of 2), natural (Sylvester) order."""
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != n:
        raise ValueError("order must be a power of two")
    return h


def orthonormal_hadamard(n: int) -> np.ndarray:
    return sylvester_hadamard(n) / math.sqrt(n)


def nearest_code(y: np.ndarray, c32: np.ndarray) -> np.ndarray:
    """Index of the nearest fp32 centroid, the lower one on a tie.

    On a sorted codebook the cell of c_k is bounded by the midpoints of its
    neighbours, so the nearest index is the number of midpoints strictly below
    y.  The midpoints of fp32 values are exact in fp64, and so is the compare.
    """
    c = np.asarray(c32, dtype=np.float32).astype(np.float64)
    m = 0.5 * (c[:-1] + c[1:])
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros(y.shape, dtype=np.int64)
    for mk in m:
        out += (y > mk)
    return out


def boundary_distance(y: np.ndarray, c32: np.ndarray) -> np.ndarray:
    """Distance of y to the nearest exact midpoint between neighbouring centroids."""
    c = c32.astype(np.float64)
    m = 0.5 * (c[:-1] + c[1:])
    return np.min(np.abs(np.asarray(y, dtype=np.float64)[..., None] - m), axis=-1)


def quantize_def(x_blocks: np.ndarray, bits: int, c32: np.ndarray | None = None):
    """Tier D on (..., L) float blocks.

    Returns (codes, norm fp64, y fp64) with y = (x / n) @ H_orth * sqrt(L).
    """
    x = np.asarray(x_blocks, dtype=np.float64)
    L = x.shape[-1]
    if c32 is None:
        c32, _ = lloyd_max.table(bits)
    n = np.sqrt(np.sum(x * x, axis=-1))
    safe = np.where(n > 0.0, n, 1.0)
    u = np.where((n > 0.0)[..., None], x / safe[..., None], 0.0)
    y = (u @ orthonormal_hadamard(L)) * math.sqrt(L)
    return nearest_code(y, c32), n, y


def dequantize_def(codes: np.ndarray, norms: np.ndarray, bits: int,
                   c32: np.ndarray | None = None) -> np.ndarray:
    """Tier D inverse: n * (c[codes] @ H_orth^T) / sqrt(L), fp64, unrounded."""
    if c32 is None:
        c32, _ = lloyd_max.table(bits)
    v = c32.astype(np.float64)[np.asarray(codes)]
    L = v.shape[-1]
    z = v @ orthonormal_hadamard(L).T
    return np.asarray(norms, dtype=np.float64)[..., None] * z / math.sqrt(L)


# --------------------------------------------------------------------------
# Tier C: canonical fp32 operation order
# --------------------------------------------------------------------------

def pair_sumsq_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """RN32(a*a + RN32(b*b)): one pair of squares as a fused multiply-add forms it.

    a*a is exact in fp64 for bf16 a (at most 16 significant bits) and RN32(b*b)
    is an fp32 value, so their fp64 sum is either exact or lies so close to one
    of the two terms (the other below 2^-29 of it, far from any fp32 rounding
    boundary) that rounding it to fp32 gives the correctly rounded sum.
    """
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    a2 = a.astype(np.float64) * a.astype(np.float64)
    b2 = (b * b).astype(np.float64)
    return (a2 + b2).astype(np.float32)


def norm_tree_f32(x: np.ndarray) -> np.ndarray:
    """Sum of squares by the adjacent-pair tree, then a correctly rounded sqrt.

    Level 0 forms every pair (x_2i, x_2i+1) as RN(x_2i^2 + RN(x_2i+1^2)) (one
    fused multiply-add); every further level adds neighbouring partial sums.
    """
    x = np.asarray(x, dtype=np.float32)
    s = pair_sumsq_f32(x[..., 0::2], x[..., 1::2])
    while s.shape[-1] > 1:
        s = s[..., 0::2] + s[..., 1::2]
    return np.sqrt(s[..., 0])


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Unnormalised +-1 Walsh-Hadamard transform along the last axis.

    Stages at strides h = 1, 2, 4, ...: every pair (i, i + h) inside a group of
    2h entries becomes (a + b, a - b); each add is one fp32 rounding.
    """
    v = np.array(x, dtype=np.float32, copy=True)
    lead = v.shape[:-1]
    L = v.shape[-1]
    h = 1
    while h < L:
        g = v.reshape(lead + (L // (2 * h), 2, h))
        a = g[..., 0, :]
        b = g[..., 1, :]
        v = np.stack((a + b, a - b), axis=-2).reshape(lead + (L,))
        h *= 2
    return v


def codes_from_y(y: np.ndarray, b32: np.ndarray) -> np.ndarray:
    """code = number of fp32 thresholds strictly below y (fp32 compares)."""
    y = np.asarray(y, dtype=np.float32)
    out = np.zeros(y.shape, dtype=np.int64)
    for b in np.asarray(b32, dtype=np.float32):
        out += (y > b)
    return out


def quantize_vectors_c(x: np.ndarray, bits: int, tables=None):
    """Tier C on (..., L) float32 vectors: returns (codes, n32, n16, y)."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle inputs must be finite")
    c32, b32 = tables if tables is not None else lloyd_max.table(bits)
    n = norm_tree_f32(x)
    n16 = n.astype(np.float16)
    with np.errstate(divide="ignore"):
        r = np.where(n >= FLT_MIN, np.float32(1.0) / n, np.float32(0.0)).astype(np.float32)
    z = fwht_f32(x)
    y = z * r[..., None]
    return codes_from_y(y, b32), n, n16, y


def dequantize_vectors_c(codes: np.ndarray, n16: np.ndarray, bits: int, tables=None) -> np.ndarray:
    """Tier C inverse on (..., L) codes: returns float32 before the bf16 rounding."""
    c32, _ = tables if tables is not None else lloyd_max.table(bits)
    v = c32[np.asarray(codes)]
    L = v.shape[-1]
    z = fwht_f32(v)
    # H H = L I for the +-1 matrix, so the inverse rotation divides by L; n16 / L
    # is exact in fp32 for every fp16 value.
    scale = np.asarray(n16, dtype=np.float16).astype(np.float32) * np.float32(1.0 / L)
    return z * scale[..., None]


def quantize_c(w_bits: np.ndarray, bits: int, tables=None):
    """Tier C quantize of one bf16 matrix (rows, in).

    Returns packed uint8 (rows, n_blocks, 16 * bits) and fp16 norms (rows, n_blocks).
    """
    if bits not in (3, 5):
        raise ValueError("bits must be 5 or 3")
    x, nb = blocks_from_rows(w_bits)
    codes, _, n16, _ = quantize_vectors_c(x, bits, tables)
    return pack_codes(codes, bits), n16


def dequantize_c(packed: np.ndarray, n16: np.ndarray, n_in: int, bits: int, tables=None) -> np.ndarray:
    """Tier C dequantize: packed (rows, nb, 16*bits), norms (rows, nb) -> bf16 bits (rows, in)."""
    codes = unpack_codes(packed, bits)
    w = dequantize_vectors_c(codes, n16, bits, tables)
    rows = w.shape[0]
    w = w.reshape(rows, -1)[:, :n_in]
    return f32_to_bf16_rne(w)


def quantize_codes8_c(w_bits: np.ndarray, bits: int, tables=None):
    """Tier C quantize with one code per byte ("Gemma-4-26B-A4B-it-HLWQ-Q5",
    "Technical Details": int8 codes and fp16 norms): codes uint8
    (rows, n_blocks, 128), fp16 norms (rows, n_blocks)."""
    x, nb = blocks_from_rows(w_bits)
    codes, _, n16, _ = quantize_vectors_c(x, bits, tables)
    return codes.astype(np.uint8), n16


def dequantize_codes8_c(codes: np.ndarray, n16: np.ndarray, n_in: int, bits: int, tables=None) -> np.ndarray:
    """Inverse of quantize_codes8_c: -> bf16 bits (rows, in)."""
    w = dequantize_vectors_c(np.asarray(codes, dtype=np.int64), n16, bits, tables)
    return f32_to_bf16_rne(w.reshape(w.shape[0], -1)[:, :n_in])


def kv_quantize_c(kv_bits: np.ndarray, n_residual: int = 128, bits: int = 3, tables=None):
    """Tier C KV-cache quantize of [B, H, T, 256] bf16.

    Tokens t < T - n_residual are quantised; the newest n_residual tokens stay
    bf16 and are not part of the output.  Returns packed [B, H, Tq, 32 * bits]
    and fp16 norms [B, H, Tq].
    """
    kv_bits = np.asarray(kv_bits, dtype=np.uint16)
    B, H, T, D = kv_bits.shape
    if D != KV_DIM:
        raise ValueError("head_dim must be 256")
    tq = max(T - n_residual, 0)
    x = bf16_to_f32(kv_bits[:, :, :tq, :])
    codes, _, n16, _ = quantize_vectors_c(x, bits, tables)
    return pack_codes(codes, bits), n16


def kv_dequantize_c(packed: np.ndarray, n16: np.ndarray, bits: int = 3, tables=None) -> np.ndarray:
    """Inverse of kv_quantize_c: -> bf16 bits [B, H, Tq, 256]."""
    codes = unpack_codes(packed, bits)
    return f32_to_bf16_rne(dequantize_vectors_c(codes, n16, bits, tables))


def kv_stream_c(chunks, n_residual: int = 128, bits: int = 3, tables=None):
    """Tier C streaming KV cache, token by token.

    Tokens arrive in chunks (bf16 bits [B, H, n, 256] each).  Every arriving
    token enters the window of the newest n_residual tokens, which are kept
    unquantised ("Qwopus3.6-27B-v2 · HLWQ Q5", "Methodology notes": a residual
    buffer holds recent tokens unquantised); when the window overflows, its
    oldest token leaves and is encoded.  Returns (packed [B, H, Tq, 32 * bits],
    norms [B, H, Tq], window [B, H, min(T, n_residual), 256] oldest first).
    """
    window = collections.deque()
    packed, norms = [], []
    shape = None
    for chunk in chunks:
        chunk = np.asarray(chunk, dtype=np.uint16)
        shape = chunk.shape[:2]
        for j in range(chunk.shape[2]):
            window.append(chunk[:, :, j, :])
            if len(window) > n_residual:
                old = bf16_to_f32(window.popleft())
                codes, _, n16, _ = quantize_vectors_c(old, bits, tables)
                packed.append(pack_codes(codes, bits))
                norms.append(n16)
    B, H = shape
    out_p = np.stack(packed, axis=2) if packed else np.zeros((B, H, 0, 32 * bits), np.uint8)
    out_n = np.stack(norms, axis=2) if norms else np.zeros((B, H, 0), np.float16)
    out_w = np.stack(list(window), axis=2) if window else np.zeros((B, H, 0, KV_DIM), np.uint16)
    return out_p, out_n, out_w


# --------------------------------------------------------------------------
# dequantize -> INT4 group-128 (the step after HLWQ in the pages' pipeline)
# --------------------------------------------------------------------------

INT4_LEVELS = 15  # codes 0..15


def int4_quantize_c(w_bits: np.ndarray, group: int = BLOCK):
    """Asymmetric 4-bit quantisation with one scale and zero point per group
    of `group` consecutive columns of a row ("Qwopus3.6-27B-v2 · HLWQ Q5",
    "Pipeline": dequantize per Linear to BF16, then a 4-bit weight-only
    quantisation with group size 128 of the 128-aligned Linears; "Qwen3.5-9B —
    HLWQ INT4", "Why HLWQ INT4 is Better": dequant -> INT4).

    Readings (plain asymmetric min-max quantiser, fp32):
      lo = min(0, min w), hi = max(0, max w) over the group (zero exactly
      representable); scale = RN((hi - lo) / 15), 1 if that is 0;
      inv = RN(1 / scale); zero point zp = clamp(rint(RN(-lo * inv)), 0, 15);
      q = clamp(rint(RN(w * inv)) + zp, 0, 15), rint = round half to even.
    Dequantised value: (q - zp) * scale.

    w_bits: bf16 bits [rows, in], in % group == 0.  Returns q uint8 [rows, in]
    (0..15), scales float32 [rows, in // group], zeros uint8 [rows, in // group].
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    rows, n_in = w_bits.shape
    if n_in % group:
        raise ValueError("in must be a multiple of the group size")
    w = bf16_to_f32(w_bits).reshape(rows, n_in // group, group)
    f = np.float32
    lo = np.minimum(w.min(axis=-1), f(0))
    hi = np.maximum(w.max(axis=-1), f(0))
    scale = ((hi - lo) / f(INT4_LEVELS)).astype(f)
    scale = np.where(scale == 0, f(1), scale).astype(f)
    inv = (f(1) / scale).astype(f)
    zp = np.clip(np.rint((-lo * inv).astype(f)), 0, INT4_LEVELS).astype(np.int64)
    t = (w * inv[..., None]).astype(f)
    q = np.clip(np.rint(t).astype(np.int64) + zp[..., None], 0, INT4_LEVELS)
    return q.reshape(rows, n_in).astype(np.uint8), scale, zp.astype(np.uint8)


def int4_pack(q: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, element 2i in the low nibble: [..., n] -> [..., n / 2]."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def int4_dequantize(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group: int = BLOCK) -> np.ndarray:
    """(q - zp) * scale, fp32 [rows, in]."""
    rows, n_in = q.shape
    qq = q.reshape(rows, n_in // group, group).astype(np.float32)
    z = zeros.astype(np.float32)[..., None]
    return ((qq - z) * scales[..., None]).astype(np.float32).reshape(rows, n_in)


def dequantize_to_int4_c(packed: np.ndarray, n16: np.ndarray, n_in: int, bits: int, tables=None):
    """HLWQ dequantize (tier C, bf16) followed by int4_quantize_c: returns packed
    nibbles uint8 [rows, in / 2], scales float32 [rows, nb], zeros uint8 [rows, nb]."""
    w = dequantize_c(packed, n16, n_in, bits, tables)
    q, scales, zeros = int4_quantize_c(w)
    return int4_pack(q), scales, zeros
