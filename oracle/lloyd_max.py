"""Lloyd-Max scalar codebooks for the unit Gaussian (oracle, fp64).

TEST INFRASTRUCTURE ONLY: see the package docstring of ``oracle``.

HLWQ snaps every rotated, normalised weight to the nearest of K centroids that
are MSE-optimal for N(0, 1): 32 centroids for Q5 ("Qwen3.6-35B-A3B — HLWQ Q5",
section "Method", step [4]; "Qwopus3.6-27B-v2 · HLWQ Q5", "Methodology notes",
weight bullet: centroids computed for a unit Gaussian) and 8 centroids for the
3-bit KV cache (same card, "Methodology notes", KV bullet).

Lloyd's iteration, written out for the Gaussian density phi and its CDF Phi:

* decision thresholds are the midpoints of neighbouring centroids,
  b_k = (c_k + c_{k+1}) / 2, with b_{-1} = -inf and b_{K-1} = +inf;
* every centroid moves to the conditional mean of its cell,
  c_k = (phi(b_{k-1}) - phi(b_k)) / (Phi(b_k) - Phi(b_{k-1})).

The Gaussian is log-concave, so the fixed point is unique and the start point
only changes the iteration count.  The result is symmetrised so c_k = -c_{K-1-k}
holds exactly.

The stored tables are fp32: the centroids are rounded to nearest, and a
decision threshold is the largest fp32 value not above the exact midpoint of two
neighbouring fp32 centroids.  With that choice, ``code = #{k : y > b_k}`` equals
the index of the nearest fp32 centroid, ties going to the lower index.
"""
from __future__ import annotations

import functools
import math

import numpy as np
from scipy.special import ndtr, ndtri


def _gauss_pdf(t: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return np.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)


def _cell_mass(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    """P(lo < X < hi) for X ~ N(0, 1), taking the tail that avoids cancellation."""
    upper = lo >= 0.0
    return np.where(upper, ndtr(-lo) - ndtr(-hi), ndtr(hi) - ndtr(lo))


def lloyd_max_gaussian(K: int, tol: float = 1e-15, max_iter: int = 200_000):
    """Return (centroids fp64 ascending, iterations) for K levels on N(0, 1)."""
    if K < 2:
        raise ValueError("K must be at least 2")
    c = ndtri((np.arange(K) + 0.5) / K)
    it = 0
    for it in range(1, max_iter + 1):
        b = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([-np.inf], b))
        hi = np.concatenate((b, [np.inf]))
        c_new = (_gauss_pdf(lo) - _gauss_pdf(hi)) / _cell_mass(lo, hi)
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol:
            break
    else:
        raise RuntimeError(f"Lloyd iteration for K={K} did not converge")
    c = 0.5 * (c - c[::-1])
    return c, it


def distortion(c: np.ndarray) -> float:
    """Mean squared error E[(X - Q(X))^2] of the nearest-centroid quantizer."""
    b = 0.5 * (c[:-1] + c[1:])
    lo = np.concatenate(([-np.inf], b))
    hi = np.concatenate((b, [np.inf]))
    p = _cell_mass(lo, hi)
    return float(1.0 - np.sum(p * c * c))


def centroids_f32(K: int) -> np.ndarray:
    """The fp32 centroid table c32[K], ascending."""
    c, _ = lloyd_max_gaussian(K)
    return c.astype(np.float32)


def thresholds_f32(c32: np.ndarray) -> np.ndarray:
    """Decision thresholds b32[K-1]: round-down of the exact fp32-centroid midpoints."""
    c64 = np.asarray(c32, dtype=np.float32).astype(np.float64)
    m = 0.5 * (c64[:-1] + c64[1:])  # exact in fp64
    b = m.astype(np.float32)
    above = b.astype(np.float64) > m
    b[above] = np.nextafter(b[above], np.float32(-np.inf))
    return b


@functools.lru_cache(maxsize=None)
def _table(bits: int):
    c32 = centroids_f32(1 << bits)
    return c32, thresholds_f32(c32)


def table(bits: int):
    """(c32, b32) for a 2**bits-level codebook (fresh copies of a cached table)."""
    c32, b32 = _table(bits)
    return c32.copy(), b32.copy()
