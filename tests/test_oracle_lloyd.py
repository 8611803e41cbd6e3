"""Pins for the oracle's Lloyd-Max codebooks (CPU only).

Each check ties the oracle to something other than itself: the classical
optimum-quantizer table, a closed form, an independent numerical integral, or a
brute-force search.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import integrate

from oracle import hlwq_ref as ref
from oracle import lloyd_max as lm

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def test_two_level_closed_form():
    # Two levels: the centroid of the half line is E[X | X > 0] = sqrt(2 / pi).
    c, _ = lm.lloyd_max_gaussian(2)
    assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-12
    assert abs(lm.distortion(c) - (1 - 2 / math.pi)) < 1e-12


@pytest.mark.parametrize("K", [2, 4, 8])
def test_matches_classical_table(K):
    g = json.load(open(os.path.join(GOLD, "max1960_gaussian.json")))
    c, _ = lm.lloyd_max_gaussian(K)
    pos = c[K // 2:]
    want = np.array(g["levels"][str(K)])
    assert np.max(np.abs(pos - want)) < g["tolerance"]
    assert abs(lm.distortion(c) - g["mse"][str(K)]) < 1e-4


@pytest.mark.parametrize("K", [8, 32])
def test_fixed_point_by_quadrature(K):
    # Every centroid is the conditional mean of its cell, computed here by
    # adaptive quadrature rather than the closed form the iteration uses.
    c, _ = lm.lloyd_max_gaussian(K)
    b = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
    for k in range(K):
        lo, hi = b[k], b[k + 1]
        m1 = integrate.quad(lambda x: x * _phi(x), lo, hi, epsabs=1e-15, epsrel=1e-13)[0]
        m0 = integrate.quad(_phi, lo, hi, epsabs=1e-15, epsrel=1e-13)[0]
        assert abs(c[k] - m1 / m0) < 1e-9, (k, c[k], m1 / m0)


@pytest.mark.parametrize("K", [4, 8, 32])
def test_symmetric_and_sorted(K):
    c, _ = lm.lloyd_max_gaussian(K)
    assert np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])
    c32, b32 = lm.table(int(math.log2(K)))
    assert np.array_equal(c32, -c32[::-1])
    assert b32[K // 2 - 1] == 0.0


def _grid_mse(c, lo=-9.0, hi=9.0, n=2_000_001):
    x = np.linspace(lo, hi, n)
    w = np.exp(-0.5 * x * x) / math.sqrt(2 * math.pi) * (x[1] - x[0])
    q = c[np.argmin(np.abs(x[:, None] - c[None, :]), axis=1)]
    return float(np.sum((x - q) ** 2 * w))


@pytest.mark.parametrize("K", [8, 32])
def test_distortion_brute_force_and_local_optimum(K):
    c, _ = lm.lloyd_max_gaussian(K)
    d = _grid_mse(c)
    assert abs(d - lm.distortion(c)) < 1e-6
    # nudging any centroid must not lower the brute-force distortion
    for k in (0, K // 2, K - 1):
        for eps in (-1e-2, 1e-2):
            c2 = c.copy()
            c2[k] += eps
            assert _grid_mse(np.sort(c2)) > d


def test_q5_distortion_value():
    # sqrt(1 - D32) is the cosine expected between Gaussian data and its Q5
    # reconstruction; it must clear the 0.996 quoted on the Gemma-4 card.
    c, _ = lm.lloyd_max_gaussian(32)
    d = lm.distortion(c)
    assert 0.0024 < d < 0.0026
    assert math.sqrt(1 - d) > 0.996


@pytest.mark.parametrize("bits", [2, 3, 5])
def test_thresholds_are_round_down_of_midpoints(bits):
    c32, b32 = lm.table(bits)
    m = 0.5 * (c32[:-1].astype(np.float64) + c32[1:].astype(np.float64))
    assert np.all(b32.astype(np.float64) <= m)
    up = np.nextafter(b32, np.float32(np.inf)).astype(np.float64)
    assert np.all(up > m)


@pytest.mark.parametrize("bits", [3, 5])
def test_threshold_count_is_nearest_centroid(bits):
    # Brute force: "#thresholds below y" must equal the nearest fp32 centroid
    # (first index on a tie) for random y and for every fp32 value within a
    # few ulps of every midpoint and every centroid.
    c32, b32 = lm.table(bits)
    rng = np.random.default_rng(1)
    ys = [rng.standard_normal(20_000).astype(np.float32) * np.float32(1.5),
          np.float32([0.0, -0.0, 12.0, -12.0])]
    m = 0.5 * (c32[:-1].astype(np.float64) + c32[1:].astype(np.float64))
    for p in np.concatenate((m.astype(np.float32), c32)):
        v = np.float32(p)
        lo = v
        hi = v
        near = [v]
        for _ in range(4):
            lo = np.nextafter(lo, np.float32(-np.inf))
            hi = np.nextafter(hi, np.float32(np.inf))
            near += [lo, hi]
        ys.append(np.array(near, dtype=np.float32))
    y = np.concatenate(ys)
    # argmin |y - c_k| with exact rational distances (first index on a tie)
    cf = [Fraction(float(c)) for c in c32]
    want = []
    for v in y:
        fv = Fraction(float(v))
        d = [abs(fv - c) for c in cf]
        want.append(d.index(min(d)))
    want = np.array(want)
    assert np.array_equal(ref.codes_from_y(y, b32), want)
    assert np.array_equal(ref.nearest_code(y, c32), want)


@pytest.mark.parametrize("K", [4, 8, 32])
def test_fp32_table_is_unambiguous(K):
    # The fp64 fixed point sits far (> 1e-10) from every fp32 rounding
    # boundary, so any converged Lloyd implementation rounds to the same fp32
    # table; the residual iteration error is below 1e-12.
    c, _ = lm.lloyd_max_gaussian(K)
    c32 = c.astype(np.float32)
    up = np.nextafter(c32, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(c32, np.float32(-np.inf)).astype(np.float64)
    mid_up = 0.5 * (c32.astype(np.float64) + up)
    mid_dn = 0.5 * (c32.astype(np.float64) + dn)
    assert np.min(np.minimum(np.abs(c - mid_up), np.abs(c - mid_dn))) > 1e-10
