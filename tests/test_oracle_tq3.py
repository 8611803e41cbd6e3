"""Pins for the TQ3 (scalar HIGGS) oracle ("Qwen3.6-35B-A3B-TQ3-native",
section "What TQ3 actually does"; CPU only)."""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import hlwq_ref as ref
from oracle import lloyd_max as lm
from oracle import tq3_ref as tq

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gauss_groups(n, seed, sigma=0.02):
    return synth.bf16_bits_to_f32(synth.random_bf16((n, 128), seed=seed, key=31, sigma=sigma))


def test_splitmix64_known_answers():
    with open(os.path.join(GOLD, "splitmix64.json")) as f:
        gold = json.load(f)
    for seed, outs in gold["outputs"].items():
        want = [int(v, 0) for v in outs]
        assert tq.splitmix64(int(seed), len(want)) == want


def test_sign_vectors_are_balanced_signs():
    d1, d2 = tq.sign_vectors(42)
    assert d1.shape == d2.shape == (128,)
    assert set(np.unique(np.concatenate([d1, d2]))) <= {-1, 1}
    assert not np.array_equal(d1, d2)
    # bit 63 of SplitMix64 is a fair coin: over 256 seeds x 256 draws the count
    # of -1 stays within 5 sigma of half
    neg = sum(int(np.sum(np.concatenate(tq.sign_vectors(s)) < 0)) for s in range(256))
    n = 256 * 256
    assert abs(neg - n / 2) < 5 * math.sqrt(n) / 2
    # a different seed gives different vectors
    assert not np.array_equal(tq.sign_vectors(43)[0], d1)


def test_rotation_is_orthogonal_and_places_the_signs():
    d1, d2 = tq.sign_vectors(42)
    R = tq.rotation_matrix(d1, d2)
    assert np.allclose(R @ R.T, np.eye(128), atol=1e-13)
    h = ref.sylvester_hadamard(128)
    # D1 acts on the input: flipping input coordinate i flips the image of e_i;
    # D2 acts on the output: it flips coordinate j of every image
    ones = np.ones(128, dtype=np.int8)
    for i in (0, 5, 77, 127):
        e = np.zeros(128)
        e[i] = 1.0
        assert np.array_equal(tq.rotation_matrix(d1, ones) @ e * math.sqrt(128), d1[i] * h[:, i])
        assert np.array_equal(tq.rotation_matrix(ones, d2) @ e * math.sqrt(128), d2 * h[:, i])


def test_tier_c_rotation_matches_the_matrix():
    d1, d2 = tq.sign_vectors(42)
    x = _gauss_groups(64, 1)
    codes, g, y = tq.quantize_groups_c(x, d1, d2)
    _, gd, yd, n = tq.quantize_def(x, d1, d2)
    assert np.allclose(y, yd, rtol=0, atol=2e-5)
    d = ref.boundary_distance(yd, lm.table(3)[0])
    cd = ref.nearest_code(yd, lm.table(3)[0])
    far = d > 1e-4
    assert far.mean() > 0.99
    assert np.array_equal(codes[far], cd[far])
    rows_exact = np.all(codes == cd, axis=-1)
    assert np.allclose(g[rows_exact], gd[rows_exact], rtol=2e-6)


def test_without_signs_the_codes_are_hlwq_q3():
    x = _gauss_groups(256, 2)
    ones = np.ones(128, dtype=np.int8)
    codes, g, _ = tq.quantize_groups_c(x, ones, ones)
    hcodes, n, _, _ = ref.quantize_vectors_c(x, 3)
    assert np.array_equal(codes, hcodes)


def test_input_signs_act_as_a_flipped_input():
    d1, _ = tq.sign_vectors(42)
    ones = np.ones(128, dtype=np.int8)
    x = _gauss_groups(256, 3)
    codes, _, _ = tq.quantize_groups_c(x, d1, ones)
    hcodes, _, _, _ = ref.quantize_vectors_c(x * d1.astype(np.float32), 3)
    assert np.array_equal(codes, hcodes)


def test_output_signs_mirror_the_codes():
    # code(-y) = 7 - code(y) on the symmetric threshold set, except where y is
    # itself a threshold (then 6 - code(y))
    _, d2 = tq.sign_vectors(42)
    ones = np.ones(128, dtype=np.int8)
    x = _gauss_groups(256, 4)
    codes, _, _ = tq.quantize_groups_c(x, ones, d2)
    hcodes, _, _, y = ref.quantize_vectors_c(x, 3)
    b32 = lm.table(3)[1]
    on_thr = np.isin(y, b32)
    want = np.where(d2 < 0, 7 - hcodes - on_thr, hcodes)
    assert np.array_equal(codes, want)


def test_shape_gain_restores_the_norm():
    d1, d2 = tq.sign_vectors(42)
    x = synth.bf16_bits_to_f32(synth.random_bf16((128, 128), seed=5, key=1, dist="student_t5")).astype(np.float64)
    codes, g, _, n = tq.quantize_def(x, d1, d2)
    xr = tq.dequantize_def(codes, g, d1, d2)
    assert np.allclose(np.linalg.norm(xr, axis=-1), n, rtol=1e-12)
    # and the shape is the normalised reconstruction
    c32 = lm.table(3)[0].astype(np.float64)
    unit = (c32[codes] @ tq.rotation_matrix(d1, d2))
    unit /= np.linalg.norm(unit, axis=-1, keepdims=True)
    assert np.allclose(xr, n[:, None] * unit, rtol=0, atol=1e-12 * n.max())


def test_power_of_two_scaling_is_exact():
    d1, d2 = tq.sign_vectors(42)
    x = _gauss_groups(128, 6)
    codes, g, _ = tq.quantize_groups_c(x, d1, d2)
    for k in (-20, 7, 40):
        s = np.float32(2.0 ** k)
        c2, g2, _ = tq.quantize_groups_c(x * s, d1, d2)
        assert np.array_equal(c2, codes)
        assert np.array_equal(g2, g * s)


def test_zero_group():
    d1, d2 = tq.sign_vectors(42)
    x = np.zeros((2, 128), dtype=np.float32)
    codes, g, y = tq.quantize_groups_c(x, d1, d2)
    assert np.all(codes == 3)  # thresholds 0, 1, 2 lie below 0; threshold 3 is 0
    assert np.all(g == 0)
    out = tq.dequantize_groups_c(codes, g, d1, d2)
    assert np.all(out == 0)


def test_codes_brute_force():
    d1, d2 = tq.sign_vectors(7)
    x = _gauss_groups(16, 8)
    codes, _, y = tq.quantize_groups_c(x, d1, d2)
    c = lm.table(3)[0].astype(np.float64)
    dist = np.abs(y.astype(np.float64)[..., None] - c)
    assert np.array_equal(codes, np.argmin(dist, axis=-1))


def test_tier_c_dequant_within_bf16_of_definition():
    d1, d2 = tq.sign_vectors(42)
    x = _gauss_groups(64, 9)
    codes, g, _ = tq.quantize_groups_c(x, d1, d2)
    want = tq.dequantize_def(codes, g.astype(np.float64), d1, d2)
    got = tq.dequantize_groups_c(codes, g, d1, d2)
    # fp32 butterflies over 7 stages: error below ~8 ulp of the row's scale g
    tol = 2e-6 * g.astype(np.float64)[:, None]
    assert np.all(np.abs(got - want) <= tol)
    b = ref.bf16_to_f32(ref.f32_to_bf16_rne(got))
    assert np.all(np.abs(b - want) <= np.abs(want) * 2.0 ** -8 + tol)


def test_quality_matches_max_distortion():
    # for N(0, 1) coordinates the 8-level Lloyd-Max distortion per coordinate is
    # Max's 0.03454; the shape-gain rescale adds only a second-order term
    with open(os.path.join(GOLD, "max1960_gaussian.json")) as f:
        mse8 = json.load(f)["mse"]["8"]
    d1, d2 = tq.sign_vectors(42)
    x = _gauss_groups(4096, 10).astype(np.float64)
    codes, g, _, n = tq.quantize_def(x, d1, d2)
    xr = tq.dequantize_def(codes, g, d1, d2)
    rel = np.sum((xr - x) ** 2) / np.sum(x * x)
    assert abs(rel - mse8) < 0.1 * mse8


def test_shape_gain_error_is_close_to_raw_norm_error():
    # storing the raw L2 norm instead of the shape-gain: on Gaussian groups the
    # two reconstruction errors agree to within a few percent (the shape-gain
    # one slightly lower); the page's factor of two does not appear here
    d1, d2 = tq.sign_vectors(42)
    x = _gauss_groups(4096, 13).astype(np.float64)
    codes, g, _, n = tq.quantize_def(x, d1, d2)
    err = lambda a: np.sum((a - x) ** 2) / np.sum(x * x)
    e_gain, e_raw = err(tq.dequantize_def(codes, g, d1, d2)), err(tq.dequantize_def(codes, n, d1, d2))
    assert e_gain < e_raw < 1.05 * e_gain


def test_matrix_tail_group_is_zero_padded():
    w = synth.random_bf16((3, 200), seed=11, key=2)
    packed, g = tq.quantize_c(w, 42)
    assert packed.shape == (3, 2, 48) and g.shape == (3, 2) and g.dtype == np.float32
    x = np.zeros((3, 256), dtype=np.float32)
    x[:, :200] = ref.bf16_to_f32(w)
    d1, d2 = tq.sign_vectors(42)
    codes, g2, _ = tq.quantize_groups_c(x.reshape(3, 2, 128), d1, d2)
    assert np.array_equal(ref.unpack_codes(packed, 3), codes)
    assert np.array_equal(g, g2)
    back = tq.dequantize_c(packed, g, 200, 42)
    assert back.shape == (3, 200)
    err = ref.bf16_to_f32(back) - ref.bf16_to_f32(w)
    assert np.sum(err.astype(np.float64) ** 2) < 0.06 * np.sum(ref.bf16_to_f32(w).astype(np.float64) ** 2)


def test_reconstruction_sum_is_exactly_rounded():
    # the fp64 sum of the squared centroids equals the exactly rounded sum
    # (math.fsum), on codes drawn uniformly and on the extremes
    c32 = lm.table(3)[0]
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 8, (500, 128))
    codes[0] = 0
    codes[1] = 3
    codes[2] = np.arange(128) % 8
    got = tq.recon_sumsq_f32(codes, c32)
    e = (c32 * c32).astype(np.float32)
    for row, g in zip(codes, got):
        assert g == np.float32(math.fsum(float(e[k]) for k in row))


def test_kappa_is_the_rounded_inverse_sqrt():
    # RN(1 / sqrt(128)) = RN(sqrt(2)) / 16 (a power-of-two scaling is exact)
    assert np.float32(1.0 / math.sqrt(128)) == np.float32(math.sqrt(2.0)) / np.float32(16)
