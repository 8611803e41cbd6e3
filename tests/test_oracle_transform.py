"""Pins for the oracle's rotation, norm and packing steps (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import hlwq_ref as ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _popcount(a):
    return bin(int(a)).count("1")


@pytest.mark.parametrize("n", [2, 8, 128, 256])
def test_sylvester_closed_form_and_orthogonality(n):
    h = ref.sylvester_hadamard(n)
    want = np.array([[(-1) ** _popcount(i & j) for j in range(n)] for i in range(n)], dtype=np.float64)
    assert np.array_equal(h, want)
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h.T, n * np.eye(n))
    ho = ref.orthonormal_hadamard(n)
    assert np.allclose(ho @ ho.T, np.eye(n), atol=1e-14)


@pytest.mark.parametrize("n", [128, 256])
def test_fwht_equals_dense_matrix_on_integers(n):
    # Small integers keep every fp32 partial sum exact, so the butterflies must
    # reproduce the dense Sylvester product exactly.
    rng = np.random.default_rng(0)
    x = rng.integers(-1000, 1000, size=(64, n)).astype(np.float32)
    want = (x.astype(np.float64) @ ref.sylvester_hadamard(n)).astype(np.float32)
    assert np.array_equal(ref.fwht_f32(x), want)
    assert np.array_equal(ref.fwht_f32(ref.fwht_f32(x)), np.float32(n) * x)


def _fwht_scalar_loop(v):
    """In-place textbook FWHT on a Python list of np.float32 (ascending strides)."""
    v = [np.float32(t) for t in v]
    n = len(v)
    h = 1
    while h < n:
        for start in range(0, n, 2 * h):
            for i in range(start, start + h):
                a, b = v[i], v[i + h]
                v[i], v[i + h] = np.float32(a + b), np.float32(a - b)
        h *= 2
    return np.array(v, dtype=np.float32)


def test_fwht_rounding_order_brute_force():
    # Random floats make every stage round; the vectorised stages must match the
    # scalar in-place loop bit for bit.
    rng = np.random.default_rng(2)
    for n in (4, 16, 128):
        for _ in range(20):
            x = (rng.standard_normal(n) * np.exp(rng.uniform(-8, 8, n))).astype(np.float32)
            assert np.array_equal(ref.fwht_f32(x[None])[0].view(np.uint32),
                                  _fwht_scalar_loop(x).view(np.uint32))


def test_norm_tree_exact_cases():
    x = np.zeros((3, 128), dtype=np.float32)
    x[0, 5], x[0, 77] = 3.0, 4.0              # 3-4-5
    x[1, :] = 1.0                              # sqrt(128), correctly rounded
    n = ref.norm_tree_f32(x)
    assert n[0] == np.float32(5.0)
    assert n[1] == np.sqrt(np.float32(128.0))
    assert n[2] == 0.0


def test_norm_tree_pairing_order():
    # squares 1, 2^-24, 2^-24, 0, ...: pairing (0,1) gives 1 + 2^-24 -> 1 (tie to
    # even), pairing (2,3) gives 2^-24; then 1 + 2^-24 -> 1 again.  With x[3]
    # also 2^-12 the pair (2,3) is 2^-23 and survives: sqrt(1 + 2^-23).
    x = np.zeros((2, 128), dtype=np.float32)
    x[:, 0] = 1.0
    x[:, 1] = 2.0 ** -12
    x[:, 2] = 2.0 ** -12
    x[1, 3] = 2.0 ** -12
    n = ref.norm_tree_f32(x)
    assert n[0] == np.float32(1.0)
    assert n[1] == np.sqrt(np.float32(1.0) + np.float32(2.0 ** -23))


def test_norm_tree_close_to_library_norm():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((1000, 128)) * 0.02).astype(np.float32)
    got = ref.norm_tree_f32(x).astype(np.float64)
    want = np.linalg.norm(x.astype(np.float64), axis=1)
    assert np.max(np.abs(got / want - 1)) < 4e-7


@pytest.mark.parametrize("L", [128, 256])
def test_rotation_preserves_norm(L):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((500, L)) * 0.02).astype(np.float32)
    _, n, _, y = ref.quantize_vectors_c(x, 5 if L == 128 else 3)
    ss = np.sum(y.astype(np.float64) ** 2, axis=-1)
    assert np.max(np.abs(ss / L - 1)) < 1e-5
    _, nd, yd = ref.quantize_def(x, 5)
    assert np.max(np.abs(np.sum(yd ** 2, axis=-1) / L - 1)) < 1e-13
    assert np.allclose(nd, np.linalg.norm(x.astype(np.float64), axis=-1), rtol=1e-15)


def test_pack_golden_bytes():
    g = json.load(open(os.path.join(GOLD, "pack_examples.json")))
    for case in g["cases"]:
        codes = np.array(case["codes"])[None]
        got = ref.pack_codes(codes, case["bits"])[0]
        assert got.tolist() == case["bytes"], case
        assert ref.unpack_codes(got[None], case["bits"])[0].tolist() == case["codes"]


def test_pack_roundtrip_3bit_exhaustive():
    # all 8^8 groups, in chunks
    base = np.arange(8 ** 8, dtype=np.int64)
    for lo in range(0, 8 ** 8, 1 << 21):
        v = base[lo:lo + (1 << 21)]
        codes = np.stack([(v >> (3 * i)) & 7 for i in range(8)], axis=-1)
        packed = ref.pack_codes(codes, 3)
        assert packed.shape == (v.size, 3)
        # the 24-bit little-endian integer of the 3 bytes is the group index
        val = packed[:, 0].astype(np.int64) | (packed[:, 1].astype(np.int64) << 8) | (packed[:, 2].astype(np.int64) << 16)
        assert np.array_equal(val, v)
        assert np.array_equal(ref.unpack_codes(packed, 3), codes)


def test_pack_roundtrip_5bit():
    # every (position, value) pair in isolation, then random groups
    for pos in range(8):
        for val in range(32):
            codes = np.zeros((1, 8), dtype=np.int64)
            codes[0, pos] = val
            p = ref.pack_codes(codes, 5)[0]
            as_int = sum(int(b) << (8 * m) for m, b in enumerate(p))
            assert as_int == val << (5 * pos)
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 32, size=(1_000_000, 128))
    assert np.array_equal(ref.unpack_codes(ref.pack_codes(codes, 5), 5), codes)


def test_storage_density():
    # 0.625 byte per weight for Q5 ("Qwopus3.6-27B-v2 · HLWQ Q5", Methodology
    # notes); with one fp16 norm per 128 weights, 33.62e9 quantised weights
    # take 21.55 GB ("Qwen3.6-35B-A3B — HLWQ Q5", Compression Pipeline table).
    codes = np.zeros((1, 128), dtype=np.int64)
    assert ref.pack_codes(codes, 5).shape[-1] == 80
    assert ref.pack_codes(codes, 3).shape[-1] == 48
    assert ref.pack_codes(np.zeros((1, 256), dtype=np.int64), 3).shape[-1] == 96
    assert 80 / 128 == 0.625
    total = 33.62e9 * (80 + 2) / 128
    assert abs(total / 21.55e9 - 1) < 1e-3


def _rn32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even) by search."""
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - q), int(np.float32(v).view(np.uint32)) & 1))


def test_first_tree_level_is_a_fused_pair():
    # RN(a^2 + RN(b^2)) with exact rationals, on normal, tiny (squares in the
    # fp32 denormal range) and mixed-magnitude bf16 pairs; a two-rounding
    # RN(RN(a^2) + RN(b^2)) differs from it on some of the tiny ones.
    rng = np.random.default_rng(6)
    mags = np.exp(rng.uniform(-105, 40, (4000, 2)))
    v = synth_bf16((rng.standard_normal((4000, 2)) * mags).astype(np.float32))
    a, b = v[:, 0], v[:, 1]
    got = ref.pair_sumsq_f32(a, b)
    want = np.array([_rn32(Fraction(float(x)) ** 2 + Fraction(float(np.float32(y) * np.float32(y))))
                     for x, y in zip(a, b)], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # a pair whose squares fall in the fp32 denormal range, where rounding the
    # first square separately changes the sum: 2^-138 * 1.125^2 + 2^-140 * 1.546875^2
    a = np.uint32([0x1B900000]).view(np.float32)
    b = np.uint32([0x1B460000]).view(np.float32)
    fused = ref.pair_sumsq_f32(a, b)[0]
    assert fused == _rn32(Fraction(float(a[0])) ** 2 + Fraction(float(b[0] * b[0])))
    assert fused != np.float32(a[0] * a[0] + b[0] * b[0])


def synth_bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16).view(np.float32)
