"""Pins for the oracle's end-to-end quantize / dequantize (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import hlwq_ref as ref
from oracle import lloyd_max as lm

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 30, 200_000))).astype(np.float32)
    # include exact ties: low 16 bits == 0x8000
    ties = (rng.integers(0, 2 ** 16, 5000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ref.f32_to_bf16_rne(x), want)
    assert np.array_equal(synth.f32_to_bf16_bits(x), want)
    back = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(ref.bf16_to_f32(want), back)


@pytest.mark.parametrize("bits", [5, 3])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_one_hot_block(bits, sign):
    # x = a e_i: n = |a| exactly, y = +-column i of the +-1 Hadamard matrix, so
    # every code is the one of centroid nearest +-1 (1.0488 for Q5, 0.7560 for
    # Q3), and the dequantised block is exactly RN(c * n16) e_i with +0 elsewhere.
    c32, b32 = lm.table(bits)
    a = np.float32(sign * 0.03125)
    i = 37
    w = np.zeros((1, 128), dtype=np.uint16)
    w[0, i] = synth.f32_to_bf16_bits(np.array([a]))[0]
    packed, n16 = ref.quantize_c(w, bits)
    assert n16[0, 0] == np.float16(abs(a))
    codes = ref.unpack_codes(packed, bits)[0, 0]
    hcol = ref.sylvester_hadamard(128)[:, i] * np.sign(a)
    K = 1 << bits
    up = int(np.argmin(np.abs(c32 - 1.0)))
    assert np.array_equal(codes, np.where(hcol > 0, up, K - 1 - up))
    out = ref.bf16_to_f32(ref.dequantize_c(packed, n16, 128, bits))[0]
    want = np.zeros(128, dtype=np.float32)
    want[i] = np.float32(sign) * (c32[up] * np.float32(n16[0, 0]))
    assert np.array_equal(out.view(np.uint32), ref.bf16_to_f32(ref.f32_to_bf16_rne(want)).view(np.uint32))


@pytest.mark.parametrize("bits", [5, 3])
def test_constant_block(bits):
    # x = a * ones: z = (128 a, 0, ..., 0) exactly; y_0 = sqrt(128) -> top code,
    # the 127 exact zeros sit on the middle threshold 0 and take the lower code.
    K = 1 << bits
    c32, _ = lm.table(bits)
    w = np.full((1, 128), synth.f32_to_bf16_bits(np.array([0.015625], np.float32))[0], dtype=np.uint16)
    packed, n16 = ref.quantize_c(w, bits)
    codes = ref.unpack_codes(packed, bits)[0, 0]
    assert codes[0] == K - 1
    assert np.all(codes[1:] == K // 2 - 1)
    out = ref.bf16_to_f32(ref.dequantize_c(packed, n16, 128, bits))[0].astype(np.float64)
    n = float(n16[0, 0])
    cm = float(c32[K // 2 - 1])
    ct = float(c32[K - 1])
    assert abs(out[0] - n * (ct + 127 * cm) / 128) <= 2 ** -8 * abs(out[0]) + 1e-12
    want_rest = n * (ct - cm) / 128
    assert np.all(np.abs(out[1:] - want_rest) <= 2 ** -8 * abs(want_rest))


@pytest.mark.parametrize("bits", [5, 3])
def test_zero_block(bits):
    K = 1 << bits
    w = np.zeros((2, 128), dtype=np.uint16)
    packed, n16 = ref.quantize_c(w, bits)
    assert np.all(n16.view(np.uint16) == 0)
    assert np.all(ref.unpack_codes(packed, bits) == K // 2 - 1)
    out = ref.dequantize_c(packed, n16, 128, bits)
    # butterflies of the constant centroid c_{K/2-1} < 0 leave 128 c at entry 0
    # and exact +0 elsewhere; times a zero scale: -0 at entry 0, +0 elsewhere.
    assert out[0, 0] == 0x8000 and np.all(out[:, 1:] == 0)


def test_tail_block_padding():
    w = synth.random_bf16((8, 704), seed=1)
    packed, n16 = ref.quantize_c(w, 5)
    assert packed.shape == (8, 6, 80) and n16.shape == (8, 6)
    x = ref.bf16_to_f32(w).astype(np.float64)
    tail_norm = np.linalg.norm(x[:, 640:], axis=1)
    assert np.allclose(n16[:, 5].astype(np.float64), tail_norm, rtol=2 ** -10)
    full = np.zeros((8, 768), dtype=np.uint16)
    full[:, :704] = w
    p2, n2 = ref.quantize_c(full, 5)
    assert np.array_equal(p2, packed) and np.array_equal(n2.view(np.uint16), n16.view(np.uint16))
    out = ref.dequantize_c(packed, n16, 704, 5)
    assert out.shape == (8, 704)
    assert np.array_equal(out, ref.dequantize_c(p2, n2, 768, 5)[:, :704])


def _cos(a, b):
    a = a.astype(np.float64).ravel()
    b = b.astype(np.float64).ravel()
    return float(a @ b / math.sqrt((a @ a) * (b @ b)))


@pytest.mark.parametrize("dist,ofrac", [("normal", 0.0), ("normal", 0.001), ("student_t5", 0.0)])
def test_quality_q5_and_q3(dist, ofrac):
    # cos_sim > 0.996 for Q5 ("Gemma-4-26B-A4B-it-HLWQ-Q5", Method: HLWQ);
    # on Gaussian-like data it should sit at sqrt(1 - D_K).
    w = synth.random_bf16((256, 1024), seed=7, dist=dist, outlier_frac=ofrac, outlier_mult=20.0)
    x = ref.bf16_to_f32(w)
    for bits, floor in ((5, 0.996), (3, 0.975)):
        packed, n16 = ref.quantize_c(w, bits)
        xh = ref.bf16_to_f32(ref.dequantize_c(packed, n16, 1024, bits))
        c = _cos(x, xh)
        d = lm.distortion(lm.lloyd_max_gaussian(1 << bits)[0])
        assert c > floor
        assert abs(c - math.sqrt(1 - d)) < 2e-3


@pytest.mark.parametrize("bits,L", [(5, 128), (3, 128), (3, 256)])
def test_canonical_tier_vs_definition(bits, L):
    # Tier C (fp32) may only disagree with Tier D (fp64) on values that sit
    # within 1e-5 of a decision boundary; such flips must be rare.  Norms agree
    # to fp16 rounding, dequant to 1e-3 per unit of block norm.
    rng = np.random.default_rng(11)
    w = synth.f32_to_bf16_bits((rng.standard_normal((20000, L)) * 0.02).astype(np.float32))
    x = ref.bf16_to_f32(w)
    tables = lm.table(bits)
    codes_c, _, n16, _ = ref.quantize_vectors_c(x, bits, tables)
    codes_d, nd, yd = ref.quantize_def(x, bits, tables[0])
    diff = codes_c != codes_d
    dist = ref.boundary_distance(yd, tables[0])
    assert np.all(dist[diff] < 1e-5)
    assert diff.mean() < 1e-5
    assert np.mean(n16 != nd.astype(np.float16)) < 1e-3
    assert np.all(np.abs(n16.astype(np.float64) / nd - 1) <= 2 ** -11)
    deq_c = ref.dequantize_vectors_c(codes_c, n16, bits, tables).astype(np.float64)
    deq_d = ref.dequantize_def(codes_c, n16.astype(np.float64), bits, tables[0])
    assert np.all(np.abs(deq_c - deq_d) <= 1e-3 * nd[..., None] + 1e-30)


@pytest.mark.parametrize("bits", [5, 3])
def test_requantization_is_idempotent(bits):
    # dequantize -> quantize returns the same codes: rescaling the centroid
    # vector to unit mean square moves every centroid far less than its
    # distance to a threshold.
    w = synth.random_bf16((512, 512), seed=9)
    packed, n16 = ref.quantize_c(w, bits)
    again, n16b = ref.quantize_c(ref.dequantize_c(packed, n16, 512, bits), bits)
    assert np.array_equal(again, packed)


def test_kv_path():
    kv = synth.random_bf16((1, 2, 300, 256), seed=3, sigma=1.0)
    packed, n16 = ref.kv_quantize_c(kv, n_residual=128, bits=3)
    assert packed.shape == (1, 2, 172, 96) and n16.shape == (1, 2, 172)
    # each quantised token equals the same transform applied to that vector alone
    x = ref.bf16_to_f32(kv[0, 1, 100])
    codes, _, n, _ = ref.quantize_vectors_c(x[None], 3)
    assert np.array_equal(ref.pack_codes(codes, 3)[0], packed[0, 1, 100])
    assert n[0] == n16[0, 1, 100]
    out = ref.kv_dequantize_c(packed, n16, 3)
    assert out.shape == (1, 2, 172, 256)
    c = _cos(ref.bf16_to_f32(kv[:, :, :172]), ref.bf16_to_f32(out))
    assert abs(c - math.sqrt(1 - lm.distortion(lm.lloyd_max_gaussian(8)[0]))) < 3e-3
    # fewer tokens than the residual window: nothing is quantised
    p0, n0 = ref.kv_quantize_c(kv[:, :, :100], n_residual=128)
    assert p0.shape == (1, 2, 0, 96) and n0.shape == (1, 2, 0)


def test_linear_golden_regression():
    # Stored by tests/golden/make_golden.py (oracle only); guards the oracle
    # against silent drift.
    g = json.load(open(os.path.join(GOLD, "linear_64x256_q5.json")))
    w = synth.weight("linear_64x256", "W")
    assert synth.bf16_bits_to_f32(w).dtype == np.float32
    packed, n16 = ref.quantize_c(w, 5)
    assert bytes(packed.ravel()).hex() == g["packed_hex"]
    assert bytes(n16.view(np.uint16).astype("<u2").ravel().view(np.uint8)).hex() == g["norms_hex"]
    out = ref.dequantize_c(packed, n16, 256, 5)
    assert bytes(out.astype("<u2").ravel().view(np.uint8)).hex() == g["dequant_hex"]


def test_underflowing_squares_reach():
    # Squares below 2^-150 vanish from the fp32 norm sum, so a block of such
    # values next to one larger value gets a norm far below its exact one and
    # rotated values far beyond sqrt(L); the code is still the nearest centroid
    # (the top one).  The bound |y| < sqrt(L * (1 + R / 2)), R the roundings of
    # the norm sum, is what sizes the kernels' search tables.
    for L, bits, rounds in ((128, 5, 191), (256, 3, 383)):
        v = np.full(L, np.float32(255 / 256 * 2.0 ** -75))
        v[0] = np.float32(1.5 * 2.0 ** -75)
        codes, n, _, y = ref.quantize_vectors_c(v[None], bits)
        assert n[0] == np.float32(2.0 ** -74.5)            # only the first square survives
        assert abs(float(y[0, 0]) - (1.5 + (L - 1) * 255 / 256) * 2.0 ** -0.5) < 1e-3 * L
        assert np.abs(y).max() < math.sqrt(L * (1 + rounds / 2))
        assert codes[0, 0] == (1 << bits) - 1


def test_kv_stream_hand_example():
    # window of 2: tokens a, b, c, d arrive one by one; a and b leave (in that
    # order) and are encoded, c and d stay unquantised
    toks = synth.random_bf16((1, 1, 4, 256), seed=21, sigma=1.0)
    packed, norms, window = ref.kv_stream_c([toks[:, :, i:i + 1] for i in range(4)], n_residual=2)
    assert packed.shape == (1, 1, 2, 96) and norms.shape == (1, 1, 2)
    assert np.array_equal(window, toks[:, :, 2:])
    for i in range(2):
        codes, _, n16, _ = ref.quantize_vectors_c(ref.bf16_to_f32(toks[:, :, i]), 3)
        assert np.array_equal(packed[:, :, i], ref.pack_codes(codes, 3))
        assert np.array_equal(norms[:, :, i].view(np.uint16), n16.view(np.uint16))
    # a window of 0 encodes every token on arrival
    p0, n0, w0 = ref.kv_stream_c([toks], n_residual=0)
    assert p0.shape[2] == 4 and w0.shape[2] == 0


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("chunks", [(1,) * 40, (7, 1, 30, 2), (200,), (130, 3, 5)])
def test_kv_stream_equals_static_cache(bits, chunks):
    # however the tokens arrive, the streamed cache is the static one: every
    # token but the newest n_residual encoded, the newest kept as they came
    T = sum(chunks)
    kv = synth.random_bf16((2, 2, T, 256), seed=T + bits, sigma=1.0)
    n_res = 16
    parts, t = [], 0
    for n in chunks:
        parts.append(kv[:, :, t:t + n])
        t += n
    packed, norms, window = ref.kv_stream_c(parts, n_residual=n_res, bits=bits)
    sp, sn = ref.kv_quantize_c(kv, n_residual=n_res, bits=bits)
    assert np.array_equal(packed, sp)
    assert np.array_equal(norms.view(np.uint16), sn.view(np.uint16))
    assert np.array_equal(window, kv[:, :, max(T - n_res, 0):])


def test_kv_q2_quality():
    # 4 Lloyd-Max levels: cosine near sqrt(1 - D_4), D_4 = 0.1175 (Max, 1960)
    kv = synth.random_bf16((1, 2, 300, 256), seed=31, sigma=1.0)
    packed, n16 = ref.kv_quantize_c(kv, n_residual=128, bits=2)
    assert packed.shape == (1, 2, 172, 64)
    out = ref.bf16_to_f32(ref.kv_dequantize_c(packed, n16, bits=2)).astype(np.float64)
    x = ref.bf16_to_f32(kv[:, :, :172]).astype(np.float64)
    c = float(np.mean(np.sum(x * out, -1) / np.linalg.norm(x, axis=-1) / np.linalg.norm(out, axis=-1)))
    assert abs(c - math.sqrt(1 - 0.1175)) < 5e-3


@pytest.mark.parametrize("bits", [5, 3])
def test_codes8_layout_is_the_unpacked_codes(bits):
    # one code per byte (int8 codes) holds exactly the codes the packed layout
    # packs, and decodes to the same weights
    w = synth.random_bf16((40, 300), seed=50 + bits)
    codes, n16 = ref.quantize_codes8_c(w, bits)
    packed, n16p = ref.quantize_c(w, bits)
    assert codes.dtype == np.uint8 and codes.shape == (40, 3, 128)
    assert np.array_equal(codes, ref.unpack_codes(packed, bits))
    assert np.array_equal(n16.view(np.uint16), n16p.view(np.uint16))
    assert np.array_equal(ref.dequantize_codes8_c(codes, n16, 300, bits), ref.dequantize_c(packed, n16p, 300, bits))
