"""Pins for the oracle's INT4 group-128 step (CPU only)."""
import numpy as np
import pytest

import synth
from oracle import hlwq_ref as ref


def _bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_levels_on_the_grid_are_exact():
    # a group whose values are -3..12 times 2^-6: lo = -3/64, hi = 12/64,
    # scale = 1/64 exactly, zero point 3, every value sits on a level
    vals = (np.arange(-3, 13, dtype=np.float32) / 64).repeat(8)
    q, s, z = ref.int4_quantize_c(_bits(vals)[None])
    assert s[0, 0] == np.float32(1 / 64) and z[0, 0] == 3
    assert np.array_equal(q[0], (np.arange(-3, 13) + 3).repeat(8))
    assert np.array_equal(ref.int4_dequantize(q, s, z)[0], ref.bf16_to_f32(_bits(vals)))


def test_zero_group_and_one_signed_groups():
    q, s, z = ref.int4_quantize_c(np.zeros((1, 256), np.uint16))
    assert np.all(q == 0) and np.all(s == 1) and np.all(z == 0)
    pos = np.linspace(0, 1, 128, dtype=np.float32)
    q, s, z = ref.int4_quantize_c(_bits(pos)[None])
    assert z[0, 0] == 0 and q[0, 0] == 0 and q[0, -1] == 15   # range [0, max]
    q, s, z = ref.int4_quantize_c(_bits(-pos)[None])
    assert z[0, 0] == 15 and q[0, 0] == 15 and q[0, -1] == 0  # range [min, 0]


def test_nearest_level_within_half_a_step():
    # every value lands on one of the two levels around it: the error is at
    # most half a step (plus the fp32 rounding of w / scale), and no other
    # level is closer by more than that rounding
    w = synth.random_bf16((64, 1024), seed=3, dist="student_t5", sigma=0.02)
    q, s, z = ref.int4_quantize_c(w)
    x = ref.bf16_to_f32(w).astype(np.float64).reshape(64, 8, 128)
    levels = (np.arange(16)[None, None, :] - z[..., None].astype(np.float64)) * s[..., None]   # [64, 8, 16]
    err = np.abs(x[..., None] - levels[:, :, None, :])                                           # [64, 8, 128, 16]
    best = err.min(axis=-1)
    got = np.take_along_axis(err, q.reshape(64, 8, 128, 1).astype(np.int64), axis=-1)[..., 0]
    step = s.astype(np.float64)[..., None]
    assert np.all(got <= best + 1e-6 * step)
    assert np.all(got <= 0.5 * step * (1 + 1e-6))


def test_pack_nibbles():
    q = np.array([[1, 2, 15, 0, 7, 8]], np.uint8)
    assert ref.int4_pack(q).tolist() == [[0x21, 0x0F, 0x87]]


def test_dequantize_to_int4_follows_the_bf16_dequant():
    w = synth.random_bf16((32, 256), seed=4)
    packed, n16 = ref.quantize_c(w, 5)
    p4, s, z = ref.dequantize_to_int4_c(packed, n16, 256, 5)
    q, s2, z2 = ref.int4_quantize_c(ref.dequantize_c(packed, n16, 256, 5))
    assert np.array_equal(p4, ref.int4_pack(q)) and np.array_equal(s, s2) and np.array_equal(z, z2)
    assert p4.shape == (32, 128) and s.shape == (32, 2)
    with pytest.raises(ValueError):
        ref.int4_quantize_c(np.zeros((2, 200), np.uint16))
