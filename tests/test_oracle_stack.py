"""Pins of the stack glue (oracle.stack.rms_norm) by closed forms and exact
invariants: a constant row maps to +-target, a one-hot row to
+-target*sqrt(H) at its index, a zero row to zeros, the output RMS is the
target, and scaling the input by a power of two changes nothing."""
import numpy as np

import synth
from oracle import stack


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_constant_rows():
    t = 2.2338308
    x = _bits([[3.0] * 64, [-0.5] * 64])
    y = stack.rms_norm(x, t)
    assert np.allclose(y[0], t, rtol=1e-15, atol=0)
    assert np.allclose(y[1], -t, rtol=1e-15, atol=0)


def test_one_hot_and_zero_rows():
    H, t = 256, 1.5
    x = np.zeros((2, H), np.float32)
    x[0, 17] = -7.0
    y = stack.rms_norm(_bits(x), t)
    assert np.isclose(y[0, 17], -t * np.sqrt(H), rtol=1e-15)
    assert np.count_nonzero(y[0]) == 1
    assert np.all(y[1] == 0.0)


def test_output_rms_and_power_of_two_invariance():
    rng = np.random.default_rng(5)
    x = _bits(rng.standard_normal((8, 2560)) * np.array([[0.01], [0.1], [1], [3], [10], [30], [100], [1000]]))
    t = np.sqrt(4.99)
    y = stack.rms_norm(x, t)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), t, rtol=1e-12)
    x4 = (x.astype(np.uint32) + (2 << 7)).astype(np.uint16)       # exponent + 2: x * 4, exact
    assert np.array_equal(stack.rms_norm(x4, t), y)
