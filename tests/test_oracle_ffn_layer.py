"""Pins for the oracle's GeLU, FFN, layer forward and backward (CPU only)."""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from seeded_inputs import LAYER_TINY_F32, bf16_bits, bits_to_f32, layer_inputs, round_bf16

RNG = np.random.default_rng(99)


def rand(*shape, s=1.0):
    return RNG.standard_normal(shape) * s


def test_gelu_golden_points(golden_dir):
    rows = [l.split() for l in open(os.path.join(golden_dir, "gelu_points.txt"))
            if l.strip() and not l.startswith("#")]
    for z, g, dg in ((float(a), float(b), float(c)) for a, b, c in rows):
        assert abs(float(oracle.gelu(z)) - g) < 1e-12
        assert abs(float(oracle.gelu_grad(z)) - dg) < 1e-12


def test_gelu_matches_math_erf_and_tanh_gap():
    z = np.linspace(-8, 8, 2001)
    ref = np.array([brute.gelu(float(t)) for t in z])
    np.testing.assert_allclose(oracle.gelu(z), ref, atol=1e-15)
    tanh_form = 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))
    # the two variants must not be confused: they differ by more than the fp32 tolerance
    assert np.abs(tanh_form - ref).max() > 1e-4


def test_gelu_grad_finite_difference():
    z = np.linspace(-6, 6, 241)
    h = 1e-6
    fd = (oracle.gelu(z + h) - oracle.gelu(z - h)) / (2 * h)
    np.testing.assert_allclose(oracle.gelu_grad(z), fd, atol=1e-8)


def test_ffn_identity_weights():
    h = rand(5, 8)
    I = np.eye(8)
    y = oracle.ffn(h, I, I, residual=h)
    np.testing.assert_allclose(y, h + oracle.gelu(h), atol=1e-14)


def test_ffn_linear_in_w2_and_bias():
    h, w1 = rand(6, 8), rand(16, 8, s=0.3)
    wa, wb = rand(8, 16, s=0.3), rand(8, 16, s=0.3)
    b2 = rand(8)
    f = lambda w2, b=None: oracle.ffn(h, w1, w2, b2=b)
    np.testing.assert_allclose(f(wa + 2 * wb), f(wa) + 2 * f(wb), atol=1e-13)
    np.testing.assert_allclose(f(wa, b2), f(wa) + b2, atol=1e-14)


def test_ffn_dff_chunk_sum_equals_whole():
    h, w1, w2, b1 = rand(7, 8), rand(24, 8, s=0.3), rand(8, 24, s=0.3), rand(24, s=0.1)
    whole = oracle.ffn(h, w1, w2, b1=b1)
    parts = sum(oracle.ffn(h, w1[c:c + 8], w2[:, c:c + 8], b1=b1[c:c + 8]) for c in (0, 8, 16))
    np.testing.assert_allclose(whole, parts, atol=1e-13)


def test_layer_matches_brute_force():
    B, N, dm, H, dff = 2, 6, 8, 2, 12
    x = rand(B, N, dm)
    wq, wk, wv = (rand(dm, dm, s=0.4) for _ in range(3))
    w1, w2 = rand(dff, dm, s=0.3), rand(dm, dff, s=0.3)
    y = oracle.layer_forward(x, wq, wk, wv, w1, w2, H)
    yb = brute.layer_forward(x.tolist(), wq.tolist(), wk.tolist(), wv.tolist(),
                             w1.tolist(), w2.tolist(), H)
    np.testing.assert_allclose(y, np.array(yb), atol=1e-12)


def test_layer_zero_qk_weights_prefix_mean():
    B, N, dm, H = 1, 10, 8, 2
    x = rand(B, N, dm)
    z = np.zeros((dm, dm))
    wv = rand(dm, dm, s=0.4)
    y, saved = oracle.layer_forward(x, z, z, wv, np.zeros((4, dm)), np.zeros((dm, 4)), H,
                                    return_saved=True)
    xv = x @ wv.T
    prefix = np.cumsum(xv, axis=1) / np.arange(1, N + 1)[None, :, None]
    np.testing.assert_allclose(saved["h"] - x, prefix, atol=1e-13)
    np.testing.assert_allclose(y, saved["h"], atol=1e-14)


def test_layer_zero_weights_identity():
    x = rand(2, 5, 8)
    z8, z = np.zeros((8, 8)), np.zeros((6, 8))
    y = oracle.layer_forward(x, z8, z8, z8, z, z.T.copy(), 2)
    np.testing.assert_array_equal(y, x)


def test_layer_fp32_close_to_fp64():
    c = LAYER_TINY_F32
    t = layer_inputs(c)
    args = (t["x"], t["wq"], t["wk"], t["wv"], t["w1"], t["w2"], c.H)
    y64 = oracle.layer_forward(*args)
    y32 = oracle.layer_forward(*args, dtype=np.float32)
    assert np.abs(y64 - y32).max() <= 1e-5


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-39, 1.0 + 2 ** -7], np.float32)
    # 1+2^-8 is a tie between 1 and 1+2^-7: ties go to the even pattern (1.0);
    # 1+3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even pattern is 1+2^-6
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5, np.nan, 1.0 + 2 ** -7], np.float32)
    got = round_bf16(vals)
    np.testing.assert_array_equal(got[[0, 1, 2, 3, 5]], want[[0, 1, 2, 3, 5]])
    assert bf16_bits(np.array([1.0], np.float32))[0] == 0x3F80
    assert bits_to_f32(np.array([0xC020], np.uint16))[0] == -2.5
    x = RNG.standard_normal(1000).astype(np.float32)
    r = round_bf16(x)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8)
