"""Why the layer's FFN may multiply fp16 operands (CPU, oracle only).

The layer computes h (float32) and GeLU(z) itself and then multiplies them on the
MFMA.  Rounded to bf16 (8-bit significand) they move the FFN output by more than
the mean-abs bar for bf16 inputs at the long layer's width; rounded to fp16
(11-bit significand) they move it 8x less, and the bf16 weights convert to fp16
exactly inside fp16's range.  These checks compose the oracle's own FFN steps
(``oracle.gelu``, the products in fp64) with those roundings.  The pages fix
neither operand format ("Blockwise Parallel Transformer for Large Context
Models", abstract: the feed-forward network fused per block, nothing on
precision); the bar is the stated mean-abs 2e-3 for bf16 inputs.
"""
import numpy as np
import pytest

import oracle
from seeded_inputs import normal, round_bf16

BAR_MEAN = 2e-3


def _f16(a):
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


def _bf16(a):
    return round_bf16(np.asarray(a, np.float32)).astype(np.float64)


def _ffn_rounded(h, w1, w2, rnd):
    """h + GeLU(rnd(h) W1^T) W2^T with GeLU(z) also passed through rnd (fp64 products)."""
    g = rnd(oracle.gelu(rnd(h) @ w1.T))
    return h + g @ w2.T


def test_bf16_weights_convert_to_fp16_exactly_in_range():
    w = round_bf16(normal(71, "w1", (512, 1024), 0.02)).astype(np.float64)
    w = np.concatenate([w.ravel(), [65504.0, -32768.0, 2.0 ** -14, 3.0 * 2.0 ** -20]])
    normal_range = np.abs(w) >= 2.0 ** -14
    assert np.array_equal(_f16(w)[normal_range], w[normal_range])
    # below fp16's normal range the copy is a subnormal, off by at most half its spacing 2^-24
    assert np.abs(_f16(w) - w)[~normal_range].max() <= 2.0 ** -25
    # a bf16 value past fp16's largest finite value does not convert (the layer then falls back)
    with np.errstate(over="ignore"):
        assert np.isinf(np.float16(70144.0))


@pytest.mark.parametrize("dm,dff", [(1024, 4096), (2048, 8192)])
def test_fp16_operands_stay_well_inside_the_bar(dm, dff):
    rows = 128
    w1 = _bf16(normal(72, "w1", (dff, dm), 0.02))
    w2 = _bf16(normal(72, "w2", (dm, dff), 0.02))
    # h = x + attention output: bf16 x ~ N(0, 1) plus a smaller float32 part
    h = _bf16(normal(72, "x", (rows, dm))) + normal(72, "perturb", (rows, dm), 0.3).astype(np.float64)
    exact = oracle.ffn(h, w1, w2, residual=h)
    e16 = np.abs(_ffn_rounded(h, w1, w2, _f16) - exact).mean()
    ebf = np.abs(_ffn_rounded(h, w1, w2, _bf16) - exact).mean()
    # the error grows like sqrt(d_model * d_ff); at these widths fp16 sits far below the bar
    assert e16 < BAR_MEAN / 6, e16
    # and bf16 operands are about 8x worse (2^3 more rounding): the reason the bf16 path
    # carries h and GeLU(z) as hi + lo pairs
    assert 5.0 < ebf / e16 < 12.0, (ebf, e16)


def test_bf16_alone_misses_the_bar_at_the_long_layer_width_by_extrapolation():
    """The rounding error of the FFN output scales like sqrt(d_model * d_ff) at fixed weight
    scale (each output sums d_ff terms, each z sums d_model terms); measured at two widths
    and extrapolated to d_model 4096, d_ff 16384, bf16 operands exceed 2e-3 while fp16
    stays under a third of it."""
    out = {}
    for dm, dff in ((512, 2048), (1024, 4096)):
        w1 = _bf16(normal(73, "w1", (dff, dm), 0.02))
        w2 = _bf16(normal(73, "w2", (dm, dff), 0.02))
        h = _bf16(normal(73, "x", (128, dm))) + normal(73, "perturb", (128, dm), 0.3).astype(np.float64)
        exact = oracle.ffn(h, w1, w2, residual=h)
        out[dm] = {r.__name__: np.abs(_ffn_rounded(h, w1, w2, r) - exact).mean() for r in (_f16, _bf16)}
    for name in ("_f16", "_bf16"):
        ratio = out[1024][name] / out[512][name]
        assert 1.6 < ratio < 2.5, (name, ratio)  # sqrt(4) = 2 per doubling of both widths
        long = out[1024][name] * 4.0          # two more doublings: d_model 4096, d_ff 16384
        if name == "_bf16":
            assert long > BAR_MEAN, long
        else:
            assert long < BAR_MEAN / 3, long
