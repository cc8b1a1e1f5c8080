"""Pins of the oracle's RMS normalization producer (y = x / sqrt(mean(x^2) + eps) * gamma, then BF16,
then MXFP8 of the BF16 y; vLLM PR #57977 "[Perf][DSv4.1] Keep activations MXFP8 between DeepGEMM
kernels", before/after diagrams and Pieces).

Each pin is fixed by arithmetic, not by the oracle itself: a hand-computed row (mean, not sum; the
square root; eps inside it), constant rows (exactly +-gamma), scale invariance under powers of two
(exact in floating point), the unit output RMS at gamma = 1, linearity in gamma, all-zero rows, and
the MXFP8 output being the oracle quantizer's of the BF16 y.
"""
import math

import numpy as np
import pytest
import torch

import synth_inputs as si
from oracle import mxfp8_ref as mx
from oracle import rmsnorm_ref as rn

K = 128


def bf16(vals):
    t = torch.tensor(np.asarray(vals, dtype=np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


ONES = bf16(np.ones(K))


@pytest.mark.parametrize("eps", [0.0, 0.1])
def test_hand_computed_row(eps):
    row = np.zeros(K)
    row[0], row[1] = 3.0, 4.0                       # mean of squares: 25 / 128
    y = rn.rmsnorm(bf16(row)[None, :], ONES, eps)[0]
    r = 1.0 / math.sqrt(25.0 / 128.0 + eps)
    assert y[0] == pytest.approx(3.0 * r, rel=1e-15) and y[1] == pytest.approx(4.0 * r, rel=1e-15)
    assert np.all(y[2:] == 0.0)


@pytest.mark.parametrize("c", [3.0, -0.375, 2.0 ** 20, -(2.0 ** -30)])
def test_constant_row_is_plus_minus_gamma(c):
    g = bf16(np.linspace(-2.0, 2.0, K))
    y = rn.rmsnorm(bf16(np.full(K, c))[None, :], g, 0.0)[0]
    assert np.array_equal(y, np.sign(c) * mx.bf16_decode(g))


@pytest.mark.parametrize("alpha", [4.0, 0.25, 2.0 ** 10])
def test_power_of_two_scale_invariance(alpha):
    x = si.quant_sweep_input(3, K, seed=1234)
    g = bf16(np.linspace(0.5, 1.5, K))
    xs = bf16(mx.bf16_decode(x) * alpha)           # exact: a power of two times a BF16 value
    assert np.array_equal(rn.rmsnorm(xs, g, 0.0), rn.rmsnorm(x, g, 0.0))


def test_unit_output_rms_and_gamma_linearity():
    x = si.quant_sweep_input(5, K, seed=99)
    y1 = rn.rmsnorm(x, ONES, 0.0)
    assert np.allclose(np.sqrt(np.mean(y1 * y1, axis=1)), 1.0, rtol=1e-14, atol=0)
    g = bf16(np.linspace(-3.0, 3.0, K))
    assert np.allclose(rn.rmsnorm(x, g, 0.0), y1 * mx.bf16_decode(g)[None, :], rtol=1e-15, atol=0)


def test_eps_matters_only_near_zero_and_zero_rows_stay_zero():
    rows = np.zeros((2, K))
    rows[1, :] = 1e-3
    y = rn.rmsnorm(bf16(rows), ONES, 1e-6)
    assert np.all(y[0] == 0.0)
    ms = mx.bf16_decode(bf16([1e-3]))[0] ** 2
    assert y[1, 0] == pytest.approx(math.sqrt(ms) / math.sqrt(ms + 1e-6), rel=1e-15)


def test_mxfp8_output_is_the_quantized_bf16_y():
    x = si.quant_sweep_input(7, 7168)
    g = si.rmsnorm_gamma(7168)
    y_bits, q, sf = rn.rmsnorm_quantize(x, g, 1e-6)
    assert np.array_equal(y_bits, mx.bf16_round(rn.rmsnorm(x, g, 1e-6)))
    q2, sf2 = mx.quantize(y_bits)
    assert np.array_equal(q, q2) and np.array_equal(sf, sf2)
    # the sweep rows scaled by 1e3 and the all-zero rows both normalize to O(1) or zero
    yd = mx.bf16_decode(y_bits)
    assert np.all(np.abs(yd) < 64.0)


def test_negative_eps_is_rejected():
    with pytest.raises(ValueError):
        rn.rmsnorm(bf16(np.ones((1, K))), ONES, -1.0)
