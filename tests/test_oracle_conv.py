"""Pins of the oracle's causal depthwise conv1d against references that do not
come from it: numpy's convolve, the impulse response, causality and the SiLU of a
library sigmoid.  A wrong tap order, a missing shift, a bias applied after the SiLU
or a convolution that leaks future tokens fails one of them.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_matches_numpy_convolve(K):
    r = _rng(K)
    x = r.standard_normal((2, 3, 37))
    w = r.standard_normal((3, K))
    out = oracle.causal_conv1d(x, w, None, apply_silu=False)
    for b in range(2):
        for d in range(3):
            # np.convolve flips its second argument: the tap on the current token is
            # w[d, K-1], so the flipped taps convolve; the first L outputs are causal
            ref = np.convolve(x[b, d], w[d, ::-1], mode="full")[:37]
            assert np.allclose(out[b, d], ref, rtol=0, atol=1e-12)


def test_impulse_response_is_the_reversed_taps_shifted():
    w = np.array([[0.5, -1.0, 2.0, 3.0]])
    x = np.zeros((1, 1, 9))
    x[0, 0, 2] = 1.0
    out = oracle.causal_conv1d(x, w, None, apply_silu=False)[0, 0]
    # the impulse at t = 2 shows w[K-1] at t = 2, w[K-2] at t = 3, ... and nothing before
    assert np.array_equal(out, [0, 0, 3.0, 2.0, -1.0, 0.5, 0, 0, 0])


def test_causal_and_bias_before_silu():
    r = _rng(5)
    x = r.standard_normal((1, 4, 50))
    w = r.standard_normal((4, 4))
    b = r.standard_normal(4)
    y = oracle.causal_conv1d(x, w, b, apply_silu=True)
    x2 = x.copy()
    x2[:, :, 30:] += r.standard_normal((1, 4, 20))
    y2 = oracle.causal_conv1d(x2, w, b, apply_silu=True)
    assert np.array_equal(y[:, :, :30], y2[:, :, :30])
    assert not np.allclose(y[:, :, 30:], y2[:, :, 30:])
    pre = oracle.causal_conv1d(x, w, None, apply_silu=False) + b[None, :, None]
    assert np.allclose(y, pre * expit(pre), rtol=1e-13, atol=1e-15)


def test_channels_are_independent():
    r = _rng(9)
    x = r.standard_normal((2, 5, 20))
    w = r.standard_normal((5, 4))
    full = oracle.causal_conv1d(x, w, None)
    part = oracle.causal_conv1d(x[:, 2:3], w[2:3], None)
    assert np.array_equal(full[:, 2:3], part)
