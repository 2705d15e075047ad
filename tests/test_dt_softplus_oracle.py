"""The oracle's step activation (oracle.dt_softplus) against closed forms of
softplus, and planted mistakes that they must catch."""
import math

import numpy as np
import pytest

import oracle


def _pins(f):
    """Raise AssertionError if f(dt_raw, dt_bias) is not softplus(raw + bias)."""
    # softplus(0) = ln 2, at every head when the bias is zero
    assert np.allclose(f(np.zeros((3, 4)), np.zeros(4)), math.log(2.0), rtol=0, atol=1e-15)
    # softplus(v) - softplus(-v) = v
    v = np.linspace(-30.0, 30.0, 61)[:, None]
    d = f(v, None) - f(-v, None)
    assert np.allclose(d, v, rtol=0, atol=1e-12)
    # large v: softplus(v) = v + log1p(e^-v); very negative v: softplus(v) ~ e^v
    assert abs(f(np.array([[40.0]]), None)[0, 0] - 40.0) < 1e-15
    assert abs(f(np.array([[-40.0]]), None)[0, 0] / math.exp(-40.0) - 1.0) < 1e-12
    # the bias of head h shifts column h only
    raw = np.array([[0.5, -1.0, 2.0]])
    bias = np.array([0.25, -0.5, 1.0])
    want = [math.log1p(math.exp(0.75)), math.log1p(math.exp(-1.5)), math.log1p(math.exp(3.0))]
    assert np.allclose(f(raw, bias)[0], want, rtol=0, atol=1e-15)


def test_dt_softplus_pins():
    _pins(oracle.dt_softplus)


MUTANTS = {
    "no_activation": lambda raw, b: raw + (0 if b is None else b),
    "bias_after_activation": lambda raw, b: np.logaddexp(0.0, raw) + (0 if b is None else b),
    "bias_of_head_0": lambda raw, b: np.logaddexp(0.0, raw + (0 if b is None else b[0])),
    "exp_not_softplus": lambda raw, b: np.exp(raw + (0 if b is None else b)),
    "relu": lambda raw, b: np.maximum(raw + (0 if b is None else b), 0.0),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_dt_softplus_mutant_is_caught(name):
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            _pins(MUTANTS[name])
