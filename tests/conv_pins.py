"""Checks that pin the convolution-front oracle (``oracle/conv.py``) to facts
fixed outside itself.

Each ``pin_*`` takes a module with ``silu``, ``causal_conv`` and
``conv_front`` (the oracle, or a copy with a planted mistake in
test_conv_oracle.py) and raises AssertionError when it disagrees with:
  * a hand-worked three-token example (values derived in the docstring);
  * numpy's full discrete convolution (np.convolve), the textbook definition
    a causal filter reduces to when the history is zero;
  * scipy's logistic function for the activation, and the identity
    silu(v) - silu(-v) = v;
  * causality (a change at token t moves no output before t);
  * continuation (one call over a sequence equals two calls, the second
    given the history the first returned);
  * packing (sequences packed together give what each gives alone), and the
    routing of the packed channels to x, B and C.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import expit

from oracle_pins import rel_err


def _rand(rng, L, ch, K):
    return (rng.standard_normal((L, ch)), 0.5 * rng.standard_normal((ch, K)),
            0.3 * rng.standard_normal(ch))


def pin_conv_worked_example(m):
    """One channel, K = 3, u = (1, 2, 3), weight = (0.5, -1, 2) (oldest tap
    first), bias 0.25, zero history:
      pre_0 = 2*1                 + 0.25 = 2.25
      pre_1 = 2*2 - 1*1           + 0.25 = 3.25
      pre_2 = 2*3 - 1*2 + 0.5*1   + 0.25 = 4.75
    out_t = pre_t / (1 + e^-pre_t); the history afterwards is (2, 3)."""
    out, h = m.causal_conv(np.array([[1.0], [2.0], [3.0]]), np.array([[0.5, -1.0, 2.0]]),
                           np.array([0.25]))
    pre = [2.25, 3.25, 4.75]
    want = [p / (1.0 + math.exp(-p)) for p in pre]
    assert np.allclose(out[:, 0], want, rtol=0, atol=1e-15), out
    assert np.array_equal(h[:, 0], [2.0, 3.0]), h


def pin_conv_is_np_convolve(m):
    """Zero history, no activation: channel c is np.convolve(u_c, reversed
    weight_c) truncated to the first L outputs, plus the bias."""
    rng = np.random.default_rng(31)
    for K in (2, 3, 4):
        u, w, b = _rand(rng, 23, 5, K)
        out, _ = m.causal_conv(u, w, b, activation=False)
        for c in range(5):
            ref = np.convolve(u[:, c], w[c, ::-1])[:23] + b[c]
            assert rel_err(out[:, c], ref) < 1e-14, ("convolve", K, c)


def pin_silu_closed_forms(m):
    """silu(v) = v * expit(v); silu(v) - silu(-v) = v; silu(0) = 0;
    silu(ln 3) = (3/4) ln 3."""
    v = np.linspace(-30.0, 30.0, 601)
    s = m.silu(v)
    assert rel_err(s, v * expit(v)) < 1e-15, "silu vs expit"
    assert np.allclose(s - m.silu(-v), v, rtol=1e-15, atol=1e-14), "odd part"
    assert m.silu(np.array([0.0]))[0] == 0.0
    assert abs(m.silu(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15


def pin_conv_causal(m):
    """Perturbing token t changes nothing before t, and (with K taps) nothing
    from t + K on."""
    rng = np.random.default_rng(32)
    u, w, b = _rand(rng, 20, 4, 4)
    base, _ = m.causal_conv(u, w, b)
    u2 = u.copy()
    u2[9] += 1.0
    pert, _ = m.causal_conv(u2, w, b)
    assert np.array_equal(base[:9], pert[:9]), "output before the change moved"
    assert np.array_equal(base[13:], pert[13:]), "output beyond the filter moved"
    assert np.all(np.abs(base[9:13] - pert[9:13]) > 0), "filter window did not see the change"


def pin_conv_continuation(m):
    """conv over u equals conv over u[:L1] then u[L1:] with the returned
    history, for split points before, inside and past the first K - 1
    tokens (a short first part carries part of the initial history)."""
    rng = np.random.default_rng(33)
    u, w, b = _rand(rng, 17, 3, 4)
    h0 = rng.standard_normal((3, 3))
    full, hf = m.causal_conv(u, w, b, h0)
    for L1 in (0, 1, 2, 3, 9, 17):
        o1, h1 = m.causal_conv(u[:L1], w, b, h0)
        o2, h2 = m.causal_conv(u[L1:], w, b, h1)
        assert rel_err(np.concatenate([o1, o2]), full) < 1e-15, ("continuation", L1)
        assert np.array_equal(h2, hf), ("history", L1)
    # the history is the last K - 1 inputs, oldest first
    assert np.array_equal(hf, u[-3:])
    _, hs = m.causal_conv(u[:1], w, b, h0)
    assert np.array_equal(hs, np.concatenate([h0[1:], u[:1]])), "short sequence history"


def pin_conv_front_packing_and_routing(m):
    """Packed sequences (one empty) equal separate runs; the channels route
    to x, B, C in order; tokens of one sequence never reach another."""
    rng = np.random.default_rng(34)
    x_dim, bc_dim, K = 4, 2, 3
    ch = x_dim + 2 * bc_dim
    cu = [0, 5, 5, 6, 14]
    T = cu[-1]
    xbc, w, b = _rand(rng, T, ch, K)
    hist = rng.standard_normal((4, K - 1, ch))
    bounds = [(cu[i], cu[i + 1]) for i in range(4)]
    x, B, C, ho = m.conv_front(xbc, w, b, bounds, x_dim, bc_dim, hist)
    packed = np.concatenate([x, B, C], axis=1)
    for s, (a, e) in enumerate(bounds):
        o, h = m.causal_conv(xbc[a:e], w, b, hist[s])
        if e > a:
            assert rel_err(packed[a:e], o) < 1e-15, ("packed", s)
        assert np.array_equal(ho[s], h), ("history", s)
    assert np.array_equal(ho[1], hist[1]), "empty sequence keeps its history"
    # routing: scale each part's bias so the parts differ, zero the taps
    zw = np.zeros_like(w)
    bb = np.concatenate([np.full(x_dim, 1.0), np.full(bc_dim, 2.0), np.full(bc_dim, 3.0)])
    x, B, C, _ = m.conv_front(xbc, zw, bb, bounds, x_dim, bc_dim)
    for part, v in ((x, 1.0), (B, 2.0), (C, 3.0)):
        assert np.allclose(part, v / (1.0 + math.exp(-v)), rtol=1e-15), "routing"
    # no leak: changing the last token of sequence 2 (token 5) leaves sequence
    # 3 (tokens 6..13) and its history untouched
    xbc2 = xbc.copy()
    xbc2[5] += 5.0
    x2, B2, C2, h2 = m.conv_front(xbc2, w, b, bounds, x_dim, bc_dim, hist)
    x1, B1, C1, h1 = m.conv_front(xbc, w, b, bounds, x_dim, bc_dim, hist)
    assert np.array_equal(np.concatenate([x1, B1, C1], 1)[6:], np.concatenate([x2, B2, C2], 1)[6:])
    assert np.array_equal(h1[3], h2[3]), "leak into the next sequence's history"


ALL_CONV_PINS = [(f.__name__, f) for f in (
    pin_conv_worked_example, pin_conv_is_np_convolve, pin_silu_closed_forms, pin_conv_causal,
    pin_conv_continuation, pin_conv_front_packing_and_routing)]
