"""Checks that pin the backward oracle (``oracle/backward.py``) to facts fixed
outside itself.

Each ``pin_*`` takes a module with ``ssd_backward`` (the oracle, or a copy
with a planted mistake in test_backward_oracle.py) and raises AssertionError
when it disagrees with:
  * a hand-worked two-token example (values derived in the docstring);
  * central finite differences of the loss L = <dy, y> + <dhT, hT> computed by
    the forward sequence oracle (the C recurrence, itself pinned to the dense
    quadratic form), along a random direction of every input;
  * exact identities of a loss that is linear or affine in an input: L is
    linear in (x, h0) jointly, and affine in B, in C and in D, so
    <dx, x> + <dh0, h0> = L and <dB, B> = L - L(B = 0), and likewise for C
    and D;
  * packing (sequences packed together give what each gives alone) and
    grouping (a group's dB, dC is the sum over its heads' own).
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from oracle_pins import rel_err


def _problem(rng, lens=(5, 4), H=2, G=1, P=3, N=2, with_D=True, with_h0=True):
    T = sum(lens)
    return dict(x=rng.standard_normal((T, H, P)),
                dt=np.logaddexp(0.0, rng.standard_normal((T, H)) - 1.0),
                A=-np.exp(rng.uniform(-1.0, 1.0, size=H)),
                B=rng.standard_normal((T, G, N)), C=rng.standard_normal((T, G, N)),
                D=rng.standard_normal(H) if with_D else None,
                h0=rng.standard_normal((len(lens), H, P, N)) if with_h0 else None,
                seq_lens=list(lens),
                dy=rng.standard_normal((T, H, P)),
                dhT=rng.standard_normal((len(lens), H, P, N)))


def _loss(p, **over):
    """L = <dy, y> + <dhT, hT> by the forward sequence oracle."""
    q = dict(p)
    q.update(over)
    y, hT = oracle.ssd_recurrence(q["x"], q["dt"], q["A"], q["B"], q["C"], q["D"], q["h0"],
                                  q["seq_lens"])
    return float(np.sum(q["dy"] * y) + np.sum(q["dhT"] * hT))


def _grads(m, p):
    return m.ssd_backward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"],
                          p["seq_lens"], p["dy"], p["dhT"])


def pin_bwd_worked_example(m):
    """One head, P = N = 1, two tokens: x = (1, 2), dt = (0.5, 1), A = -1,
    B = (2, -1), C = (1, 3), D = 0.25, h0 = 0.5, dy = (1, -2), dhT = 0.5.
    Forward: h_0 = 0.5 e^-0.5 + 1, h_1 = e^-1 h_0 - 2.
    Backward, G starting at dhT = 0.5:
      t = 1: G = 0.5 + (-2)(3) = -5.5; dC_1 = -2 h_1; dx_1 = 0.25(-2) + 1(-5.5)(-1) = 5;
             dB_1 = 1(-5.5)(2) = -11; ddt_1 = (-5.5)(2)(-1) + (-1) e^-1 (-5.5) h_0;
             dA gets 1 e^-1 (-5.5) h_0; G -> -5.5 e^-1
      t = 0: G = -5.5 e^-1 + 1 (1) = 1 - 5.5 e^-1 =: g0; dC_0 = h_0; dx_0 = 0.25 + 0.5 g0 (2);
             dB_0 = 0.5 g0 (1); ddt_0 = g0 (1)(2) + (-1) e^-0.5 g0 (0.5);
             dA gets 0.5 e^-0.5 g0 (0.5); dD = 1 (1) + (-2)(2) = -3; dh0 = e^-0.5 g0."""
    e1, eh = math.exp(-1.0), math.exp(-0.5)
    h_0 = 0.5 * eh + 1.0
    h_1 = e1 * h_0 - 2.0
    g0 = 1.0 - 5.5 * e1
    want = dict(
        dx=[0.25 + g0, 5.0], dB=[0.5 * g0, -11.0], dC=[h_0, -2.0 * h_1],
        ddt=[2.0 * g0 - 0.5 * eh * g0, 11.0 + 5.5 * e1 * h_0],
        dA=[-5.5 * e1 * h_0 + 0.25 * eh * g0], dD=[-3.0], dh0=[eh * g0])
    r = m.ssd_backward(np.array([[[1.0]], [[2.0]]]), np.array([[0.5], [1.0]]), np.array([-1.0]),
                       np.array([[[2.0]], [[-1.0]]]), np.array([[[1.0]], [[3.0]]]),
                       np.array([0.25]), np.array([[[[0.5]]]]), [2],
                       np.array([[[1.0]], [[-2.0]]]), np.array([[[[0.5]]]]))
    for k, v in want.items():
        assert np.allclose(r[k].ravel(), v, rtol=0, atol=1e-14), (k, r[k].ravel(), v)


def pin_bwd_finite_differences(m):
    """<d theta, v> equals the central difference of L along v, for every
    input theta (directions drawn at random; dt stays positive)."""
    rng = np.random.default_rng(41)
    p = _problem(rng, lens=(5, 4), H=2, G=1, P=3, N=2)
    g = _grads(m, p)
    pairs = [("x", "dx"), ("dt", "ddt"), ("A", "dA"), ("B", "dB"), ("C", "dC"), ("D", "dD"),
             ("h0", "dh0")]
    for name, gname in pairs:
        v = rng.standard_normal(p[name].shape)
        eps = 1e-6
        fd = (_loss(p, **{name: p[name] + eps * v}) - _loss(p, **{name: p[name] - eps * v})) / (2 * eps)
        an = float(np.sum(g[gname] * v))
        assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (name, fd, an)


def pin_bwd_linear_identities(m):
    """L is linear in (x, h0) jointly and affine in B, C and D: the gradient
    contracted with the input equals the loss difference exactly (up to
    rounding), at full accuracy rather than the finite-difference bound."""
    rng = np.random.default_rng(42)
    p = _problem(rng, lens=(6, 3, 7), H=4, G=2, P=3, N=4)
    g = _grads(m, p)
    L = _loss(p)
    tol = 1e-11 * (1.0 + abs(L))
    assert abs(np.sum(g["dx"] * p["x"]) + np.sum(g["dh0"] * p["h0"]) - L) <= tol, "x, h0"
    for name, gname in (("B", "dB"), ("C", "dC"), ("D", "dD")):
        L0 = _loss(p, **{name: np.zeros_like(p[name])})
        assert abs(np.sum(g[gname] * p[name]) - (L - L0)) <= tol, name


def pin_bwd_packing_and_groups(m):
    """Packed sequences give what each gives alone; with G = 1, dB and dC are
    the sums over the heads of a run where every head has its own copy of B
    and C (G = H)."""
    rng = np.random.default_rng(43)
    p = _problem(rng, lens=(4, 1, 6), H=3, G=1, P=2, N=3)
    g = _grads(m, p)
    start = 0
    for s, L in enumerate(p["seq_lens"]):
        r = slice(start, start + L)
        q = dict(x=p["x"][r], dt=p["dt"][r], A=p["A"], B=p["B"][r], C=p["C"][r], D=p["D"],
                 h0=p["h0"][s:s + 1], seq_lens=[L], dy=p["dy"][r], dhT=p["dhT"][s:s + 1])
        gs = _grads(m, q)
        for k in ("dx", "ddt", "dB", "dC"):
            assert rel_err(g[k][r], gs[k]) < 1e-13, ("packing", k, s)
        assert rel_err(g["dh0"][s:s + 1], gs["dh0"]) < 1e-13, ("packing dh0", s)
        start += L
    q = dict(p)
    q["B"] = np.repeat(p["B"], 3, axis=1)
    q["C"] = np.repeat(p["C"], 3, axis=1)
    gq = _grads(m, q)
    assert rel_err(g["dB"][:, 0], gq["dB"].sum(axis=1)) < 1e-13, "group dB"
    assert rel_err(g["dC"][:, 0], gq["dC"].sum(axis=1)) < 1e-13, "group dC"
    assert rel_err(g["dx"], gq["dx"]) < 1e-13 and rel_err(g["ddt"], gq["ddt"]) < 1e-13


ALL_BWD_PINS = [(f.__name__, f) for f in (
    pin_bwd_worked_example, pin_bwd_finite_differences, pin_bwd_linear_identities,
    pin_bwd_packing_and_groups)]
