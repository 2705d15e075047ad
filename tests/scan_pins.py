"""Checks that pin the selective-scan oracle (``oracle/selective_scan.py``) to
facts fixed outside itself.

Each ``pin_*`` takes a module with ``selective_scan`` (the oracle, or a copy
with a planted mistake in test_scan_oracle.py) and raises AssertionError when
it disagrees with:
  * a hand-worked two-token example (values derived in the comments);
  * the SSD recurrence (the C oracle, itself pinned to the dense quadratic
    form) when A is one scalar per head of P channels and the step is shared
    by the head's channels -- the restriction that turns the selective SSM
    into Mamba-2's layer (QbitAI "Mamba-2" article, srwj168 repost, section
    "Mamba-2: stronger learning, faster training and inference");
  * closed forms: constant inputs with a different A for every state index
    (geometric series), A = 0 (running sum), the reset limit step*A -> -inf
    and the freeze limit step -> 0 (tj-hxxt.cn long read, part III item 3);
  * channel independence (a subset of channels runs as in the full run).
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from oracle_pins import rel_err


def _case(rng, batch, L, Dm, N, with_D=True, with_h0=True):
    return dict(
        x=rng.standard_normal((batch, L, Dm)),
        delta=np.logaddexp(0.0, rng.standard_normal((batch, L, Dm)) - 1.0),
        A=-np.exp(rng.uniform(-1.0, 1.0, size=(Dm, N))),
        B=rng.standard_normal((batch, L, N)),
        C=rng.standard_normal((batch, L, N)),
        D=rng.standard_normal(Dm) if with_D else None,
        h0=rng.standard_normal((batch, Dm, N)) if with_h0 else None)


def _run(m, c, **kw):
    return m.selective_scan(c["x"], c["delta"], c["A"], c["B"], c["C"], c["D"], c["h0"], **kw)


def pin_scan_worked_example(m):
    """One channel, N = 2, two tokens, zero initial state, no D:
    x = (1, 2), step = (0.5, 1), A = (-1, -2), B_0 = (1, 1), B_1 = (0, 1),
    C_0 = (1, 1), C_1 = (2, 0).
      t = 0: h = 0.5 * 1 * (1, 1) = (0.5, 0.5);            y_0 = 0.5 + 0.5 = 1
      t = 1: h = (0.5 e^-1, 0.5 e^-2) + 1 * 2 * (0, 1)
               = (0.5 e^-1, 0.5 e^-2 + 2);                  y_1 = 2 * 0.5 e^-1 = e^-1
    """
    x = np.array([[[1.0], [2.0]]])
    delta = np.array([[[0.5], [1.0]]])
    A = np.array([[-1.0, -2.0]])
    B = np.array([[[1.0, 1.0], [0.0, 1.0]]])
    C = np.array([[[1.0, 1.0], [2.0, 0.0]]])
    y, h = m.selective_scan(x, delta, A, B, C, None, None)
    assert np.allclose(y[0, :, 0], [1.0, math.exp(-1.0)], rtol=0, atol=1e-15), y
    assert np.allclose(h[0, 0], [0.5 * math.exp(-1.0), 0.5 * math.exp(-2.0) + 2.0],
                       rtol=0, atol=1e-15), h


def pin_scan_reduces_to_ssd(m):
    """A[d, n] = A_h and step[b, t, d] = dt[b, t, h] for the P channels of
    head h: the scan equals the SSD recurrence with one B, C group."""
    rng = np.random.default_rng(21)
    batch, L, H, P, N = 2, 37, 3, 4, 5
    dt = np.logaddexp(0.0, rng.standard_normal((batch, L, H)) - 1.0)
    Ah = -np.exp(rng.uniform(-1.0, 1.0, size=H))
    xs = rng.standard_normal((batch, L, H, P))
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    Dh = rng.standard_normal(H)
    h0 = rng.standard_normal((batch, H, P, N))
    head = np.repeat(np.arange(H), P)                      # channel d = h * P + p
    y, hT = m.selective_scan(xs.reshape(batch, L, H * P), dt[:, :, head],
                             np.repeat(Ah[head][:, None], N, axis=1), B, C, Dh[head],
                             h0.reshape(batch, H * P, N))
    T = batch * L
    yr, hr = oracle.ssd_recurrence(xs.reshape(T, H, P), dt.reshape(T, H), Ah,
                                   B.reshape(T, 1, N), C.reshape(T, 1, N), Dh, h0,
                                   [L] * batch)
    assert rel_err(y, yr.reshape(batch, L, H * P)) < 1e-12, "y vs SSD"
    assert rel_err(hT, hr.reshape(batch, H * P, N)) < 1e-12, "state vs SSD"


def pin_scan_closed_form_constant(m):
    """Constant step, x, B, C per sequence and channel, a different A for
    every state index: h_k[n] = a_n^k h0[n] + step x B_n (1 - a_n^k) / (1 - a_n)
    with a_n = exp(step A[d, n]); y_k = sum_n C_n h_k[n] + D x."""
    rng = np.random.default_rng(22)
    batch, L, Dm, N = 2, 25, 3, 4
    A = -np.exp(rng.uniform(-2.0, 1.0, size=(Dm, N)))
    step = np.array([[0.3, 0.05, 1.2], [0.7, 0.2, 0.01]])
    xi = rng.standard_normal((batch, Dm))
    b = rng.standard_normal((batch, N))
    c = rng.standard_normal((batch, N))
    D = rng.standard_normal(Dm)
    h0 = rng.standard_normal((batch, Dm, N))
    rep = lambda v: np.repeat(v[:, None], L, axis=1)
    y, hT = m.selective_scan(rep(xi), rep(step), A, rep(b), rep(c), D, h0)
    a = np.exp(step[:, :, None] * A[None])                  # (batch, Dm, N)
    for k in (1, 2, 13, L):
        hk = a ** k * h0 + (step * xi)[:, :, None] * b[:, None, :] * (1 - a ** k) / (1 - a)
        yk = np.einsum("bdn,bn->bd", hk, c) + D[None] * xi
        assert rel_err(y[:, k - 1], yk) < 1e-12, ("closed form y", k)
        if k == L:
            assert rel_err(hT, hk) < 1e-12, "closed form state"


def pin_scan_a_zero_running_sum(m):
    """A = 0: the state is h0 plus the running sum of step x B (cumsum)."""
    rng = np.random.default_rng(23)
    c = _case(rng, 2, 9, 3, 4)
    c["A"] = np.zeros_like(c["A"])
    y, hT = _run(m, c)
    terms = (c["delta"] * c["x"])[..., None] * c["B"][:, :, None, :]   # (b, L, Dm, N)
    states = c["h0"][:, None] + np.cumsum(terms, axis=1)
    yy = np.einsum("btdn,btn->btd", states, c["C"]) + c["D"][None, None] * c["x"]
    assert rel_err(y, yy) < 1e-12 and rel_err(hT, states[:, -1]) < 1e-12, "A=0"


def pin_scan_reset_limit(m):
    """step*A -> -inf: every token forgets the state before it;
    y_t = step_t (C_t . B_t) x_t + D x_t."""
    rng = np.random.default_rng(24)
    c = _case(rng, 2, 6, 3, 4)
    c["A"] = np.full_like(c["A"], -1.0e4)
    c["delta"] = 0.05 + rng.uniform(size=c["delta"].shape)
    y, hT = _run(m, c)
    cb = np.sum(c["C"] * c["B"], axis=-1)                   # (batch, L)
    assert rel_err(y, c["delta"] * cb[..., None] * c["x"] + c["D"] * c["x"]) < 1e-12, "reset y"
    last = (c["delta"][:, -1] * c["x"][:, -1])[..., None] * c["B"][:, -1, None, :]
    assert rel_err(hT, last) < 1e-12, "reset state"


def pin_scan_freeze_limit(m):
    """step = 0: the state is kept exactly; y_t = C_t . h0 + D x_t."""
    rng = np.random.default_rng(25)
    c = _case(rng, 2, 5, 3, 4)
    c["delta"] = np.zeros_like(c["delta"])
    y, hT = _run(m, c)
    assert np.array_equal(hT, c["h0"]), "freeze state"
    assert rel_err(y, np.einsum("bdn,btn->btd", c["h0"], c["C"]) + c["D"] * c["x"]) < 1e-12


def pin_scan_channels_independent(m):
    """Running a subset of channels reproduces those channels of the full run."""
    rng = np.random.default_rng(26)
    c = _case(rng, 2, 11, 6, 3)
    y, hT = _run(m, c)
    sel = np.array([4, 1, 5])
    ys, hs = _run(m, c, channels=sel)
    assert rel_err(ys, y[:, :, sel]) < 1e-15 and rel_err(hs, hT[:, sel]) < 1e-15, "subset"


ALL_SCAN_PINS = [(f.__name__, f) for f in (
    pin_scan_worked_example, pin_scan_reduces_to_ssd, pin_scan_closed_form_constant,
    pin_scan_a_zero_running_sum, pin_scan_reset_limit, pin_scan_freeze_limit,
    pin_scan_channels_independent)]
