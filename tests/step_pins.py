"""Checks that pin the decode-step oracle (``oracle/step.py``) to facts fixed
outside itself.

Each ``pin_*`` takes a module with ``ssd_step`` / ``ssd_steps`` (the oracle,
or a copy with a planted mistake in test_step_oracle.py) and raises
AssertionError when it disagrees with:
  * the hand-worked examples under tests/golden/, stepped token by token;
  * the sequence oracle (the C recurrence, itself pinned to the dense
    quadratic form), with several heads per group;
  * closed forms: constant inputs (geometric series), A = 0 (a running sum
    of outer products), the reset limit dt*A -> -inf and the freeze limit
    dt -> 0 (tj-hxxt.cn long read of the Mamba-1 paper, part III item 3 on
    the step size);
  * linearity in (x, state).
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle_pins import load_golden, rel_err


def _case(rng, batch, H, P, N, G, T=1, with_D=True):
    return dict(
        x=rng.standard_normal((T, batch, H, P)),
        dt=np.logaddexp(0.0, rng.standard_normal((T, batch, H)) - 1.0),
        A=-np.exp(rng.uniform(0.0, 2.0, size=H)),
        B=rng.standard_normal((T, batch, G, N)),
        C=rng.standard_normal((T, batch, G, N)),
        D=rng.standard_normal(H) if with_D else None,
        h0=rng.standard_normal((batch, H, P, N)))


def pin_step_golden(m):
    """Every hand-worked fixture, run one token at a time per sequence."""
    for name in ("worked_single_head.txt", "worked_two_seq_two_head.txt"):
        g = load_golden(name)
        start = 0
        for s, L in enumerate(g["seq_lens"]):
            sl = slice(start, start + L)
            y, hT = m.ssd_steps(g["x"][sl, None], g["dt"][sl, None], g["A"],
                                g["B"][sl, None], g["C"][sl, None], g["D"],
                                g["h0"][s:s + 1])
            assert np.allclose(y[:, 0], g["y"][sl], rtol=0, atol=1e-12), (name, s)
            assert np.allclose(hT[0], g["h_final"][s], rtol=0, atol=1e-12), (name, s)
            start += L


def pin_step_matches_sequence_oracle(m):
    """T steps from h0 equal the C recurrence over T tokens, per sequence,
    with 2 and 3 heads per group."""
    rng = np.random.default_rng(11)
    for batch, H, P, N, G, T in ((3, 4, 3, 5, 2, 9), (2, 6, 2, 4, 2, 5), (1, 3, 4, 3, 1, 12)):
        c = _case(rng, batch, H, P, N, G, T=T)
        y, hT = m.ssd_steps(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["h0"])
        # the same tokens as a packed stream of `batch` sequences of length T
        flat = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1)).reshape((-1,) + a.shape[2:])
        yr, hr = oracle.ssd_recurrence(flat(c["x"]), flat(c["dt"]), c["A"], flat(c["B"]),
                                       flat(c["C"]), c["D"], c["h0"], [T] * batch)
        assert rel_err(flat(y), yr) < 1e-12, ("y", batch, H, G)
        assert rel_err(hT, hr) < 1e-12, ("state", batch, H, G)


def pin_step_closed_form_constant(m):
    """Constant dt, x, B, C per (sequence, head): after k steps from h0,
    h = a^k h0 + dt x b^T (1 - a^k) / (1 - a), a = exp(dt A); y = h c + D x."""
    rng = np.random.default_rng(5)
    batch, H, P, N, T = 2, 3, 4, 5, 30
    A = np.array([-0.5, -2.0, -0.05])
    delta = np.array([[0.3, 0.1, 1.5], [0.02, 0.7, 0.2]])
    xi = rng.standard_normal((batch, H, P))
    b = rng.standard_normal((batch, 1, N))
    c = rng.standard_normal((batch, 1, N))
    D = np.array([0.5, -1.0, 2.0])
    h0 = rng.standard_normal((batch, H, P, N))
    rep = lambda v: np.broadcast_to(v, (T,) + v.shape)
    y, hT = m.ssd_steps(rep(xi), rep(delta), A, rep(b), rep(c), D, h0)
    a = np.exp(delta * A[None, :])                          # (batch, H)
    for k in (1, 2, 17, T):
        ak = a ** k
        hk = (ak[..., None, None] * h0 + (delta[..., None] * xi)[..., None] * b[:, :, None, :]
              * ((1 - ak) / (1 - a))[..., None, None])
        yk = np.einsum("bhpn,bn->bhp", hk, c[:, 0]) + D[None, :, None] * xi
        assert rel_err(y[k - 1], yk) < 1e-12, ("closed form y", k)
        if k == T:
            assert rel_err(hT, hk) < 1e-12, "closed form state"


def pin_step_a_zero_running_sum(m):
    """A = 0: the state is h0 plus the running sum of dt x B^T (linear
    attention), here accumulated with numpy's cumsum."""
    rng = np.random.default_rng(6)
    batch, H, P, N, G, T = 2, 4, 3, 2, 2, 8
    c = _case(rng, batch, H, P, N, G, T=T)
    A = np.zeros(H)
    y, hT = m.ssd_steps(c["x"], c["dt"], A, c["B"], c["C"], c["D"], c["h0"])
    grp = np.repeat(np.arange(G), H // G)
    terms = (c["dt"][..., None, None] * c["x"][..., None]) * c["B"][:, :, grp, None, :]
    states = c["h0"][None] + np.cumsum(terms, axis=0)     # (T, batch, H, P, N)
    yy = np.einsum("tbhpn,tbhn->tbhp", states, c["C"][:, :, grp, :]) + c["D"][None, None, :, None] * c["x"]
    assert rel_err(y, yy) < 1e-12, "A=0 y"
    assert rel_err(hT, states[-1]) < 1e-12, "A=0 state"


def pin_step_reset_limit(m):
    """dt*A -> -inf: the old state is forgotten; state = dt x B^T and
    y = dt (C.B) x + D x."""
    rng = np.random.default_rng(8)
    batch, H, P, N, G = 3, 2, 4, 3, 1
    c = _case(rng, batch, H, P, N, G)
    A = np.full(H, -1.0e4)
    dt = 0.05 + rng.uniform(size=(batch, H))
    y, h = m.ssd_step(c["x"][0], dt, A, c["B"][0], c["C"][0], c["D"], c["h0"])
    cb = np.sum(c["C"][0, :, 0] * c["B"][0, :, 0], axis=-1)          # (batch,)
    assert rel_err(y, dt[..., None] * cb[:, None, None] * c["x"][0]
                   + c["D"][None, :, None] * c["x"][0]) < 1e-12, "reset y"
    assert rel_err(h, dt[..., None, None] * c["x"][0][..., None]
                   * c["B"][0][:, :, None, :]) < 1e-12, "reset state"


def pin_step_freeze_limit(m):
    """dt = 0: the state is kept exactly and the input ignored; y = C h + D x."""
    rng = np.random.default_rng(9)
    batch, H, P, N, G = 2, 4, 2, 5, 4
    c = _case(rng, batch, H, P, N, G)
    dt = np.zeros((batch, H))
    y, h = m.ssd_step(c["x"][0], dt, c["A"], c["B"][0], c["C"][0], c["D"], c["h0"])
    assert np.array_equal(h, c["h0"]), "freeze state"
    assert rel_err(y, np.einsum("bhpn,bhn->bhp", c["h0"], c["C"][0])
                   + c["D"][None, :, None] * c["x"][0]) < 1e-12, "freeze y"


def pin_step_linearity(m):
    """y and the new state are linear in (x, state) jointly."""
    rng = np.random.default_rng(10)
    c = _case(rng, 2, 4, 3, 4, 2)
    y1, h1 = m.ssd_step(c["x"][0], c["dt"][0], c["A"], c["B"][0], c["C"][0], c["D"], c["h0"])
    y2, h2 = m.ssd_step(-2.5 * c["x"][0], c["dt"][0], c["A"], c["B"][0], c["C"][0], c["D"],
                        -2.5 * c["h0"])
    assert rel_err(y2, -2.5 * y1) < 1e-13 and rel_err(h2, -2.5 * h1) < 1e-13, "linearity"


ALL_STEP_PINS = [(f.__name__, f) for f in (
    pin_step_golden, pin_step_matches_sequence_oracle, pin_step_closed_form_constant,
    pin_step_a_zero_running_sum, pin_step_reset_limit, pin_step_freeze_limit,
    pin_step_linearity)]
