"""Checks that pin the fp64 oracle to facts fixed outside itself.

Each ``pin_*`` function runs the oracle (optionally a given build of it) and
raises AssertionError when the oracle disagrees with:
  * the hand-worked examples under tests/golden/ (values derived by hand in
    the fixture's comments),
  * the dense quadratic form (a second formulation: the semiseparable-matrix
    view of the QbitAI "Mamba-2" article, section "Unifying SSM and
    attention"),
  * closed forms: constant inputs (geometric series), A = 0 (prefix sum /
    linear attention), the reset limit dt*A -> -inf and the freeze limit
    dt -> 0 (tj-hxxt.cn long read of the Mamba-1 paper, part III item 3 on
    the step size: a tiny step keeps the state and ignores the input, a huge
    one resets the state to the current input),
  * structural facts: chunk snapshots equal prefix runs, split-and-continue.
The same functions run against mutated oracle builds in
test_oracle_mutants.py, where each must be caught by at least one pin.
"""
from __future__ import annotations

import os

import numpy as np

import oracle
from oracle.dense import ssd_dense

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            vals[key] = [float(v) for v in rest]
    T, H, P, N, G = (int(vals[k][0]) for k in ("T", "H", "P", "N", "G"))
    S = len(vals["seq_lens"])
    return dict(
        x=np.array(vals["x"]).reshape(T, H, P),
        dt=np.array(vals["dt"]).reshape(T, H),
        A=np.array(vals["A"]), D=np.array(vals["D"]),
        B=np.array(vals["B"]).reshape(T, G, N),
        C=np.array(vals["C"]).reshape(T, G, N),
        h0=np.array(vals["h0"]).reshape(S, H, P, N),
        seq_lens=[int(v) for v in vals["seq_lens"]],
        y=np.array(vals["y"]).reshape(T, H, P),
        h_final=np.array(vals["h_final"]).reshape(S, H, P, N))


def rel_err(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(float(np.max(np.abs(b))), 1e-300) if b.size else 1.0
    return float(np.max(np.abs(a - b))) / scale if a.size else 0.0


def random_case(rng, T_lens, H, P, N, G, with_h0=True, with_D=True,
                log_neg_a=(0.0, 2.0)):
    T = int(sum(T_lens))
    S = len(T_lens)
    return dict(
        x=rng.standard_normal((T, H, P)),
        dt=np.logaddexp(0.0, rng.standard_normal((T, H)) - 1.0),
        A=-np.exp(rng.uniform(*log_neg_a, size=H)),
        B=rng.standard_normal((T, G, N)),
        C=rng.standard_normal((T, G, N)),
        D=rng.standard_normal(H) if with_D else None,
        h0=rng.standard_normal((S, H, P, N)) if with_h0 else None,
        seq_lens=list(T_lens))


def _run(case, lib=None, **kw):
    return oracle.ssd_recurrence(case["x"], case["dt"], case["A"], case["B"],
                                 case["C"], case.get("D"), case.get("h0"),
                                 case.get("seq_lens"), lib=lib, **kw)


def pin_golden(name: str, lib=None):
    g = load_golden(name)
    y, hT = _run(g, lib)
    assert np.allclose(y, g["y"], rtol=0, atol=1e-12), (name, y, g["y"])
    assert np.allclose(hT, g["h_final"], rtol=0, atol=1e-12), (name, hT)


def pin_dense(lib=None, seed=0):
    rng = np.random.default_rng(seed)
    cases = [
        random_case(rng, [37], H=1, P=3, N=4, G=1),
        random_case(rng, [50], H=4, P=2, N=5, G=2),                 # 2 heads/group
        random_case(rng, [5, 0, 17, 1, 9], H=4, P=3, N=2, G=2),    # varlen incl. empty
        random_case(rng, [64, 31], H=6, P=4, N=3, G=3, with_D=False),
        random_case(rng, [40], H=2, P=2, N=3, G=1, with_h0=False),
    ]
    for i, c in enumerate(cases):
        y, hT = _run(c, lib)
        yd, hd = ssd_dense(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"],
                           c["h0"], c["seq_lens"])
        assert rel_err(y, yd) < 1e-12, ("dense y", i, rel_err(y, yd))
        assert rel_err(hT, hd) < 1e-12, ("dense h", i, rel_err(hT, hd))


def pin_closed_form_constant(lib=None):
    """Constant dt, B, C, x: h_t = a^(t+1) h0 + dt x b^T (1 - a^(t+1)) / (1 - a)."""
    T, H, P, N = 40, 2, 3, 4
    rng = np.random.default_rng(7)
    delta = np.array([0.3, 0.05])
    A = np.array([-1.7, -0.4])
    b = rng.standard_normal(N)
    c = rng.standard_normal(N)
    xi = rng.standard_normal((H, P))
    D = np.array([0.25, -1.5])
    h0 = rng.standard_normal((1, H, P, N))
    case = dict(x=np.broadcast_to(xi, (T, H, P)).copy(),
                dt=np.broadcast_to(delta, (T, H)).copy(), A=A,
                B=np.broadcast_to(b, (T, 1, N)).copy(),
                C=np.broadcast_to(c, (T, 1, N)).copy(), D=D, h0=h0,
                seq_lens=[T])
    y, hT = _run(case, lib)
    for h in range(H):
        a = np.exp(delta[h] * A[h])
        for t in range(T):
            k = t + 1
            ht = a ** k * h0[0, h] + delta[h] * np.outer(xi[h], b) * (1 - a ** k) / (1 - a)
            want = ht @ c + D[h] * xi[h]
            assert np.allclose(y[t, h], want, rtol=1e-12, atol=1e-12), (t, h)
        assert np.allclose(hT[0, h], ht, rtol=1e-12, atol=1e-12)


def pin_a_zero_prefix_sum(lib=None):
    """A = 0: y_t = C_t . (h0 + sum_{s<=t} dt_s x_s B_s^T) + D x_t (linear attention)."""
    rng = np.random.default_rng(11)
    c = random_case(rng, [30], H=3, P=2, N=3, G=1)
    c["A"] = np.zeros(3)
    y, hT = _run(c, lib)
    outer = np.einsum("th,thp,tn->thpn", c["dt"], c["x"], c["B"][:, 0, :])
    states = np.cumsum(outer, axis=0) + c["h0"][0][None]
    want = np.einsum("thpn,tn->thp", states, c["C"][:, 0, :]) + c["D"][None, :, None] * c["x"]
    assert rel_err(y, want) < 1e-12
    assert rel_err(hT[0], states[-1]) < 1e-12


def pin_reset_limit(lib=None):
    """dt*A -> -inf: each step forgets everything, y_t = dt_t (C_t.B_t) x_t + D x_t."""
    rng = np.random.default_rng(13)
    c = random_case(rng, [25], H=2, P=3, N=4, G=1)
    c["A"] = np.array([-1e6, -3e6])
    y, hT = _run(c, lib)
    cb = np.einsum("tn,tn->t", c["C"][:, 0], c["B"][:, 0])
    want = (c["dt"] * cb[:, None])[:, :, None] * c["x"] + c["D"][None, :, None] * c["x"]
    assert rel_err(y, want) < 1e-12
    last = np.einsum("h,hp,n->hpn", c["dt"][-1], c["x"][-1], c["B"][-1, 0])
    assert rel_err(hT[0], last) < 1e-12


def pin_freeze_limit(lib=None):
    """dt -> 0: the state is kept and the input ignored, y_t = C_t . h0 + D x_t."""
    rng = np.random.default_rng(17)
    c = random_case(rng, [20], H=2, P=2, N=3, G=1)
    c["dt"] = np.full_like(c["dt"], 1e-13)
    y, hT = _run(c, lib)
    want = np.einsum("hpn,tn->thp", c["h0"][0], c["C"][:, 0]) + c["D"][None, :, None] * c["x"]
    assert rel_err(y, want) < 1e-9
    assert rel_err(hT, c["h0"]) < 1e-9


def pin_snapshots_are_prefix_states(lib=None, Q=8):
    """The snapshot before chunk k is the final state of the first k*Q tokens,
    which the dense form gives in closed form."""
    rng = np.random.default_rng(19)
    c = random_case(rng, [21, 16, 3], H=2, P=2, N=3, G=1)
    y, hT, snaps = _run(c, lib, snap_every=Q)
    start = 0
    idx = 0
    for s, L in enumerate(c["seq_lens"]):
        for k in range((L + Q - 1) // Q):
            sl = slice(start, start + k * Q)
            _, hd = ssd_dense(c["x"][sl], c["dt"][sl], c["A"], c["B"][sl],
                              c["C"][sl], None, c["h0"][s:s + 1], [k * Q])
            assert rel_err(snaps[idx], hd[0]) < 1e-12, (s, k)
            idx += 1
        start += L
    assert idx == snaps.shape[0]


def pin_split_continuity(lib=None):
    """Running [0, t) then [t, L) with final -> initial equals one run."""
    rng = np.random.default_rng(23)
    c = random_case(rng, [45], H=2, P=3, N=2, G=1)
    y, hT = _run(c, lib)
    for cut in (1, 17, 44):
        a = {k: (v[:cut] if k in ("x", "dt", "B", "C") else v) for k, v in c.items()}
        a["seq_lens"] = [cut]
        b = {k: (v[cut:] if k in ("x", "dt", "B", "C") else v) for k, v in c.items()}
        b["seq_lens"] = [45 - cut]
        ya, ha = _run(a, lib)
        b["h0"] = ha
        yb, hb = _run(b, lib)
        assert rel_err(np.concatenate([ya, yb]), y) < 1e-13
        assert rel_err(hb, hT) < 1e-13


ALL_PINS = [
    ("golden_single", lambda lib: pin_golden("worked_single_head.txt", lib)),
    ("golden_two_seq", lambda lib: pin_golden("worked_two_seq_two_head.txt", lib)),
    ("dense", pin_dense),
    ("closed_form", pin_closed_form_constant),
    ("a_zero", pin_a_zero_prefix_sum),
    ("reset", pin_reset_limit),
    ("freeze", pin_freeze_limit),
    ("snapshots", pin_snapshots_are_prefix_states),
    ("split", pin_split_continuity),
]
