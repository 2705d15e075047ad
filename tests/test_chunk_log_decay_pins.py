"""Pins of ``oracle.chunk_log_decay``, the per-chunk log-decay prefix the GPU
path's cumsum step is checked against (CPU only).

The decay of one step is exp(dt_t * A_h) (tj-hxxt.cn long read of the Mamba-1
paper, part III (二) and item 3 on the step size), so the decay from a
chunk's start through token l is the product of those factors, whose natural
log is the inclusive sum of dt * A over the chunk's tokens up to l. Chunks
restart at every sequence start (same page, item 2.3 "Boundary Resetting").

Each pin is fixed by something other than the function's own formula:
  * hand values: the worked fixtures under tests/golden/ use A = -ln 2, so
    the prefix is -ln 2 times the running sum of the steps, worked out in the
    comments below;
  * the state ratio: with no input (x = 0) the recurrence only decays its
    state, so the C recurrence (pinned on its own in test_oracle_pins.py),
    snapshotted before every token, gives exp(prefix) as the ratio of two
    snapshots;
  * closed forms: constant dt gives dt * A * (l + 1); A = 0 gives zeros.
Plausible mistakes (exclusive prefix, log base 2, no restart at a chunk or a
sequence start, dt of the wrong head, no NaN past a partial chunk) are planted
in copies below and each must be caught.
"""
import math

import numpy as np
import pytest

import oracle
from oracle_pins import load_golden

LN2 = math.log(2.0)


def pin_hand_single(f):
    # worked_single_head.txt: dt = 1, 1, 2 and A = -ln 2, one sequence of 3.
    # Q = 2: chunk 0 holds tokens 0, 1 -> -ln2 * (1, 1 + 1) = (-ln2, -2 ln2);
    #        chunk 1 holds token 2     -> -ln2 * 2 = -2 ln2, then past its end.
    g = load_golden("worked_single_head.txt")
    cs = f(g["dt"], g["A"], g["seq_lens"], 2)
    assert cs.shape == (2, 1, 2), cs.shape
    assert np.allclose(cs[0, 0], [-LN2, -2 * LN2], rtol=0, atol=1e-15), cs[0, 0]
    assert abs(cs[1, 0, 0] + 2 * LN2) < 1e-15, cs[1, 0]
    assert np.isnan(cs[1, 0, 1]), cs[1, 0]


def pin_hand_two_seq(f):
    # worked_two_seq_two_head.txt: sequences of 2 and 1 tokens; head 0 has
    # A = -ln 2, head 1 has A = 0. Steps per token (head 0, head 1):
    # t0 (1, 1), t1 (1, 2), t2 (2, 1).
    # Q = 4: sequence 0 is one chunk: head 0 -> (-ln2, -2 ln2), head 1 -> 0;
    #        sequence 1 restarts: head 0 -> (-2 ln2), head 1 -> 0.
    g = load_golden("worked_two_seq_two_head.txt")
    cs = f(g["dt"], g["A"], g["seq_lens"], 4)
    assert cs.shape == (2, 2, 4), cs.shape
    assert np.allclose(cs[0, 0, :2], [-LN2, -2 * LN2], rtol=0, atol=1e-15), cs[0, 0]
    assert np.array_equal(cs[0, 1, :2], [0.0, 0.0]), cs[0, 1]
    assert abs(cs[1, 0, 0] + 2 * LN2) < 1e-15 and cs[1, 1, 0] == 0.0, cs[1]
    assert np.isnan(cs[0, :, 2:]).all() and np.isnan(cs[1, :, 1:]).all()
    # Q = 1: every token is its own chunk; the prefix is that token's dt * A
    cs1 = f(g["dt"], g["A"], g["seq_lens"], 1)
    assert np.allclose(cs1[:, 0, 0], [-LN2, -LN2, -2 * LN2], rtol=0, atol=1e-15), cs1[:, 0]
    assert np.array_equal(cs1[:, 1, 0], [0.0, 0.0, 0.0])


def pin_state_ratio(f):
    """x = 0 and a positive initial state: the state only decays, so the
    ratio of the recurrence's snapshots (taken before every token) between a
    chunk's start and just after token l is exp(prefix[l])."""
    rng = np.random.default_rng(5)
    lens = [13, 0, 5, 16, 1]
    T, H, P, N, Q = sum(lens), 3, 1, 1, 4
    dt = np.logaddexp(0.0, rng.standard_normal((T, H)) - 1.0)
    A = -np.exp(rng.uniform(0.0, 2.0, size=H))
    h0 = np.full((len(lens), H, P, N), 1.0)
    _, hT, snaps = oracle.ssd_recurrence(
        np.zeros((T, H, P)), dt, A, rng.standard_normal((T, 1, N)),
        rng.standard_normal((T, 1, N)), None, h0, lens, snap_every=1)
    # snapshot i of a sequence = state before its token i; the state after the
    # sequence's last token is its final state
    after, k = [], 0
    for s, L in enumerate(lens):
        seq = [snaps[k + i, :, 0, 0] for i in range(L)] + [hT[s, :, 0, 0]]
        after.append(np.array(seq))
        k += L
    cs = f(dt, A, lens, Q)
    c = 0
    for s, L in enumerate(lens):
        for c0 in range(0, L, Q):
            n = min(Q, L - c0)
            want = np.log(after[s][c0 + 1:c0 + n + 1] / after[s][c0][None, :])  # (n, H)
            assert np.allclose(cs[c, :, :n].T, want, rtol=1e-12, atol=1e-12), (s, c0)
            assert np.isnan(cs[c, :, n:]).all()
            c += 1
    assert c == cs.shape[0]


def pin_closed_forms(f):
    T, H, Q = 20, 2, 8
    dt = np.tile(np.array([0.3, 0.05]), (T, 1))
    A = np.array([-1.7, -0.4])
    cs = f(dt, A, [T], Q)
    for c in range(3):
        n = min(Q, T - c * Q)
        for h in range(H):
            want = dt[0, h] * A[h] * np.arange(1, n + 1)
            assert np.allclose(cs[c, h, :n], want, rtol=1e-14, atol=1e-15), (c, h)
    z = f(dt, np.zeros(H), [7, 13], Q)
    assert np.array_equal(z[np.isfinite(z)], np.zeros(np.isfinite(z).sum()))
    assert np.isfinite(z).sum() == 20 * H


PINS = [("hand_single", pin_hand_single), ("hand_two_seq", pin_hand_two_seq),
        ("state_ratio", pin_state_ratio), ("closed_forms", pin_closed_forms)]


@pytest.mark.parametrize("name,pin", PINS, ids=[n for n, _ in PINS])
def test_pin(name, pin):
    pin(oracle.chunk_log_decay)


# ---- planted mistakes: each must fail at least one pin -----------------------
def _mutant(kind):
    def f(dt, A, seq_lens, Q):
        dt = np.asarray(dt, np.float64)
        A = np.asarray(A, np.float64)
        T, H = dt.shape
        starts, lens = oracle.seq_layout(T, seq_lens)
        if kind == "no_sequence_restart":      # chunks cut from the packed stream
            starts, lens = np.array([0]), np.array([T])
        out = []
        carry = np.zeros(H)
        for a, L in zip(starts, lens):
            for c0 in range(0, int(L), Q):
                n = min(Q, int(L) - c0)
                v = dt[a + c0:a + c0 + n] * (A[None, :] if kind != "head_0_A" else A[0])
                if kind == "exclusive":
                    s = np.cumsum(v, axis=0) - v
                elif kind == "log2":
                    s = np.cumsum(v, axis=0) / LN2
                elif kind == "no_chunk_restart":
                    s = np.cumsum(v, axis=0) + carry
                    carry = s[-1]
                else:
                    s = np.cumsum(v, axis=0)
                block = np.full((H, Q), 0.0 if kind == "zero_past_end" else np.nan)
                block[:, :n] = s.T
                out.append(block)
            carry = np.zeros(H)
        return np.stack(out) if out else np.zeros((0, H, Q))
    return f


@pytest.mark.parametrize("kind", ["exclusive", "log2", "no_chunk_restart", "no_sequence_restart",
                                  "head_0_A", "zero_past_end"])
def test_mutant_is_caught(kind):
    caught = []
    for name, pin in PINS:
        try:
            pin(_mutant(kind))
        except (AssertionError, ValueError, IndexError):
            caught.append(name)
    assert caught, "mutant %s passed every pin" % kind


def test_unmutated_copy_passes():
    """The mutant generator with no mistake passes every pin (so the pins
    reject the mistakes, not the generator)."""
    for _, pin in PINS:
        pin(_mutant("none"))
