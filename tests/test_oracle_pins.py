"""The oracle pinned to facts fixed outside itself (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle.dense import ssd_dense
from oracle_pins import ALL_PINS, load_golden, random_case, rel_err


@pytest.mark.parametrize("name,pin", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_pin(name, pin):
    pin(None)


@pytest.mark.parametrize("fixture", ["worked_single_head.txt",
                                     "worked_two_seq_two_head.txt"])
def test_dense_form_matches_golden(fixture):
    g = load_golden(fixture)
    y, hT = ssd_dense(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"],
                      g["seq_lens"])
    assert np.allclose(y, g["y"], atol=1e-12)
    assert np.allclose(hT, g["h_final"], atol=1e-12)


def test_linearity_in_x_and_h0():
    rng = np.random.default_rng(31)
    c = random_case(rng, [33, 12], H=3, P=2, N=3, G=1)
    y, hT = oracle.ssd_recurrence(c["x"], c["dt"], c["A"], c["B"], c["C"],
                                  c["D"], c["h0"], c["seq_lens"])
    y2, h2 = oracle.ssd_recurrence(2.5 * c["x"], c["dt"], c["A"], c["B"], c["C"],
                                   c["D"], 2.5 * c["h0"], c["seq_lens"])
    assert rel_err(y2, 2.5 * y) < 1e-13 and rel_err(h2, 2.5 * hT) < 1e-13


def test_head_permutation_equivariance():
    rng = np.random.default_rng(37)
    c = random_case(rng, [29], H=4, P=2, N=3, G=1)
    perm = np.array([2, 0, 3, 1])
    y, hT = oracle.ssd_recurrence(c["x"], c["dt"], c["A"], c["B"], c["C"],
                                  c["D"], c["h0"], c["seq_lens"])
    yp, hp = oracle.ssd_recurrence(c["x"][:, perm], c["dt"][:, perm],
                                   c["A"][perm], c["B"], c["C"], c["D"][perm],
                                   c["h0"][:, perm], c["seq_lens"])
    assert rel_err(yp, y[:, perm]) < 1e-14 and rel_err(hp, hT[:, perm]) < 1e-14


def test_group_map_is_contiguous():
    """H = 4 heads on G = 2 groups: heads 0,1 read group 0, heads 2,3 group 1
    (reading of the multi-input SSM). Equivalent to G = H with each head's
    group copied out."""
    rng = np.random.default_rng(41)
    c = random_case(rng, [26], H=4, P=2, N=3, G=2)
    y, hT = oracle.ssd_recurrence(c["x"], c["dt"], c["A"], c["B"], c["C"],
                                  c["D"], c["h0"], c["seq_lens"])
    idx = np.array([0, 0, 1, 1])
    ye, he = oracle.ssd_recurrence(c["x"], c["dt"], c["A"], c["B"][:, idx],
                                   c["C"][:, idx], c["D"], c["h0"], c["seq_lens"])
    assert rel_err(y, ye) < 1e-15 and rel_err(hT, he) < 1e-15


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(43)
    c = random_case(rng, [0, 5, 0], H=2, P=2, N=2, G=1)
    y, hT = oracle.ssd_recurrence(c["x"], c["dt"], c["A"], c["B"], c["C"],
                                  c["D"], c["h0"], c["seq_lens"])
    assert np.array_equal(hT[0], c["h0"][0]) and np.array_equal(hT[2], c["h0"][2])


def test_sampled_pairs_equal_full_run():
    rng = np.random.default_rng(47)
    c = random_case(rng, [19, 7, 30], H=4, P=3, N=2, G=2)
    y, hT = oracle.ssd_recurrence(c["x"], c["dt"], c["A"], c["B"], c["C"],
                                  c["D"], c["h0"], c["seq_lens"])
    starts = np.concatenate([[0], np.cumsum(c["seq_lens"])])
    got = oracle.ssd_pairs(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"],
                           c["h0"], c["seq_lens"], [(0, 3), (2, 1), (1, 2)])
    for (s, h), (ys, hs) in got.items():
        assert np.array_equal(ys, y[starts[s]:starts[s + 1], h])
        assert np.array_equal(hs, hT[s, h])
