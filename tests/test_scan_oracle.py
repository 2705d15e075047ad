"""The selective-scan oracle against its pins, and planted mistakes in copies
of it (on the CPU) that the pins must catch."""
import importlib.util
import os
import warnings

import pytest

import oracle.selective_scan as scan_oracle
from scan_pins import ALL_SCAN_PINS

SRC = scan_oracle.__file__


@pytest.mark.parametrize("name,pin", ALL_SCAN_PINS, ids=[n for n, _ in ALL_SCAN_PINS])
def test_scan_oracle_pin(name, pin):
    pin(scan_oracle)


MUTANTS = {
    "add_then_decay": [(
        "h = decay * h + (step * x[:, t, :])[:, :, None] * B[:, t, None, :]",
        "h = decay * (h + (step * x[:, t, :])[:, :, None] * B[:, t, None, :])")],
    "output_from_old_state": [(
        "        h = decay * h + (step * x[:, t, :])[:, :, None] * B[:, t, None, :]\n"
        "        y[:, t, :] = np.einsum(\"bdn,bn->bd\", h, C[:, t, :])",
        "        y[:, t, :] = np.einsum(\"bdn,bn->bd\", h, C[:, t, :])\n"
        "        h = decay * h + (step * x[:, t, :])[:, :, None] * B[:, t, None, :]")],
    "decay_of_state_0": [("np.exp(step[:, :, None] * A[None, :, :])",
                          "np.exp(step[:, :, None] * A[None, :, :1])")],
    "decay_of_channel_0": [("np.exp(step[:, :, None] * A[None, :, :])",
                            "np.exp(step[:, :, None] * A[None, :1, :])")],
    "sign_of_A": [("np.exp(step[:, :, None] * A[None, :, :])",
                   "np.exp(-step[:, :, None] * A[None, :, :])")],
    "zoh_input_factor": [("(step * x[:, t, :])[:, :, None] * B[:, t, None, :]",
                          "((decay - 1) / np.where(A == 0, -1.0, A)[None]) * x[:, t, :, None]"
                          " * B[:, t, None, :]")],
    "swap_B_C": [("* B[:, t, None, :]", "* C[:, t, None, :]"),
                 ('np.einsum("bdn,bn->bd", h, C[:, t, :])', 'np.einsum("bdn,bn->bd", h, B[:, t, :])')],
    "drop_D": [("y[:, t, :] += D[None, :] * x[:, t, :]", "pass")],
    "step_of_previous_token": [("step = delta[:, t, :]", "step = delta[:, max(t - 1, 0), :]")],
    "ignore_initial_state": [("h = np.zeros((batch, Dm, N)) if h0 is None else h0.copy()",
                              "h = np.zeros((batch, Dm, N))")],
    "C_of_next_token": [('np.einsum("bdn,bn->bd", h, C[:, t, :])',
                         'np.einsum("bdn,bn->bd", h, C[:, min(t + 1, L - 1), :])')],
    "step_squared": [("(step * x[:, t, :])", "(step * step * x[:, t, :])")],
}


def _load_mutant(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, ("mutation anchor not unique/found", name, old)
        src = src.replace(old, new)
    path = os.path.join(str(tmp_path), "scan_%s.py" % name)
    with open(path, "w") as f:
        f.write(src)
    spec = importlib.util.spec_from_file_location("scan_%s" % name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_scan_mutant_is_caught(name, tmp_path):
    m = _load_mutant(name, tmp_path)
    caught = []
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for pin_name, pin in ALL_SCAN_PINS:
            try:
                pin(m)
            except (AssertionError, FloatingPointError):
                caught.append(pin_name)
    assert caught, "mutant %s passed every pin" % name
