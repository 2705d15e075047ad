"""The decode-step oracle against its pins, and planted mistakes in copies of
it (on the CPU) that the pins must catch."""
import importlib.util
import os

import pytest

import oracle.step as step_oracle
from step_pins import ALL_STEP_PINS

SRC = step_oracle.__file__


@pytest.mark.parametrize("name,pin", ALL_STEP_PINS, ids=[n for n, _ in ALL_STEP_PINS])
def test_step_oracle_pin(name, pin):
    pin(step_oracle)


MUTANTS = {
    "add_then_decay": [(
        "new_state = (a[:, :, None, None] * state\n"
        "                 + (dt[:, :, None] * x)[:, :, :, None] * Bh[:, :, None, :])",
        "new_state = a[:, :, None, None] * (state\n"
        "                 + (dt[:, :, None] * x)[:, :, :, None] * Bh[:, :, None, :])")],
    "output_from_old_state": [('np.einsum("bhpn,bhn->bhp", new_state, Ch)',
                               'np.einsum("bhpn,bhn->bhp", state, Ch)')],
    "zoh_input_factor": [("(dt[:, :, None] * x)[:, :, :, None]",
                          "(np.where(A[None, :] != 0, (a - 1) / np.where(A == 0, 1, A)[None, :],"
                          " dt)[:, :, None] * x)[:, :, :, None]")],
    "interleaved_groups": [("group = np.arange(H) // (H // G)", "group = np.arange(H) % G")],
    "drop_D": [("y = y + D[None, :, None] * x", "y = y")],
    "sign_of_A": [("a = np.exp(dt * A[None, :])", "a = np.exp(-dt * A[None, :])")],
    "swap_B_C": [("Bh = B[:, group, :]", "Bh = C[:, group, :]"),
                 ("Ch = C[:, group, :]", "Ch = B[:, group, :]")],
    "dt_squared": [("(dt[:, :, None] * x)", "(dt[:, :, None] ** 2 * x)")],
    "state_not_decayed": [("a[:, :, None, None] * state", "state")],
    "state_dropped": [("a[:, :, None, None] * state", "0.0 * state")],
    "decay_of_head_0": [("a = np.exp(dt * A[None, :])", "a = np.exp(dt * A[None, :1])")],
    "x_of_head_0_in_output": [("y = y + D[None, :, None] * x", "y = y + D[None, :, None] * x[:, :1]")],
}


def _load_mutant(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, ("mutation anchor not unique/found", name, old)
        src = src.replace(old, new)
    path = os.path.join(str(tmp_path), "step_%s.py" % name)
    with open(path, "w") as f:
        f.write(src)
    spec = importlib.util.spec_from_file_location("step_%s" % name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_step_mutant_is_caught(name, tmp_path):
    m = _load_mutant(name, tmp_path)
    caught = []
    for pin_name, pin in ALL_STEP_PINS:
        try:
            pin(m)
        except (AssertionError, ValueError):
            caught.append(pin_name)
    assert caught, "mutant %s passed every pin" % name
