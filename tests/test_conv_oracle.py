"""The convolution-front oracle against its pins, and planted mistakes in
copies of it (on the CPU) that the pins must catch."""
import importlib.util
import os
import warnings

import pytest

import oracle.conv as conv_oracle
from conv_pins import ALL_CONV_PINS

SRC = conv_oracle.__file__


@pytest.mark.parametrize("name,pin", ALL_CONV_PINS, ids=[n for n, _ in ALL_CONV_PINS])
def test_conv_oracle_pin(name, pin):
    pin(conv_oracle)


MUTANTS = {
    "taps_not_reversed": [("pre = pre + weight[None, :, k] * e[k:k + L]",
                           "pre = pre + weight[None, :, K - 1 - k] * e[k:k + L]")],
    "drop_bias": [("pre = np.zeros((L, ch)) if bias is None else np.repeat(bias[None, :], L, axis=0)",
                   "pre = np.zeros((L, ch))")],
    "sees_next_token": [("e = np.concatenate([history, u], axis=0)",
                         "e = np.concatenate([history[1:], u, u[-1:]], axis=0)")],
    "one_tap_short": [("for k in range(K):", "for k in range(1, K):")],
    "sigmoid_not_silu": [("return v / (1.0 + np.exp(-v))", "return 1.0 / (1.0 + np.exp(-v))")],
    "history_ignored": [("if history is None:\n        history = np.zeros((K - 1, ch))",
                         "history = np.zeros((K - 1, ch))")],
    "history_newest_first": [("e = np.concatenate([history, u], axis=0)",
                              "e = np.concatenate([history[::-1], u], axis=0)")],
    "history_from_outputs": [("return out, e[len(e) - (K - 1):].copy()",
                              "return out, np.concatenate([history, out])[len(e) - (K - 1):].copy()")],
    "B_C_swapped": [("return (out[:, :x_dim], out[:, x_dim:x_dim + bc_dim], out[:, x_dim + bc_dim:], hist_out)",
                     "return (out[:, :x_dim], out[:, x_dim + bc_dim:], out[:, x_dim:x_dim + bc_dim], hist_out)")],
    "sequences_not_reset": [("o, h = m_causal(xbc[a:b], weight, bias,", None)],
    "no_activation_anywhere": [("out = silu(pre) if activation else pre", "out = pre")],
}
# packed sequences run as one stream: the second sequence starts from the first's tail
MUTANTS["sequences_not_reset"] = [(
    "        o, h = causal_conv(xbc[a:b], weight, bias,\n"
    "                           None if history is None else history[s], activation)",
    "        o, h = causal_conv(xbc[a:b], weight, bias,\n"
    "                           (None if history is None else history[s]) if s == 0 or a < K - 1\n"
    "                           else xbc[a - (K - 1):a], activation)")]


def _load_mutant(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, ("mutation anchor not unique/found", name, old)
        src = src.replace(old, new)
    path = os.path.join(str(tmp_path), "conv_%s.py" % name)
    with open(path, "w") as f:
        f.write(src)
    spec = importlib.util.spec_from_file_location("conv_%s" % name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_conv_mutant_is_caught(name, tmp_path):
    m = _load_mutant(name, tmp_path)
    caught = []
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for pin_name, pin in ALL_CONV_PINS:
            try:
                pin(m)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(pin_name)
    assert caught, "mutant %s passed every pin" % name
