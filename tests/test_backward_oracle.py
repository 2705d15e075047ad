"""The backward oracle against its pins, and planted mistakes in copies of it
(on the CPU) that the pins must catch."""
import importlib.util
import os
import warnings

import pytest

import oracle.backward as bwd_oracle
from backward_pins import ALL_BWD_PINS

SRC = bwd_oracle.__file__


@pytest.mark.parametrize("name,pin", ALL_BWD_PINS, ids=[n for n, _ in ALL_BWD_PINS])
def test_backward_oracle_pin(name, pin):
    pin(bwd_oracle)


MUTANTS = {
    "adjoint_not_decayed": [("            Gs = a[:, None, None] * Gs\n", "")],
    "output_grad_after_use": [(
        "            Gs += dy[t][:, :, None] * Ch[:, None, :]\n", ""),
        ("            Gs = a[:, None, None] * Gs\n",
         "            Gs = a[:, None, None] * Gs\n            Gs += dy[t][:, :, None] * Ch[:, None, :]\n")],
    "dC_from_previous_state": [('np.einsum("hp,hpn->hn", dy[t], hs[k + 1])',
                                'np.einsum("hp,hpn->hn", dy[t], hs[k])')],
    "dx_without_step": [('dt[t][:, None] * np.einsum("hpn,hn->hp", Gs, Bh)',
                         'np.einsum("hpn,hn->hp", Gs, Bh)')],
    "dx_without_skip": [("out[\"dx\"][t] = Dv[:, None] * dy[t] + ", "out[\"dx\"][t] = ")],
    "dB_without_step": [('dt[t][:, None] * np.einsum("hpn,hp->hn", Gs, x[t])',
                         'np.einsum("hpn,hp->hn", Gs, x[t])')],
    "ddt_missing_decay_term": [(" + A * a * gh", "")],
    "ddt_decay_sign": [(" + A * a * gh", " - A * a * gh")],
    "dA_missing_step": [('out["dA"] += dt[t] * a * gh', 'out["dA"] += a * gh')],
    "decay_grad_from_current_state": [('gh = np.einsum("hpn,hpn->h", Gs, hs[k])',
                                       'gh = np.einsum("hpn,hpn->h", Gs, hs[k + 1])')],
    "final_state_grad_ignored": [("Gs = np.zeros((H, P, N)) if dhT is None else dhT[s].copy()",
                                  "Gs = np.zeros((H, P, N))")],
    "dh0_not_decayed_last": [("            Gs = a[:, None, None] * Gs\n        out[\"dh0\"][s] = Gs",
                              None)],
    "group_of_head_0": [("Bh, Ch = B[t, grp], C[t, grp]\n            Gs +=",
                         "Bh, Ch = B[t, 0 * grp], C[t, 0 * grp]\n            Gs +=")],
    "dD_missing": [('out["dD"] += np.einsum("hp,hp->h", dy[t], x[t])', "pass")],
}
# dh0 taken before the first token's decay: the adjoint is not propagated through a_0
MUTANTS["dh0_not_decayed_last"] = [(
    "            Gs = a[:, None, None] * Gs\n        out[\"dh0\"][s] = Gs",
    "            if k > 0:\n                Gs = a[:, None, None] * Gs\n        out[\"dh0\"][s] = Gs")]


def _load_mutant(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, ("mutation anchor not unique/found", name, old)
        src = src.replace(old, new)
    path = os.path.join(str(tmp_path), "bwd_%s.py" % name)
    with open(path, "w") as f:
        f.write(src)
    spec = importlib.util.spec_from_file_location("bwd_%s" % name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(name, tmp_path):
    m = _load_mutant(name, tmp_path)
    caught = []
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for pin_name, pin in ALL_BWD_PINS:
            try:
                pin(m)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(pin_name)
    assert caught, "mutant %s passed every pin" % name
