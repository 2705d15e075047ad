"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them."""
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

MUTANTS = {
    "swap_B_C": [("row[n] = decay * row[n] + u * bt[n];", "row[n] = decay * row[n] + u * ct[n];"),
                 ("acc += ct[n] * row[n];", "acc += bt[n] * row[n];")],
    "add_then_decay": [("row[n] = decay * row[n] + u * bt[n];",
                        "row[n] = decay * (row[n] + u * bt[n]);")],
    "output_before_update": [("row[n] = decay * row[n] + u * bt[n];\n          acc += ct[n] * row[n];",
                              "acc += ct[n] * row[n];\n          row[n] = decay * row[n] + u * bt[n];")],
    "sign_of_A": [("exp(step * A[h])", "exp(-step * A[h])")],
    "drop_D": [("yt[p] = acc + d_skip * xt[p];", "yt[p] = acc;")],
    "interleaved_groups": [("g = h / heads_per_group", "g = h % G")],
    "zoh_input_factor": [("const double u = step * xt[p];",
                          "const double u = (A[h] != 0.0 ? (decay - 1.0) / A[h] : step) * xt[p];")],
    "ignore_initial_state": [("if (h0)\n", "if (0)\n")],
    "dt_of_previous_token": [("const double step = dt[t * H + h];",
                              "const double step = dt[(t > 0 ? t - 1 : t) * H + h];")],
    "snapshot_off_by_one": [("i % snap_every == 0", "i % snap_every == 1")],
    "group_ignored": [("const double *bt = B + (t * G + g) * N;",
                       "const double *bt = B + (t * G) * N;")],
    "decay_of_head_0": [("exp(step * A[h])", "exp(step * A[0])")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, ("mutation anchor not unique/found", name, old)
        src = src.replace(old, new)
    cfile = tmp_path / ("%s.c" % name)
    cfile.write_text(src)
    so = tmp_path / ("lib%s.so" % name)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                    "-o", str(so), str(cfile), "-lm"], check=True)
    lib = oracle._load(str(so))
    caught = []
    for pin_name, pin in ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin_name)
    assert caught, "mutant %s passed every pin" % name
