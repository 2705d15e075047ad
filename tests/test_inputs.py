"""Seeded input generator: shapes, determinism, recipe (CPU only)."""
import numpy as np
import torch

import ssd_inputs as si


def test_config0_shapes_and_determinism():
    a = si.make_inputs(si.CONFIGS[0])
    b = si.make_inputs(si.CONFIGS[0])
    assert a["x"].shape == (1, 256, 4, 32) and a["x"].dtype == torch.float32
    assert a["B"].shape == (1, 256, 1, 16) and a["dt"].shape == (1, 256, 4)
    assert a["h0"] is None and a["cu_seqlens"] is None
    for k in ("x", "dt", "A", "B", "C", "D"):
        assert torch.equal(a[k], b[k])
    assert bool((a["dt"] > 0).all()) and bool((a["A"] < 0).all())
    assert float(a["A"].min()) >= -np.exp(2.0) - 1e-5 and float(a["A"].max()) <= -1.0 + 1e-6


def test_varlen_layout():
    w = si.scaled(si.CONFIGS[4], nheads=2, headdim=8, dstate=4, num_seqs=5,
                  len_range=(16, 64))
    inp = si.make_inputs(w)
    cu = inp["cu_seqlens"]
    assert cu.dtype == torch.int32 and cu.shape == (6,) and int(cu[0]) == 0
    assert int(cu[-1]) == inp["x"].shape[1] and inp["x"].shape[0] == 1
    lens = np.diff(cu.numpy())
    assert (lens >= 16).all() and (lens <= 64).all()
    assert inp["x"].dtype == torch.bfloat16


def test_dt_bias_solver_hits_target():
    rng = np.random.default_rng(5)
    z = rng.standard_normal((20000, 64))
    A = -np.exp(rng.uniform(0, 2, size=64))
    b = si.solve_dt_bias(z, A, 0.9)
    m = np.mean(np.exp(np.logaddexp(0, z + b) * A[None]))
    assert abs(m - 0.9) < 1e-6
    assert -4.2 < b < -3.3      # same neighbourhood as the large-state workload's draw


def test_h0_std():
    w = si.scaled(si.CONFIGS[2], batch=2, seqlen=8, nheads=4, headdim=16, dstate=32)
    inp = si.make_inputs(w)
    assert inp["h0"].shape == (2, 4, 16, 32) and inp["h0"].dtype == torch.float32
    assert 0.08 < float(inp["h0"].std()) < 0.12
