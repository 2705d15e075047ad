"""ssd_forward_dt_softplus: the step's pre-activation goes in, every kernel
applies softplus(dt + dt_bias[h]); checked against the oracle recurrence run
on oracle.dt_softplus of the same raw values, on every kernel path."""
import numpy as np
import pytest
import torch

import mamba_ssd_sequence_fwd_amd as ssd
import oracle
import ssd_inputs as si
from gpu_helpers import PATHS, flat_inputs, rel_err, seq_lens_of, tol_of

pytestmark = pytest.mark.gpu

CASES = {
    "bf16-N128-h0": si.scaled(si.CONFIGS[2], batch=2, seqlen=600, nheads=4, seed=2501),
    "bf16-N256-G2-slow": si.scaled(si.STRESS["S1"], batch=1, seqlen=700, nheads=4, dstate=256,
                                   ngroups=2, seed=2502),
    "bf16-varlen": si.scaled(si.CONFIGS[4], nheads=4, num_seqs=4, seq_lens=(1, 300, 0, 520),
                             h0_std=0.1, seed=2503),
    "fp32-N64": si.scaled(si.CONFIGS[2], batch=1, seqlen=333, nheads=3, dstate=64,
                          dtype="fp32", seed=2504),
}


def _raw_inputs(w):
    """The workload's inputs with dt replaced by a raw pre-activation
    z ~ N(0, 1) (in the dtype) and a per-head fp32 bias ~ -2 + N(0, 0.5^2)."""
    inp = si.make_inputs(w)
    rng = np.random.default_rng(w.seed + 77)
    z = rng.standard_normal(tuple(inp["dt"].shape)).astype(np.float32)
    raw = torch.from_numpy(z).to(inp["dt"].dtype)
    bias = torch.from_numpy((-2.0 + 0.5 * rng.standard_normal(w.nheads)).astype(np.float32))
    return inp, raw, bias


# The generic FMA kernels run every dtype alike: the fp32 cases cover them.
PARAMS = [(n, p) for n in sorted(CASES) for p in PATHS] + \
         [(n, "generic") for n in sorted(CASES) if CASES[n].dtype == "fp32"]


@pytest.mark.parametrize("name,path", PARAMS)
def test_dt_softplus_parity(name, path):
    w = CASES[name]
    inp, raw, bias = _raw_inputs(w)
    kw = dict(PATHS.get(path, {}))
    if path == "generic":
        kw = {"generic": True}
    dev = lambda t: None if t is None else t.cuda()
    plan = ssd.Plan(dev(inp["x"]), dev(raw), dev(inp["A"]), dev(inp["B"]), dev(inp["C"]),
                    dev(inp["D"]), dev(inp["h0"]), chunk_size=w.chunk,
                    cu_seqlens=inp["cu_seqlens"], dt_softplus=True, dt_bias=dev(bias), **kw)
    print("[gpu] dt softplus %s %s" % (name, path), flush=True)
    y, hT = plan.run()
    torch.cuda.synchronize()
    assert plan.chain_error() == 0
    T, H = plan.tokens, w.nheads
    f = oracle._np                                          # exact fp64 upcast
    x, _, B, C = flat_inputs(inp)
    dt_eff = oracle.dt_softplus(raw.reshape(T, H), bias)
    yr, hr = oracle.ssd_recurrence(f(x), dt_eff, f(inp["A"]), f(B), f(C), f(inp["D"]),
                                   None if inp["h0"] is None else f(inp["h0"]),
                                   seq_lens_of(inp))
    ey = rel_err(y.reshape(T, H, -1).double().cpu().numpy(), yr)
    eh = rel_err(hT.double().cpu().numpy(), hr)
    print("  y err %.3e  final err %.3e" % (ey, eh), flush=True)
    assert ey <= tol_of(inp) and eh <= tol_of(inp)


def test_dt_softplus_equals_precomputed_step():
    """fp32: softplus fused in the kernels = the same step computed first."""
    w = CASES["fp32-N64"]
    inp, raw, bias = _raw_inputs(w)
    step = torch.nn.functional.softplus(raw + bias)
    dev = lambda t: None if t is None else t.cuda()
    y1, h1 = ssd.Plan(dev(inp["x"]), dev(raw), dev(inp["A"]), dev(inp["B"]), dev(inp["C"]),
                      dev(inp["D"]), dev(inp["h0"]), chunk_size=w.chunk, dt_softplus=True,
                      dt_bias=dev(bias)).run()
    y2, h2 = ssd.forward(dev(inp["x"]), dev(step), dev(inp["A"]), dev(inp["B"]), dev(inp["C"]),
                         dev(inp["D"]), dev(inp["h0"]), chunk_size=w.chunk)
    torch.cuda.synchronize()
    assert rel_err(y1.double().cpu().numpy(), y2.double().cpu().numpy()) < 1e-5
    assert rel_err(h1.double().cpu().numpy(), h2.double().cpu().numpy()) < 1e-5
