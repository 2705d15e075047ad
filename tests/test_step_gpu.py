"""Decode step (ssd_step) on the GPU against the fp64 step oracle.

Every test calls the C ABI through the binding and compares normwise
(max |gpu - ref| / max |ref| per tensor): y within the dtype's bound (fp32
1e-4, bf16 2e-2: y is rounded to bf16), the fp32 state within 1e-5 (fp32
arithmetic on inputs that are exact in fp32, plus the hardware exp2).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_ssd_sequence_fwd_amd as ssd
import ssd_inputs as si
from gpu_helpers import TOL
from oracle.step import ssd_step as oracle_step, ssd_steps as oracle_steps
from oracle_pins import rel_err

pytestmark = pytest.mark.gpu
STATE_TOL = 1e-5

SHAPES = {
    # name: (batch, H, P, N, G, dtype)
    "2.7b-bf16": (8, 80, 64, 128, 1, "bf16"),
    "2.7b-fp32": (8, 80, 64, 128, 1, "fp32"),
    "large-state-bf16": (4, 64, 64, 256, 8, "bf16"),
    "odd-N48-fp32": (3, 6, 16, 48, 3, "fp32"),          # 12 of 16 lanes per row active
    "N16-bf16": (5, 4, 32, 16, 2, "bf16"),               # a wave spans two heads
    "P128-N80-fp32": (2, 3, 128, 80, 1, "fp32"),
    "ragged-block-bf16": (1, 5, 16, 16, 1, "bf16"),      # 80 rows: one partial block
    "single-fp32": (1, 1, 16, 16, 1, "fp32"),
}


def _dev(inp, t=None):
    pick = (lambda v: v[t]) if t is not None else (lambda v: v)
    return {k: pick(inp[k]).cuda() for k in ("x", "dt", "B", "C")}


def _step_case(name, seed, with_D=True):
    batch, H, P, N, G, dtype = SHAPES[name]
    inp = si.make_step_inputs(batch, H, P, N, G, dtype, seed)
    d = _dev(inp, 0)
    A, D = inp["A"].cuda(), inp["D"].cuda() if with_D else None
    state = inp["state"].cuda()
    print("[gpu] ssd_step %s seed=%d D=%s" % (name, seed, with_D), flush=True)
    y = ssd.step(d["x"], d["dt"], A, d["B"], d["C"], D, state)
    torch.cuda.synchronize()
    yr, hr = oracle_step(inp["x"][0], inp["dt"][0], inp["A"], inp["B"][0], inp["C"][0],
                         inp["D"] if with_D else None, inp["state"])
    return y.double().cpu().numpy(), state.double().cpu().numpy(), yr, hr, dtype


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_step_parity(name):
    y, h, yr, hr, dtype = _step_case(name, seed=2000 + sorted(SHAPES).index(name))
    assert rel_err(y, yr) < TOL[dtype], rel_err(y, yr)
    assert rel_err(h, hr) < STATE_TOL, rel_err(h, hr)


def test_step_parity_without_D():
    y, h, yr, hr, dtype = _step_case("2.7b-bf16", seed=2100, with_D=False)
    assert rel_err(y, yr) < TOL[dtype]
    assert rel_err(h, hr) < STATE_TOL


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_step_sequence_of_steps(dtype):
    """32 consecutive steps on the same state buffer follow the oracle run
    step by step (errors do not build up)."""
    batch, H, P, N, G = 8, 80, 64, 128, 1
    T = 32
    inp = si.make_step_inputs(batch, H, P, N, G, dtype, seed=2200, steps=T)
    A, D, state = inp["A"].cuda(), inp["D"].cuda(), inp["state"].cuda()
    print("[gpu] ssd_step x%d %s" % (T, dtype), flush=True)
    ys = []
    for t in range(T):
        d = _dev(inp, t)
        ys.append(ssd.step(d["x"], d["dt"], A, d["B"], d["C"], D, state).double())
    torch.cuda.synchronize()
    yr, hr = oracle_steps(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                          inp["state"])
    y = torch.stack(ys).cpu().numpy()
    for t in (0, 1, T // 2, T - 1):
        assert rel_err(y[t], yr[t]) < TOL[dtype], (t, rel_err(y[t], yr[t]))
    assert rel_err(state.double().cpu().numpy(), hr) < STATE_TOL


def test_step_continues_a_prefilled_sequence():
    """Prefill 300 tokens with ssd_forward, then one ssd_step with token 301:
    y and the state match the oracle over all 301 tokens, and ssd_forward
    run over the 301 tokens at once."""
    w = si.scaled(si.CONFIGS[2], batch=2, seqlen=301, nheads=8, seed=2300)
    inp = si.make_inputs(w)
    dev = lambda t: t.cuda()
    x, dt, B, C = (dev(inp[k]) for k in ("x", "dt", "B", "C"))
    A, D, h0 = dev(inp["A"]), dev(inp["D"]), dev(inp["h0"])
    print("[gpu] prefill 300 + ssd_step vs ssd_forward 301", flush=True)
    _, h_pre = ssd.forward(x[:, :300].contiguous(), dt[:, :300].contiguous(), A,
                           B[:, :300].contiguous(), C[:, :300].contiguous(), D, h0)
    state = h_pre.clone()
    y_last = ssd.step(x[:, 300].contiguous(), dt[:, 300].contiguous(), A,
                      B[:, 300].contiguous(), C[:, 300].contiguous(), D, state)
    y_full, h_full = ssd.forward(x, dt, A, B, C, D, h0)
    torch.cuda.synchronize()
    import oracle
    T = 2 * 301
    f64 = lambda t, *shape: t.double().reshape(*shape).numpy()    # exact upcast
    yr, hr = oracle.ssd_recurrence(f64(inp["x"], T, 8, 64), f64(inp["dt"], T, 8),
                                   f64(inp["A"], 8), f64(inp["B"], T, 1, 128),
                                   f64(inp["C"], T, 1, 128), f64(inp["D"], 8),
                                   f64(inp["h0"], 2, 8, 64, 128), [301, 301])
    yr_last = yr.reshape(2, 301, 8, 64)[:, 300]
    y_step = y_last.double().cpu().numpy()
    assert rel_err(y_step, yr_last) < TOL["bf16"]
    assert rel_err(state.double().cpu().numpy(), hr) < TOL["bf16"]
    y_fwd = y_full[:, 300].double().cpu().numpy()
    assert rel_err(y_step, y_fwd) < TOL["bf16"]
    assert rel_err(state.double().cpu().numpy(), h_full.double().cpu().numpy()) < TOL["bf16"]


def test_step_empty_batch():
    x = torch.empty((0, 4, 16), device="cuda", dtype=torch.bfloat16)
    dt = torch.empty((0, 4), device="cuda", dtype=torch.bfloat16)
    B = torch.empty((0, 1, 16), device="cuda", dtype=torch.bfloat16)
    A = torch.full((4,), -1.0, device="cuda")
    state = torch.empty((0, 4, 16, 16), device="cuda")
    y = ssd.step(x, dt, A, B, B, None, state)
    assert y.shape == (0, 4, 16)


def test_step_large_batch_sampled():
    """batch 1024 at the 2.7B shapes (a 2.7 GB state): sampled sequences
    against the oracle."""
    batch, H, P, N, G = 1024, 80, 64, 128, 1
    inp = si.make_step_inputs(batch, H, P, N, G, "bf16", seed=2400)
    d = _dev(inp, 0)
    A, D, state = inp["A"].cuda(), inp["D"].cuda(), inp["state"].cuda()
    print("[gpu] ssd_step batch %d" % batch, flush=True)
    y = ssd.step(d["x"], d["dt"], A, d["B"], d["C"], D, state)
    torch.cuda.synchronize()
    pick = np.array([0, 1, 511, 512, 1000, 1023])
    yr, hr = oracle_step(inp["x"][0][pick], inp["dt"][0][pick], inp["A"], inp["B"][0][pick],
                         inp["C"][0][pick], inp["D"], inp["state"][pick])
    pick_t = torch.as_tensor(pick, device="cuda")
    assert rel_err(y[pick_t].double().cpu().numpy(), yr) < TOL["bf16"]
    assert rel_err(state[pick_t].double().cpu().numpy(), hr) < STATE_TOL
