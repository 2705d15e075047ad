"""The Mamba-1 selective scan (ssd_selective_scan) on the GPU against the fp64
scan oracle, and against the SSD path where the two layers coincide.

Normwise bounds (max |gpu - ref| / max |ref| per tensor): y within the
dtype's bound (fp32 1e-4, bf16 2e-2: y is rounded to bf16); the state is
fp32 throughout, from inputs that are exact in fp32, so within 1e-4.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_ssd_sequence_fwd_amd as ssd
import ssd_inputs as si
from gpu_helpers import TOL
from oracle.selective_scan import selective_scan as oracle_scan
from oracle_pins import rel_err

pytestmark = pytest.mark.gpu
STATE_TOL = 1e-4

CASES = {
    # name: (batch, L, dim, N, dtype, h0_std)
    "N16-bf16-ragged-h0": (2, 300, 128, 16, "bf16", 0.1),
    "N16-fp32": (1, 257, 64, 16, "fp32", 0.0),
    "N32-bf16": (2, 100, 128, 32, "bf16", 0.1),
    "N64-fp32-h0": (1, 65, 192, 64, "fp32", 0.5),
    "N128-bf16": (1, 96, 64, 128, "bf16", 0.1),
    "N256-bf16": (2, 40, 64, 256, "bf16", 0.1),
    "N16-L1": (3, 1, 64, 16, "bf16", 0.1),
    "N16-L31": (1, 31, 128, 16, "bf16", 0.0),
}


def _gpu(inp, with_D=True):
    dev = lambda t: None if t is None else t.cuda()
    return ssd.selective_scan(dev(inp["x"]), dev(inp["delta"]), dev(inp["A"]), dev(inp["B"]),
                              dev(inp["C"]), dev(inp["D"]) if with_D else None, dev(inp["h0"]))


@pytest.mark.parametrize("name", sorted(CASES))
def test_scan_parity(name):
    batch, L, dim, N, dtype, h0_std = CASES[name]
    inp = si.make_scan_inputs(batch, L, dim, N, dtype, seed=3000 + sorted(CASES).index(name),
                              h0_std=h0_std)
    print("[gpu] selective scan %s" % name, flush=True)
    y, hT = _gpu(inp)
    torch.cuda.synchronize()
    yr, hr = oracle_scan(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["h0"])
    ey = rel_err(y.double().cpu().numpy(), yr)
    eh = rel_err(hT.double().cpu().numpy(), hr)
    print("  y err %.3e  state err %.3e" % (ey, eh), flush=True)
    assert ey < TOL[dtype] and eh < STATE_TOL, (ey, eh)


def test_scan_without_D_and_zero_tokens():
    inp = si.make_scan_inputs(2, 50, 64, 16, "bf16", seed=3100, h0_std=0.2)
    y, hT = _gpu(inp, with_D=False)
    torch.cuda.synchronize()
    yr, hr = oracle_scan(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], None, inp["h0"])
    assert rel_err(y.double().cpu().numpy(), yr) < TOL["bf16"]
    assert rel_err(hT.double().cpu().numpy(), hr) < STATE_TOL
    # no tokens: the final state is the initial state
    empty = {k: (v[:, :0] if k in ("x", "delta", "B", "C") else v) for k, v in inp.items()}
    y0, h0 = _gpu(empty)
    torch.cuda.synchronize()
    assert y0.shape == (2, 0, 64)
    assert torch.equal(h0.cpu(), inp["h0"])


def test_scan_matches_ssd_forward_when_A_is_per_head():
    """A[d, n] = A_h and delta shared by the channels of a head: the scan and
    the SSD path compute the same layer (both on the GPU, and the oracle)."""
    w = si.scaled(si.CONFIGS[2], batch=2, seqlen=520, nheads=4, seed=3200)
    inp = si.make_inputs(w)
    b, L, H, P, N = 2, 520, 4, 64, 128
    head = torch.arange(H).repeat_interleave(P)
    x = inp["x"].reshape(b, L, H * P)
    delta = inp["dt"][:, :, head].contiguous()
    A = inp["A"][head][:, None].expand(H * P, N).contiguous()
    B, C = inp["B"][:, :, 0].contiguous(), inp["C"][:, :, 0].contiguous()
    D = inp["D"][head].contiguous()
    h0 = inp["h0"].reshape(b, H * P, N)
    print("[gpu] selective scan vs ssd_forward", flush=True)
    ys, hs = ssd.selective_scan(x.cuda(), delta.cuda(), A.cuda(), B.cuda(), C.cuda(), D.cuda(),
                                h0.cuda())
    yf, hf = ssd.forward(inp["x"].cuda(), inp["dt"].cuda(), inp["A"].cuda(), inp["B"].cuda(),
                         inp["C"].cuda(), inp["D"].cuda(), inp["h0"].cuda())
    torch.cuda.synchronize()
    yr, hr = oracle_scan(x, delta, A, B, C, D, h0)
    ys_ = ys.double().cpu().numpy()
    assert rel_err(ys_, yr) < TOL["bf16"] and rel_err(hs.double().cpu().numpy(), hr) < STATE_TOL
    assert rel_err(ys_, yf.reshape(b, L, H * P).double().cpu().numpy()) < TOL["bf16"]
    assert rel_err(hs.double().cpu().numpy(),
                   hf.reshape(b, H * P, N).double().cpu().numpy()) < TOL["bf16"]


def test_scan_full_workload_sampled():
    """The comparator workload (batch 8, 2048 tokens, 5120 channels, N 16):
    sampled channels against the oracle (each channel is independent)."""
    inp = si.make_scan_inputs(8, 2048, 5120, 16, "bf16", seed=3300)
    print("[gpu] selective scan full workload", flush=True)
    y, hT = _gpu(inp)
    torch.cuda.synchronize()
    ch = np.array([0, 1, 63, 64, 2500, 4095, 5119])
    yr, hr = oracle_scan(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["h0"], channels=ch)
    sel = torch.as_tensor(ch)
    assert rel_err(y[:, :, sel.cuda()].double().cpu().numpy(), yr) < TOL["bf16"]
    assert rel_err(hT[:, sel.cuda()].double().cpu().numpy(), hr) < STATE_TOL
