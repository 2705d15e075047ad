"""The convolution front (ssd_conv1d_silu) on the GPU against the fp64 conv
oracle.

Bounds, per element, from the arithmetic: the kernel computes in fp32 from
inputs exact in fp32, |pre| stays below ~10 for these inputs and takes K + 1
rounded terms, and the activation uses the hardware exp and reciprocal (a few
ulp), so an fp32 output is within 1e-5 + 1e-5 |ref|. A bf16 output is that
value rounded to nearest, within 2^-9 of it relatively: 2^-8 |ref| + 2e-5.
Histories are copies of inputs and must match exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_ssd_sequence_fwd_amd as ssd
import oracle
import ssd_inputs as si
from gpu_helpers import TOL
from oracle.conv import conv_front, dense_bounds, varlen_bounds
from oracle_pins import rel_err

pytestmark = pytest.mark.gpu

BOUND = {"fp32": (1e-5, 1e-5), "bf16": (2.0 ** -8, 2e-5)}   # (rtol, atol)

CASES = {
    # name: (batch, seqlen, seq_lens, x_dim, bc_dim, K, dtype, history, lead, pad, bias)
    "bf16-K4-dense-ragged-hist": (2, 300, None, 128, 32, 4, "bf16", True, 0, 0, True),
    "fp32-K4-dense": (3, 65, None, 64, 16, 4, "fp32", False, 0, 0, True),
    "bf16-K3-packed-short-empty": (1, 0, [1, 0, 37, 2, 100, 0, 64, 3], 64, 16, 3, "bf16", True,
                                   0, 0, True),
    "bf16-K2-packed-empty-tail": (1, 0, [5, 40, 0, 0], 32, 8, 2, "bf16", True, 0, 0, False),
    "fp32-K3-slice-of-wider-rows": (2, 50, None, 64, 16, 3, "fp32", True, 64, 32, True),
    "bf16-K4-packed-slice": (1, 0, [33, 31, 64, 1], 256, 64, 4, "bf16", False, 128, 64, True),
    "bf16-K4-decode-L1": (5, 1, None, 64, 16, 4, "bf16", True, 0, 0, True),
    "bf16-K4-no-x-part": (2, 70, None, 0, 16, 4, "bf16", True, 0, 0, True),
}


def _bounds(inp, seq_lens):
    if seq_lens is None:
        return dense_bounds(inp["batch"], inp["seqlen"])
    return varlen_bounds(inp["cu_seqlens"].tolist())


def _run_gpu(inp, x_dim, bc_dim, seq_lens, lead=0, with_bias=True):
    """One ssd_conv1d_silu call on the device copy of ``inp``; xbc is the
    column slice [lead, lead + ch) of the full rows. Returns x, B, C flattened
    to (tokens, channels) and the final history."""
    ch = x_dim + 2 * bc_dim
    xbc = inp["xbc_full"].cuda()[:, lead:lead + ch]
    if seq_lens is None:
        xbc = xbc.view(inp["batch"], inp["seqlen"], ch)
    h = inp["history"]
    x, B, C, ho = ssd.conv1d_silu(xbc, inp["weight"].cuda(),
                                  inp["bias"].cuda() if with_bias else None, x_dim, bc_dim,
                                  None if h is None else h.cuda(),
                                  None if seq_lens is None else inp["cu_seqlens"])
    torch.cuda.synchronize()
    flat = lambda t: t.reshape(inp["T"], t.shape[-1])
    return flat(x), flat(B), flat(C), ho


def _check(name, got, want, dtype):
    rtol, atol = BOUND[dtype]
    g = got.double().cpu().numpy().reshape(want.shape)
    err = np.abs(g - want) - (atol + rtol * np.abs(want))
    worst = float(err.max()) if err.size else -1.0
    print("  %s: max |err| %.3e" % (name, float(np.abs(g - want).max()) if err.size else 0.0),
          flush=True)
    assert worst <= 0, (name, worst)


@pytest.mark.parametrize("name", sorted(CASES))
def test_conv_parity(name):
    batch, seqlen, seq_lens, x_dim, bc_dim, K, dtype, hist, lead, pad, bias = CASES[name]
    inp = si.make_conv_inputs(batch, seqlen, x_dim, bc_dim, K, dtype,
                              seed=4000 + sorted(CASES).index(name), seq_lens=seq_lens,
                              history=hist, lead_cols=lead, pad_cols=pad)
    print("[gpu] conv front %s" % name, flush=True)
    x, B, C, ho = _run_gpu(inp, x_dim, bc_dim, seq_lens, lead, with_bias=bias)
    rx, rB, rC, rh = conv_front(inp["xbc"], inp["weight"], inp["bias"] if bias else None,
                                _bounds(inp, seq_lens), x_dim, bc_dim, inp["history"])
    _check("x", x, rx, dtype)
    _check("B", B, rB, dtype)
    _check("C", C, rC, dtype)
    assert np.array_equal(ho.double().cpu().numpy(), rh), "history"


def test_conv_continuation_across_calls():
    """Three calls over consecutive token ranges, each given the history the
    last returned, equal one call over the whole range (and the oracle)."""
    x_dim, bc_dim, K = 64, 16, 4
    inp = si.make_conv_inputs(3, 90, x_dim, bc_dim, K, "bf16", seed=4100, history=True)
    ch = x_dim + 2 * bc_dim
    xbc = inp["xbc"].view(3, 90, ch).cuda()
    w, b = inp["weight"].cuda(), inp["bias"].cuda()
    print("[gpu] conv front continuation", flush=True)
    full = ssd.conv1d_silu(xbc, w, b, x_dim, bc_dim, inp["history"].cuda())
    h = inp["history"].cuda()
    parts = []
    for a, e in ((0, 1), (1, 41), (41, 90)):
        o = ssd.conv1d_silu(xbc[:, a:e].contiguous(), w, b, x_dim, bc_dim, h)
        parts.append(o[:3])
        h = o[3]
    torch.cuda.synchronize()
    for k in range(3):
        assert torch.equal(torch.cat([p[k] for p in parts], dim=1), full[k]), k
    assert torch.equal(h, full[3])


def test_conv_zero_tokens_keep_history():
    """Dense rows without tokens: the history passes through unchanged (or
    zeros without one); nothing else is written."""
    x_dim, bc_dim, K = 32, 8, 3
    ch = x_dim + 2 * bc_dim
    hist = torch.randn(4, K - 1, ch).to(torch.bfloat16).cuda()
    w = torch.randn(ch, K).cuda()
    xbc = torch.empty(4, 0, ch, dtype=torch.bfloat16, device="cuda")
    print("[gpu] conv front zero tokens", flush=True)
    x, B, C, ho = ssd.conv1d_silu(xbc, w, None, x_dim, bc_dim, hist)
    _, _, _, hz = ssd.conv1d_silu(xbc, w, None, x_dim, bc_dim, None)
    torch.cuda.synchronize()
    assert x.shape == (4, 0, x_dim) and B.shape == (4, 0, bc_dim)
    assert torch.equal(ho, hist)
    assert torch.count_nonzero(hz) == 0


def test_conv_then_ssd_forward_matches_oracle_chain():
    """The front's outputs go into ssd_forward as they are (x viewed as
    (batch, L, H, P), B and C as (batch, L, G, N), no copy), and the GPU chain
    matches the fp64 oracle chain (conv oracle, then the SSD oracle) within
    the bf16 bound of the SSD parity tests."""
    H, P, G, N, K, L = 4, 64, 1, 64, 4, 300
    x_dim, bc_dim = H * P, G * N
    inp = si.make_conv_inputs(2, L, x_dim, bc_dim, K, "bf16", seed=4200, history=True)
    ref = si.make_inputs(si.scaled(si.CONFIGS[1], batch=2, seqlen=L, nheads=H, seed=4201))
    print("[gpu] conv front into ssd_forward", flush=True)
    xbc = inp["xbc"].view(2, L, -1).cuda()
    x, B, C, _ = ssd.conv1d_silu(xbc, inp["weight"].cuda(), inp["bias"].cuda(), x_dim, bc_dim,
                                 inp["history"].cuda())
    xv, Bv, Cv = x.view(2, L, H, P), B.view(2, L, G, N), C.view(2, L, G, N)
    assert xv.data_ptr() == x.data_ptr()
    y, hT = ssd.forward(xv, ref["dt"].cuda(), ref["A"].cuda(), Bv, Cv, ref["D"].cuda(),
                        chunk_size=256)
    torch.cuda.synchronize()
    rx, rB, rC, _ = conv_front(inp["xbc"], inp["weight"], inp["bias"], dense_bounds(2, L),
                               x_dim, bc_dim, inp["history"])
    f = oracle._np
    ry, rh = oracle.ssd_recurrence(rx.reshape(2 * L, H, P), f(ref["dt"]).reshape(2 * L, H),
                                   f(ref["A"]), rB.reshape(2 * L, G, N), rC.reshape(2 * L, G, N),
                                   f(ref["D"]), None, [L, L])
    ey = rel_err(y.reshape(2 * L, H, P).double().cpu().numpy(), ry)
    eh = rel_err(hT.double().cpu().numpy(), rh)
    print("  y err %.3e  state err %.3e" % (ey, eh), flush=True)
    assert ey < TOL["bf16"] and eh < TOL["bf16"], (ey, eh)


def test_conv_full_workload_sampled():
    """The 2.7B-shaped front (batch 8, 2048 tokens, x 5120 channels, B and C
    128 each, K 4, bf16) in the launch configuration the benchmark times;
    sampled channel groups against the oracle (channels are independent)."""
    x_dim, bc_dim, K = 5120, 128, 4
    inp = si.make_conv_inputs(8, 2048, x_dim, bc_dim, K, "bf16", seed=4300, history=True)
    ch = x_dim + 2 * bc_dim
    print("[gpu] conv front full workload", flush=True)
    x, B, C, ho = _run_gpu(inp, x_dim, bc_dim, None)
    out = torch.cat([x, B, C], dim=1)
    assert ch == out.shape[1]
    groups = [0, 1, 63, 64, 200, 639, 640, 655, 656, 671]
    cols = np.concatenate([np.arange(8 * g, 8 * g + 8) for g in groups])
    sel = torch.as_tensor(cols)
    xs, _, _, hs = conv_front(inp["xbc"][:, sel], inp["weight"][sel], inp["bias"][sel],
                              dense_bounds(8, 2048), len(cols), 0, inp["history"][:, :, sel])
    _check("sampled", out[:, sel.cuda()], xs, "bf16")
    assert np.array_equal(ho[:, :, sel.cuda()].double().cpu().numpy(), hs)
