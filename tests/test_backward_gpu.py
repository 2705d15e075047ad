"""The backward pass (ssd_backward) on the GPU against the fp64 backward
oracle.

Both sides recompute the forward states from the inputs. Every gradient is
compared normwise, max |gpu - ref| / max |ref| per tensor, within the bf16 bound
2e-2: the products round their operands to bf16 (2^-9 relative each) and
accumulate in fp32, and the gradients are rounded to bf16 once.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_ssd_sequence_fwd_amd as ssd
import oracle
import ssd_inputs as si
from gpu_helpers import TOL
from oracle.backward import ssd_backward as oracle_backward
from oracle_pins import rel_err

pytestmark = pytest.mark.gpu
BASE = si.CONFIGS[2]

CASES = {
    "dense-N64-Q128-ragged": si.scaled(BASE, batch=2, seqlen=300, nheads=4, dstate=64, chunk=128,
                                       seed=5001),
    "dense-N128-Q256-G2": si.scaled(BASE, batch=1, seqlen=520, nheads=4, ngroups=2, seed=5002),
    "varlen-short-empty": si.scaled(BASE, batch=1, nheads=2, num_seqs=5,
                                    seq_lens=(40, 0, 300, 1, 257), seed=5003),
    "slow-decay-N64": si.scaled(BASE, batch=1, seqlen=600, nheads=2, dstate=64, chunk=128,
                                log_neg_a=(-7.0, -5.0), seed=5004),
    "no-D-no-h0": si.scaled(BASE, batch=2, seqlen=256, nheads=2, h0_std=0.0, seed=5005),
    "single-chunk-Q256": si.scaled(BASE, batch=3, seqlen=100, nheads=2, seed=5006),
    # the dB / dC kernel walks a group's heads in pairs: an odd count and a
    # single head take its tail path
    "odd-heads-per-group": si.scaled(BASE, batch=1, seqlen=400, nheads=3, seed=5007),
    "one-head-N64-Q128": si.scaled(BASE, batch=2, seqlen=200, nheads=1, dstate=64, chunk=128,
                                   seed=5008),
}


def _run(w, no_D=False, dhT_std=0.1):
    inp = si.make_inputs(w)
    gin = si.make_grad_inputs(w, inp, dhT_std=dhT_std)
    dev = {k: (None if inp[k] is None else inp[k].cuda())
           for k in ("x", "dt", "A", "B", "C", "D", "h0")}
    if no_D:
        dev["D"] = None
    print("[gpu] ssd_backward %s seed=%d" % (w.name, w.seed), flush=True)
    g = ssd.backward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["h0"],
                     gin["dy"].cuda(), None if gin["dhT"] is None else gin["dhT"].cuda(),
                     chunk_size=w.chunk, cu_seqlens=inp["cu_seqlens"])
    torch.cuda.synchronize()
    return inp, gin, g


def _flat(inp, w):
    x = inp["x"]
    T = x.shape[0] * x.shape[1]
    return T, (inp["seq_lens"] or [w.seqlen] * w.batch)


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_parity(name):
    w = CASES[name]
    no_D = name.startswith("no-D")
    inp, gin, g = _run(w, no_D=no_D, dhT_std=0.0 if no_D else 0.1)
    T, lens = _flat(inp, w)
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    f = oracle._np
    ref = oracle_backward(f(inp["x"]).reshape(T, H, P), f(inp["dt"]).reshape(T, H), f(inp["A"]),
                          f(inp["B"]).reshape(T, G, N), f(inp["C"]).reshape(T, G, N),
                          None if no_D else f(inp["D"]),
                          None if inp["h0"] is None else f(inp["h0"]), lens,
                          f(gin["dy"]).reshape(T, H, P),
                          None if gin["dhT"] is None else f(gin["dhT"]))
    got = {"dx": g["dx"].reshape(T, H, P), "ddt": g["ddt"].reshape(T, H),
           "dB": g["dB"].reshape(T, G, N), "dC": g["dC"].reshape(T, G, N),
           "dA": g["dA"], "dD": g["dD"], "dh0": g["dinitial_state"]}
    errs = {k: rel_err(v.double().cpu().numpy(), ref[k]) for k, v in got.items()}
    print("  " + "  ".join("%s %.2e" % kv for kv in errs.items()), flush=True)
    bad = {k: e for k, e in errs.items() if not e < TOL["bf16"]}
    assert not bad, bad


def test_backward_zero_tokens_pass_the_state_gradient():
    """Dense rows without tokens: dL/dh0 = dL/d(final state); dA = dD = 0."""
    w = si.scaled(BASE, batch=2, seqlen=0, nheads=2, seed=5100)
    inp = si.make_inputs(w)
    dhT = torch.randn(2, 2, 64, 128)
    dev = {k: (None if inp[k] is None else inp[k].cuda()) for k in ("x", "dt", "A", "B", "C",
                                                                    "D", "h0")}
    print("[gpu] ssd_backward zero tokens", flush=True)
    g = ssd.backward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["h0"],
                     torch.empty_like(dev["x"]), dhT.cuda(), chunk_size=256)
    torch.cuda.synchronize()
    assert torch.equal(g["dinitial_state"].cpu(), dhT)
    assert torch.count_nonzero(g["dA"]) == 0 and torch.count_nonzero(g["dD"]) == 0


def test_backward_full_workload_sampled():
    """The 2.7B-shaped workload (batch 8 x 2048 tokens, 80 heads, P 64, N 128,
    chunk 256) in the launch configuration the benchmark times. dx, ddt and
    dh0 of sampled (sequence, head) pairs against the oracle run on those
    pairs alone (heads are independent there); dB, dC, dD and the whole
    problem through the identities of a loss affine in B, C and D,
    L - L(B = 0) = <dB, B> etc., with L from the forward C oracle."""
    w = BASE
    inp, gin, g = _run(w)
    T, lens = _flat(inp, w)
    H, P, N, G, L = w.nheads, w.headdim, w.dstate, w.ngroups, w.seqlen
    f = oracle._np
    x, dt, A, B, C, D, h0 = (f(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "h0"))
    dy, dhT = f(gin["dy"]), f(gin["dhT"])
    for b, h in ((0, 0), (3, 41), (7, 79)):
        r = oracle_backward(x[b, :, h:h + 1], dt[b, :, h:h + 1], A[h:h + 1], B[b], C[b],
                            D[h:h + 1], h0[b:b + 1, h:h + 1], [L], dy[b, :, h:h + 1],
                            dhT[b:b + 1, h:h + 1])
        for k, gk, sl in (("dx", "dx", (b, slice(None), h)), ("ddt", "ddt", (b, slice(None), h)),
                          ("dh0", "dinitial_state", (b, h))):
            e = rel_err(g[gk][sl].double().cpu().numpy(), r[k].reshape(g[gk][sl].shape))
            print("  (%d, %d) %s %.2e" % (b, h, k, e), flush=True)
            assert e < TOL["bf16"], (b, h, k, e)

    # dA and dD of one head over every sequence (a head's own recurrence)
    h = 41
    r = oracle_backward(x[:, :, h:h + 1].reshape(T, 1, P), dt[:, :, h:h + 1].reshape(T, 1),
                        A[h:h + 1], B.reshape(T, G, N), C.reshape(T, G, N), D[h:h + 1],
                        h0[:, h:h + 1], lens, dy[:, :, h:h + 1].reshape(T, 1, P),
                        dhT[:, h:h + 1])
    for k in ("dA", "dD"):
        e = rel_err(g[k][h:h + 1].double().cpu().numpy(), r[k])
        print("  head %d %s %.2e" % (h, k, e), flush=True)
        assert e < TOL["bf16"], (k, e)

    def loss(**over):
        q = dict(x=x.reshape(T, H, P), dt=dt.reshape(T, H), A=A, B=B.reshape(T, G, N),
                 C=C.reshape(T, G, N), D=D, h0=h0)
        q.update(over)
        y, hT = oracle.ssd_recurrence(q["x"], q["dt"], q["A"], q["B"], q["C"], q["D"], q["h0"],
                                      lens)
        return float(np.sum(dy.reshape(T, H, P) * y) + np.sum(dhT * hT))

    L0 = loss()
    for name, gk, shape in (("B", "dB", (T, G, N)), ("C", "dC", (T, G, N)), ("D", "dD", (H,))):
        val = dict(B=B, C=C, D=D)[name].reshape(shape)
        want = L0 - loss(**{name: np.zeros(shape)})
        got = float(np.sum(g[gk].double().cpu().numpy().reshape(shape) * val))
        print("  <d%s, %s> %.6e vs %.6e" % (name, name, got, want), flush=True)
        assert abs(got - want) <= TOL["bf16"] * abs(want), (name, got, want)


def test_backward_is_deterministic():
    """Every gradient is bit-identical across repeated passes: the kernels sum
    in a fixed order (no float atomics), whatever order their waves run in."""
    w = si.scaled(BASE, batch=2, seqlen=1024, nheads=16, seed=5050)
    inp = si.make_inputs(w)
    gin = si.make_grad_inputs(w, inp)
    d = {k: (None if inp[k] is None else inp[k].cuda()) for k in ("x", "dt", "A", "B", "C", "D", "h0")}
    plan = ssd.BackwardPlan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                            gin["dy"].cuda(), gin["dhT"].cuda(), w.chunk)
    print("[gpu] backward determinism %r" % plan.prob, flush=True)
    first = {k: v.clone() for k, v in plan.run().items()}
    for _ in range(4):
        again = plan.run()
        torch.cuda.synchronize()
        for k, v in first.items():
            assert torch.equal(v, again[k]), k
