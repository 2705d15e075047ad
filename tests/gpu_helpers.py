"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the C-ABI path, run the oracle, compare normwise."""
from __future__ import annotations

import numpy as np
import torch

import mamba_ssd_sequence_fwd_amd as ssd
import oracle

# Normwise max relative error bounds: max|gpu - ref| / max|ref| per tensor.
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def to_device(inp: dict, dev="cuda") -> dict:
    out = {}
    for k in ("x", "dt", "A", "B", "C", "D", "h0"):
        out[k] = None if inp[k] is None else inp[k].to(dev)
    out["cu_seqlens"] = inp["cu_seqlens"]
    return out


# Kernel paths of the library: the default (chained per-(chunk, head)
# workgroups for bf16), the per-(sequence, head) fused kernel, and one kernel
# per step of the method.
PATHS = {"default": {}, "per_sequence": {"per_sequence": True}, "unfused": {"unfused": True}}


def plan_for(inp: dict, chunk=None, generic=False, unfused=False, per_sequence=False,
             dev="cuda") -> ssd.Plan:
    d = to_device(inp, dev)
    w = inp["workload"]
    return ssd.Plan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                    chunk_size=chunk or w.chunk, cu_seqlens=d["cu_seqlens"],
                    generic=generic, unfused=unfused, per_sequence=per_sequence)


def run_gpu(inp: dict, chunk=None, generic=False, unfused=False, per_sequence=False):
    """(y (T, H, P) fp64, final_state fp64, plan) after one ssd_forward."""
    plan = plan_for(inp, chunk, generic, unfused, per_sequence)
    print("[gpu] ssd_forward %s seed=%d %r" % (inp["workload"].name, inp["workload"].seed,
                                               plan.prob), flush=True)
    y, hT = plan.run()
    torch.cuda.synchronize()
    assert plan.chain_error() == 0, "a chained workgroup timed out waiting for its state"
    T = plan.tokens
    y64 = y.reshape(T, y.shape[2], y.shape[3]).to(torch.float64).cpu().numpy()
    return y64, hT.to(torch.float64).cpu().numpy(), plan


def seq_lens_of(inp: dict):
    if inp["seq_lens"] is not None:
        return list(inp["seq_lens"])
    b, L = inp["x"].shape[:2]
    return [L] * b


def flat_inputs(inp: dict):
    """(x, dt, B, C) reshaped to the packed-token view the oracle takes."""
    x = inp["x"]
    T = x.shape[0] * x.shape[1]
    return (x.reshape(T, x.shape[2], x.shape[3]), inp["dt"].reshape(T, x.shape[2]),
            inp["B"].reshape(T, inp["B"].shape[2], inp["B"].shape[3]),
            inp["C"].reshape(T, inp["C"].shape[2], inp["C"].shape[3]))


def run_oracle(inp: dict, snap_every=0):
    x, dt, B, C = flat_inputs(inp)
    f = oracle._np
    return oracle.ssd_recurrence(f(x), f(dt), f(inp["A"]), f(B), f(C), f(inp["D"]),
                                 None if inp["h0"] is None else f(inp["h0"]),
                                 seq_lens_of(inp), snap_every=snap_every)


def rel_err(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    scale = float(np.max(np.abs(b)))
    return float(np.max(np.abs(a - b))) / max(scale, 1e-30)


def tol_of(inp: dict) -> float:
    return TOL[inp["workload"].dtype]


def compare_every_pair(inp: dict, outs: dict, block_tokens: int = 16384):
    """Compare GPU outputs with the oracle over EVERY (sequence, head) pair.

    ``outs`` maps a label (a kernel path) to (y (T, H, P) tensor on the CPU,
    final_state (S, H, P, N) tensor on the CPU). The oracle runs once, over
    blocks of whole sequences of about ``block_tokens`` tokens, and every
    label is compared against the same reference. Returns per label a dict:
    normwise errors of y and of the final state over the whole tensor
    (max|gpu - ref| / max|ref|), the worst per-(sequence, head) slice error
    of each (the same ratio within the slice), and the pair it occurs at.
    """
    x, dt, B, C = flat_inputs(inp)
    lens = seq_lens_of(inp)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    H = x.shape[1]
    f = oracle._np
    acc = {k: dict(dy=0.0, ry=0.0, dh=0.0, rh=0.0, wy=0.0, wy_at=None, wh=0.0, wh_at=None)
           for k in outs}
    s0 = 0
    while s0 < len(lens):
        s1, tok = s0, 0
        while s1 < len(lens) and (s1 == s0 or tok + lens[s1] <= block_tokens):
            tok += lens[s1]
            s1 += 1
        a, b = int(starts[s0]), int(starts[s1])
        h0 = None if inp["h0"] is None else f(inp["h0"][s0:s1])
        yr, hr = oracle.ssd_recurrence(f(x[a:b]), f(dt[a:b]), f(inp["A"]), f(B[a:b]), f(C[a:b]),
                                       f(inp["D"]), h0, lens[s0:s1])
        for k, (y, hT) in outs.items():
            r = acc[k]
            yg = y[a:b].to(torch.float64).numpy()
            hg = hT[s0:s1].to(torch.float64).numpy()
            dy = np.abs(yg - yr)
            dh = np.abs(hg - hr)
            r["dy"] = max(r["dy"], float(dy.max()) if dy.size else 0.0)
            r["ry"] = max(r["ry"], float(np.abs(yr).max()) if yr.size else 0.0)
            r["dh"] = max(r["dh"], float(dh.max()))
            r["rh"] = max(r["rh"], float(np.abs(hr).max()))
            for j in range(s1 - s0):
                ja, jb = int(starts[s0 + j]) - a, int(starts[s0 + j + 1]) - a
                for h in range(H):
                    if jb > ja:
                        e = float(dy[ja:jb, h].max()) / max(float(np.abs(yr[ja:jb, h]).max()), 1e-30)
                        if e > r["wy"]:
                            r["wy"], r["wy_at"] = e, (s0 + j, h)
                    e = float(dh[j, h].max()) / max(float(np.abs(hr[j, h]).max()), 1e-30)
                    if e > r["wh"]:
                        r["wh"], r["wh_at"] = e, (s0 + j, h)
        s0 = s1
    res = {}
    for k, r in acc.items():
        res[k] = dict(y=r["dy"] / max(r["ry"], 1e-30), final=r["dh"] / max(r["rh"], 1e-30),
                      worst_y=r["wy"], worst_y_at=r["wy_at"], worst_final=r["wh"],
                      worst_final_at=r["wh_at"], pairs=len(lens) * H)
    return res
