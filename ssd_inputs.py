"""Seeded synthetic inputs for the SSD forward pass.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic and is imported by both the GPU-path tests/benchmark and
the oracle tests, which is the one thing the two sides share.

Workloads (the shapes of a Mamba-2 block's SSD layer; the pages train on
The Pile at sequence length 2048/8192 with 125M-3B models and state sizes up
to 256, so every input here is synthetic with those shapes):

  id  name               batch  L      H   P   N    G  Q    dtype
  0   tiny-fp32          1      256    4   32  16   1  64   fp32
  1   small-bf16         4      2048   24  64  128  1  256  bf16
  2   2.7b-bf16          8      2048   80  64  128  1  256  bf16  (+ h0 ~ N(0, 0.1^2))
  3   large-state-long   2      16384  64  64  256  8  256  bf16  (dt bias solved: mean exp(dt A) = 0.9)
  4   varlen-packed      64 sequences, lengths ~ U[16, 4096], packed; H 80, P 64, N 128, G 1, Q 256, bf16

Decode steps (make_step_inputs): a dense batch of sequences advancing one token
each, e.g. batch 8 or 256 at H 80, P 64, N 128, with the same value recipe and
a random fp32 state ~ N(0, 0.1^2).

Value recipe (all configs unless stated): x, B, C, D ~ N(0, 1);
dt = softplus(z + bias) with z ~ N(0, 1) and bias = -2; A_h = -exp(U(0, 2));
zero initial state. Draw order from numpy.random.default_rng(seed):
sequence lengths (varlen only), x, B, C, z, u (for A), D, h0.
Floating inputs are drawn in float32/float64 and then rounded once to the
config dtype; A, D and h0 stay float32. The oracle consumes exactly these
rounded values, upcast to float64.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int = 1
    seqlen: int = 256
    nheads: int = 4
    headdim: int = 32
    dstate: int = 16
    ngroups: int = 1
    chunk: int = 64
    dtype: str = "fp32"            # "fp32" or "bf16": x, dt, B, C, y
    h0_std: float = 0.0            # > 0: random fp32 initial state of this std
    dt_bias: float = -2.0
    target_mean_decay: Optional[float] = None   # solve dt_bias for this mean of exp(dt*A)
    log_neg_a: tuple = (0.0, 2.0)  # A_h = -exp(U(lo, hi))
    a_zero: bool = False           # A_h = 0 (linear attention special case)
    num_seqs: int = 0              # > 0: varlen, batch must be 1
    len_range: tuple = (16, 4096)  # inclusive, varlen lengths ~ U[lo, hi]
    seq_lens: Optional[tuple] = None   # explicit varlen lengths (overrides the draw)
    seed: int = 1000


CONFIGS = {
    0: Workload("tiny-fp32", batch=1, seqlen=256, nheads=4, headdim=32, dstate=16,
                ngroups=1, chunk=64, dtype="fp32", seed=1000),
    1: Workload("small-bf16", batch=4, seqlen=2048, nheads=24, headdim=64,
                dstate=128, ngroups=1, chunk=256, dtype="bf16", seed=1001),
    2: Workload("2.7b-bf16", batch=8, seqlen=2048, nheads=80, headdim=64,
                dstate=128, ngroups=1, chunk=256, dtype="bf16", h0_std=0.1,
                seed=1002),
    3: Workload("large-state-long", batch=2, seqlen=16384, nheads=64, headdim=64,
                dstate=256, ngroups=8, chunk=256, dtype="bf16",
                target_mean_decay=0.9, seed=1003),
    4: Workload("varlen-packed", batch=1, seqlen=0, nheads=80, headdim=64,
                dstate=128, ngroups=1, chunk=256, dtype="bf16", num_seqs=64,
                len_range=(16, 4096), seed=1004),
}

# Stress workloads: the configs' decay is so fast that a chunk's carried
# state is numerically invisible, so these make it visible.
STRESS = {
    # config-2 shapes, per-step decay ~0.999, random initial state
    "S1": replace(CONFIGS[2], name="S1-slow-decay", log_neg_a=(-7.0, -5.0),
                  h0_std=0.1, seed=1101),
    # A = 0 at config-1 shapes (pure linear attention / prefix sum)
    "S2": replace(CONFIGS[1], name="S2-a-zero", a_zero=True, seed=1102),
    # config 4 with slow decay: carries across chunks inside a sequence
    "S3": replace(CONFIGS[4], name="S3-varlen-slow", log_neg_a=(-7.0, -5.0),
                  seed=1103),
}


def _softplus(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def solve_dt_bias(z: np.ndarray, A: np.ndarray, target: float) -> float:
    """Bias b such that mean over (t, h) of exp(softplus(z + b) * A_h) = target.

    A generator calibration (bisection on the drawn z and A), not part of the
    method.
    """
    lo, hi = -20.0, 5.0
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        m = float(np.mean(np.exp(_softplus(z + mid) * A[None, :])))
        if m > target:      # decays too little: dt too small -> raise bias
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def make_inputs(w: Workload) -> dict:
    """Draw one seeded input set for workload ``w`` (CPU torch tensors).

    Returns dict with x (batch, L, H, P), dt (batch, L, H), A (H,) fp32,
    B, C (batch, L, G, N), D (H,) fp32, h0 (batch|num_seqs, H, P, N) fp32 or
    None, cu_seqlens int32 (num_seqs+1,) or None, seq_lens list or None, plus
    'workload' and 'dt_bias'.
    """
    rng = np.random.default_rng(w.seed)
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    cu = None
    lens = None
    if w.num_seqs > 0:
        if w.seq_lens is not None:
            lens = [int(v) for v in w.seq_lens]
        else:
            lo, hi = w.len_range
            lens = [int(v) for v in rng.integers(lo, hi + 1, size=w.num_seqs)]
        batch, L = 1, int(sum(lens))
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
        nstate = len(lens)
    else:
        batch, L = w.batch, w.seqlen
        nstate = batch
    x = rng.standard_normal((batch, L, H, P), dtype=np.float32)
    B = rng.standard_normal((batch, L, G, N), dtype=np.float32)
    C = rng.standard_normal((batch, L, G, N), dtype=np.float32)
    z = rng.standard_normal((batch, L, H))
    u = rng.uniform(w.log_neg_a[0], w.log_neg_a[1], size=H)
    A = np.zeros(H) if w.a_zero else -np.exp(u)
    D = rng.standard_normal(H)
    h0 = None
    if w.h0_std > 0:
        h0 = torch.from_numpy(
            rng.normal(0.0, w.h0_std, size=(nstate, H, P, N)).astype(np.float32))
    bias = w.dt_bias
    if w.target_mean_decay is not None:
        bias = solve_dt_bias(z.reshape(-1, H), A, w.target_mean_decay)
    dt = _softplus(z + bias)
    return dict(
        x=_cast(x, w.dtype), dt=_cast(dt, w.dtype),
        A=torch.from_numpy(A.astype(np.float32)),
        B=_cast(B, w.dtype), C=_cast(C, w.dtype),
        D=torch.from_numpy(D.astype(np.float32)),
        h0=h0, cu_seqlens=cu, seq_lens=lens, workload=w, dt_bias=bias)


def scaled(w: Workload, **kw) -> Workload:
    """A smaller copy of a workload (same value recipe, new shape/seed)."""
    return replace(w, **kw)


def tokens(inp: dict) -> int:
    x = inp["x"]
    return int(x.shape[0] * x.shape[1])


def make_step_inputs(batch: int, nheads: int, headdim: int, dstate: int, ngroups: int,
                     dtype: str, seed: int, state_std: float = 0.1, steps: int = 1) -> dict:
    """Seeded inputs of ``steps`` decode steps (one token per sequence each),
    with the value recipe of the workloads above and a random fp32 state.

    Draw order: x, B, C, z, u (for A), D, state. Returns x (steps, batch, H, P),
    dt (steps, batch, H), B, C (steps, batch, G, N) in ``dtype``; A, D (H,)
    fp32; state (batch, H, P, N) fp32.
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((steps, batch, nheads, headdim), dtype=np.float32)
    B = rng.standard_normal((steps, batch, ngroups, dstate), dtype=np.float32)
    C = rng.standard_normal((steps, batch, ngroups, dstate), dtype=np.float32)
    z = rng.standard_normal((steps, batch, nheads))
    u = rng.uniform(0.0, 2.0, size=nheads)
    D = rng.standard_normal(nheads)
    state = rng.standard_normal((batch, nheads, headdim, dstate), dtype=np.float32) * np.float32(state_std)
    return dict(x=_cast(x, dtype), dt=_cast(_softplus(z - 2.0), dtype),
                A=torch.from_numpy((-np.exp(u)).astype(np.float32)),
                B=_cast(B, dtype), C=_cast(C, dtype),
                D=torch.from_numpy(D.astype(np.float32)),
                state=torch.from_numpy(state))


def make_scan_inputs(batch: int, seqlen: int, dim: int, dstate: int, dtype: str, seed: int,
                     h0_std: float = 0.0) -> dict:
    """Seeded inputs of the Mamba-1 selective scan, with the value recipe of
    the workloads above: x, B, C, D ~ N(0, 1); delta = softplus(z - 2);
    A[d, n] = -exp(U(0, 2)), one rate per channel and state index; an
    optional fp32 initial state ~ N(0, h0_std^2).

    Draw order: x, B, C, z, u (for A), D, h0. Returns x, delta (batch, L, dim)
    and B, C (batch, L, dstate) in ``dtype``; A (dim, dstate), D (dim,) and
    h0 (batch, dim, dstate) or None in fp32.
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, seqlen, dim), dtype=np.float32)
    B = rng.standard_normal((batch, seqlen, dstate), dtype=np.float32)
    C = rng.standard_normal((batch, seqlen, dstate), dtype=np.float32)
    z = rng.standard_normal((batch, seqlen, dim), dtype=np.float32)
    u = rng.uniform(0.0, 2.0, size=(dim, dstate))
    D = rng.standard_normal(dim)
    h0 = None
    if h0_std > 0:
        h0 = torch.from_numpy(rng.standard_normal((batch, dim, dstate), dtype=np.float32)
                              * np.float32(h0_std))
    return dict(x=_cast(x, dtype), delta=_cast(_softplus(z - 2.0), dtype),
                A=torch.from_numpy((-np.exp(u)).astype(np.float32)),
                B=_cast(B, dtype), C=_cast(C, dtype),
                D=torch.from_numpy(D.astype(np.float32)), h0=h0)


def make_conv_inputs(batch: int, seqlen: int, x_dim: int, bc_dim: int, width: int, dtype: str,
                     seed: int, seq_lens=None, history: bool = False, pad_cols: int = 0,
                     lead_cols: int = 0) -> dict:
    """Seeded inputs of the convolution front (packed x, B, C channels).

    Dense (``seq_lens`` None): ``batch`` rows of ``seqlen`` tokens. Packed
    (``seq_lens`` a list, batch 1): those lengths back to back, with
    cu_seqlens. The packed input rows are ``lead_cols + channels + pad_cols``
    wide and the channels start at ``lead_cols``, as when xBC is a slice of a
    wider projection output (``xbc`` is that slice, ``xbc_full`` the whole).

    Value recipe: inputs ~ N(0, 1); weight and bias ~ U(-1/sqrt(K),
    1/sqrt(K)), the usual fan-in bound of a K-tap filter; optional history
    ~ N(0, 1). Draw order: the full input rows, weight, bias, history.
    Inputs and history are rounded once to ``dtype``; weight and bias stay
    float32.
    """
    rng = np.random.default_rng(seed)
    ch = x_dim + 2 * bc_dim
    cu = None
    if seq_lens is not None:
        lens = [int(v) for v in seq_lens]
        T, nseq = int(sum(lens)), len(lens)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    else:
        T, nseq = batch * seqlen, batch
    full = rng.standard_normal((T, lead_cols + ch + pad_cols), dtype=np.float32)
    bound = 1.0 / np.sqrt(width)
    w = rng.uniform(-bound, bound, size=(ch, width)).astype(np.float32)
    b = rng.uniform(-bound, bound, size=ch).astype(np.float32)
    hist = None
    if history:
        hist = _cast(rng.standard_normal((nseq, width - 1, ch), dtype=np.float32), dtype)
    xbc_full = _cast(full, dtype)
    return dict(xbc_full=xbc_full, xbc=xbc_full[:, lead_cols:lead_cols + ch],
                weight=torch.from_numpy(w), bias=torch.from_numpy(b), history=hist,
                cu_seqlens=cu, num_seqs=0 if seq_lens is None else nseq, T=T,
                batch=batch if seq_lens is None else 1,
                seqlen=seqlen if seq_lens is None else T)


def make_grad_inputs(w: Workload, inp: dict, dhT_std: float = 0.1) -> dict:
    """Upstream gradients for the backward pass of workload ``w``: dy ~ N(0, 1)
    in the config dtype, shaped like x, and an fp32 dL/d(final state) ~
    N(0, dhT_std^2) shaped like the final state (None when dhT_std is 0).
    Drawn from their own stream (seed + 500) so the forward inputs of
    ``make_inputs(w)`` are unchanged. Draw order: dy, dhT."""
    rng = np.random.default_rng(w.seed + 500)
    x = inp["x"]
    dy = rng.standard_normal(tuple(x.shape), dtype=np.float32)
    nstate = len(inp["seq_lens"]) if inp["seq_lens"] is not None else x.shape[0]
    dhT = None
    if dhT_std > 0:
        dhT = torch.from_numpy(rng.standard_normal((nstate, w.nheads, w.headdim, w.dstate),
                                                   dtype=np.float32) * np.float32(dhT_std))
    return dict(dy=_cast(dy, w.dtype), dhT=dhT)
