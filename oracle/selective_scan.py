"""fp64 oracle of the Mamba-1 selective scan (S6), the comparator of the SSD
forward pass.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it, and the product library shares no code with it.

The selective SSM makes the step size and B, C functions of the input and
discretises with exp(step * A) (tj-hxxt.cn long read of the Mamba-1 paper,
part III (二), the selection mechanism, and item 3 on the roles of the step,
A, B and C). Its A is a diagonal N x D matrix, broadcast over the expanded
state of every channel, and the step has the shape of the input, batch x
length x channels (kuaisou snippet mapping the selective SSM to linear
attention). Mamba-2's core layer restricts A to one scalar per head; the pages
credit that restriction with a 2-8x speed-up over this scan (QbitAI CSDN
repost, abstract; briefgpt TL;DR).

For every sequence b, channel d and state index n, with the input term taken
as step * B * x (the same reading as the SSD oracle):

    h[b,d,n]  <- exp(delta[b,t,d] * A[d,n]) * h[b,d,n] + delta[b,t,d] * B[b,t,n] * x[b,t,d]
    y[b,t,d]   = sum_n C[b,t,n] * h[b,d,n] + D[d] * x[b,t,d]

Plain numpy in fp64: a loop over tokens, whole (batch, channel, state)
arrays per token.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        import torch
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def selective_scan(x, delta, A, B, C, D=None, h0=None, channels=None):
    """Run the scan over every token.

    x, delta (batch, L, Dm); A (Dm, N); B, C (batch, L, N); D (Dm,) or None;
    h0 (batch, Dm, N) or None (zeros). ``channels`` (optional index array)
    restricts the run to those channels; each channel is an independent
    recurrence, so the result for a channel does not depend on the others.
    Returns ``(y (batch, L, Dm'), h_final (batch, Dm', N))`` in fp64, Dm' the
    selected channels.
    """
    x, delta, A, B, C, D, h0 = (_f64(v) for v in (x, delta, A, B, C, D, h0))
    if channels is not None:
        channels = np.asarray(channels)
        x, delta, A = x[:, :, channels], delta[:, :, channels], A[channels]
        D = None if D is None else D[channels]
        h0 = None if h0 is None else h0[:, channels]
    batch, L, Dm = x.shape
    N = A.shape[1]
    h = np.zeros((batch, Dm, N)) if h0 is None else h0.copy()
    y = np.zeros((batch, L, Dm))
    for t in range(L):
        step = delta[:, t, :]                                  # (batch, Dm)
        decay = np.exp(step[:, :, None] * A[None, :, :])       # (batch, Dm, N)
        h = decay * h + (step * x[:, t, :])[:, :, None] * B[:, t, None, :]
        y[:, t, :] = np.einsum("bdn,bn->bd", h, C[:, t, :])
        if D is not None:
            y[:, t, :] += D[None, :] * x[:, t, :]
    return y, h
