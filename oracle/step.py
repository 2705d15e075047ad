"""fp64 oracle of one decode step of the SSD layer (the recurrent mode).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it, and the product library shares no code with it.

Generating one token at a time needs only the state of each (sequence, head):
the discretised SSM runs as a recurrence (tj-hxxt.cn long read of the Mamba-1
paper, part II (一), "from continuous systems to discrete modelling": S4's
discrete form can be evaluated recurrently or as a convolution), and the state
cache is what makes generation linear in the sequence length (same page, part
IV (五), "computational efficiency", the inference-speed item). One step is one
iteration of the token recurrence that the sequence oracle runs, with the same
readings (Euler input term dt*x*B^T, decay exp(dt*A) applied before the input
is added, output read from the updated state, D as a per-head skip, heads
mapped to groups contiguously).

For every sequence b and head h, with group g = h // (H / G):

    a              = exp(dt[b, h] * A[h])
    state'[b,h]    = a * state[b,h] + dt[b,h] * outer(x[b,h], B[b,g])    (P x N)
    y[b,h,p]       = sum_n C[b,g,n] * state'[b,h,p,n] + D[h] * x[b,h,p]

Plain numpy in fp64, no blocking or reordering.
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


def ssd_step(x, dt, A, B, C, D, state):
    """One decode step.

    x (batch, H, P); dt (batch, H), already positive; A (H,); B, C (batch, G, N);
    D (H,) or None (no skip term); state (batch, H, P, N). Any float dtype, taken
    exactly as fp64. Returns ``(y (batch, H, P), new_state (batch, H, P, N))``
    in fp64; the input state is not modified.
    """
    x, dt, A, B, C, D, state = (_f64(v) for v in (x, dt, A, B, C, D, state))
    batch, H, P = x.shape
    G = B.shape[1]
    if H % G != 0:
        raise ValueError("nheads %d not divisible by ngroups %d" % (H, G))
    group = np.arange(H) // (H // G)          # head h reads group h // (H/G)
    Bh = B[:, group, :]                       # (batch, H, N)
    Ch = C[:, group, :]
    a = np.exp(dt * A[None, :])               # per-step decay, (batch, H)
    new_state = (a[:, :, None, None] * state
                 + (dt[:, :, None] * x)[:, :, :, None] * Bh[:, :, None, :])
    y = np.einsum("bhpn,bhn->bhp", new_state, Ch)
    if D is not None:
        y = y + D[None, :, None] * x
    return y, new_state


def ssd_steps(x, dt, A, B, C, D, state):
    """``ssd_step`` applied to T tokens in order: x (T, batch, H, P), dt
    (T, batch, H), B, C (T, batch, G, N). Returns ``(y (T, batch, H, P),
    final_state)``."""
    x, dt, B, C = (_f64(v) for v in (x, dt, B, C))
    h = _f64(state)
    ys = []
    for t in range(x.shape[0]):
        y, h = ssd_step(x[t], dt[t], A, B[t], C[t], D, h)
        ys.append(y)
    return np.stack(ys), h
