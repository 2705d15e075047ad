"""fp64 oracle of the SSD layer's backward pass: the gradients of a scalar
loss through the token recurrence.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it, and the product library shares no code with it.

The forward recurrence (the same readings as the sequence oracle), per
sequence and head h with group g = h // (H / G):

    a_t   = exp(dt_t A_h)
    h_t   = a_t h_{t-1} + dt_t x_t B_t^T                 (P x N; h_{-1} = h0)
    y_t   = h_t C_t + D_h x_t

Training needs the gradients of a loss L given dL/dy_t (dy) and dL/dh_final
(dhT); the selective-scan kernel recomputes the states in the backward pass
instead of storing them (tj-hxxt.cn long read of the Mamba-1 paper, part III
(三), the efficient implementation: recomputation). This oracle stores every
state (it is small-input test infrastructure) and walks the tokens backwards
with the adjoint state G_t = dL/dh_t:

    G   <- dhT                                       (after the last token)
    for t from last to first:
        G       += dy_t C_t^T                        (y_t reads h_t)
        dC_t    += sum_p dy_t[p] h_t[p, :]           (summed over the group's heads)
        dx_t     = D_h dy_t + dt_t G B_t
        dB_t    += dt_t G^T x_t                      (summed over the group's heads)
        ddt_t    = <G, x_t B_t^T> + A_h a_t <G, h_{t-1}>
        dA_h    += dt_t a_t <G, h_{t-1}>
        dD_h    += <dy_t, x_t>
        G        = a_t G                             (h_t reads h_{t-1})
    dh0 = G

Packed sequences are independent: the adjoint restarts from dhT of each
sequence at its last token and stops at its first. Plain numpy in fp64, one
token at a time over whole (head, P, N) arrays.
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


def ssd_backward(x, dt, A, B, C, D, h0, seq_lens, dy, dhT=None):
    """Gradients of the SSD recurrence over a packed token stream.

    Shapes (T tokens, S sequences): x (T, H, P); dt (T, H) (positive, as the
    recurrence uses it); A (H,); B, C (T, G, N); D (H,) or None; h0
    (S, H, P, N) or None; seq_lens: S lengths summing to T; dy (T, H, P);
    dhT (S, H, P, N) or None (zero). Without D the layer has no skip term;
    dD is then the gradient at D = 0.

    Returns a dict of fp64 arrays: dx (T, H, P), ddt (T, H), dA (H,),
    dB (T, G, N), dC (T, G, N), dD (H,), dh0 (S, H, P, N), and the forward
    outputs y (T, H, P) and hT (S, H, P, N) it recomputed on the way.
    """
    x, dt, A, B, C, D, h0, dy, dhT = (_f64(v) for v in (x, dt, A, B, C, D, h0, dy, dhT))
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    grp = np.arange(H) // (H // G)                 # group of each head
    S = len(seq_lens)
    Dv = np.zeros(H) if D is None else D
    out = dict(dx=np.zeros((T, H, P)), ddt=np.zeros((T, H)), dA=np.zeros(H),
               dB=np.zeros((T, G, N)), dC=np.zeros((T, G, N)), dD=np.zeros(H),
               dh0=np.zeros((S, H, P, N)), y=np.zeros((T, H, P)), hT=np.zeros((S, H, P, N)))
    start = 0
    for s, L in enumerate(seq_lens):
        rows = range(start, start + L)
        # forward, keeping every state: hs[k] = state after token start + k - 1
        hs = np.zeros((L + 1, H, P, N))
        hs[0] = 0.0 if h0 is None else h0[s]
        for k, t in enumerate(rows):
            a = np.exp(dt[t] * A)                                   # (H,)
            Bh, Ch = B[t, grp], C[t, grp]                           # (H, N)
            hs[k + 1] = a[:, None, None] * hs[k] + \
                (dt[t][:, None] * x[t])[:, :, None] * Bh[:, None, :]
            out["y"][t] = np.einsum("hpn,hn->hp", hs[k + 1], Ch) + Dv[:, None] * x[t]
        out["hT"][s] = hs[L]
        # backward
        Gs = np.zeros((H, P, N)) if dhT is None else dhT[s].copy()
        for k in reversed(range(L)):
            t = start + k
            a = np.exp(dt[t] * A)
            Bh, Ch = B[t, grp], C[t, grp]
            Gs += dy[t][:, :, None] * Ch[:, None, :]
            np.add.at(out["dC"][t], grp, np.einsum("hp,hpn->hn", dy[t], hs[k + 1]))
            out["dx"][t] = Dv[:, None] * dy[t] + dt[t][:, None] * np.einsum("hpn,hn->hp", Gs, Bh)
            np.add.at(out["dB"][t], grp, dt[t][:, None] * np.einsum("hpn,hp->hn", Gs, x[t]))
            gh = np.einsum("hpn,hpn->h", Gs, hs[k])                 # <G, h_{t-1}>
            out["ddt"][t] = np.einsum("hpn,hp,hn->h", Gs, x[t], Bh) + A * a * gh
            out["dA"] += dt[t] * a * gh
            out["dD"] += np.einsum("hp,hp->h", dy[t], x[t])
            Gs = a[:, None, None] * Gs
        out["dh0"][s] = Gs
        start += L
    return out
