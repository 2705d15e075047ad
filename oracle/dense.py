"""Quadratic (masked-attention) form of the SSD forward pass, numpy fp64.

TEST INFRASTRUCTURE ONLY -- used to pin the recurrence in ``ssd_oracle.c`` on
tiny inputs; never called by the product library.

QbitAI "Mamba-2" article (srwj168 repost), section "Unifying SSM and
attention": a selective SSM is the multiplication of the input sequence by a
semiseparable matrix, and a masked attention with a semiseparable mask is the
same map; the kuaisou "mamba model explained" snippets identify C, B and the
input with query, key and value. Written out for one sequence and one head
(g = h // (H/G)), with log-decay a_k = dt_k * A_h:

    M[i, j] = (C_i . B_j) * exp(sum_{k=j+1..i} a_k) * dt_j      for i >= j
            = 0                                                 for i <  j
    y_i     = sum_j M[i, j] x_j  +  exp(sum_{k<=i} a_k) * (h0 C_i)  +  D_h x_i
    h_final = exp(sum_k a_k) * h0  +  sum_j exp(sum_{k>j} a_k) dt_j x_j B_j^T

No chunking and no reordering beyond these sums: the whole L x L matrix is
formed, so this is O(L^2) per head and only for small L.
"""
from __future__ import annotations

import numpy as np


def _segsum_exp(a: np.ndarray) -> np.ndarray:
    """E[i, j] = exp(sum_{k=j+1..i} a_k) for i >= j, 0 above the diagonal.

    The sums are taken explicitly (a double loop over the lower triangle with
    a running sum per column), not as differences of a prefix sum.
    """
    L = a.shape[0]
    E = np.zeros((L, L))
    for j in range(L):
        run = 0.0
        E[j, j] = 1.0
        for i in range(j + 1, L):
            run += a[i]
            E[i, j] = np.exp(run)
    return E


def ssd_dense(x, dt, A, B, C, D=None, h0=None, seq_lens=None):
    """Same signature and shapes as :func:`oracle.ssd_recurrence`."""
    x = np.asarray(x, np.float64)
    T, H, P = x.shape
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    G, N = B.shape[1], B.shape[2]
    if seq_lens is None:
        seq_lens = [T]
    S = len(seq_lens)
    y = np.zeros((T, H, P))
    hT = np.zeros((S, H, P, N))
    start = 0
    for s, L in enumerate(seq_lens):
        sl = slice(start, start + L)
        for h in range(H):
            g = h // (H // G)
            a = dt[sl, h] * A[h]                       # per-token log-decay
            E = _segsum_exp(a)                          # L x L, lower
            CB = C[sl, g, :] @ B[sl, g, :].T            # L x L, (C_i . B_j)
            M = CB * E * dt[sl, h][None, :]             # semiseparable mask
            ys = M @ x[sl, h, :]
            to_end = np.array([np.exp(a[j + 1:].sum()) for j in range(L)])
            hs = (x[sl, h, :] * (dt[sl, h] * to_end)[:, None]).T @ B[sl, g, :]
            if h0 is not None:
                h0sh = np.asarray(h0, np.float64)[s, h]     # P x N
                from_start = np.array([np.exp(a[:i + 1].sum()) for i in range(L)])
                ys = ys + from_start[:, None] * (C[sl, g, :] @ h0sh.T)
                hs = hs + np.exp(a.sum()) * h0sh
            if D is not None:
                ys = ys + float(np.asarray(D)[h]) * x[sl, h, :]
            y[sl, h, :] = ys
            hT[s, h] = hs
        start += L
    return y, hT
