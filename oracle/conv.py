"""fp64 oracle of the convolution front of the SSD layer: a causal depthwise
1-D convolution over the packed (x, B, C) channels, then an activation.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it, and the product library shares no code with it.

What the pages fix: in the Mamba-2 model one part of the input projection goes
through a 1-D convolution that picks up local dependencies along the sequence,
and nothing may look at later tokens (CSDN csdn_xmj page, related-article
snippet on implementing the Mamba-2 model). The Mamba block puts an activation
where H3 put a gate, and H3 itself has a local convolution between its gates
(tj-hxxt.cn long read of the Mamba-1 paper, part II, the table of related
models, and part III, the closing paragraph on the selection mechanism).

Readings where the pages are silent:
  * depthwise: one filter of ``width`` taps per channel, no mixing of channels;
  * causal with the ``width - 1`` inputs before a sequence's first token taken
    from a per-sequence history (the inputs a previous call ended with), or
    zeros; packed sequences never see each other's tokens;
  * tap ``k`` of channel ``c`` multiplies the input ``width - 1 - k`` tokens
    back (``weight[c, width - 1]`` weighs the current token), plus a bias;
  * the activation is SiLU, v * sigmoid(v);
  * the channels are packed as [x (x_dim) | B (bc_dim) | C (bc_dim)], and the
    three parts come out as separate arrays.

For each sequence with inputs u_0 .. u_{L-1} (one row of channels per token)
and history rows h_0 .. h_{K-2} (oldest first), let e = [h_0 .. h_{K-2}, u_0 ..
u_{L-1}]. Then

    pre[t, c]  = bias[c] + sum_{k=0}^{K-1} weight[c, k] * e[t + k, c]
    out[t, c]  = pre[t, c] / (1 + exp(-pre[t, c]))
    history'   = the last K - 1 rows of e

Plain numpy in fp64: a loop over taps, whole (token, channel) arrays per tap.
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


def silu(v):
    """v * sigmoid(v), written as v / (1 + exp(-v))."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def causal_conv(u, weight, bias=None, history=None, activation=True):
    """One sequence: u (L, channels), weight (channels, K), bias (channels,)
    or None, history (K - 1, channels) or None (zeros).
    Returns (out (L, channels), history' (K - 1, channels))."""
    u, weight, bias, history = (_f64(v) for v in (u, weight, bias, history))
    L, ch = u.shape
    K = weight.shape[1]
    if history is None:
        history = np.zeros((K - 1, ch))
    e = np.concatenate([history, u], axis=0)               # (K - 1 + L, ch)
    pre = np.zeros((L, ch)) if bias is None else np.repeat(bias[None, :], L, axis=0)
    for k in range(K):
        pre = pre + weight[None, :, k] * e[k:k + L]
    out = silu(pre) if activation else pre
    return out, e[len(e) - (K - 1):].copy()


def conv_front(xbc, weight, bias, seq_bounds, x_dim, bc_dim, history=None,
               activation=True):
    """The packed front: xbc (T, x_dim + 2 * bc_dim) holds the tokens of the
    sequences ``seq_bounds`` [(start, end), ...] (each a half-open token
    range); history (num_seqs, K - 1, channels) or None.

    Returns (x (T, x_dim), B (T, bc_dim), C (T, bc_dim),
    history' (num_seqs, K - 1, channels)). Tokens outside every sequence stay
    zero."""
    xbc, weight, bias, history = (_f64(v) for v in (xbc, weight, bias, history))
    T, ch = xbc.shape
    assert ch == x_dim + 2 * bc_dim
    K = weight.shape[1]
    out = np.zeros((T, ch))
    hist_out = np.zeros((len(seq_bounds), K - 1, ch))
    for s, (a, b) in enumerate(seq_bounds):
        o, h = causal_conv(xbc[a:b], weight, bias,
                           None if history is None else history[s], activation)
        out[a:b] = o
        hist_out[s] = h
    return (out[:, :x_dim], out[:, x_dim:x_dim + bc_dim], out[:, x_dim + bc_dim:], hist_out)


def dense_bounds(batch, seqlen):
    """The sequences of a dense batch: row b holds tokens [b L, (b + 1) L)."""
    return [(b * seqlen, (b + 1) * seqlen) for b in range(batch)]


def varlen_bounds(cu_seqlens):
    """The sequences of a packed batch from its cumulative offsets."""
    cu = [int(v) for v in cu_seqlens]
    return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
