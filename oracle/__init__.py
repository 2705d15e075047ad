"""fp64 CPU oracle of the Mamba-2 SSD forward pass.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
library (``mamba_ssd_sequence_fwd_amd``) never imports it and shares no code
with it; the two meet only through the seeded inputs of ``ssd_inputs``.

Two independent formulations of the same linear map:

* :func:`ssd_recurrence` -- the token-by-token recurrence in C (``ssd_oracle.c``),
  fp64, OpenMP over (sequence, head) pairs. This is the oracle proper.
* :func:`oracle.dense.ssd_dense` -- the quadratic "masked attention" form
  y = (L o C B^T) (dt o x) + decay * C h0 + D x, in numpy, for tiny inputs.
  It pins the recurrence (QbitAI "Mamba-2" article, srwj168 repost, section
  "Unifying SSM and attention": an SSM is multiplication by a semiseparable
  matrix, equivalently a masked attention whose mask is that matrix).

A third module, :mod:`oracle.step`, is the decode step (one token of the
recurrence per sequence, the state carried by the caller), a fourth,
:mod:`oracle.selective_scan`, the Mamba-1 selective scan (a diagonal A per
channel) that the SSD layer is compared with, and a fifth, :mod:`oracle.conv`,
the causal depthwise convolution and activation that produce the layer's x,
B and C, and a sixth, :mod:`oracle.backward`, the gradients of the recurrence
(the backward pass), all in numpy.

Every function here is plain and slow on purpose.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile ``ssd_oracle.c`` into ``libssd_oracle.so`` with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load(path: str | None = None):
    """Load the oracle library (``path`` selects another build of the same
    source, e.g. a deliberately mutated copy in a test)."""
    global _lib
    with _lock:
        if path is None and _lib is not None:
            return _lib
        if path is None:
            build()
        lib = ctypes.CDLL(path or _LIB_PATH)
        f = lib.ssd_oracle_forward
        i64 = ctypes.c_int64
        dp = ctypes.c_void_p
        f.argtypes = [i64, dp, dp, i64, i64, i64, i64, dp, dp, dp, dp, dp,
                      dp, dp, dp, dp, i64, dp, ctypes.c_int]
        f.restype = ctypes.c_int
        if path is None:
            _lib = lib
    return lib


def _f64(a, shape=None):
    if a is None:
        return None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError("oracle: expected shape %s, got %s" % (shape, arr.shape))
    return arr


def _ptr(a):
    return None if a is None else a.ctypes.data


def seq_layout(total_tokens: int, seq_lens=None):
    """Start offset and length of each sequence in the packed token stream."""
    if seq_lens is None:
        seq_lens = [total_tokens]
    lens = np.asarray(seq_lens, dtype=np.int64)
    starts = np.zeros_like(lens)
    if len(lens) > 1:
        starts[1:] = np.cumsum(lens)[:-1]
    if lens.sum() != total_tokens:
        raise ValueError("sequence lengths do not add up to the token count")
    return starts, lens


def ssd_recurrence(x, dt, A, B, C, D=None, h0=None, seq_lens=None,
                   snap_every: int = 0, threads: int = 0, lib=None):
    """Run the fp64 recurrence over a packed token stream.

    Shapes (T = total tokens, S = number of sequences):
      x (T, H, P); dt (T, H), already positive; A (H,); B, C (T, G, N);
      D (H,) or None; h0 (S, H, P, N) or None; seq_lens: S lengths summing to T
      (None = one sequence). A dense batch of shape (batch, L, ...) is the same
      stream with ``seq_lens = [L] * batch``.

    Returns ``(y (T, H, P), h_final (S, H, P, N))`` and, with ``snap_every=Q``,
    also the states entering each Q-chunk, ``(sum_s ceil(len_s/Q), H, P, N)``.
    """
    x = _f64(x)
    T, H, P = x.shape
    dt = _f64(dt, (T, H))
    A = _f64(A, (H,))
    B = _f64(B)
    G, N = B.shape[1], B.shape[2]
    B = _f64(B, (T, G, N))
    C = _f64(C, (T, G, N))
    D = _f64(D, (H,))
    starts, lens = seq_layout(T, seq_lens)
    S = len(lens)
    h0 = _f64(h0, (S, H, P, N))
    y = np.zeros((T, H, P))
    hT = np.zeros((S, H, P, N))
    snaps = None
    if snap_every:
        nsnap = int(sum((int(L) + snap_every - 1) // snap_every for L in lens))
        snaps = np.zeros((nsnap, H, P, N))
    rc = (lib or _load()).ssd_oracle_forward(
        S, _ptr(starts), _ptr(lens), H, P, N, G, _ptr(x), _ptr(dt), _ptr(A),
        _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(hT),
        int(snap_every), _ptr(snaps), int(threads))
    if rc != 0:
        raise RuntimeError("ssd_oracle_forward failed with code %d" % rc)
    if snap_every:
        return y, hT, snaps
    return y, hT


def ssd_pairs(x, dt, A, B, C, D, h0, seq_lens, pairs, threads: int = 0):
    """Oracle outputs for a sample of (sequence, head) pairs only.

    ``x``... are full-size CPU arrays or tensors in any float dtype (upcast
    exactly to fp64 slice by slice); ``pairs`` lists (s, h). Returns a dict
    {(s, h): (y_slice (len_s, P), h_final_slice (P, N))}. Each pair is an
    independent run of the recurrence, so sampling changes nothing in what is
    computed for that pair.
    """
    T, H, P = x.shape
    G = B.shape[1]
    starts, lens = seq_layout(T, seq_lens)
    pairs = [(int(s), int(h)) for s, h in pairs]

    def one(pair):
        s, h = pair
        a, L = int(starts[s]), int(lens[s])
        g = h // (H // G)
        y, hT = ssd_recurrence(
            _np(x[a:a + L, h:h + 1, :]), _np(dt[a:a + L, h:h + 1]),
            _np(A[h:h + 1]), _np(B[a:a + L, g:g + 1, :]),
            _np(C[a:a + L, g:g + 1, :]),
            None if D is None else _np(D[h:h + 1]),
            None if h0 is None else _np(h0[s:s + 1, h:h + 1]),
            threads=1)
        return pair, (y[:, 0, :], hT[0, 0])

    # The C call releases the GIL, so a thread pool runs the pairs in
    # parallel; each pair is an independent run of the recurrence.
    workers = threads if threads > 0 else default_threads()
    with ThreadPoolExecutor(max_workers=max(1, min(workers, len(pairs)))) as ex:
        return dict(ex.map(one, pairs))


def default_threads() -> int:
    """Host threads the oracle may use: OMP_NUM_THREADS if set, else the CPUs
    this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _np(a):
    """Exact fp64 numpy view of a numpy array or a CPU torch tensor."""
    if hasattr(a, "detach"):
        import torch
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def chunk_log_decay(dt, A, seq_lens, Q: int):
    """Natural-log decay from each chunk's start through each of its tokens:
    sum of dt_k * A_h over the chunk's tokens up to and including token l
    (the log of the product of the per-step decays exp(dt*A)).

    Returns (chunks, H, Q) fp64 with chunks numbered sequence by sequence and
    NaN past a partial chunk's end -- the same numbering as the snapshots of
    :func:`ssd_recurrence`.
    """
    dt = np.asarray(_np(dt), np.float64)
    A = np.asarray(_np(A), np.float64)
    T, H = dt.shape
    starts, lens = seq_layout(T, seq_lens)
    out = []
    for a, L in zip(starts, lens):
        for c0 in range(0, int(L), Q):
            n = min(Q, int(L) - c0)
            block = np.full((H, Q), np.nan)
            block[:, :n] = np.cumsum(dt[a + c0:a + c0 + n] * A[None, :], axis=0).T
            out.append(block)
    return np.stack(out) if out else np.zeros((0, H, Q))


def dt_softplus(dt_raw, dt_bias=None):
    """The step as the recurrence uses it when the caller passes the step's
    pre-activation: softplus(dt_raw + dt_bias[h]), in fp64.

    The selection mechanism makes the step a function of the input and passes
    it through the softplus activation (tj-hxxt.cn long read of the Mamba-1
    paper, part III (二), the step's activation tau_delta); dt_bias is the
    learned per-head offset added before it. dt_raw (..., H) in any float
    dtype, dt_bias (H,) or None. softplus(v) = log(1 + e^v), evaluated as
    logaddexp(0, v) so that large v does not overflow.
    """
    v = _np(dt_raw)
    if dt_bias is not None:
        v = v + _np(dt_bias)
    return np.logaddexp(0.0, v)
