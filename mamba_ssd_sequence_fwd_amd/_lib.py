"""ctypes binding of ``libssd.so`` (declared in ``include/ssd.h``).

Argument marshalling only: torch provides device memory and the current HIP
stream; every step of the SSD forward pass runs in the library's kernels.
There is no CPU fallback -- if the library is missing, import succeeds but
every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssd.so")

SSD_OK, SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP = range(5)
SSD_DTYPE_F32, SSD_DTYPE_BF16 = 0, 1
SSD_FLAG_GENERIC_KERNELS = 1
SSD_FLAG_UNFUSED = 2
SSD_FLAG_PER_SEQUENCE = 4


class SSDError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, _status_string(status), detail))


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("dstate", ctypes.c_int32), ("ngroups", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]

    def __repr__(self):
        return "Problem(%s)" % ", ".join("%s=%s" % (f, getattr(self, f)) for f, _ in self._fields_)


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [("chunk_cumsum", ctypes.c_size_t), ("chunk_states", ctypes.c_size_t),
                ("chunk_table", ctypes.c_size_t), ("chunk_records", ctypes.c_int64),
                ("max_chunks", ctypes.c_int64), ("chain_sync", ctypes.c_size_t),
                ("chain_sync_words", ctypes.c_int64), ("chain_chunks_per_unit", ctypes.c_int64),
                ("chain_ranges", ctypes.c_int64)]


class ScanProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("dstate", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class ConvProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("x_dim", ctypes.c_int32),
                ("bc_dim", ctypes.c_int32), ("width", ctypes.c_int32),
                ("in_stride", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


MAX_STAGES = 12


class StageTimes(ctypes.Structure):
    _fields_ = [("num_stages", ctypes.c_int32), ("iterations", ctypes.c_int32),
                ("names", (ctypes.c_char * 24) * MAX_STAGES),
                ("ms", ctypes.c_float * MAX_STAGES), ("total_ms", ctypes.c_float)]

    def as_dict(self):
        """{kernel name: mean ms per launch}, plus '_total_ms' (all iterations)."""
        out = {self.names[k].value.decode(): self.ms[k] / max(self.iterations, 1)
               for k in range(self.num_stages)}
        out["_total_ms"] = self.total_ms
        return out


EXPORTED = ("ssd_validate", "ssd_validate_cu_seqlens", "ssd_workspace_size",
            "ssd_forward", "ssd_forward_noalloc", "ssd_forward_dt_softplus",
            "ssd_forward_timed", "ssd_step",
            "ssd_selective_scan", "ssd_conv1d_silu",
            "ssd_backward_workspace_size", "ssd_backward", "ssd_backward_timed",
            "ssd_get_workspace_layout",
            "ssd_status_string", "ssd_last_error_detail")

_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH):
    """Load libssd.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                "libssd.so is not built (%s); run `python -m mamba_ssd_sequence_fwd_amd.build`"
                % path)
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER(Problem)
        vp = ctypes.c_void_p
        lib.ssd_validate.argtypes = [P]
        lib.ssd_validate_cu_seqlens.argtypes = [P, vp]
        lib.ssd_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        lib.ssd_get_workspace_layout.argtypes = [P, ctypes.POINTER(WorkspaceLayout)]
        lib.ssd_forward.argtypes = [P] + [vp] * 11 + [ctypes.c_size_t, vp]
        lib.ssd_forward_noalloc.argtypes = [P] + [vp] * 11
        lib.ssd_forward_timed.argtypes = ([P] + [vp] * 11 + [ctypes.c_size_t, vp, ctypes.c_int32,
                                          ctypes.POINTER(StageTimes)])
        lib.ssd_step.argtypes = [P] + [vp] * 9
        lib.ssd_forward_dt_softplus.argtypes = [P] + [vp] * 12 + [ctypes.c_size_t, vp]
        lib.ssd_selective_scan.argtypes = [ctypes.POINTER(ScanProblem)] + [vp] * 10
        lib.ssd_conv1d_silu.argtypes = [ctypes.POINTER(ConvProblem)] + [vp] * 10
        lib.ssd_backward_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        lib.ssd_backward.argtypes = [P] + [vp] * 18 + [ctypes.c_size_t, vp]
        lib.ssd_backward_timed.argtypes = ([P] + [vp] * 18 + [ctypes.c_size_t, vp,
                                           ctypes.c_int32, ctypes.POINTER(StageTimes)])
        for f in ("ssd_validate", "ssd_validate_cu_seqlens", "ssd_workspace_size",
                  "ssd_get_workspace_layout", "ssd_forward", "ssd_forward_noalloc",
                  "ssd_forward_timed", "ssd_step",
                  "ssd_selective_scan", "ssd_forward_dt_softplus"):
            getattr(lib, f).restype = ctypes.c_int
        lib.ssd_status_string.argtypes = [ctypes.c_int]
        lib.ssd_status_string.restype = ctypes.c_char_p
        lib.ssd_last_error_detail.argtypes = []
        lib.ssd_last_error_detail.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _status_string(st: int) -> str:
    try:
        return load().ssd_status_string(st).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "status %d" % st


def _check(st: int, where: str):
    if st != SSD_OK:
        raise SSDError(st, where, load().ssd_last_error_detail().decode())


def make_problem(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size,
                 num_seqs=0, dtype=SSD_DTYPE_BF16, flags=0) -> Problem:
    return Problem(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size,
                   num_seqs, dtype, flags)


def validate(prob: Problem):
    _check(load().ssd_validate(ctypes.byref(prob)), "ssd_validate")


def validate_cu_seqlens(prob: Problem, cu_host):
    cu = torch.as_tensor(cu_host, dtype=torch.int32).contiguous().cpu()
    _check(load().ssd_validate_cu_seqlens(ctypes.byref(prob), ctypes.c_void_p(cu.data_ptr())),
           "ssd_validate_cu_seqlens")


def workspace_size(prob: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(load().ssd_workspace_size(ctypes.byref(prob), ctypes.byref(n)), "ssd_workspace_size")
    return int(n.value)


def workspace_layout(prob: Problem) -> WorkspaceLayout:
    lay = WorkspaceLayout()
    _check(load().ssd_get_workspace_layout(ctypes.byref(prob), ctypes.byref(lay)),
           "ssd_get_workspace_layout")
    return lay


_DTYPES = {torch.bfloat16: SSD_DTYPE_BF16, torch.float32: SSD_DTYPE_F32}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _same_device(dev, **tensors):
    """Every tensor a kernel reads or writes must live on ``dev`` (the device
    of the first input): a host pointer handed to a kernel would fault the GPU
    instead of raising. Checked before anything is launched."""
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError("%s is on %s, but the other inputs are on %s" % (name, t.device, dev))


def _on_gpu(dev):
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU (got %s)" % dev)


class Plan:
    """A prepared ssd_forward call: validated problem, outputs and workspace
    allocated once; :meth:`run` only enqueues the kernels.

    Shapes: x (batch, L, H, P); dt (batch, L, H); A (H,) fp32; B, C
    (batch, L, G, N); D (H,) fp32 or None; initial_state (batch | num_seqs,
    H, P, N) fp32 or None; cu_seqlens (num_seqs + 1,) int32 (CPU or GPU) or
    None. x, dt, B, C share the dtype (bfloat16 or float32).

    With ``dt_softplus=True`` dt holds the step's pre-activation and the
    kernels use softplus(dt + dt_bias[h]) (ssd_forward_dt_softplus); dt_bias
    is (H,) fp32 or None.
    """

    def __init__(self, x, dt, A, B, C, D=None, initial_state=None, chunk_size=256,
                 cu_seqlens=None, *, want_final_state=True, generic=False,
                 unfused=False, per_sequence=False, check_cu_seqlens=True,
                 dt_softplus=False, dt_bias=None):
        if x.dim() != 4:
            raise ValueError("x must be (batch, seqlen, nheads, headdim)")
        batch, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        dev = x.device
        _same_device(dev, dt=dt, A=A, B=B, C=C, D=D, initial_state=initial_state,
                     dt_bias=dt_bias)
        _on_gpu(dev)
        if x.dtype not in _DTYPES:
            raise ValueError("x must be bfloat16 or float32")
        for name, t, shape in (("dt", dt, (batch, L, H)), ("B", B, (batch, L, G, N)),
                               ("C", C, (batch, L, G, N))):
            if tuple(t.shape) != shape or t.dtype != x.dtype or t.device != dev:
                raise ValueError("%s must be %s %s on %s" % (name, shape, x.dtype, dev))
        if tuple(A.shape) != (H,) or A.dtype != torch.float32:
            raise ValueError("A must be (H,) float32")
        if D is not None and (tuple(D.shape) != (H,) or D.dtype != torch.float32):
            raise ValueError("D must be (H,) float32")
        num_seqs = 0
        cu_dev = None
        if cu_seqlens is not None:
            if batch != 1:
                raise ValueError("cu_seqlens needs batch == 1")
            num_seqs = int(cu_seqlens.numel()) - 1
        nstate = num_seqs if num_seqs else batch
        if initial_state is not None and (
                tuple(initial_state.shape) != (nstate, H, P, N)
                or initial_state.dtype != torch.float32):
            raise ValueError("initial_state must be (%d, %d, %d, %d) float32" % (nstate, H, P, N))
        self.prob = make_problem(batch, L, H, P, N, G, chunk_size, num_seqs,
                                 _DTYPES[x.dtype],
                                 (SSD_FLAG_GENERIC_KERNELS if generic else 0)
                                 | (SSD_FLAG_UNFUSED if unfused else 0)
                                 | (SSD_FLAG_PER_SEQUENCE if per_sequence else 0))
        validate(self.prob)
        if cu_seqlens is not None:
            if check_cu_seqlens or cu_seqlens.device.type == "cpu":
                validate_cu_seqlens(self.prob, cu_seqlens.detach().cpu())
            cu_dev = cu_seqlens.to(device=dev, dtype=torch.int32).contiguous()
        if dt_bias is not None:
            if not dt_softplus:
                raise ValueError("dt_bias needs dt_softplus=True")
            if tuple(dt_bias.shape) != (H,) or dt_bias.dtype != torch.float32 or dt_bias.device != dev:
                raise ValueError("dt_bias must be (H,) float32 on %s" % dev)
            dt_bias = dt_bias.contiguous()
        self.dt_softplus = bool(dt_softplus)
        self.dt_bias = dt_bias
        self.inputs = [t.contiguous() if t is not None else None
                       for t in (x, dt, A, B, C, D, initial_state)]
        self.cu = cu_dev
        self.y = torch.empty_like(x)
        self.final_state = (torch.empty((nstate, H, P, N), device=dev, dtype=torch.float32)
                            if want_final_state else None)
        self.ws_bytes = workspace_size(self.prob)
        self.workspace = torch.empty(max(self.ws_bytes, 256), device=dev, dtype=torch.uint8)
        self.tokens = batch * L

    def run(self, stream=None):
        """Enqueue one forward pass on ``stream`` (default: torch's current)."""
        if stream is None:
            stream = torch.cuda.current_stream(self.y.device)
        x, dt, A, B, C, D, h0 = self.inputs
        if self.dt_softplus:
            _check(load().ssd_forward_dt_softplus(
                ctypes.byref(self.prob), _ptr(x), _ptr(dt), _ptr(self.dt_bias), _ptr(A),
                _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(self.cu), _ptr(self.y),
                _ptr(self.final_state), _ptr(self.workspace),
                ctypes.c_size_t(self.workspace.numel()), ctypes.c_void_p(stream.cuda_stream)),
                "ssd_forward_dt_softplus")
            return self.y, self.final_state
        _check(load().ssd_forward(
            ctypes.byref(self.prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(h0), _ptr(self.cu), _ptr(self.y), _ptr(self.final_state),
            _ptr(self.workspace), ctypes.c_size_t(self.workspace.numel()),
            ctypes.c_void_p(stream.cuda_stream)), "ssd_forward")
        return self.y, self.final_state

    def run_timed(self, iterations: int, stream=None) -> StageTimes:
        """``iterations`` passes with a HIP event after every kernel; waits for
        them and returns the per-kernel times (see ssd_forward_timed)."""
        if self.dt_softplus:
            raise ValueError("run_timed times ssd_forward; it has no raw-step variant")
        if stream is None:
            stream = torch.cuda.current_stream(self.y.device)
        x, dt, A, B, C, D, h0 = self.inputs
        times = StageTimes()
        _check(load().ssd_forward_timed(
            ctypes.byref(self.prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(h0), _ptr(self.cu), _ptr(self.y), _ptr(self.final_state),
            _ptr(self.workspace), ctypes.c_size_t(self.workspace.numel()),
            ctypes.c_void_p(stream.cuda_stream), int(iterations), ctypes.byref(times)),
            "ssd_forward_timed")
        return times

    def layout(self) -> WorkspaceLayout:
        return workspace_layout(self.prob)

    def chain_error(self) -> int:
        """Error word of the chained kernel after the passes run so far
        (synchronises): nonzero if a workgroup gave up waiting for its
        predecessor's state. 0 when the problem does not use that kernel."""
        lay = self.layout()
        if lay.chain_sync_words == 0:
            return 0
        torch.cuda.synchronize(self.workspace.device)
        w = self.workspace[lay.chain_sync:lay.chain_sync + 8].view(torch.int32)
        return int(w[1].item())

    def check(self):
        """Wait for the passes run so far and raise SSDError if the chained
        kernel's error word is set (see :meth:`chain_error`)."""
        err = self.chain_error()
        if err:
            raise SSDError(SSD_ERR_HIP, "ssd_forward",
                           "a chained workgroup timed out waiting for its predecessor's "
                           "state (error word %d); the outputs are invalid" % err)


def forward(x, dt, A, B, C, D=None, initial_state=None, chunk_size=256, cu_seqlens=None,
            *, check=False, **kw):
    """SSD forward pass: returns (y, final_state).

    With ``check=True`` the call waits for the pass and raises SSDError if a
    chained workgroup gave up waiting for its predecessor's state (the error
    word of the workspace; the outputs are then wrong)."""
    plan = Plan(x, dt, A, B, C, D, initial_state, chunk_size, cu_seqlens, **kw)
    y, hT = plan.run()
    if check:
        plan.check()
    return y, hT


def forward_noalloc(x, dt, A, B, C, D, initial_state, y, final_state, chunk_size=256,
                    cu_seqlens=None, *, stream=None):
    """ssd_forward_noalloc: the forward pass into caller-provided ``y`` and
    ``final_state`` (or None) with the library's fixed device scratch area as
    the workspace; nothing is allocated. Tensors as for :class:`Plan`, all on
    one GPU; ``cu_seqlens`` int32 on that GPU (no host copy, no check of its
    values here). Calls that may overlap on one GPU race on the scratch area.
    """
    if x.dim() != 4:
        raise ValueError("x must be (batch, seqlen, nheads, headdim)")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    _same_device(dev, dt=dt, A=A, B=B, C=C, D=D, initial_state=initial_state, y=y,
                 final_state=final_state, cu_seqlens=cu_seqlens)
    _on_gpu(dev)
    if x.dtype not in _DTYPES:
        raise ValueError("x must be bfloat16 or float32")
    num_seqs = 0 if cu_seqlens is None else int(cu_seqlens.numel()) - 1
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or batch != 1):
        raise ValueError("cu_seqlens must be int32 with batch == 1")
    nstate = num_seqs if num_seqs else batch
    for name, t, shape, dtype in (
            ("dt", dt, (batch, L, H), x.dtype), ("B", B, (batch, L, G, N), x.dtype),
            ("C", C, (batch, L, G, N), x.dtype), ("A", A, (H,), torch.float32),
            ("D", D, (H,), torch.float32), ("y", y, (batch, L, H, P), x.dtype),
            ("initial_state", initial_state, (nstate, H, P, N), torch.float32),
            ("final_state", final_state, (nstate, H, P, N), torch.float32)):
        if t is None and name in ("dt", "B", "C", "A", "y"):
            raise ValueError("%s is required" % name)
        if t is not None and (tuple(t.shape) != shape or t.dtype != dtype
                              or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous %s %s tensor" % (name, shape, dtype))
    for name, t in (("x", x), ("cu_seqlens", cu_seqlens)):
        if t is not None and not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    prob = make_problem(batch, L, H, P, N, G, chunk_size, num_seqs, _DTYPES[x.dtype], 0)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _check(load().ssd_forward_noalloc(
        ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(initial_state), _ptr(cu_seqlens), _ptr(y), _ptr(final_state),
        ctypes.c_void_p(stream.cuda_stream)), "ssd_forward_noalloc")
    return y, final_state


def step(x, dt, A, B, C, D=None, state=None, *, y=None, stream=None):
    """One decode step (ssd_step): every sequence advances by one token and
    ``state`` is updated IN PLACE; returns y.

    Shapes: x (batch, H, P); dt (batch, H); A (H,) fp32; B, C (batch, G, N);
    D (H,) fp32 or None; state (batch, H, P, N) fp32, contiguous; y (optional
    output) like x. x, dt, B, C share the dtype (bfloat16 or float32).
    """
    if x.dim() != 3:
        raise ValueError("x must be (batch, nheads, headdim)")
    batch, H, P = x.shape
    if B.dim() != 3:
        raise ValueError("B must be (batch, ngroups, dstate)")
    G, N = B.shape[1], B.shape[2]
    dev = x.device
    _same_device(dev, dt=dt, A=A, B=B, C=C, D=D, state=state, y=y)
    _on_gpu(dev)
    if x.dtype not in _DTYPES:
        raise ValueError("x must be bfloat16 or float32")
    for name, t, shape in (("dt", dt, (batch, H)), ("B", B, (batch, G, N)),
                           ("C", C, (batch, G, N))):
        if tuple(t.shape) != shape or t.dtype != x.dtype or t.device != dev:
            raise ValueError("%s must be %s %s on %s" % (name, shape, x.dtype, dev))
    if tuple(A.shape) != (H,) or A.dtype != torch.float32:
        raise ValueError("A must be (H,) float32")
    if D is not None and (tuple(D.shape) != (H,) or D.dtype != torch.float32):
        raise ValueError("D must be (H,) float32")
    if (state is None or tuple(state.shape) != (batch, H, P, N)
            or state.dtype != torch.float32 or not state.is_contiguous()
            or state.device != dev):
        raise ValueError("state must be a contiguous (%d, %d, %d, %d) float32 tensor on %s"
                         % (batch, H, P, N, dev))
    if y is None:
        y = torch.empty_like(x, memory_format=torch.contiguous_format)
    elif tuple(y.shape) != (batch, H, P) or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("y must be a contiguous (%d, %d, %d) %s tensor" % (batch, H, P, x.dtype))
    prob = make_problem(batch, 1, H, P, N, G, 0, 0, _DTYPES[x.dtype], 0)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    # copies of non-contiguous inputs are made on the stream the kernel runs
    # on, so they are complete before it reads them and their memory is not
    # reused before it has run
    with torch.cuda.stream(stream):
        x, dt, A, B, C = (t.contiguous() for t in (x, dt, A, B, C))
        D = D.contiguous() if D is not None else None
    _check(load().ssd_step(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                           _ptr(D), _ptr(state), _ptr(y), ctypes.c_void_p(stream.cuda_stream)),
           "ssd_step")
    return y


def selective_scan(x, delta, A, B, C, D=None, initial_state=None, *, want_final_state=True,
                   y=None, final_state=None, stream=None):
    """The Mamba-1 selective scan (ssd_selective_scan): returns (y, final_state).

    Shapes: x, delta (batch, L, dim); A (dim, N) fp32; B, C (batch, L, N);
    D (dim,) fp32 or None; initial_state (batch, dim, N) fp32 or None. x,
    delta, B, C share the dtype (bfloat16 or float32); dim must be a multiple
    of 64 and N one of 16, 32, 64, 128, 256.
    """
    if x.dim() != 3:
        raise ValueError("x must be (batch, seqlen, dim)")
    batch, L, Dm = x.shape
    if A.dim() != 2 or A.shape[0] != Dm or A.dtype != torch.float32:
        raise ValueError("A must be (dim, dstate) float32")
    N = A.shape[1]
    dev = x.device
    _same_device(dev, delta=delta, A=A, B=B, C=C, D=D, initial_state=initial_state, y=y,
                 final_state=final_state)
    _on_gpu(dev)
    if x.dtype not in _DTYPES:
        raise ValueError("x must be bfloat16 or float32")
    for name, t, shape in (("delta", delta, (batch, L, Dm)), ("B", B, (batch, L, N)),
                           ("C", C, (batch, L, N))):
        if tuple(t.shape) != shape or t.dtype != x.dtype or t.device != dev:
            raise ValueError("%s must be %s %s on %s" % (name, shape, x.dtype, dev))
    if D is not None and (tuple(D.shape) != (Dm,) or D.dtype != torch.float32):
        raise ValueError("D must be (dim,) float32")
    if initial_state is not None and (tuple(initial_state.shape) != (batch, Dm, N)
                                      or initial_state.dtype != torch.float32):
        raise ValueError("initial_state must be (%d, %d, %d) float32" % (batch, Dm, N))
    prob = ScanProblem(batch, L, Dm, N, _DTYPES[x.dtype], 0)
    if y is not None and (tuple(y.shape) != (batch, L, Dm) or y.dtype != x.dtype
                          or not y.is_contiguous()):
        raise ValueError("y must be a contiguous (%d, %d, %d) %s tensor" % (batch, L, Dm, x.dtype))
    if final_state is not None and (tuple(final_state.shape) != (batch, Dm, N)
                                    or final_state.dtype != torch.float32
                                    or not final_state.is_contiguous()):
        raise ValueError("final_state must be a contiguous (%d, %d, %d) float32 tensor"
                         % (batch, Dm, N))
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    # copies and outputs are made on the stream the kernel runs on (see step())
    with torch.cuda.stream(stream):
        x, delta, A, B, C = (t.contiguous() for t in (x, delta, A, B, C))
        D = D.contiguous() if D is not None else None
        h0 = initial_state.contiguous() if initial_state is not None else None
        if y is None:
            y = torch.empty_like(x)
        if final_state is None and want_final_state:
            final_state = torch.empty((batch, Dm, N), device=dev, dtype=torch.float32)
    _check(load().ssd_selective_scan(ctypes.byref(prob), _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                                     _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(final_state),
                                     ctypes.c_void_p(stream.cuda_stream)),
           "ssd_selective_scan")
    return y, final_state


def _check_offsets(cu, tokens: int):
    """Host check of packed offsets: 0 = cu[0] <= ... <= cu[-1] = tokens."""
    c = cu.detach().to("cpu", torch.int64)
    if c.dim() != 1 or c.numel() < 2 or int(c[0]) != 0 or int(c[-1]) != tokens or \
            bool((c[1:] < c[:-1]).any()):
        raise ValueError("cu_seqlens must rise from 0 to the token count %d" % tokens)


def conv1d_silu(xbc, weight, bias, x_dim, bc_dim, history=None, cu_seqlens=None, *,
                want_history=True, x=None, B=None, C=None, history_out=None,
                check_cu_seqlens=True, stream=None):
    """The convolution front (ssd_conv1d_silu): causal depthwise conv1d over
    the packed channels [x | B | C], then SiLU. Returns (x, B, C,
    history_out).

    xbc is (batch, L, ch) (dense) or (tokens, ch) with ``cu_seqlens``, ch =
    x_dim + 2 * bc_dim, channels contiguous; its rows may be a slice of wider
    rows (the row stride is passed through). weight (ch, K) and bias (ch,) are
    float32; history (sequences, K - 1, ch) in xbc's dtype or None. Outputs
    have xbc's leading shape with x_dim, bc_dim, bc_dim channels.
    """
    _same_device(xbc.device, weight=weight, bias=bias, history=history, x=x, B=B, C=C,
                 history_out=history_out)
    _on_gpu(xbc.device)
    if xbc.dtype not in _DTYPES:
        raise ValueError("xbc must be bfloat16 or float32")
    ch = x_dim + 2 * bc_dim
    if xbc.shape[-1] != ch or xbc.stride(-1) != 1:
        raise ValueError("xbc must end in %d contiguous channels" % ch)
    dev = xbc.device
    if cu_seqlens is not None:
        if xbc.dim() != 2:
            raise ValueError("packed xbc must be (tokens, channels)")
        batch, L = 1, int(xbc.shape[0])
        num_seqs = int(cu_seqlens.numel()) - 1
        if check_cu_seqlens or cu_seqlens.device.type == "cpu":
            _check_offsets(cu_seqlens, L)
        cu_dev = cu_seqlens.to(device=dev, dtype=torch.int32).contiguous()
        nseq, lead = num_seqs, (L,)
        in_stride = xbc.stride(0) if L > 1 else ch
    else:
        if xbc.dim() != 3:
            raise ValueError("dense xbc must be (batch, seqlen, channels)")
        batch, L = int(xbc.shape[0]), int(xbc.shape[1])
        num_seqs, cu_dev, nseq, lead = 0, None, batch, (batch, L)
        # token row t = b * L + l sits at b * stride(0) + l * stride(1)
        if L > 1:
            if batch > 1 and xbc.stride(0) != L * xbc.stride(1):
                raise ValueError("the token rows of xbc must be evenly spaced")
            in_stride = xbc.stride(1)
        else:
            in_stride = xbc.stride(0) if batch > 1 else ch
    K = int(weight.shape[1]) if weight.dim() == 2 else 0
    if tuple(weight.shape) != (ch, K) or weight.dtype != torch.float32:
        raise ValueError("weight must be (%d, K) float32" % ch)
    if bias is not None and (tuple(bias.shape) != (ch,) or bias.dtype != torch.float32):
        raise ValueError("bias must be (%d,) float32" % ch)
    hshape = (nseq, K - 1, ch)
    if history is not None and (tuple(history.shape) != hshape or history.dtype != xbc.dtype):
        raise ValueError("history must be %s %s" % (hshape, xbc.dtype))
    for name, t, shape in (("x", x, lead + (x_dim,)), ("B", B, lead + (bc_dim,)),
                           ("C", C, lead + (bc_dim,)), ("history_out", history_out, hshape)):
        if t is not None and (tuple(t.shape) != shape or t.dtype != xbc.dtype
                              or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous %s %s tensor" % (name, shape, xbc.dtype))
    prob = ConvProblem(batch, L, num_seqs, x_dim, bc_dim, K, in_stride, _DTYPES[xbc.dtype], 0)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    # copies and outputs are made on the stream the kernel runs on (see step())
    with torch.cuda.stream(stream):
        weight = weight.contiguous()
        bias = bias.contiguous() if bias is not None else None
        history = history.contiguous() if history is not None else None
        if x is None:
            x = torch.empty(lead + (x_dim,), device=dev, dtype=xbc.dtype)
        if B is None:
            B = torch.empty(lead + (bc_dim,), device=dev, dtype=xbc.dtype)
        if C is None:
            C = torch.empty(lead + (bc_dim,), device=dev, dtype=xbc.dtype)
        if history_out is None and want_history:
            history_out = torch.empty(hshape, device=dev, dtype=xbc.dtype)
    _check(load().ssd_conv1d_silu(ctypes.byref(prob), _ptr(xbc), _ptr(weight), _ptr(bias),
                                  _ptr(history), _ptr(cu_dev), _ptr(x), _ptr(B), _ptr(C),
                                  _ptr(history_out), ctypes.c_void_p(stream.cuda_stream)),
           "ssd_conv1d_silu")
    return x, B, C, history_out


class BackwardPlan:
    """A prepared ssd_backward call for one forward problem: the problem is
    validated and the gradient outputs and workspace allocated once; :meth:`run`
    only enqueues the kernels.

    Takes the forward inputs (as for :class:`Plan`; bf16) and dL/dy, and
    optionally dL/d(final state); the states are recomputed. Returns from :meth:`run` a dict
    with dx, ddt, dA, dB, dC, dD, dinitial_state (dD without D is the gradient
    at D = 0; dinitial_state without an initial state the gradient at zero).
    """

    def __init__(self, x, dt, A, B, C, D, initial_state, dy, dfinal_state=None,
                 chunk_size=256, cu_seqlens=None, *, check_cu_seqlens=True):
        if x.dim() != 4:
            raise ValueError("x must be (batch, seqlen, nheads, headdim)")
        batch, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        dev = x.device
        _same_device(dev, dt=dt, A=A, B=B, C=C, D=D, initial_state=initial_state, dy=dy,
                     dfinal_state=dfinal_state)
        _on_gpu(dev)
        if x.dtype != torch.bfloat16:
            raise ValueError("the backward pass takes bfloat16 problems")
        for name, t, shape in (("dt", dt, (batch, L, H)), ("B", B, (batch, L, G, N)),
                               ("C", C, (batch, L, G, N)), ("dy", dy, tuple(x.shape))):
            if tuple(t.shape) != shape or t.dtype != x.dtype or t.device != dev:
                raise ValueError("%s must be %s %s on %s" % (name, shape, x.dtype, dev))
        if tuple(A.shape) != (H,) or A.dtype != torch.float32:
            raise ValueError("A must be (H,) float32")
        if D is not None and (tuple(D.shape) != (H,) or D.dtype != torch.float32):
            raise ValueError("D must be (H,) float32")
        num_seqs = 0
        if cu_seqlens is not None:
            if batch != 1:
                raise ValueError("cu_seqlens needs batch == 1")
            num_seqs = int(cu_seqlens.numel()) - 1
        nstate = num_seqs if num_seqs else batch
        for name, t in (("initial_state", initial_state), ("dfinal_state", dfinal_state)):
            if t is not None and (tuple(t.shape) != (nstate, H, P, N) or t.dtype != torch.float32):
                raise ValueError("%s must be (%d, %d, %d, %d) float32" % (name, nstate, H, P, N))
        self.prob = make_problem(batch, L, H, P, N, G, chunk_size, num_seqs, SSD_DTYPE_BF16, 0)
        validate(self.prob)
        self.cu = None
        if cu_seqlens is not None:
            if check_cu_seqlens or cu_seqlens.device.type == "cpu":
                validate_cu_seqlens(self.prob, cu_seqlens.detach().cpu())
            self.cu = cu_seqlens.to(device=dev, dtype=torch.int32).contiguous()
        n = ctypes.c_size_t(0)
        _check(load().ssd_backward_workspace_size(ctypes.byref(self.prob), ctypes.byref(n)),
               "ssd_backward_workspace_size")
        self.inputs = [t.contiguous() if t is not None else None
                       for t in (x, dt, A, B, C, D, initial_state, dy, dfinal_state)]
        self.grads = dict(
            dx=torch.empty_like(x), ddt=torch.empty_like(dt),
            dA=torch.empty(H, device=dev, dtype=torch.float32),
            dB=torch.empty_like(B), dC=torch.empty_like(C),
            dD=torch.empty(H, device=dev, dtype=torch.float32),
            dinitial_state=torch.empty((nstate, H, P, N), device=dev, dtype=torch.float32))
        self.workspace = torch.empty(max(n.value, 256), device=dev, dtype=torch.uint8)
        self.tokens = batch * L

    def _args(self, stream):
        x, dt, A, B, C, D, h0, dy, dhT = self.inputs
        g = self.grads
        return [ctypes.byref(self.prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                _ptr(h0), _ptr(self.cu), _ptr(dy), _ptr(dhT), _ptr(g["dx"]),
                _ptr(g["ddt"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
                _ptr(g["dinitial_state"]), _ptr(self.workspace),
                ctypes.c_size_t(self.workspace.numel()), ctypes.c_void_p(stream.cuda_stream)]

    def run(self, stream=None):
        """Enqueue one backward pass on ``stream`` (default: torch's current)."""
        if stream is None:
            stream = torch.cuda.current_stream(self.workspace.device)
        _check(load().ssd_backward(*self._args(stream)), "ssd_backward")
        return self.grads

    def run_timed(self, iterations: int, stream=None) -> StageTimes:
        """``iterations`` passes with a HIP event after every kernel; waits for
        them and returns the per-kernel times (see ssd_backward_timed)."""
        if stream is None:
            stream = torch.cuda.current_stream(self.workspace.device)
        times = StageTimes()
        _check(load().ssd_backward_timed(*self._args(stream), int(iterations),
                                         ctypes.byref(times)), "ssd_backward_timed")
        return times


def backward(x, dt, A, B, C, D, initial_state, dy, dfinal_state=None, chunk_size=256,
             cu_seqlens=None):
    """SSD backward pass (ssd_backward): a dict of gradients (see BackwardPlan)."""
    return BackwardPlan(x, dt, A, B, C, D, initial_state, dy, dfinal_state, chunk_size,
                        cu_seqlens).run()
