"""The C-ABI library on the host: exports, validation, workspace sizing.

No kernel is launched; everything here runs without a GPU.
"""
import ctypes
import os
import re

import pytest

import mamba_ssd_sequence_fwd_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "ssd.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.LIB_PATH):
        pytest.fail("libssd.so not built; run python -m mamba_ssd_sequence_fwd_amd.build")
    return ssd.load()


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert set(names) == set(ssd.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def P(**kw):
    base = dict(batch=2, seqlen=1000, nheads=8, headdim=64, dstate=128, ngroups=2,
                chunk_size=256, num_seqs=0, dtype=ssd.SSD_DTYPE_BF16, flags=0)
    base.update(kw)
    return ssd.make_problem(**base)


def status_of(fn, *a):
    try:
        fn(*a)
    except ssd.SSDError as e:
        return e.status
    return ssd.SSD_OK


@pytest.mark.parametrize("kw,status", [
    ({}, ssd.SSD_OK),
    ({"seqlen": 0}, ssd.SSD_OK),
    ({"batch": 0}, ssd.SSD_ERR_INVALID_ARG),
    ({"nheads": 0}, ssd.SSD_ERR_INVALID_ARG),
    ({"ngroups": 3}, ssd.SSD_ERR_INVALID_ARG),
    ({"num_seqs": 4}, ssd.SSD_ERR_INVALID_ARG),          # batch must be 1
    ({"batch": 1, "num_seqs": 4}, ssd.SSD_OK),
    ({"seqlen": -1}, ssd.SSD_ERR_INVALID_ARG),
    ({"flags": 8}, ssd.SSD_ERR_INVALID_ARG),
    ({"flags": ssd.SSD_FLAG_UNFUSED}, ssd.SSD_OK),
    ({"flags": ssd.SSD_FLAG_PER_SEQUENCE}, ssd.SSD_OK),
    ({"dtype": 7}, ssd.SSD_ERR_UNSUPPORTED),
    ({"headdim": 48}, ssd.SSD_ERR_UNSUPPORTED),
    ({"dstate": 24}, ssd.SSD_ERR_UNSUPPORTED),
    ({"dstate": 272}, ssd.SSD_ERR_UNSUPPORTED),
    ({"chunk_size": 100}, ssd.SSD_ERR_UNSUPPORTED),
    ({"chunk_size": 512}, ssd.SSD_ERR_UNSUPPORTED),
    ({"seqlen": 2 ** 30}, ssd.SSD_ERR_UNSUPPORTED),
])
def test_validate(lib, kw, status):
    assert status_of(ssd.validate, P(**kw)) == status


def test_error_detail_names_the_problem(lib):
    with pytest.raises(ssd.SSDError) as ei:
        ssd.validate(P(ngroups=3))
    assert "ngroups" in str(ei.value)


@pytest.mark.parametrize("cu,status", [
    ([0, 10, 10, 25, 40], ssd.SSD_OK),            # an empty sequence is allowed
    ([0, 0, 0, 0, 40], ssd.SSD_OK),
    ([1, 10, 20, 30, 40], ssd.SSD_ERR_INVALID_ARG),
    ([0, 10, 5, 30, 40], ssd.SSD_ERR_INVALID_ARG),
    ([0, 10, 20, 30, 39], ssd.SSD_ERR_INVALID_ARG),
    # malformed in the ways the device plan kernel guards against: negative
    # offsets, offsets past the stream, a sequence running backwards past 0,
    # int32 extremes (none may make either side index out of bounds)
    ([0, -5, 20, 30, 40], ssd.SSD_ERR_INVALID_ARG),
    ([0, 10, 50, 30, 40], ssd.SSD_ERR_INVALID_ARG),
    ([0, 41, 41, 41, 40], ssd.SSD_ERR_INVALID_ARG),
    ([0, 2 ** 31 - 1, 20, 30, 40], ssd.SSD_ERR_INVALID_ARG),
    ([0, -2 ** 31, 20, 30, 40], ssd.SSD_ERR_INVALID_ARG),
    ([-2 ** 31, 10, 20, 30, 40], ssd.SSD_ERR_INVALID_ARG),
])
def test_validate_cu_seqlens(lib, cu, status):
    prob = P(batch=1, seqlen=40, num_seqs=4)
    assert status_of(ssd.validate_cu_seqlens, prob, cu) == status


def test_workspace_layout_dense(lib):
    prob = P(flags=ssd.SSD_FLAG_UNFUSED)
    lay = ssd.workspace_layout(prob)
    nc = 2 * 4                                   # batch 2, ceil(1000/256) = 4
    assert lay.max_chunks == nc
    assert lay.chunk_cumsum % 256 == 0 and lay.chunk_states % 256 == 0
    assert lay.chunk_states >= lay.chunk_cumsum + nc * 8 * 256 * 4
    size = ssd.workspace_size(prob)
    assert size >= lay.chunk_states + nc * 8 * 64 * 128 * 4


def test_workspace_layout_varlen_bound(lib):
    prob = P(batch=1, seqlen=5000, num_seqs=7)
    lay = ssd.workspace_layout(prob)
    assert lay.max_chunks == 5000 // 256 + 7
    assert lay.chunk_records >= 3 + 7 and lay.chunk_records % 4 == 0


def test_workspace_layout_chain_counters(lib):
    """The default bf16 path (chained workgroups) has a status word and a
    decay word per (chunk, head) after a 576-word header (ticket, error word
    and eight queue counters 64 words apart), then the state
    leaving every chunk and (one-chunk units) every chunk's aggregate, fp32
    P x N each; the other paths have none."""
    lay = ssd.workspace_layout(P())
    nc = 2 * 4                                   # batch 2, ceil(1000/256) = 4
    assert lay.chain_sync_words == 576 + 2 * nc * 8 and lay.chain_sync % 256 == 0
    assert lay.chain_chunks_per_unit == 1        # 64 units: one chunk each, aggregates kept
    assert ssd.workspace_size(P()) >= lay.chain_sync + 4 * lay.chain_sync_words + \
        2 * nc * 8 * 64 * 128 * 4
    lay_v = ssd.workspace_layout(P(batch=1, seqlen=5000, num_seqs=7))
    assert lay_v.chain_sync_words == 576 + 2 * (5000 // 256 + 7) * 8
    for flags in (ssd.SSD_FLAG_UNFUSED, ssd.SSD_FLAG_PER_SEQUENCE, ssd.SSD_FLAG_GENERIC_KERNELS):
        assert ssd.workspace_layout(P(flags=flags)).chain_sync_words == 0


def test_workspace_lookback_slots_up_to_1536_units(lib):
    """One state slot and one aggregate per (chunk, head) on grids of up to
    1536 one-chunk units (the look-back kernel), two state slots per
    (sequence, head) above that."""
    state = 64 * 128 * 4
    look = ssd.workspace_size(P(seqlen=2048, nheads=96, ngroups=1))    # 2 x 8 x 96 = 1536
    assert look >= 2 * 1536 * state
    plain = ssd.workspace_size(P(seqlen=2048, nheads=100, ngroups=1))  # 1600 units
    assert plain < 1600 * state and plain >= 2 * 2 * 100 * state


def test_workspace_grows_with_problem(lib):
    a = ssd.workspace_size(P(seqlen=1000))
    b = ssd.workspace_size(P(seqlen=2000))
    assert b > a
    # generic kernels need no C.B^T buffer; the per-sequence fused kernel
    # keeps the per-chunk states on chip (the chained kernel publishes the
    # state leaving every chunk, and one-chunk units every chunk's aggregate)
    unf = ssd.workspace_size(P(flags=ssd.SSD_FLAG_UNFUSED))
    assert ssd.workspace_size(P(flags=ssd.SSD_FLAG_GENERIC_KERNELS)) < unf
    assert ssd.workspace_size(P(flags=ssd.SSD_FLAG_PER_SEQUENCE)) < unf


def test_forward_rejects_bad_arguments_before_launch(lib):
    prob = P()
    vp = ctypes.c_void_p
    fake = vp(1 << 20)        # never dereferenced: validation fails first
    st = lib.ssd_forward(ctypes.byref(prob), fake, fake, fake, fake, fake, None, None,
                         None, fake, None, None, ctypes.c_size_t(0), None)
    assert st == ssd.SSD_ERR_WORKSPACE
    st = lib.ssd_forward(ctypes.byref(prob), None, fake, fake, fake, fake, None, None,
                         None, fake, None, vp(1 << 21), ctypes.c_size_t(1 << 40), None)
    assert st == ssd.SSD_ERR_INVALID_ARG
    st = lib.ssd_forward(ctypes.byref(prob), vp((1 << 20) + 2), fake, fake, fake, fake,
                         None, None, None, fake, None, vp(1 << 21), ctypes.c_size_t(1 << 40),
                         None)
    assert st == ssd.SSD_ERR_INVALID_ARG      # misaligned x
    st = lib.ssd_forward(ctypes.byref(prob), fake, fake, fake, fake, fake, None, None,
                         fake, fake, None, vp(1 << 21), ctypes.c_size_t(1 << 40), None)
    assert st == ssd.SSD_ERR_INVALID_ARG      # cu_seqlens in dense mode


def test_status_strings(lib):
    for st in range(5):
        assert lib.ssd_status_string(st)


def _step_status(lib, prob, ptrs=None):
    """ssd_step's status for pointer values that are never dereferenced: each
    case below is rejected (or is empty) before anything is enqueued."""
    vp = ctypes.c_void_p
    if ptrs is None:
        ptrs = [vp(4096 * (i + 1)) for i in range(8)]   # 16-byte aligned, never touched
    return lib.ssd_step(ctypes.byref(prob), *ptrs, vp(None))


@pytest.mark.parametrize("kw,status", [
    ({"seqlen": 2}, ssd.SSD_ERR_INVALID_ARG),
    ({"seqlen": 0}, ssd.SSD_ERR_INVALID_ARG),
    ({"batch": 1, "num_seqs": 1}, ssd.SSD_ERR_INVALID_ARG),
    ({"batch": -1}, ssd.SSD_ERR_INVALID_ARG),
    ({"nheads": 0}, ssd.SSD_ERR_INVALID_ARG),
    ({"ngroups": 3}, ssd.SSD_ERR_INVALID_ARG),
    ({"flags": ssd.SSD_FLAG_UNFUSED}, ssd.SSD_ERR_INVALID_ARG),
    ({"dtype": 7}, ssd.SSD_ERR_UNSUPPORTED),
    ({"headdim": 48}, ssd.SSD_ERR_UNSUPPORTED),
    ({"dstate": 24}, ssd.SSD_ERR_UNSUPPORTED),
    ({"dstate": 272}, ssd.SSD_ERR_UNSUPPORTED),
    ({"batch": 2 ** 30, "nheads": 8}, ssd.SSD_ERR_UNSUPPORTED),   # batch * H above 32 bits
])
def test_step_validate(lib, kw, status):
    kw = dict({"seqlen": 1}, **kw)
    assert _step_status(lib, P(**kw)) == status


def test_step_empty_batch_is_a_no_op(lib):
    # batch 0: nothing to do, no pointer needed and nothing enqueued
    prob = P(seqlen=1, batch=0)
    assert _step_status(lib, prob, [ctypes.c_void_p(None)] * 8) == ssd.SSD_OK


def test_step_rejects_null_and_misaligned_pointers(lib):
    prob = P(seqlen=1)
    vp = ctypes.c_void_p
    good = [vp(4096 * (i + 1)) for i in range(8)]
    for i in (0, 1, 2, 3, 4, 6, 7):          # every pointer but D is required
        ptrs = list(good)
        ptrs[i] = vp(None)
        assert _step_status(lib, prob, ptrs) == ssd.SSD_ERR_INVALID_ARG, i
    for i in (0, 3, 4, 6, 7):                # x, B, C, state, y: 16-byte aligned
        ptrs = list(good)
        ptrs[i] = vp(4096 * (i + 1) + 8)
        assert _step_status(lib, prob, ptrs) == ssd.SSD_ERR_INVALID_ARG, i
    assert "aligned" in lib.ssd_last_error_detail().decode()


def _scan_status(lib, prob, ptrs=None):
    """ssd_selective_scan's status for pointer values that are never
    dereferenced: each case is rejected (or empty) before anything is enqueued."""
    vp = ctypes.c_void_p
    if ptrs is None:
        ptrs = [vp(4096 * (i + 1)) for i in range(9)]
    return lib.ssd_selective_scan(ctypes.byref(prob), *ptrs, vp(None))


def SP(**kw):
    base = dict(batch=2, seqlen=100, dim=128, dstate=16, dtype=ssd.SSD_DTYPE_BF16, flags=0)
    base.update(kw)
    return ssd.ScanProblem(**base)


@pytest.mark.parametrize("kw,status", [
    ({"batch": -1}, ssd.SSD_ERR_INVALID_ARG),
    ({"seqlen": -1}, ssd.SSD_ERR_INVALID_ARG),
    ({"dim": 0}, ssd.SSD_ERR_INVALID_ARG),
    ({"flags": 1}, ssd.SSD_ERR_INVALID_ARG),
    ({"dtype": 5}, ssd.SSD_ERR_UNSUPPORTED),
    ({"dstate": 24}, ssd.SSD_ERR_UNSUPPORTED),
    ({"dstate": 512}, ssd.SSD_ERR_UNSUPPORTED),
    ({"dim": 96}, ssd.SSD_ERR_UNSUPPORTED),
    ({"batch": 70000}, ssd.SSD_ERR_UNSUPPORTED),
])
def test_scan_validate(lib, kw, status):
    assert _scan_status(lib, SP(**kw)) == status


def test_scan_empty_batch_is_a_no_op(lib):
    assert _scan_status(lib, SP(batch=0), [ctypes.c_void_p(None)] * 9) == ssd.SSD_OK


def test_scan_rejects_null_and_misaligned_pointers(lib):
    vp = ctypes.c_void_p
    good = [vp(4096 * (i + 1)) for i in range(9)]
    # x, delta, A, B, C, y are required when there are tokens (D, h0, hT optional)
    for i in (0, 1, 2, 3, 4, 7):
        ptrs = list(good)
        ptrs[i] = vp(None)
        assert _scan_status(lib, SP(), ptrs) == ssd.SSD_ERR_INVALID_ARG, i
    for i in (0, 1, 2, 3, 4, 6, 7, 8):
        ptrs = list(good)
        ptrs[i] = vp(4096 * (i + 1) + 4)
        assert _scan_status(lib, SP(), ptrs) == ssd.SSD_ERR_INVALID_ARG, i


def _conv_status(lib, prob, ptrs=None):
    """ssd_conv1d_silu's status for pointer values that are never
    dereferenced: each case is rejected (or empty) before anything is enqueued.
    Pointer order: xbc, weight, bias, history_in, cu_seqlens, x, B, C,
    history_out."""
    vp = ctypes.c_void_p
    if ptrs is None:
        ptrs = [vp(4096 * (i + 1)) for i in range(9)]
    return lib.ssd_conv1d_silu(ctypes.byref(prob), *ptrs, vp(None))


def CP(**kw):
    base = dict(batch=2, seqlen=100, num_seqs=0, x_dim=64, bc_dim=16, width=4, in_stride=96,
                dtype=ssd.SSD_DTYPE_BF16, flags=0)
    base.update(kw)
    return ssd.ConvProblem(**base)


@pytest.mark.parametrize("kw,status", [
    ({"batch": -1}, ssd.SSD_ERR_INVALID_ARG),
    ({"seqlen": -1}, ssd.SSD_ERR_INVALID_ARG),
    ({"num_seqs": -1}, ssd.SSD_ERR_INVALID_ARG),
    ({"x_dim": -8}, ssd.SSD_ERR_INVALID_ARG),
    ({"flags": 1}, ssd.SSD_ERR_INVALID_ARG),
    ({"x_dim": 0, "bc_dim": 0, "in_stride": 8}, ssd.SSD_ERR_INVALID_ARG),
    ({"in_stride": 88}, ssd.SSD_ERR_INVALID_ARG),              # narrower than the 96 channels
    ({"in_stride": 100}, ssd.SSD_ERR_INVALID_ARG),             # 200 bytes: not 16-byte rows
    ({"num_seqs": 3}, ssd.SSD_ERR_INVALID_ARG),                # packed needs batch 1
    ({"dtype": 5}, ssd.SSD_ERR_UNSUPPORTED),
    ({"width": 1}, ssd.SSD_ERR_UNSUPPORTED),
    ({"width": 5}, ssd.SSD_ERR_UNSUPPORTED),
    ({"x_dim": 60, "in_stride": 96}, ssd.SSD_ERR_UNSUPPORTED),
    ({"bc_dim": 12, "in_stride": 96}, ssd.SSD_ERR_UNSUPPORTED),
    ({"seqlen": 1 << 30, "batch": 4}, ssd.SSD_ERR_UNSUPPORTED),
])
def test_conv_validate(lib, kw, status):
    assert _conv_status(lib, CP(**kw)) == status


def test_conv_packed_needs_offsets(lib):
    vp = ctypes.c_void_p
    ptrs = [vp(4096 * (i + 1)) for i in range(9)]
    ptrs[4] = vp(None)
    assert _conv_status(lib, CP(batch=1, num_seqs=3), ptrs) == ssd.SSD_ERR_INVALID_ARG


def test_conv_nothing_to_do_is_a_no_op(lib):
    nulls = [ctypes.c_void_p(None)] * 9
    assert _conv_status(lib, CP(batch=0), nulls) == ssd.SSD_OK
    # no tokens and no history to write
    assert _conv_status(lib, CP(seqlen=0), nulls) == ssd.SSD_OK


def test_conv_rejects_null_and_misaligned_pointers(lib):
    vp = ctypes.c_void_p
    good = [vp(4096 * (i + 1)) for i in range(9)]
    for i in (0, 1, 5, 6, 7):               # xbc, weight, x, B, C are required
        ptrs = list(good)
        ptrs[i] = vp(None)
        assert _conv_status(lib, CP(), ptrs) == ssd.SSD_ERR_INVALID_ARG, i
    for i in (0, 3, 5, 6, 7, 8):            # xbc, histories, x, B, C: 16-byte aligned
        ptrs = list(good)
        ptrs[i] = vp(4096 * (i + 1) + 8)
        assert _conv_status(lib, CP(), ptrs) == ssd.SSD_ERR_INVALID_ARG, i
    assert "aligned" in lib.ssd_last_error_detail().decode()


def _bwd_status(lib, prob, ptrs=None, ws_bytes=1 << 30):
    """ssd_backward's status for pointer values that are never dereferenced.
    Pointer order: x, dt, A, B, C, D, h0, cu, dy, dhT, dx, ddt, dA, dB, dC, dD,
    dh0, workspace."""
    vp = ctypes.c_void_p
    if ptrs is None:
        ptrs = [vp(4096 * (i + 1)) for i in range(18)]
        ptrs[7] = vp(None)                        # dense: no cu_seqlens
    return lib.ssd_backward(ctypes.byref(prob), *ptrs, ctypes.c_size_t(ws_bytes), vp(None))


@pytest.mark.parametrize("kw,status", [
    ({"flags": ssd.SSD_FLAG_UNFUSED}, ssd.SSD_ERR_INVALID_ARG),
    ({"dtype": ssd.SSD_DTYPE_F32}, ssd.SSD_ERR_UNSUPPORTED),
    ({"headdim": 32}, ssd.SSD_ERR_UNSUPPORTED),
    ({"dstate": 256}, ssd.SSD_ERR_UNSUPPORTED),
    ({"chunk_size": 64}, ssd.SSD_ERR_UNSUPPORTED),
    ({"nheads": 6, "ngroups": 4}, ssd.SSD_ERR_INVALID_ARG),
])
def test_backward_validate(lib, kw, status):
    assert _bwd_status(lib, P(**kw)) == status


def test_backward_workspace_size_and_checks(lib):
    n = ctypes.c_size_t(0)
    prob = P()
    assert lib.ssd_backward_workspace_size(ctypes.byref(prob), ctypes.byref(n)) == ssd.SSD_OK
    fwd = ssd.workspace_size(P(flags=ssd.SSD_FLAG_UNFUSED))
    # the per-step forward layout plus final states, gradient states and partials
    assert n.value >= fwd + 2 * 2 * 8 * 64 * 128 * 4
    assert _bwd_status(lib, prob, ws_bytes=n.value - 1) == ssd.SSD_ERR_WORKSPACE
    vp = ctypes.c_void_p
    good = [vp(4096 * (i + 1)) for i in range(18)]
    good[7] = vp(None)
    for i in (0, 1, 2, 3, 4, 8, 10, 12, 13, 14):  # x dt A B C dy dx dA dB dC
        ptrs = list(good)
        ptrs[i] = vp(None)
        assert _bwd_status(lib, prob, ptrs) == ssd.SSD_ERR_INVALID_ARG, i
    for i in (0, 3, 4, 8, 9, 10, 13, 14, 16):       # 16-byte aligned tensors
        ptrs = list(good)
        ptrs[i] = vp(4096 * (i + 1) + 8)
        assert _bwd_status(lib, prob, ptrs) == ssd.SSD_ERR_INVALID_ARG, i
    ptrs = list(good)
    ptrs[17] = vp(4096 * 18 + 128)                  # workspace not 256-byte aligned
    assert _bwd_status(lib, prob, ptrs) == ssd.SSD_ERR_WORKSPACE


# ---- the Python binding refuses tensors on another device ----------------------
# Every tensor a kernel touches must sit on the device of the first input:
# a host pointer handed to a kernel would fault the GPU instead of raising.
# The check runs before the GPU check and before any launch, so it is
# exercised here with inputs on torch's "meta" device and one tensor on the CPU.
import torch  # noqa: E402


def _meta(*shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device="meta")


def _fwd_args(**over):
    b, L, H, P, N, G = 2, 64, 4, 64, 128, 1
    a = dict(x=_meta(b, L, H, P), dt=_meta(b, L, H), A=_meta(H, dtype=torch.float32),
             B=_meta(b, L, G, N), C=_meta(b, L, G, N), D=_meta(H, dtype=torch.float32),
             initial_state=_meta(b, H, P, N, dtype=torch.float32))
    a.update(over)
    return a


@pytest.mark.parametrize("name,shape", [("A", (4,)), ("D", (4,)),
                                        ("initial_state", (2, 4, 64, 128)),
                                        ("dt", None), ("B", None)])
def test_forward_rejects_tensor_on_another_device(name, shape):
    a = _fwd_args()
    a[name] = torch.zeros(shape or a[name].shape, dtype=a[name].dtype)   # on the CPU
    with pytest.raises(ValueError, match=name):
        ssd.Plan(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["initial_state"])


def test_forward_on_meta_device_is_not_a_gpu():
    a = _fwd_args()
    with pytest.raises(ValueError, match="GPU"):
        ssd.Plan(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["initial_state"])


@pytest.mark.parametrize("name", ["A", "D", "state"])
def test_step_rejects_tensor_on_another_device(name):
    b, H, P, N = 3, 4, 64, 128
    a = dict(x=_meta(b, H, P), dt=_meta(b, H), A=_meta(H, dtype=torch.float32),
             B=_meta(b, 1, N), C=_meta(b, 1, N), D=_meta(H, dtype=torch.float32),
             state=_meta(b, H, P, N, dtype=torch.float32))
    a[name] = torch.zeros(a[name].shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match=name):
        ssd.step(**a)


@pytest.mark.parametrize("name", ["A", "D", "initial_state", "final_state"])
def test_selective_scan_rejects_tensor_on_another_device(name):
    b, L, Dm, N = 2, 16, 64, 16
    a = dict(x=_meta(b, L, Dm), delta=_meta(b, L, Dm), A=_meta(Dm, N, dtype=torch.float32),
             B=_meta(b, L, N), C=_meta(b, L, N), D=_meta(Dm, dtype=torch.float32),
             initial_state=_meta(b, Dm, N, dtype=torch.float32),
             final_state=_meta(b, Dm, N, dtype=torch.float32))
    a[name] = torch.zeros(a[name].shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match=name):
        ssd.selective_scan(**a)


@pytest.mark.parametrize("name", ["A", "D", "initial_state", "dfinal_state"])
def test_backward_rejects_tensor_on_another_device(name):
    a = _fwd_args()
    a["dy"] = _meta(*a["x"].shape)
    a["dfinal_state"] = _meta(*a["initial_state"].shape, dtype=torch.float32)
    a[name] = torch.zeros(a[name].shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match=name):
        ssd.BackwardPlan(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["initial_state"],
                         a["dy"], a["dfinal_state"])


@pytest.mark.parametrize("name", ["weight", "bias", "history"])
def test_conv_rejects_tensor_on_another_device(name):
    ch = 64 + 2 * 16
    a = dict(weight=_meta(ch, 4, dtype=torch.float32), bias=_meta(ch, dtype=torch.float32),
             history=_meta(2, 3, ch))
    a[name] = torch.zeros(a[name].shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match=name):
        ssd.conv1d_silu(_meta(2, 32, ch), a["weight"], a["bias"], 64, 16, a["history"])


@pytest.mark.parametrize("kw,units", [
    # 640 (sequence, head) pairs of 8 chunks, at least the 512 workgroups that
    # 256 CUs hold: balanced ranges, each walking whole sequences of 8 chunks
    (dict(batch=8, seqlen=2048, nheads=80), 8),
    (dict(batch=2, seqlen=8192, nheads=80), 1),            # 160 pairs of 32 chunks: one-chunk units
    (dict(batch=4, seqlen=2048, nheads=24), 1),            # 768 units: all fit the chip at once
    (dict(batch=2, seqlen=16384, nheads=64, dstate=256, ngroups=8), 1),   # N = 256
    (dict(batch=1, seqlen=137028, nheads=80, num_seqs=64), 12),           # packed: 5,120 pairs
    (dict(batch=1, seqlen=137028, nheads=80, num_seqs=12), 1),            # packed: 960 pairs
    (dict(batch=8, seqlen=2048, nheads=80, flags=ssd.SSD_FLAG_UNFUSED), 0),  # no chained kernel
    (dict(batch=8, seqlen=2048, nheads=80, dtype=ssd.SSD_DTYPE_F32), 0),
])
def test_chained_chunks_per_unit(lib, kw, units):
    base = dict(ngroups=1, dstate=128)
    base.update(kw)
    lay = ssd.workspace_layout(P(**base))
    assert lay.chain_chunks_per_unit == units
    # balanced ranges only for the 2.7B-shaped batch: 256 CUs (the value
    # taken without a GPU) hold 512 segment workgroups, one range each
    want = 512 if kw == dict(batch=8, seqlen=2048, nheads=80) else 0
    assert lay.chain_ranges == want


def test_noalloc_refuses_a_problem_above_its_scratch(lib):
    """The allocation-free entry point checks the workspace the problem needs
    against its fixed scratch area before touching the device."""
    prob = ssd.make_problem(1, 137028, 80, 64, 128, 1, 256, 64, ssd.SSD_DTYPE_BF16, 0)
    assert ssd.workspace_size(prob) > 64 << 20
    st = lib.ssd_forward_noalloc(ctypes.byref(prob), *([None] * 11))
    assert st == ssd.SSD_ERR_WORKSPACE
    assert b"scratch" in lib.ssd_last_error_detail()
