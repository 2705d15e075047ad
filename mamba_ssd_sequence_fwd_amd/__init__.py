"""Mamba-2 SSD forward pass for AMD Instinct MI355X (gfx950).

The hot path is the C-ABI library ``libssd.so`` (HIP kernels, declared in
``include/ssd.h``); this package is its thin Python binding. Build the library
with ``python -m mamba_ssd_sequence_fwd_amd.build``.

    y, final_state = forward(x, dt, A, B, C, D, initial_state, chunk_size=256,
                             cu_seqlens=None)
    y_t = step(x_t, dt_t, A, B_t, C_t, D, state)   # one decode step, state in place
    y, h = selective_scan(x, delta, A, B, C, D)     # the Mamba-1 scan (comparator)
    x, B, C, hist = conv1d_silu(xbc, w, b, x_dim, bc_dim)  # conv front producing x, B, C
    grads = backward(x, dt, A, B, C, D, h0, dy)  # dx, ddt, dA, dB, dC, dD, dinitial_state
"""
from ._lib import (  # noqa: F401
    EXPORTED, LIB_PATH, BackwardPlan, ConvProblem, Plan, Problem, ScanProblem, SSDError,
    StageTimes, WorkspaceLayout, backward, conv1d_silu, forward, forward_noalloc, load,
    selective_scan,
    make_problem, step, validate, validate_cu_seqlens, workspace_layout, workspace_size,
    SSD_DTYPE_BF16, SSD_DTYPE_F32, SSD_FLAG_GENERIC_KERNELS, SSD_FLAG_UNFUSED, SSD_FLAG_PER_SEQUENCE,
    SSD_OK,
    SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP,
)
