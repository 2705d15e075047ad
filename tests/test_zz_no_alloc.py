"""ssd_forward_noalloc (the entry point that allocates nothing, its workspace
a fixed scratch area in device memory) against ssd_forward on the same
inputs, through the C ABI: four calls in a row on one GPU, each smaller than
the one before (the 2.7B-shaped batch, a dense batch whose look-back slots do
not fit the scratch area, a smaller dense batch, packed sequences), so each
finds the scratch area holding the previous call's contents. The outputs
must be bit-identical: the same kernels, or the chained kernel with plain
waits against its look-back variant, which rebuilds a chunk's input state in
the same order of operations as the plain chain."""
import ctypes

import pytest
import torch

import mamba_ssd_sequence_fwd_amd as ssd
import ssd_inputs as si
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu

C = si.CONFIGS


def _noalloc(inp, w):
    d = to_device(inp)
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].cuda()
    nstate = d["x"].shape[0] if cu is None else cu.numel() - 1
    x = d["x"]
    y = torch.empty_like(x)
    hT = torch.empty((nstate,) + tuple(x.shape[2:]) + (d["B"].shape[3],), device="cuda",
                     dtype=torch.float32)
    torch.cuda.synchronize()  # everything above is allocated before the call
    ssd.forward_noalloc(x, d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], y, hT,
                        chunk_size=w.chunk, cu_seqlens=cu)
    torch.cuda.synchronize()
    return y, hT


def test_noalloc_matches_forward_on_shrinking_calls():
    # 2 x 8 chunks x 64 heads: 1,024 one-chunk units, whose per-chunk state
    # and aggregate slots (64 MiB) exceed the scratch area, so this entry
    # point takes the two-slot layout where ssd_forward takes the look-back
    cases = [C[2],
             si.scaled(C[2], batch=2, seqlen=2048, nheads=64, seed=7003),
             si.scaled(C[2], batch=2, seqlen=1100, nheads=24, seed=7001),
             si.scaled(si.STRESS["S3"], nheads=8, num_seqs=5, seq_lens=(300, 0, 900, 1, 257),
                       h0_std=0.1, seed=7002)]
    for w in cases:
        inp = si.make_inputs(w)
        print("[gpu] ssd_forward_noalloc %s seed=%d" % (w.name, w.seed), flush=True)
        y, hT = _noalloc(inp, w)
        d = to_device(inp)
        plan = ssd.Plan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                        chunk_size=w.chunk, cu_seqlens=inp["cu_seqlens"])
        yr, hr = plan.run()
        torch.cuda.synchronize()
        assert plan.chain_error() == 0
        assert torch.equal(y, yr), w.name
        assert torch.equal(hT, hr), w.name


def test_noalloc_refuses_a_problem_above_its_scratch_before_launching():
    lib = ssd.load()
    # 64 packed sequences x 80 heads: a 335 MB state hand-off ring
    prob = ssd.make_problem(1, 137028, 80, 64, 128, 1, 256, 64, ssd.SSD_DTYPE_BF16, 0)
    st = lib.ssd_forward_noalloc(ctypes.byref(prob), *([None] * 11))
    assert st == ssd.SSD_ERR_WORKSPACE
    assert b"64" in lib.ssd_last_error_detail() or b"scratch" in lib.ssd_last_error_detail()
