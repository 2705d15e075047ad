"""GPU path vs the fp64 oracle, element by element (MI355X only).

Small cases span several chunks and a ragged tail and run the full oracle;
the five workloads at full size compare sampled (sequence, head) pairs, each
a complete independent run of the recurrence, in the launch configuration the
benchmark times (one prepared ``Plan`` per workload).
Tolerance (normwise, per output tensor): 1e-4 for fp32 inputs, 2e-2 for bf16
inputs with fp32 accumulation and fp32 states.
"""
import numpy as np
import pytest
import torch

import mamba_ssd_sequence_fwd_amd as ssd

import oracle
import ssd_inputs as si
from gpu_helpers import (PATHS, compare_every_pair, flat_inputs, plan_for, rel_err, run_gpu,
                         run_oracle, seq_lens_of, tol_of)

pytestmark = pytest.mark.gpu

C = si.CONFIGS
S = si.STRESS
SMALL = {
    "cfg0-tiny-fp32": C[0],
    "cfg1-ragged": si.scaled(C[1], batch=2, seqlen=700, nheads=6, seed=2001),
    "cfg2-ragged-h0": si.scaled(C[2], batch=2, seqlen=600, nheads=4, seed=2002),
    "cfg3-groups-N256": si.scaled(C[3], batch=1, seqlen=1100, nheads=16, ngroups=4, seed=2003),
    "cfg4-varlen-edges": si.scaled(C[4], nheads=4, num_seqs=7, h0_std=0.1, seed=2004,
                                   seq_lens=(1, 255, 256, 257, 0, 600, 31)),
    "S1-slow-decay": si.scaled(S["S1"], batch=2, seqlen=900, nheads=4, seed=2011),
    "S2-a-zero": si.scaled(S["S2"], batch=1, seqlen=800, nheads=4, seed=2012),
    "S3-varlen-slow": si.scaled(S["S3"], nheads=4, num_seqs=5, len_range=(100, 900),
                                seed=2013),
    "S1-N256-h0": si.scaled(S["S1"], batch=2, seqlen=700, nheads=4, dstate=256, ngroups=2,
                            seed=2014),
    "S1-N256-Q128": si.scaled(S["S1"], batch=1, seqlen=650, nheads=4, dstate=256, chunk=128,
                              seed=2015),
    # 65 chunks x 4 groups: more than 256 (chunk, group) pairs, so the C B^T
    # kernel stages each chunk's B in LDS
    "staged-cb-G4-N64": si.scaled(C[3], batch=1, seqlen=16500, nheads=8, ngroups=4,
                                  dstate=64, seed=2025),
    # more work units (chunks x heads) than the chip holds at once: the chained
    # kernel's three-per-CU variant (smaller grids take the deep-prefetch one)
    "many-units-N128": si.scaled(C[2], batch=2, seqlen=1800, nheads=52, seed=2026),
    "many-units-N64-h0": si.scaled(C[2], batch=4, seqlen=1000, nheads=64, dstate=64, seed=2027),
    # 69 (sequence, head) pairs, an odd head count, three ragged sequences
    "odd-heads-23": si.scaled(C[2], batch=3, seqlen=700, nheads=23, h0_std=0.1, seed=2028),
    # 11 packed sequences, two of them empty, lengths from 1 to 900 tokens
    "varlen-11-seqs": si.scaled(C[4], nheads=4, num_seqs=11, h0_std=0.1, seed=2029,
                                seq_lens=(300, 0, 1, 700, 256, 257, 0, 40, 900, 5, 513)),
    # more than 768 work units on fewer than 512 (sequence, head) pairs:
    # one-chunk units handing the state over through the two-slot ring
    # (three workgroups per CU), odd chunk counts, slow decay so that every
    # carry shows.
    "seg-odd-chunks-h0": si.scaled(C[2], batch=2, seqlen=1100, nheads=80, seed=2030),
    "seg-slow-h0": si.scaled(S["S1"], batch=2, seqlen=1800, nheads=52, seed=2031),
    # packed sequences of 0 to 6 chunks with initial states, more than 768
    # units but fewer than 1,024 (sequence, head) pairs: one-chunk units
    "seg-varlen-slow": si.scaled(S["S3"], nheads=40, num_seqs=9, h0_std=0.1, seed=2032,
                                 seq_lens=(1, 600, 0, 257, 1300, 513, 40, 768, 1025)),
    # packed input with 1,040 pairs: segments of up to 12 chunks, one
    # sequence of 13 chunks (two segments, a hand-off between them), empty
    # and one-token sequences, initial states, slow decay
    "seg-varlen-long": si.scaled(S["S3"], nheads=80, num_seqs=13, h0_std=0.1, seed=2035,
                                 seq_lens=(1, 600, 0, 257, 3300, 513, 40, 768, 1025, 2000, 5,
                                           256, 100)),
    # the same at chunk 128, N = 64, two groups, no initial state: a sequence
    # of 14 chunks (segments of 12 and 2) and one of exactly 12
    "seg-varlen-q128": si.scaled(S["S3"], nheads=80, ngroups=2, dstate=64, chunk=128,
                                 num_seqs=13, h0_std=0.0, seed=2036,
                                 seq_lens=(129, 0, 1700, 64, 385, 1, 900, 256, 127, 1536, 40,
                                           700, 300)),
    # eight or more groups: one-chunk units handed out from one queue per XCD,
    # each over whole groups (N = 256 dense; packed input at N = 128 with more
    # units than the chip holds), slow decay so that every carry shows
    "gqueue-N256-G8": si.scaled(S["S1"], batch=2, seqlen=900, nheads=16, dstate=256, ngroups=8,
                                seed=2033),
    "gqueue-varlen-G8": si.scaled(S["S3"], nheads=64, ngroups=8, num_seqs=6, h0_std=0.1,
                                  seq_lens=(300, 0, 1200, 257, 900, 40), seed=2034),
    "bf16-P32-N48": si.scaled(C[1], batch=1, seqlen=333, nheads=4, headdim=32, dstate=48,
                              chunk=128, seed=2021),
    "bf16-N64": si.scaled(C[2], batch=1, seqlen=520, nheads=4, dstate=64, seed=2022),
    "fp32-P64-N128": si.scaled(C[2], batch=1, seqlen=600, nheads=3, dtype="fp32", seed=2023),
    "fp32-varlen": si.scaled(C[4], nheads=2, headdim=16, dstate=32, chunk=64, dtype="fp32",
                             num_seqs=4, seq_lens=(70, 0, 129, 5), h0_std=0.1, seed=2024),
}


@pytest.fixture(scope="module")
def small_inputs():
    return {k: si.make_inputs(w) for k, w in SMALL.items()}


@pytest.fixture(scope="module")
def small_oracle(small_inputs):
    return {k: run_oracle(v) for k, v in small_inputs.items()}


def _compare(inp, got, ref, tol=None):
    tol = tol or tol_of(inp)
    (y, hT), (yr, hr) = got, ref
    assert np.isfinite(y).all() and np.isfinite(hT).all()
    ey, eh = rel_err(y, yr), rel_err(hT, hr)
    print("  y err %.3e  final err %.3e  (tol %.0e)" % (ey, eh, tol), flush=True)
    assert ey <= tol, ("y", ey)
    assert eh <= tol, ("final_state", eh)


@pytest.mark.parametrize("case", list(SMALL))
def test_small_parity(case, small_inputs, small_oracle):
    inp = small_inputs[case]
    y, hT, _ = run_gpu(inp)
    _compare(inp, (y, hT), small_oracle[case])


@pytest.mark.parametrize("case", [k for k, w in SMALL.items() if w.dtype == "bf16"])
def test_small_parity_unfused_kernels(case, small_inputs, small_oracle):
    """One kernel per step (cumsum, chunk_state, state_passing, chunk_scan)."""
    inp = small_inputs[case]
    y, hT, _ = run_gpu(inp, unfused=True)
    _compare(inp, (y, hT), small_oracle[case])


@pytest.mark.parametrize("case", [k for k, w in SMALL.items() if w.dtype == "bf16"])
def test_small_parity_per_sequence_kernel(case, small_inputs, small_oracle):
    inp = small_inputs[case]
    y, hT, _ = run_gpu(inp, per_sequence=True)
    _compare(inp, (y, hT), small_oracle[case])


@pytest.mark.parametrize("case", [k for k, w in SMALL.items() if w.dtype == "bf16"])
def test_small_parity_generic_kernels(case, small_inputs, small_oracle):
    """The plain-FMA kernels on bf16 inputs (the MFMA path's fallback)."""
    inp = small_inputs[case]
    y, hT, _ = run_gpu(inp, generic=True)
    _compare(inp, (y, hT), small_oracle[case])


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("Q", [64, 128, 256])
@pytest.mark.parametrize("case", ["cfg2-ragged-h0", "S1-slow-decay", "fp32-P64-N128",
                                  "cfg3-groups-N256", "bf16-N64"])
def test_chunk_size_invariance(case, Q, path, small_inputs, small_oracle):
    inp = small_inputs[case]
    y, hT, _ = run_gpu(inp, chunk=Q, **PATHS[path])
    _compare(inp, (y, hT), small_oracle[case])


@pytest.mark.parametrize("case", ["S1-slow-decay", "cfg4-varlen-edges", "S3-varlen-slow",
                                  "fp32-varlen"])
def test_intermediates(case, small_inputs):
    """Chunk log-decay prefix and the state entering every chunk."""
    inp = small_inputs[case]
    Q = inp["workload"].chunk
    y, hT, plan = run_gpu(inp, unfused=True)
    lay = plan.layout()
    _, _, snaps = run_oracle(inp, snap_every=Q)
    nc = snaps.shape[0]
    H = inp["x"].shape[2]
    ws = plan.workspace
    cs = ws[lay.chunk_cumsum:lay.chunk_cumsum + nc * H * Q * 4].view(torch.float32)
    cs = cs.reshape(nc, H, Q).double().cpu().numpy() * np.log(2.0)
    x, dt, B, Cm = flat_inputs(inp)
    ref_cs = oracle.chunk_log_decay(dt, inp["A"], seq_lens_of(inp), Q)
    mask = np.isfinite(ref_cs)
    assert rel_err(cs[mask], ref_cs[mask]) < 1e-5
    P, N = inp["x"].shape[3], inp["B"].shape[3]
    st = ws[lay.chunk_states:lay.chunk_states + nc * H * P * N * 4].view(torch.float32)
    st = st.reshape(nc, H, P, N).double().cpu().numpy()
    assert rel_err(st, snaps) <= tol_of(inp), rel_err(st, snaps)


def _run_case(w):
    inp = si.make_inputs(w)
    return inp, run_gpu(inp), run_oracle(inp)


@pytest.mark.parametrize("w", [
    si.scaled(C[2], batch=1, seqlen=1, nheads=2, seed=2101),
    si.scaled(C[2], batch=3, seqlen=37, nheads=2, seed=2102),
    si.scaled(C[2], batch=1, seqlen=256, nheads=2, seed=2103),
    si.scaled(C[2], batch=1, seqlen=257, nheads=2, seed=2104),
    si.scaled(C[1], batch=1, seqlen=512, nheads=3, chunk=64, seed=2105),
    si.scaled(C[0], seqlen=1, seed=2106),
    si.scaled(C[4], nheads=2, num_seqs=3, seq_lens=(0, 0, 0), h0_std=0.1, seed=2107),
    si.scaled(C[4], nheads=2, num_seqs=1, seq_lens=(1,), seed=2108),
], ids=["L1", "L37-b3", "L256", "L257", "Q64-L512", "fp32-L1", "varlen-all-empty",
        "varlen-one-token"])
def test_edge_shapes(w):
    inp, (y, hT, _), ref = _run_case(w)
    _compare(inp, (y, hT), ref)


def test_empty_dense_batch_returns_initial_state():
    w = si.scaled(C[2], batch=2, seqlen=0, nheads=2, seed=2109)
    inp = si.make_inputs(w)
    y, hT, _ = run_gpu(inp)
    assert y.size == 0
    assert np.array_equal(hT, inp["h0"].double().numpy())


@pytest.mark.parametrize("path", list(PATHS))
def test_deterministic(small_inputs, path):
    inp = small_inputs["cfg2-ragged-h0"]
    plan = plan_for(inp, **PATHS[path])
    y1, h1 = [t.clone() for t in plan.run()]
    y2, h2 = plan.run()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_varlen_no_leakage(small_inputs):
    """Changing one packed sequence changes nothing in the others."""
    inp = dict(small_inputs["cfg4-varlen-edges"])
    cu = inp["cu_seqlens"].tolist()
    y0, h0, _ = run_gpu(inp)
    k = 3
    x = inp["x"].clone()
    x[:, cu[k]:cu[k + 1]] = x[:, cu[k]:cu[k + 1]] * 3 + 1
    inp["x"] = x
    y1, h1, _ = run_gpu(inp)
    for s in range(len(cu) - 1):
        same = np.array_equal(y0[cu[s]:cu[s + 1]], y1[cu[s]:cu[s + 1]]) and \
            np.array_equal(h0[s], h1[s])
        assert same == (s != k or cu[s] == cu[s + 1]), s


def test_split_call_continuity(small_inputs):
    """[0, t) then [t, L) with final -> initial matches one call."""
    inp = small_inputs["S1-slow-decay"]
    y, hT, _ = run_gpu(inp)
    t = 333
    first = dict(inp)
    second = dict(inp)
    for key in ("x", "dt", "B", "C"):
        first[key] = inp[key][:, :t].contiguous()
        second[key] = inp[key][:, t:].contiguous()
    ya, ha, _ = run_gpu(first)
    second["h0"] = torch.from_numpy(ha).float()
    yb, hb, _ = run_gpu(second)
    b, L = inp["x"].shape[:2]
    ya = ya.reshape(b, t, *ya.shape[1:])
    yb = yb.reshape(b, L - t, *yb.shape[1:])
    yy = np.concatenate([ya, yb], axis=1).reshape(y.shape)
    assert rel_err(yy, y) < 2e-2 and rel_err(hb, hT) < 2e-2


# ---- the five workloads and the three stress workloads at full size -------------
# Every (sequence, head) pair of the workload is compared with the oracle, in
# the launch configuration the benchmark times (one prepared Plan per path).
# The stress workloads make the state carried between chunks visible: at the
# configs' decay a 256-token chunk forgets everything (about e^-149), so a
# wrong carry would pass them. Slow decay keeps the state (tj-hxxt.cn long
# read of the Mamba-1 paper, part III item 3 on the step size: a small step
# decay keeps the state), and packed sequences reset it (same page, item 2.3
# "Boundary Resetting"). S1 is the 2.7B shapes with slow decay and an initial
# state (5,120 work units, the many-units kernel variant the benchmark
# times); S2 is A = 0 at the small shapes; S3 is the packed workload with
# slow decay, so per-sequence final states carry many chunks.
FULL = {"cfg0": C[0], "cfg1": C[1], "cfg2": C[2], "cfg3": C[3], "cfg4": C[4],
        "S1": S["S1"], "S2": S["S2"], "S3": S["S3"]}


@pytest.mark.parametrize("name", list(FULL))
def test_full_workload_every_pair(name):
    w = FULL[name]
    inp = si.make_inputs(w)
    outs = {}
    for path, kw in PATHS.items():
        plan = plan_for(inp, **kw)
        print("[gpu] full workload %s %s path=%s %r" % (name, w.name, path, plan.prob), flush=True)
        y, hT = plan.run()
        torch.cuda.synchronize()
        assert plan.chain_error() == 0, "a chained workgroup timed out waiting for its state"
        assert bool(torch.isfinite(y).all()) and bool(torch.isfinite(hT).all()), path
        T, H = plan.tokens, inp["x"].shape[2]
        outs[path] = (y.reshape(T, H, -1).cpu(), hT.cpu())
        del plan, y, hT
    res = compare_every_pair(inp, outs)
    tol = tol_of(inp)
    for path, r in res.items():
        print("  %-12s %d pairs: y err %.3e final err %.3e | worst slice y %.3e at %s, "
              "final %.3e at %s (tol %.0e)" % (path, r["pairs"], r["y"], r["final"],
                                                r["worst_y"], r["worst_y_at"], r["worst_final"],
                                                r["worst_final_at"], tol), flush=True)
    for path, r in res.items():
        assert r["y"] <= tol and r["final"] <= tol, (path, r)
        assert r["worst_y"] <= tol and r["worst_final"] <= tol, (path, r)


@pytest.mark.parametrize("path", ["default", "unfused", "fp32"])
@pytest.mark.parametrize("bad", [[1, 300, 600, 900, 1133], [0, 300, 200, 900, 1133],
                                 [0, 300, 600, 1500, 1133], [0, 300, 2 ** 31 - 1, 900, 1133],
                                 [0, -300, 600, 900, 1133]],
                         ids=["first-not-0", "decreasing", "past-the-end", "int-max", "negative"])
def test_malformed_device_cu_seqlens_are_flagged_not_followed(bad, path):
    """Offsets that only the device sees (the host check skipped) and that are
    malformed: the plan kernel flags them and leaves zero chunks, so no
    kernel reads or writes a token through them; the pass completes and the
    flag is readable in the workspace (the outputs are unspecified)."""
    w = si.scaled(C[4], nheads=4, num_seqs=4, seq_lens=(300, 300, 300, 233), h0_std=0.1,
                  seed=2110, dtype="fp32" if path == "fp32" else "bf16",
                  chunk=64 if path == "fp32" else 256, headdim=32 if path == "fp32" else 64,
                  dstate=32 if path == "fp32" else 128)
    inp = si.make_inputs(w)
    d = {k: (None if inp[k] is None else inp[k].cuda()) for k in ("x", "dt", "A", "B", "C", "D", "h0")}
    cu = torch.tensor(bad, dtype=torch.int32, device="cuda")
    plan = ssd.Plan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk_size=w.chunk,
                    cu_seqlens=cu, check_cu_seqlens=False, unfused=path == "unfused")
    print("[gpu] malformed device cu_seqlens %s path=%s %r" % (bad, path, plan.prob), flush=True)
    plan.run()
    torch.cuda.synchronize()
    assert plan.chain_error() == 0
    lay = plan.layout()
    header = plan.workspace[lay.chunk_table:lay.chunk_table + 8].view(torch.int32).cpu()
    assert int(header[0]) == 0 and int(header[1]) == 1, header.tolist()
