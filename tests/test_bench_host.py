"""Host-side logic of bench.py, on the CPU: the one-GPU contract of its
command line, the algorithmic byte and flop counts behind the roofline
(checked against the per-unit costs written out by hand for the 2.7B-shaped
workload), and the rule that a recorded HBM-traffic figure is reported only
while the kernel sources it was measured on are unchanged."""
from __future__ import annotations

import os
import subprocess
import sys

import bench
import ssd_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_chain_cost_of_the_2_7b_workload_by_hand():
    """batch 8 x 2048 tokens, 80 heads, P 64, N 128, G 1, chunk 256, bf16,
    initial state given: 8 chunks per sequence, 64 chunks in all."""
    w = si.CONFIGS[2]
    inp = si.make_inputs(w)
    e, q, P, N, H, chunks, seqs = 2, 256, 64, 128, 80, 64, 8
    tri = q * (q + 1) // 2                       # causal (l, s) pairs of a chunk
    per_chunk_head = 2 * q * P * e + q * e       # x and y, dt
    per_chunk_group = 2 * q * N * e + tri * 2    # B and C, the C B^T tiles (bf16)
    handoff = 2 * P * N * 4                      # fp32 state written and read once
    per_seq_head = 2 * P * N * 4                 # initial state in, final state out
    want = (chunks * H * per_chunk_head + chunks * per_chunk_group
            + (chunks - seqs) * H * handoff + seqs * H * per_seq_head)
    cost = bench.algorithmic_cost(w, inp)
    assert want == 686_309_376
    assert cost["ssd_chain"]["bytes"] == want
    # masked product 2 tri P, chunk state and C h_in 2 x 2 q N P, state carry 2 P N
    flops = chunks * H * (2 * tri * P + 4 * q * N * P + 2 * P * N)
    assert cost["ssd_chain"]["flops"] == flops
    # the chained kernel moves the fused minimum plus the hand-off
    assert cost["ssd_chain"]["bytes"] - cost["ssd_fused"]["bytes"] == (chunks - seqs) * H * handoff


def test_traffic_record_follows_the_kernel_sources(monkeypatch):
    rec = bench.measured_traffic("ssd_chain", "2.7b-bf16")
    assert isinstance(rec, int) and rec > 0
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda files: "0" * 64)
    assert bench.measured_traffic("ssd_chain", "2.7b-bf16") is None
    assert bench.measured_traffic("no_such_kernel", "2.7b-bf16") is None
