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
    want = chunks * H * per_chunk_head + chunks * per_chunk_group + seqs * H * per_seq_head
    cost = bench.algorithmic_cost(w, inp)
    assert want == 392_708_096
    # the roofline counts the method's bytes only ...
    assert cost["ssd_chain"]["bytes"] == want == cost["ssd_fused"]["bytes"]
    # ... and reports the state hand-off between chunk workgroups apart
    assert cost["ssd_chain"]["overhead_bytes"] == (chunks - seqs) * H * handoff == 293_601_280
    # with two chunks per work unit only every second boundary is handed off:
    # 4 units per sequence, 3 hand-offs
    two = bench.algorithmic_cost(w, inp, chunks_per_unit=2)
    assert two["ssd_chain"]["overhead_bytes"] == seqs * 3 * H * handoff == 125_829_120
    assert two["ssd_chain"]["bytes"] == want
    # 512 balanced ranges of the 5,120 (sequence, head, chunk) units, 10 chunks
    # each, in 8 queues of 64 over 80 pairs each: range t of a queue starts
    # inside a sequence of 8 chunks unless 10 t % 8 == 0, i.e. for 48 of the
    # 63 inner starts of each queue, 384 in all
    rng = bench.algorithmic_cost(w, inp, chunks_per_unit=8, ranges=512)
    assert rng["ssd_chain"]["overhead_bytes"] == 384 * handoff == 25_165_824
    assert rng["ssd_chain"]["bytes"] == want
    # masked product 2 tri P, chunk state and C h_in 2 x 2 q N P, state carry 2 P N
    flops = chunks * H * (2 * tri * P + 4 * q * N * P + 2 * P * N)
    assert cost["ssd_chain"]["flops"] == flops


def test_traffic_record_follows_the_kernel_sources(monkeypatch, tmp_path):
    """A counter record is reported only while the hash of the kernel sources
    it names matches the one written in it."""
    csrc = tmp_path / "mamba_ssd_sequence_fwd_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "k_demo.hip").write_text("// kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.TRAFFIC_PROFILES, ("demo", "w"), ("demo.md", ("k_demo.hip",)))
    digest = bench.kernel_sources_sha256(("k_demo.hip",))
    (tmp_path / "profiles" / "demo.md").write_text(
        "# demo\n\n- kernel_sources_sha256: `%s`\n- hbm_bytes_per_launch: `123456`\n" % digest)
    assert bench.measured_traffic("demo", "w") == 123456
    (csrc / "k_demo.hip").write_text("// kernel v2\n")
    assert bench.measured_traffic("demo", "w") is None
    assert bench.measured_traffic("no_such_kernel", "w") is None
