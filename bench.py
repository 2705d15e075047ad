#!/usr/bin/env python3
"""Benchmark of the SSD forward pass on one MI355X.

One step = one ssd_forward over one batch of synthetic input (every kernel of
the path). Default workload: the 2.7B-shaped config (batch 8, L 2048, H 80,
P 64, N 128, G 1, chunk 256, bf16 in / fp32 accumulate and states, random
fp32 initial state). Inputs are resident in HBM before the timed region.

Prints ONE JSON line with: whole-job tokens/s over K plain passes (HIP events
around the loop only; before them W warm-up passes and --ramp-s seconds of
untimed passes, so that the GPU's clocks have ramped up), per-kernel times
from a second run of K passes with a HIP event after every kernel, the
roofline of the dominant kernel (the method's algorithmic bytes or flops per
launch / its mean event time, with the design's own intermediate bytes
reported apart as overhead), and the fp64 CPU oracle timed on this host (a
reported baseline, not a target).

    python bench.py [--steps K] [--warmup W] [--config 0..4] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ssd_inputs as si  # noqa: E402
import mamba_ssd_sequence_fwd_amd as ssd  # noqa: E402

METRIC = "SSD fwd tokens/sec + % MFMA/HBM roofline at L=2048, H=80, P=64, N=128"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
COLD_EVICT_BYTES = 512 << 20   # twice the 256 MB Infinity Cache
MFMA_FP32_PEAK_TFLOPS = 157.3


def algorithmic_cost(w: si.Workload, inp: dict, chunks_per_unit: int = 1, ranges: int = 0) -> dict:
    """Bytes each kernel must move and flops it must do, by the method's
    definition (unique HBM bytes; causal pairs only; C B^T once per group).

    Per (chunk, head) unit with q tokens: x q*P*e, y q*P*e, dt q*e, state
    P*N*4 (fp32), cumsum q*4; per (chunk, group): B and C q*N*e each.
    ``chunks_per_unit``: consecutive chunks the chained kernel's workgroups
    walk with the state on chip (the hand-off overhead is between units);
    ``ranges`` > 0: its workgroups take that many balanced ranges of the
    (sequence, head, chunk) order instead, handing off where a range starts
    inside a sequence (dense input).
    """
    e = 2 if w.dtype == "bf16" else 4
    lens = inp["seq_lens"] or [w.seqlen] * w.batch
    H, P, N, G, Q = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    T = int(sum(lens))
    chunks = [min(Q, L - c0) for L in lens for c0 in range(0, L, Q)]
    nc = len(chunks)
    S = len(lens)
    state = P * N * 4
    causal = sum(q * (q + 1) // 2 for q in chunks)           # (l, s) pairs, s <= l
    cost = {
        "chunk_cumsum": dict(bytes=T * H * e + T * H * 4, flops=2 * T * H),
        "chunk_state": dict(bytes=T * H * P * e + T * H * (e + 4) + T * G * N * e
                            + nc * H * state, flops=2 * T * H * P * N),
        "state_passing": dict(bytes=2 * nc * H * state + 2 * S * H * state * (
            1 if inp["h0"] is not None else 0.5), flops=2 * nc * H * P * N),
        "chunk_cb": dict(bytes=2 * T * G * N * e + causal * G * 2, flops=2 * causal * G * N),
        "chunk_scan": dict(bytes=2 * T * H * P * e + T * H * e + T * G * N * e + nc * H * state
                           + T * H * 4 + causal * G * 2,
                           flops=2 * causal * H * P + 2 * T * H * N * P),
    }
    cost["ssd_fused"] = dict(
        bytes=2 * T * H * P * e + T * H * e + 2 * T * G * N * e + causal * G * 2 + S * H * state * (
            2 if inp["h0"] is not None else 1),
        flops=2 * causal * H * P + 4 * T * H * N * P + 2 * nc * H * P * N)
    # chained kernel: the method's bytes are the fused minimum; the fp32 state
    # hand-off between consecutive chunks of a sequence (written once, read
    # once) is this design's own intermediate, reported apart as overhead
    k = max(1, chunks_per_unit)
    units = sum(((L + Q - 1) // Q + k - 1) // k for L in lens)
    handoff = 2 * (units - sum(1 for L in lens if L > 0)) * H * state
    if ranges > 0:
        # one queue of ranges per XCD, each over an eighth of the (sequence,
        # head) pairs; a range starting inside a sequence takes a hand-off
        per = (lens[0] + Q - 1) // Q            # dense: chunks of every sequence
        pairs, nq = len(lens) * H, 8
        rq = ranges // nq
        n = 0
        for q in range(nq):
            units = (pairs * (q + 1) // nq - pairs * q // nq) * per
            n += sum(1 for t in range(1, rq) if (t * units // rq) % per)
        handoff = 2 * state * n
    cost["ssd_chain"] = dict(bytes=cost["ssd_fused"]["bytes"], flops=cost["ssd_fused"]["flops"],
                             overhead_bytes=handoff)
    # fp32 problems: one workgroup per (sequence, head), no C B^T tiles
    cost["ssd_f32seq"] = dict(
        bytes=2 * T * H * P * e + T * H * e + 2 * T * G * N * e + S * H * state * (
            2 if inp["h0"] is not None else 1),
        flops=2 * causal * (G * N + H * P) + 4 * T * H * N * P + 2 * nc * H * P * N)
    cost["_path"] = dict(
        bytes=2 * T * H * P * e + T * H * e + 2 * T * G * N * e + S * H * state * (
            2 if inp["h0"] is not None else 1),
        flops=2 * causal * (G * N + H * P) + 4 * T * H * N * P)
    return cost


# HBM bytes per launch of the dominant kernel, measured with rocprofv3 FETCH_SIZE
# and WRITE_SIZE passes and recorded in profiles/ with the hash of the kernel
# sources they were taken on. Reported only while the sources still match.
_CHAIN_SRC = ("k_chain.hip", "mfma_common.h", "ssd_internal.h")
TRAFFIC_PROFILES = {
    ("ssd_chain", "2.7b-bf16"): ("ssd_chain_2.7b-bf16.md", _CHAIN_SRC),
    ("ssd_chain", "small-bf16"): ("ssd_chain_small-bf16.md", _CHAIN_SRC),
    ("ssd_chain", "large-state-long"): ("ssd_chain_large-state-long.md", _CHAIN_SRC),
    ("ssd_chain", "varlen-packed"): ("ssd_chain_varlen-packed.md", _CHAIN_SRC),
    ("ssd_f32seq", "tiny-fp32"): ("ssd_f32seq_tiny-fp32.md", ("k_f32seq.hip", "ssd_internal.h")),
    ("ssd_step", "decode-2.7b-b256"): ("ssd_step_decode-2.7b-b256.md",
                                       ("k_step.hip", "step.h", "ssd_internal.h")),
    ("ssd_conv", "conv-front-2.7b"): ("ssd_conv_front-2.7b.md",
                                      ("k_conv.hip", "conv.h", "ssd_internal.h")),
    ("bwd_dx", "bwd-2.7b-bf16"): ("ssd_backward_2.7b-bf16.md",
                                   ("k_bwd.hip", "bwd.h", "mfma_common.h", "ssd_internal.h")),
}


def kernel_sources_sha256(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mamba_ssd_sequence_fwd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter profile, or None."""
    entry = TRAFFIC_PROFILES.get((kernel, workload))
    if entry is None:
        return None
    path = os.path.join(ROOT, "profiles", entry[0])
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_sources_sha256") != kernel_sources_sha256(entry[1]):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp: dict, w: si.Workload, budget_s: float, threads: int = 0) -> dict:
    """Time the fp64 oracle (as it stands) on this host over the same workload:
    (sequence, head) pairs in a seeded random order, in batches, until the time
    budget is spent (the whole workload, repeated if it takes less than the
    budget); reported as tokens of the workload per second."""
    import oracle
    threads = threads or oracle.default_threads()
    lens = inp["seq_lens"] or [w.seqlen] * w.batch
    H = w.nheads
    x = inp["x"].reshape(-1, H, w.headdim)
    dt = inp["dt"].reshape(-1, H)
    B = inp["B"].reshape(-1, w.ngroups, w.dstate)
    C = inp["C"].reshape(-1, w.ngroups, w.dstate)
    all_pairs = [(s, h) for s in range(len(lens)) for h in range(H)]
    rng = np.random.default_rng(0)
    order = [all_pairs[i] for i in rng.permutation(len(all_pairs))]
    done, tok, elapsed = 0, 0, 0.0
    n = min(len(order), threads)  # first batch: one pair per thread
    while elapsed < budget_s:
        batch = [order[(done + i) % len(order)] for i in range(n)]
        t0 = time.perf_counter()
        oracle.ssd_pairs(x, dt, inp["A"], B, C, inp["D"], inp["h0"], lens, batch,
                         threads=threads)
        elapsed += time.perf_counter() - t0
        tok += sum(lens[s] for s, _ in batch)
        done += len(batch)
        rate = elapsed / done
        n = int(min(4 * len(order), max(threads, (budget_s - elapsed) / max(rate, 1e-9))))
    # each pair is one head of one sequence; a token of the workload has H heads
    value = tok / H / elapsed
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d (sequence, head) pairs of the %s workload (%d pairs, %.2f passes), "
                      "%.1f s of fp64 recurrence over %d host threads" % (
                          done, w.name, len(order), done / len(order), elapsed, threads)}


def evict_caches(buf):
    """Read ``buf`` (COLD_EVICT_BYTES, twice the MALL) so that the L2s and the
    MALL hold its clean lines and none of the timed kernel's data. A write
    would leave dirty lines whose write-back the next kernel would pay for."""
    return torch.sum(buf)


def clock_ramp(run, stream, seconds):
    """Untimed calls of ``run`` for ``seconds`` of wall time, after the
    warm-up calls: the GPU raises its clocks only under sustained load. On
    one MI355X, the 2.7B-shaped workload after 10 warm-up passes: the next
    100 passes ran at 163.8 us each, 20 more at 151.6, then 147.9, and from
    about 40 ms of load on every batch at 142.5-143.8. Returns the calls run."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            run()
        n += 16
        stream.synchronize()
    return n


def time_launches(run, args, stream):
    """Time ``args.steps`` calls of ``run`` with HIP events on ``stream``:
    back to back (warm caches), or with ``args.cold`` each call after
    evict_caches. ``args.warmup`` untimed calls first, then untimed calls for
    ``args.ramp_s`` seconds (clock_ramp). Returns (ms per call, wall seconds
    of the timed region, calls of the clock ramp)."""
    for _ in range(args.warmup):
        run()
    ramp = clock_ramp(run, stream, args.ramp_s)
    dev = torch.device("cuda:0")
    evict = torch.zeros(COLD_EVICT_BYTES // 4, device=dev) if args.cold else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    total_ms = 0.0
    if not args.cold:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            run()
        e1.record(stream)
        e1.synchronize()
        total_ms = e0.elapsed_time(e1)
    else:
        for i in range(args.steps):
            evict_caches(evict)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            e1.synchronize()
            total_ms += e0.elapsed_time(e1)
    return total_ms / args.steps, time.perf_counter() - t0, ramp


def bench_decode(args):
    """Decode step: K back-to-back ssd_step calls on one state buffer (each
    sequence advances one token per call), timed with HIP events on the
    stream the kernel runs on. One kernel per step; it reads and writes the
    whole fp32 state, so HBM bandwidth bounds it."""
    batch, H, P, N, G = args.decode, 80, 64, 128, 1
    inp = si.make_step_inputs(batch, H, P, N, G, "bf16", seed=4000)
    dev = torch.device("cuda:0")
    x, dt, B, C = (inp[k][0].to(dev) for k in ("x", "dt", "B", "C"))
    A, D, state = inp["A"].to(dev), inp["D"].to(dev), inp["state"].to(dev)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)
    ms, wall, ramp = time_launches(lambda: ssd.step(x, dt, A, B, C, D, state, y=y, stream=stream),
                             args, stream)
    e = 2
    alg_bytes = batch * H * P * N * 4 * 2 + batch * (2 * H * P * e + H * e + 2 * G * N * e)
    alg_flops = batch * H * P * N * 6
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "SSD decode step tokens/s (one token per sequence, one layer)",
        "value": round(batch / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ramp_passes": ramp,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode-2.7b-b%d" % batch, "batch": batch, "nheads": H,
                   "headdim": P, "dstate": N, "ngroups": G,
                   "state_bytes": batch * H * P * N * 4,
                   "caches": "cold" if args.cold else "warm"},
        "roofline": {"kernel": "ssd_step", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("ssd_step", "decode-2.7b-b%d" % batch)},
        "kernels": {"ssd_step": {"ms": round(ms, 5), "alg_bytes": alg_bytes,
                                 "alg_flops": alg_flops, "GB/s": round(gbs, 1)}},
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


# Vector-ALU ceiling of the selective scan, from unit counts and clock: every
# (token, channel, state) element needs one exp2 (a transcendental, issued at
# a quarter of the full rate) and two FMAs, i.e. 6 full-rate lane-slots; a
# SIMD issues 16 lane-slots per cycle; 256 CUs x 4 SIMDs at 2.4 GHz.
SCAN_PEAK_ELEMS = 256 * 4 * 16 * 2.4e9 / 6


def bench_scan(args):
    """Mamba-1 selective scan: K back-to-back launches over the same inputs,
    timed with HIP events on the stream the kernel runs on."""
    batch, L, Dm, N = 8, 2048, 5120, args.scan
    inp = si.make_scan_inputs(batch, L, Dm, N, "bf16", seed=4100, h0_std=0.1)
    dev = torch.device("cuda:0")
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    y = torch.empty_like(d["x"])
    hT = torch.empty((batch, Dm, N), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev)
    run = lambda: ssd.selective_scan(d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                                     y=y, final_state=hT, stream=stream)
    ms, wall, ramp = time_launches(run, args, stream)
    elems = batch * L * Dm * N
    alg_bytes = batch * L * (3 * Dm * 2 + 2 * N * 2) + Dm * N * 4 + 2 * batch * Dm * N * 4
    achieved = elems / (ms * 1e-3)
    out = {
        "metric": "Mamba-1 selective scan tokens/s (the SSD layer's comparator)",
        "value": round(batch * L / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ramp_passes": ramp,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mamba1-scan-2.7b-N%d" % N, "batch": batch, "seq_len": L,
                   "dim": Dm, "dstate": N, "caches": "cold" if args.cold else "warm"},
        "roofline": {"kernel": "selective_scan", "bound": "alu",
                     "achieved": round(achieved / 1e9, 1), "peak": round(SCAN_PEAK_ELEMS / 1e9, 1),
                     "unit": "Gelem/s", "frac": round(achieved / SCAN_PEAK_ELEMS, 4),
                     "traffic": None},
        "kernels": {"selective_scan": {"ms": round(ms, 5), "alg_bytes": alg_bytes,
                                       "GB/s": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
                                       "elements": elems}},
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


def backward_cost(w: si.Workload, inp: dict) -> dict:
    """Bytes and flops of each backward kernel by the method's definition
    (unique HBM bytes; causal pairs only). The recompute stages are the
    forward's. Per (chunk, head): dy, x, dx q*P*e; ddt q*e; fp32 states P*N*4
    (h_in, the gradient state); per (chunk, group): B, C, dB, dC q*N*e.
    bwd_dx does, per head, dy x^T over the causal pairs, M^T dy, and
    two state products (g B, h_in C); bwd_dbc does dy x^T over the causal
    pairs and two state products per head, and Z B, Z^T C once per group."""
    e = 2
    lens = inp["seq_lens"] or [w.seqlen] * w.batch
    H, P, N, G, Q = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    T = int(sum(lens))
    chunks = [min(Q, L - c0) for L in lens for c0 in range(0, L, Q)]
    nc, S = len(chunks), len(lens)
    state = P * N * 4
    causal = sum(q * (q + 1) // 2 for q in chunks)
    f = algorithmic_cost(w, inp)
    cost = {k: f[k] for k in ("chunk_cumsum", "chunk_state", "state_passing")}
    cost["chunk_dstate"] = dict(bytes=T * H * P * e + T * G * N * e + T * H * 4 + nc * H * state,
                                flops=2 * T * H * P * N)
    cost["state_passing_bwd"] = dict(bytes=2 * nc * H * state + 2 * S * H * state,
                                     flops=2 * nc * H * P * N)
    cost["bwd_cbt"] = dict(bytes=2 * T * G * N * e + causal * G * 2,
                           flops=2 * causal * G * N)
    # bwd_dx also writes bf16 transposed copies of h_in and g (P*N*2 each per
    # (chunk, head)), which bwd_dbc reads in place of the fp32 states
    cost["bwd_dx"] = dict(bytes=3 * T * H * P * e + 2 * T * H * e + 2 * T * G * N * e
                          + 2 * nc * H * state + T * H * 4 + causal * G * 2
                          + 2 * nc * H * P * N * 2,
                          flops=4 * causal * H * P + 4 * T * H * P * N)
    cost["bwd_dbc"] = dict(bytes=2 * T * H * P * e + T * H * (e + 4) + 4 * T * G * N * e
                           + 2 * nc * H * P * N * 2,
                           flops=2 * causal * H * P + 4 * T * H * P * N + 4 * causal * G * N)
    cost["bwd_reduce"] = dict(bytes=2 * nc * H * 4 + 2 * H * 4, flops=2 * nc * H)
    cost["plan"] = dict(bytes=0, flops=0)
    return cost


def bench_backward(args):
    """Backward pass of the SSD layer on a workload config: K back-to-back
    plain ssd_backward calls timed with HIP events around the K calls, on the
    stream the kernels run on; after the timed region, K more calls with a HIP
    event after every kernel give the per-kernel times. The states are
    recomputed inside (no forward output is read)."""
    w = si.CONFIGS[args.config]
    inp = si.make_inputs(w)
    gin = si.make_grad_inputs(w, inp)
    dev = torch.device("cuda:0")
    d = {k: (None if inp[k] is None else inp[k].to(dev)) for k in ("x", "dt", "A", "B", "C",
                                                                   "D", "h0")}
    plan = ssd.BackwardPlan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                            gin["dy"].to(dev), gin["dhT"].to(dev), w.chunk, inp["cu_seqlens"])
    stream = torch.cuda.current_stream(dev)
    ms_per_step, wall, ramp = time_launches(lambda: plan.run(stream), args, stream)
    per_kernel_ms = plan.run_timed(args.steps, stream).as_dict()
    per_kernel_ms.pop("_total_ms")
    cost = backward_cost(w, inp)
    kernels = {}
    for name, ms in per_kernel_ms.items():
        c = cost.get(name, {"bytes": 0, "flops": 0})
        kernels[name] = {"ms": round(ms, 5), "alg_bytes": int(c["bytes"]),
                         "alg_flops": int(c["flops"]),
                         "GB/s": round(c["bytes"] / (ms * 1e-3) / 1e9, 1),
                         "TFLOP/s": round(c["flops"] / (ms * 1e-3) / 1e12, 2)}
    dom = max(per_kernel_ms, key=per_kernel_ms.get)
    kd, cd = kernels[dom], cost[dom]
    # the kernel's own roof: whichever of HBM and bf16 MFMA its algorithmic
    # bytes and flops reach first
    mfma_bound = cd["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12) > cd["bytes"] / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roofline = {"kernel": dom, "bound": "mfma", "achieved": kd["TFLOP/s"],
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(kd["TFLOP/s"] / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": measured_traffic(dom, "bwd-" + w.name)}
    else:
        roofline = {"kernel": dom, "bound": "hbm", "achieved": kd["GB/s"], "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(kd["GB/s"] / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(dom, "bwd-" + w.name),
                    "mfma_frac": round(kd["TFLOP/s"] / MFMA_BF16_PEAK_TFLOPS, 4)}
    out = {
        "metric": "SSD backward tokens/s (gradients of x, dt, A, B, C, D, h0; states "
                  "recomputed)",
        "value": round(plan.tokens / (ms_per_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ramp_passes": ramp,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bwd-" + w.name, "batch": w.batch if not w.num_seqs else 1,
                   "seq_len": plan.prob.seqlen, "nheads": w.nheads, "headdim": w.headdim,
                   "dstate": w.dstate, "ngroups": w.ngroups, "chunk_size": w.chunk,
                   "num_seqs": w.num_seqs, "tokens_per_step": plan.tokens},
        "roofline": roofline,
        "kernels": kernels,
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


def bench_conv(args):
    """Convolution front at the 2.7B shapes: batch 8, 2048 tokens, x 5120
    channels (80 heads x 64), B and C 128 channels each, 4 taps, bf16, with
    the history read and written; K back-to-back launches timed with HIP
    events on the kernel's stream. Every input is read once and every output
    written once, so HBM bandwidth bounds it."""
    batch, L, x_dim, bc_dim, K = 8, 2048, 5120, 128, 4
    ch = x_dim + 2 * bc_dim
    inp = si.make_conv_inputs(batch, L, x_dim, bc_dim, K, "bf16", seed=4300, history=True)
    dev = torch.device("cuda:0")
    xbc = inp["xbc"].view(batch, L, ch).to(dev)
    w, b, hist = inp["weight"].to(dev), inp["bias"].to(dev), inp["history"].to(dev)
    x = torch.empty((batch, L, x_dim), device=dev, dtype=torch.bfloat16)
    B = torch.empty((batch, L, bc_dim), device=dev, dtype=torch.bfloat16)
    C = torch.empty_like(B)
    ho = torch.empty_like(hist)
    stream = torch.cuda.current_stream(dev)
    ms, wall, ramp = time_launches(lambda: ssd.conv1d_silu(xbc, w, b, x_dim, bc_dim, hist, x=x, B=B,
                                                     C=C, history_out=ho, stream=stream),
                             args, stream)
    T, e = batch * L, 2
    alg_bytes = 2 * T * ch * e + 2 * batch * (K - 1) * ch * e + ch * (K + 1) * 4
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    workload = "conv-front-2.7b"
    out = {
        "metric": "SSD conv front tokens/s (causal depthwise conv1d + SiLU producing x, B, C)",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ramp_passes": ramp,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "batch": batch, "seq_len": L, "x_dim": x_dim,
                   "bc_dim": bc_dim, "width": K, "channels": ch,
                   "caches": "cold" if args.cold else "warm"},
        "roofline": {"kernel": "ssd_conv", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("ssd_conv", workload)},
        "kernels": {"ssd_conv": {"ms": round(ms, 5), "alg_bytes": alg_bytes,
                                 "alg_flops": T * ch * (2 * K + 4), "GB/s": round(gbs, 1)}},
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ramp-s", type=float, default=0.3,
                    help="after the warm-up, untimed passes for this many seconds, so that "
                         "the GPU's clocks have ramped up under load before the timed region")
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="run one kernel per step of the method instead of the fused kernel")
    ap.add_argument("--per-sequence", action="store_true",
                    help="run the fused kernel with one workgroup per (sequence, head)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads for the oracle baseline (default: all this process may use)")
    ap.add_argument("--decode", type=int, default=0, metavar="BATCH",
                    help="instead of the forward pass, time the decode step (ssd_step) "
                         "of BATCH sequences at the 2.7B shapes (H 80, P 64, N 128, bf16)")
    ap.add_argument("--scan", type=int, default=0, metavar="N",
                    help="instead of the SSD forward pass, time the Mamba-1 selective scan "
                         "(ssd_selective_scan) at the 2.7B shapes (batch 8, 2048 tokens, 5120 "
                         "channels) with state size N per channel")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the forward pass, time the backward pass (ssd_backward) "
                         "on the --config workload")
    ap.add_argument("--conv", action="store_true",
                    help="instead of the SSD forward pass, time the convolution front "
                         "(ssd_conv1d_silu) at the 2.7B shapes")
    ap.add_argument("--cold", action="store_true",
                    help="before every timed pass, read a 512 MiB buffer so that the pass "
                         "starts with the Infinity Cache (MALL) and the L2s holding none of its "
                         "data (and no dirty lines to write back)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device-to-device copy "
                         "of this many MiB (known HBM traffic) to calibrate byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the SSD forward pass here runs on a single "
              "MI355X (no sharding, no collectives); --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        # the same copy timed (events on torch's stream, which runs it): the
        # HBM rate a plain streaming read + write reaches on this GPU
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / max(args.steps, 1)
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": max(args.steps, 1), "ms_per_copy": round(ms, 5),
                          "GB/s_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}),
              flush=True)
        return

    if args.decode:
        bench_decode(args)
        return
    if args.scan:
        bench_scan(args)
        return
    if args.conv:
        bench_conv(args)
        return
    if args.backward:
        bench_backward(args)
        return

    w = si.CONFIGS[args.config]
    inp = si.make_inputs(w)
    dev = torch.device("cuda:0")
    d = {k: (None if inp[k] is None else inp[k].to(dev)) for k in ("x", "dt", "A", "B", "C",
                                                                   "D", "h0")}
    plan = ssd.Plan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                    chunk_size=w.chunk, cu_seqlens=inp["cu_seqlens"], unfused=args.unfused,
                    per_sequence=args.per_sequence)
    stream = torch.cuda.current_stream(dev)

    # Timed region (after W untimed warm-up passes and the clock ramp): K plain
    # ssd_forward passes (exactly what a caller enqueues), HIP events on the
    # kernels' stream around the whole loop only, synchronised on both sides
    # (or, with --cold, one pass at a time after an eviction read that the
    # events do not cover).
    ms_per_step, wall, ramp = time_launches(lambda: plan.run(stream), args, stream)
    if plan.chain_error():
        print("bench.py: a chained workgroup timed out waiting for its predecessor's state; "
              "the outputs of the timed passes are invalid", file=sys.stderr)
        sys.exit(3)
    tokens = plan.tokens
    value = tokens / (ms_per_step / 1e3)

    # Per-kernel durations for the roofline, from a second run of K passes of
    # the same launch sequence with a HIP event after every kernel (on the
    # kernels' stream). Each figure is a kernel's duration plus its launch
    # gap, so it can only understate the kernel's rate.
    if not args.cold:
        per_kernel_ms = plan.run_timed(args.steps, stream).as_dict()
        per_kernel_ms.pop("_total_ms")
    else:
        evict = torch.zeros(COLD_EVICT_BYTES // 4, device=dev, dtype=torch.float32)
        per_kernel_ms = {}
        for i in range(args.steps):
            evict_caches(evict)
            t = plan.run_timed(1, stream).as_dict()
            t.pop("_total_ms")
            for k, v in t.items():
                per_kernel_ms[k] = per_kernel_ms.get(k, 0.0) + v / args.steps
        del evict
    torch.cuda.synchronize()
    if plan.chain_error():
        print("bench.py: a chained workgroup timed out in the per-kernel passes",
              file=sys.stderr)
        sys.exit(3)

    lay = plan.layout()
    cost = algorithmic_cost(w, inp, int(lay.chain_chunks_per_unit), int(lay.chain_ranges))
    kernels = {}
    for name, ms in per_kernel_ms.items():
        c = cost.get(name, {"bytes": 0, "flops": 0})
        kernels[name] = {"ms": round(ms, 5), "alg_bytes": int(c["bytes"]),
                         "alg_flops": int(c["flops"]),
                         "GB/s": round(c["bytes"] / (ms * 1e-3) / 1e9, 1),
                         "TFLOP/s": round(c["flops"] / (ms * 1e-3) / 1e12, 2)}
    dom = max(per_kernel_ms, key=per_kernel_ms.get)
    kd = kernels[dom]
    # Every kernel of this path is HBM-bound by its algorithmic intensity
    # (flops/byte far below the bf16 ridge of ~312), so the roof is HBM.
    roofline = {"kernel": dom, "bound": "hbm", "achieved": kd["GB/s"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(kd["GB/s"] / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom, w.name),
                "alg_bytes": kd["alg_bytes"], "kernel_ms": kd["ms"],
                "overhead_bytes": int(cost.get(dom, {}).get("overhead_bytes", 0)),
                "mfma_frac": round(kd["TFLOP/s"] / (MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16"
                                                    else MFMA_FP32_PEAK_TFLOPS), 4)}
    path = cost["_path"]
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ramp_passes": ramp,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp32", "data": "synthetic",
        "config": {"workload": w.name, "kernels": ("unfused" if args.unfused else
                                                     "per_sequence" if args.per_sequence else
                                                     "default"), "batch": w.batch if not w.num_seqs else 1,
                   "seq_len": plan.prob.seqlen, "nheads": w.nheads, "headdim": w.headdim,
                   "dstate": w.dstate, "ngroups": w.ngroups, "chunk_size": w.chunk,
                   "num_seqs": w.num_seqs, "tokens_per_step": tokens,
                   "initial_state": inp["h0"] is not None,
                   "caches": "cold" if args.cold else "warm"},
        "roofline": roofline,
        "path": {"alg_bytes": int(path["bytes"]), "alg_flops": int(path["flops"]),
                 "GB/s": round(path["bytes"] / (ms_per_step * 1e-3) / 1e9, 1),
                 "hbm_frac": round(path["bytes"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "TFLOP/s": round(path["flops"] / (ms_per_step * 1e-3) / 1e12, 2)},
        "kernels": kernels,
        "wall_s_timed_region": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_budget, args.cpu_threads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
