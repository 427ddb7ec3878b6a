#!/usr/bin/env python3
"""Benchmark of the gated delta-rule hot path on one MI355X.

One step = one gdr_chunk_fwd call over the Gated DeltaNet workload (scalar gate,
B=8, H=16, T=8192, d_k=d_v=128, chunk 64, bf16 I/O, fp32 state), which runs every
stage of the chunkwise forward (log-gate scan, intra-chunk WY terms, state pass,
output, final state).  The headline value is tokens/s (B*T per step) with the
inputs already resident in HBM.  The decode step (256 sequences x 32 heads,
fp32 128x128 states, bf16 tokens) is timed in the same run and reported as GB/s,
and so is the serving handoff: a packed prefill of 32 prompts of log-uniform
lengths in [128, 8192] (H=16, d=128, scalar gate) through gdr_chunk_fwd_varlen,
then decode steps on the states it hands over (`handoff`), and the
preconditioner scan of the preconditioned delta rule (with forgetting) over the
workload's keys (`precond_scan`, GB/s against HBM peak), and the chunk forward
with the write keys it produced (`osdn`: phase 2, no gate, and the two phases'
tokens/s), and the backward of the chunk forward over the same workload
(`backward`: the gradients of q, k, v, beta, log a and S0 for given dO and dS_T;
`train_step_tokens_per_s` counts the forward and the backward together).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  `roofline` is for the chunk-forward kernel: algorithmic
bytes per launch (inputs read once, outputs written once) over the average
launch time measured with HIP events on the launch stream.  `cpu_baseline` is the
fp64 oracle timed on one host core over a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PROFILE_DIR = os.path.join(ROOT, "profiles")
CHUNK_SOURCES = [os.path.join(ROOT, "gated_delta_rule_21_amd", "csrc", n)
                 for n in ("chunk_prep.hip", "chunk_state.hip", "chunk_fwd.hip", "chunk_common.h", "device_common.h")]
DECODE_SOURCES = [os.path.join(ROOT, "gated_delta_rule_21_amd", "csrc", n)
                  for n in ("decode_step.hip", "device_common.h")]
PRECOND_SOURCES = [os.path.join(ROOT, "gated_delta_rule_21_amd", "csrc", n)
                   for n in ("precond_scan.hip", "chunk_common.h", "device_common.h")]
BWD_SOURCES = [os.path.join(ROOT, "gated_delta_rule_21_amd", "csrc", n)
               for n in ("chunk_bwd.hip", "bwd_common.h", "chunk_prep.hip", "chunk_common.h", "device_common.h")]


def chunk_algorithmic(wl, with_S0: bool):
    """Bytes and useful flops of one chunk-forward call.

    Bytes: q, k, v, beta, log_a (and S0 when given) read once; o and S_T written once.
    Flops per (chunk, head) with C = chunk, for the intra-chunk Gram and score
    matrices (lower triangles), the triangular solve, W and U, and the three
    state products:  C(C-1)d_k + C^3/3 + C(C+1)(2d_k+2d_v) + 6 C d_k d_v.
    """
    esz = 2 if wl.io == "bf16" else 4
    ntok = wl.B * wl.T * wl.H
    gate_w = {"none": 0, "scalar": 1, "channel": wl.d_k}[wl.gate]
    state = wl.B * wl.H * wl.d_k * wl.d_v * 4
    rd = ntok * (2 * wl.d_k + wl.d_v + 1 + gate_w) * esz + (state if with_S0 else 0)
    wr = ntok * wl.d_v * esz + state
    C, dk, dv = wl.chunk, wl.d_k, wl.d_v
    per_chunk = C * (C - 1) * dk + C ** 3 / 3 + C * (C + 1) * (2 * dk + 2 * dv) + 6 * C * dk * dv
    nchunks = -(-wl.T // C)
    return rd + wr, per_chunk * nchunks * wl.B * wl.H


def decode_bytes(wl):
    """Bytes of one decode step: each fp32 state read and written once, plus q, k,
    v, beta, log_a read and o written (bf16)."""
    esz = 2 if wl.io == "bf16" else 4
    gate_w = {"none": 0, "scalar": 1, "channel": wl.d_k}[wl.gate]
    per = 2 * 4 * wl.d_k * wl.d_v + esz * (2 * wl.d_k + 2 * wl.d_v + 1 + gate_w)
    return wl.N * wl.H * per


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic(name: str, sources):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was
    taken on the current kernel source (None otherwise)."""
    path = os.path.join(PROFILE_DIR, name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_s = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m_b or not m_s or m_s.group(1) != source_digest(sources):
        return None
    return float(m_b.group(1))


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline_child(T: int, heads: int, batches: int) -> None:
    """Run the oracle on `batches` sequences x `heads` heads x T tokens of the gated workload."""
    import numpy as np
    from oracle import forward
    from workloads import CONFIGS, slice_inputs
    wl = CONFIGS[3]
    sl = [[slice_inputs(wl, b, h, T) for h in range(heads)] for b in range(batches)]
    st = lambda n: np.stack([np.stack([s[n] for s in row], axis=1) for row in sl], axis=0)
    args = [st(n) for n in ("q", "k", "v", "beta", "log_a")]
    del sl
    t0 = time.perf_counter()
    forward(*args, None)
    dt = time.perf_counter() - t0
    print(json.dumps({"seconds": dt, "T": T, "heads": heads, "batches": batches}))


def cpu_baseline(T: int, heads: int, batches: int, H_total: int):
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    out = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child",
                          "--cpu-T", str(T), "--cpu-heads", str(heads), "--cpu-batches", str(batches)],
                         capture_output=True, text=True, env=env, check=True)
    r = json.loads(out.stdout.strip().splitlines()[-1])
    head_tok_s = r["batches"] * r["heads"] * r["T"] / r["seconds"]
    return {"value": head_tok_s / H_total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": (f"fp64 token-by-token oracle (NumPy, one thread) on {batches} sequences x {heads} of "
                       f"{H_total} heads x {T} tokens of the gated workload, S0 = 0; {r['seconds']:.1f} s; "
                       "tokens/s = head-tokens/s / H"),
            "seconds": round(r["seconds"], 2)}


def copy_calibration(log, nbytes: int = 1 << 30, reps: int = 3):
    """Streaming elementwise kernel over fp32 that reads `nbytes` and writes `nbytes`
    (torch.neg, out of place).  Profiled beside the hot path, it gives the scale
    between the HBM byte counters and bytes actually moved."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} x torch.neg over {nbytes} bytes read + {nbytes} written")
    del src, dst


# ------------------------------------------------------------------ GPU legs
def bench_chunk(args, log):
    import torch
    import gated_delta_rule_21_amd as gdr
    from workloads import CONFIGS, chunk_inputs
    wl = CONFIGS[args.chunk_config]
    log(f"generating {wl.name}")
    inp = chunk_inputs(wl)
    dev = lambda x: None if x is None else torch.from_numpy(x).to(torch.bfloat16).cuda()
    q, k, v, beta, log_a = (dev(inp[n]) for n in ("q", "k", "v", "beta", "log_a"))
    with_S0 = wl.s0_std > 0
    S0 = torch.from_numpy(inp["S0"]).cuda() if with_S0 else None
    del inp
    o = torch.empty((wl.B, wl.T, wl.H, wl.d_v), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((wl.B, wl.H, wl.d_k, wl.d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdr.chunk_workspace_size(wl.B, wl.T, wl.H, wl.d_k, wl.d_v, torch.bfloat16, wl.gate),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        gdr.chunk_fwd(q, k, v, beta, log_a, S0, o=o, S_T=S_T, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    log(f"chunk forward: {ms:.3f} ms/step (wall {1e3 * wall / args.steps:.3f} ms/step)")
    nbytes, flops = chunk_algorithmic(wl, with_S0=with_S0)
    return wl, ms, nbytes, flops, (q, k, v, beta, log_a, S0)


def bench_decode(args, log):
    import torch
    import gated_delta_rule_21_amd as gdr
    from workloads import DECODE_CONFIG, decode_inputs
    wl = DECODE_CONFIG
    n_sets = 16
    log(f"generating {wl.name} ({n_sets} token sets, reused cyclically)")
    inp = decode_inputs(wl, steps=n_sets)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    q, k, v, beta, log_a = (dev(inp[n]) for n in ("q", "k", "v", "beta", "log_a"))
    S = torch.from_numpy(inp["S0"]).cuda()
    o = torch.empty((wl.N, wl.H, wl.d_v), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(s):
        j = s % n_sets
        gdr.recurrent_step(q[j], k[j], v[j], beta[j], log_a[j], S, o=o)

    # A decode step is ~10 us: warm up over as many steps as are timed, so the
    # clocks are at their steady state however small --warmup is.
    for s in range(max(args.warmup, args.decode_steps)):
        step(s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for s in range(args.decode_steps):
        step(s)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.decode_steps
    nbytes = decode_bytes(wl)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"decode: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s")
    return {"value": round(gbs, 1), "unit": "GB/s", "us_per_step": round(ms * 1e3, 2),
            "tokens_per_s": round(wl.N / (ms * 1e-3), 1), "steps": args.decode_steps,
            "workload": wl.name, "bytes_per_step": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic("decode_step_n256h32d128_counters.md", DECODE_SOURCES)}}


def precond_bytes(B: int, T: int, H: int, d_k: int, esz: int, apf: bool) -> int:
    """Bytes of one preconditioner scan: k, beta (and r) read once, d0 read, kw and
    d_T written once."""
    ntok = B * T * H
    return ntok * (2 * d_k * esz + esz * (2 if apf else 1)) + 2 * B * H * d_k * 4


def bench_precond(args, log, wl, k, beta):
    """The preconditioner scan (with forgetting) over the keys of the chunk workload."""
    import torch
    import gated_delta_rule_21_amd as gdr
    from workloads import PRECOND_ETA, precond_factors
    log("generating the scan's retention and starting preconditioner")
    f = precond_factors(wl)
    r = torch.from_numpy(f["r"]).to(torch.bfloat16).cuda()
    d0 = torch.from_numpy(f["d0"]).cuda()
    kw = torch.empty_like(k)
    dT = torch.empty_like(d0)
    stream = torch.cuda.current_stream()

    def step():
        gdr.precond_scan(k, beta, PRECOND_ETA, r, d0, kw=kw, d_T=dT)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    nbytes = precond_bytes(wl.B, wl.T, wl.H, wl.d_k, 2, True)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"preconditioner scan: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    return kw, {"workload": "osdn_precond_scan_apf_b%dh%dt%dd%d_bf16" % (wl.B, wl.H, wl.T, wl.d_k),
            "value": round(gbs, 1), "unit": "GB/s", "us_per_launch": round(ms * 1e3, 2),
            "tokens_per_s": round(wl.B * wl.T / (ms * 1e-3), 1), "bytes_per_launch": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic("precond_scan_b8h16t8192d128_counters.md", PRECOND_SOURCES)}}


def bwd_bytes(wl, with_S0: bool):
    """Bytes of one backward call if every input were read once and every output
    written once: q, k, v, dO, beta, log_a (S0, dS_T) read; dq, dk, dv, dbeta,
    dlog_a, dS0 written.  The per-chunk records and the two sets of chunk states
    the call keeps in its workspace are not counted."""
    esz = 2
    ntok = wl.B * wl.T * wl.H
    gate_w = 1 if wl.gate == "scalar" else 0
    state = wl.B * wl.H * wl.d_k * wl.d_v * 4
    rd = ntok * (2 * wl.d_k + 2 * wl.d_v + 1 + gate_w) * esz + state * (2 if with_S0 else 1)
    wr = ntok * (2 * wl.d_k + wl.d_v + 1 + gate_w) * esz + state
    return rd + wr


def bwd_algorithmic(wl):
    """Useful flops of the backward per launch: per chunk (C = 64, d = d_k = d_v),
    the chunk-start states 4 C d^2 + C^2 d (K S, T X, K^T Delta), the reverse pass
    6 C d^2 + 3 C^2 d (P, K dS', P^T dO, T^T dDelta, Q^T dO, K^T Z) and the
    per-chunk gradients 10 C d^2 + 11 C^2 d (five state products, eleven 64-row
    products, the masked ones counted at half)."""
    C, d = 64, wl.d_k
    per_chunk = 20 * C * d * d + 15 * C * C * d
    return wl.B * wl.H * ((wl.T + C - 1) // C) * per_chunk


def bench_bwd(args, log, wl, q, k, v, beta, log_a, S0, fwd_ms):
    """The backward of the chunk forward over the same workload, with dO ~ N(0, 1)
    and dS_T ~ N(0, 1); the gradients of every input and of S0."""
    import torch
    import gated_delta_rule_21_amd as gdr
    from workloads import grad_inputs
    log("generating the output gradients")
    g = grad_inputs(wl)
    dO = torch.from_numpy(g["dO"]).to(torch.bfloat16).cuda()
    dS_T = torch.from_numpy(g["dS_T"]).cuda()
    del g
    ws = torch.empty(gdr.chunk_bwd_workspace_size(wl.B, wl.T, wl.H, wl.d_k, wl.d_v, torch.bfloat16, wl.gate),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        return gdr.chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = bwd_algorithmic(wl)
    tf = flops / (ms * 1e-3) / 1e12
    log(f"chunk backward: {ms:.3f} ms/step, {tf:.1f} TFLOP/s useful")
    return {"workload": wl.name + "_backward", "value": round(wl.B * wl.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_launch": round(ms, 4), "useful_flops_per_launch": flops,
            "train_step_tokens_per_s": round(wl.B * wl.T / ((ms + fwd_ms) * 1e-3), 1),
            "train_step_ms": round(ms + fwd_ms, 4),
            "algorithmic_bytes_per_launch": bwd_bytes(wl, S0 is not None),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": (profiled_traffic("chunk_bwd_gated_b8h16t8192d128_counters.md", BWD_SOURCES)
                                     if wl.name == "gated_deltanet_scalar_b8h16t8192d128_bf16" else None)}}


def bench_wkey(args, log, wl, q, k, v, beta, kw, scan_us):
    """Phase 2 of the preconditioned delta rule: the chunk forward with the write
    keys the scan produced (no gate), over the chunk workload's q, k, v, beta."""
    import torch
    import gated_delta_rule_21_amd as gdr
    o = torch.empty_like(v)
    S_T = torch.empty((wl.B, wl.H, wl.d_k, wl.d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdr.chunk_workspace_size(wl.B, wl.T, wl.H, wl.d_k, wl.d_v, torch.bfloat16, "none"),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        gdr.chunk_fwd(q, k, v, beta, None, None, o=o, S_T=S_T, workspace=ws, kw=kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    nbytes, _ = chunk_algorithmic(wl.replace(gate="none"), with_S0=False)
    nbytes += wl.B * wl.T * wl.H * wl.d_k * 2          # the write keys
    gbs = nbytes / (ms * 1e-3) / 1e9
    total_ms = ms + scan_us * 1e-3
    log(f"write-key forward: {ms * 1e3:.1f} us, {gbs:.0f} GB/s; scan + forward {total_ms * 1e3:.1f} us")
    return {"workload": "osdn_two_phase_b%dh%dt%dd%d_bf16" % (wl.B, wl.H, wl.T, wl.d_k),
            "forward_us": round(ms * 1e3, 2), "scan_us": scan_us,
            "tokens_per_s": round(wl.B * wl.T / (total_ms * 1e-3), 1),
            "forward_roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
            "forward_bytes_per_launch": nbytes}


def handoff_lengths(n_seq: int = 32, lo: int = 128, hi: int = 8192, seed: int = 6):
    """Prompt lengths of the serving mix: log-uniform on [lo, hi], seeded."""
    import numpy as np
    rs = np.random.RandomState(seed)
    return [int(round(x)) for x in np.exp(rs.uniform(np.log(lo), np.log(hi), size=n_seq))]


def bench_handoff(args, log):
    """Packed prefill of a batch of prompts of mixed lengths, then decode steps on the
    states it hands over (the serving steps on either side of the chunk forward)."""
    import numpy as np
    import torch
    import gated_delta_rule_21_amd as gdr
    from workloads import Workload, chunk_inputs
    lens = handoff_lengths()
    N, H, dk, dv, total = len(lens), 16, 128, 128, int(sum(lens))
    log(f"generating the handoff mix ({N} prompts, {total} tokens)")
    inp = chunk_inputs(Workload("handoff_prefill", B=1, T=total, H=H, d_k=dk, d_v=dv, io="bf16", gate="scalar",
                                s0_std=0.0, seed=6))
    n_sets = 16
    tok = chunk_inputs(Workload("handoff_tokens", B=N, T=n_sets, H=H, d_k=dk, d_v=dv, io="bf16", gate="scalar",
                                s0_std=0.0, seed=7))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()
    q, k, v, beta, log_a = (dev(inp[n]) for n in ("q", "k", "v", "beta", "log_a"))
    tq, tk, tv, tb, tl = ([dev(tok[n][:, j]) for j in range(n_sets)] for n in ("q", "k", "v", "beta", "log_a"))
    del inp, tok
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    o = torch.empty((1, total, H, dv), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((N, H, dk, dv), dtype=torch.float32, device="cuda")
    od = torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdr.chunk_varlen_workspace_size(total, N, H, dk, dv, torch.bfloat16, "scalar"),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    prefill = lambda: gdr.chunk_fwd_varlen(q, k, v, beta, log_a, cu, None, o=o, S_T=S, workspace=ws)
    decode = lambda j: gdr.recurrent_step(tq[j % n_sets], tk[j % n_sets], tv[j % n_sets], tb[j % n_sets],
                                          tl[j % n_sets], S, o=od)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    reps, dsteps = 5, 200
    for _ in range(2):
        prefill()
        decode(0)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(reps):
        prefill()
    ev[1].record(stream)
    prefill()
    decode(0)
    ev[2].record(stream)
    for j in range(1, dsteps + 1):
        decode(j)
    ev[3].record(stream)
    torch.cuda.synchronize()
    pre_ms = ev[0].elapsed_time(ev[1]) / reps
    first_ms = ev[1].elapsed_time(ev[2])
    dec_ms = ev[2].elapsed_time(ev[3]) / dsteps
    dec_bytes = N * H * (2 * 4 * dk * dv + 2 * (2 * dk + 2 * dv + 2))
    log(f"handoff: prefill {pre_ms:.3f} ms ({total / (pre_ms * 1e-3) / 1e6:.1f} M tokens/s), "
        f"decode {dec_ms * 1e3:.1f} us/step")
    return {"workload": "handoff_gated_n%d_h%d_d%d_loguniform128-8192" % (N, H, dk),
            "n_seq": N, "total_tokens": total, "min_len": min(lens), "max_len": max(lens),
            "prefill_ms": round(pre_ms, 4), "prefill_tokens_per_s": round(total / (pre_ms * 1e-3), 1),
            "prefill_plus_first_decode_ms": round(first_ms, 4),
            "decode_us_per_step": round(dec_ms * 1e3, 2), "decode_steps": dsteps,
            "decode_GBps": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The GPU's clocks ramp up over its first ~100 steps after an idle spell (the
    # input generation between legs): a chunk forward step measures 457 us after 3
    # warmup steps, 393 us after 30 and 365-367 us after 100 or more.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--chunk-config", type=int, default=3, choices=(2, 3, 4),
                    help="chunk-forward workload (3 = the gated workload of the headline metric)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-handoff", action="store_true",
                    help="skip the packed-prefill -> decode handoff leg")
    ap.add_argument("--no-precond", action="store_true", help="skip the preconditioner-scan leg")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-T", type=int, default=8192)
    ap.add_argument("--cpu-heads", type=int, default=16)
    ap.add_argument("--cpu-batches", type=int, default=4)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB streaming copy first (for scaling HBM byte counters)")
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    if args.cpu_baseline_child:
        cpu_baseline_child(args.cpu_T, args.cpu_heads, args.cpu_batches)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the hot path has no multi-GPU leg in this build.", file=sys.stderr)
        sys.exit(2)

    log = (lambda *a: None) if args.quiet else (lambda *a: print("[bench]", *a, file=sys.stderr, flush=True))
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import gated_delta_rule_21_amd as gdr
    gdr.load()
    if args.copy_calibration:
        copy_calibration(log)

    wl, ms, nbytes, flops, (q, k, v, beta, log_a, S0) = bench_chunk(args, log)
    tok_s = wl.B * wl.T / (ms * 1e-3)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    decode = None if args.no_decode else bench_decode(args, log)
    handoff = None if args.no_handoff else bench_handoff(args, log)
    precond = osdn = None
    if not args.no_precond:
        kw, precond = bench_precond(args, log, wl, k, beta)
        osdn = bench_wkey(args, log, wl, q, k, v, beta, kw, precond["us_per_launch"])
        del kw
    bwd = None if args.no_bwd else bench_bwd(args, log, wl, q, k, v, beta, log_a, S0, ms)
    del q, k, v, beta, log_a, S0
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle sample")
        cpu = cpu_baseline(args.cpu_T, args.cpu_heads, args.cpu_batches, wl.H)

    line = {
        "metric": "tokens/s + % MFMA peak, gated delta-rule chunk fwd T=8192 d=128; decode GB/s",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": wl.H, "d_k": wl.d_k, "d_v": wl.d_v,
                   "chunk": wl.chunk, "gate": wl.gate, "io": wl.io, "state": "fp32",
                   "S0": "N(0, %g^2)" % wl.s0_std if wl.s0_std > 0 else "zero",
                   "global_batch": wl.B, "seq_len": wl.T, "parallelism": "none (1 GPU)"},
        "tflops_useful": round(tflops, 2),
        "mfma_frac_useful": round(tflops / BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": (profiled_traffic("chunk_fwd_gated_b8h16t8192d128_counters.md", CHUNK_SOURCES)
                                 if args.chunk_config == 3 else None)},
        "algorithmic_bytes_per_launch": nbytes,
        "useful_flops_per_launch": flops,
        "decode": decode,
        "handoff": handoff,
        "precond_scan": precond,
        "osdn": osdn,
        "backward": bwd,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
