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
`train_step_tokens_per_s` counts the forward and the backward together; its
`training_path` times the forward that keeps the chunk-start states,
gdr_chunk_fwd_save, and the backward that takes them, gdr_chunk_bwd_saved).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Every input is generated on the host and moved to the GPU before any leg is
timed; the legs then run back to back, the headline chunk forward last, so that
no leg starts on a GPU that has idled while the host generated inputs (its
clocks take ~100 calls to come back up).  Besides the headline workload, the
other three chunk-forward workloads are timed (`configs`: the fp32 DeltaNet
B1 H1 T256 d64, the DeltaNet B4 H16 T4096 d128 with three copies of its inputs
taken in turn so the repeats do not run from the 256 MB Infinity Cache, and
the per-channel B2 H32 T32768 d128), and so is the backward on the per-channel
workload (`backward_channel`: the recomputing backward and the training path).

Prints one JSON line.  `roofline` is for the chunk-forward call: algorithmic
bytes per launch (inputs read once, outputs written once) over the average
launch time measured with HIP events on the launch stream.  `cpu_baseline` is the
fp64 oracle over the whole headline workload, its (b, h) slices split over up to
16 host processes (one BLAS thread each), with a one-process figure beside it.
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
def cpu_baseline_child(T: int, bs, hs) -> None:
    """Run the oracle on the (b, h) slices zip(bs, hs), T tokens each, of the gated
    workload (independent slices side by side as the heads of one sequence)."""
    import numpy as np
    from oracle import forward
    from workloads import CONFIGS, slice_inputs
    wl = CONFIGS[3]
    sl = [slice_inputs(wl, b, h, T) for b, h in zip(bs, hs)]
    args = [np.stack([s[n] for s in sl], axis=1)[None] for n in ("q", "k", "v", "beta", "log_a")]
    del sl
    t0 = time.perf_counter()
    forward(*args, None)
    dt = time.perf_counter() - t0
    print(json.dumps({"seconds": dt, "T": T, "slices": len(bs)}))


def host_cores() -> int:
    """Host cores for the oracle: those this process may run on, at most 16 (a GPU's share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(T: int, log):
    """The oracle over every (b, h) slice of the headline workload (T tokens each), the
    slices dealt to P = host_cores() processes run side by side; tokens/s = B T over
    the slowest process's oracle time.  Then one process alone on one of those groups."""
    from workloads import CONFIGS
    wl = CONFIGS[3]
    P = host_cores()
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    slices = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    groups = [slices[i::P] for i in range(P)]
    cmd = lambda g: [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", "--cpu-T", str(T),
                     "--cpu-b", ",".join(str(b) for b, _ in g), "--cpu-h", ",".join(str(h) for _, h in g)]
    log(f"CPU oracle: {len(slices)} slices x {T} tokens over {P} processes")
    t0 = time.perf_counter()
    procs = [subprocess.Popen(cmd(g), stdout=subprocess.PIPE, text=True, env=env) for g in groups if g]
    outs = [p.communicate()[0] for p in procs]
    wall = time.perf_counter() - t0
    if any(p.returncode != 0 for p in procs):
        raise RuntimeError("a CPU oracle process failed")
    secs = [sum(json.loads(l)["seconds"] for l in o.strip().splitlines()) for o in outs]
    value = wl.B * T / max(secs)
    log(f"CPU oracle: {max(secs):.1f} s over {len(procs)} processes; one process alone next")
    one = subprocess.run(cmd(groups[0]), capture_output=True, text=True, env=env, check=True)
    s1 = sum(json.loads(l)["seconds"] for l in one.stdout.strip().splitlines())
    per_slice_tok_s = len(groups[0]) * T / s1          # head-tokens per second on one core
    return {"value": round(value, 1), "unit": "tokens/s", "cores": len(procs), "kind": "oracle",
            "sample": (f"fp64 token-by-token oracle (NumPy, one BLAS thread per process) on all {len(slices)} "
                       f"(sequence, head) slices x {T} tokens of the gated workload, S0 = 0, dealt to "
                       f"{len(procs)} processes side by side; tokens/s = B*T / slowest process's oracle time "
                       f"({max(secs):.1f} s; wall {wall:.1f} s with input generation)"),
            "seconds": round(max(secs), 2),
            "single_core": {"value": round(per_slice_tok_s / wl.H, 1), "unit": "tokens/s", "cores": 1,
                            "sample": f"one process on {len(groups[0])} slices x {T} tokens ({s1:.1f} s); "
                                      "tokens/s = head-tokens/s / H"}}


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
def time_calls(fn, warmup: int, steps: int) -> float:
    """ms per call of fn() over `steps` calls after `warmup` untimed ones, from HIP
    events recorded on the current stream (the stream the library launches on)."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(steps):
        fn(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def chunk_traffic_profile(wl):
    """Name of the committed HBM counter summary of a chunk-forward workload."""
    return {"gated_deltanet_scalar_b8h16t8192d128_bf16": "chunk_fwd_gated_b8h16t8192d128_counters.md",
            "deltanet_b4h16t4096d128_bf16": "chunk_fwd_deltanet_b4h16t4096d128_counters.md",
            "kda_channel_b2h32t32768d128_bf16": "chunk_fwd_channel_b2h32t32768d128_counters.md"}.get(wl.name)


def prepare_chunk(cfg: int, copies: int, log):
    """Device-resident inputs, outputs and workspace of a chunk-forward workload
    (`copies` sets of inputs and outputs, taken in turn)."""
    import torch
    import gated_delta_rule_21_amd as gdr
    from workloads import CONFIGS, chunk_inputs
    wl = CONFIGS[cfg]
    log(f"generating {wl.name}")
    inp = chunk_inputs(wl)
    dt = torch.bfloat16 if wl.io == "bf16" else torch.float32
    dev = lambda x: None if x is None else torch.from_numpy(x).to(dt).cuda()
    with_S0 = wl.s0_std > 0
    sets = []
    for _ in range(copies):
        sets.append(dict(args=[dev(inp[n]) for n in ("q", "k", "v", "beta", "log_a")],
                         S0=torch.from_numpy(inp["S0"]).cuda() if with_S0 else None,
                         o=torch.empty((wl.B, wl.T, wl.H, wl.d_v), dtype=dt, device="cuda"),
                         S_T=torch.empty((wl.B, wl.H, wl.d_k, wl.d_v), dtype=torch.float32, device="cuda")))
    del inp
    ws = torch.empty(gdr.chunk_workspace_size(wl.B, wl.T, wl.H, wl.d_k, wl.d_v, dt, wl.gate),
                     dtype=torch.uint8, device="cuda")
    return dict(wl=wl, sets=sets, ws=ws, with_S0=with_S0)


def bench_chunk(prep, warmup: int, steps: int, log, label: str):
    """Time gdr_chunk_fwd on a prepared workload; returns its record."""
    import gated_delta_rule_21_amd as gdr
    wl, sets, ws = prep["wl"], prep["sets"], prep["ws"]

    def call(i):
        st = sets[i % len(sets)]
        gdr.chunk_fwd(*st["args"], st["S0"], o=st["o"], S_T=st["S_T"], workspace=ws)

    ms = time_calls(call, warmup, steps)
    nbytes, flops = chunk_algorithmic(wl, with_S0=prep["with_S0"])
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    log(f"{label} {wl.name}: {ms:.4f} ms/call, {gbs:.0f} GB/s, {tf:.1f} TFLOP/s useful")
    prof = chunk_traffic_profile(wl)
    return {"workload": wl.name, "ms_per_call": round(ms, 4), "tokens_per_s": round(wl.B * wl.T / (ms * 1e-3), 1),
            "tflops_useful": round(tf, 2), "mfma_frac_useful": round(tf / BF16_PEAK_TFLOPS, 4),
            "warmup": warmup, "steps": steps, "input_copies": len(sets),
            "algorithmic_bytes_per_launch": nbytes, "useful_flops_per_launch": flops,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic(prof, CHUNK_SOURCES) if prof else None}}


def prepare_decode(log, n_sets: int = 16):
    import torch
    from workloads import DECODE_CONFIG, decode_inputs
    wl = DECODE_CONFIG
    log(f"generating {wl.name} ({n_sets} token sets, reused cyclically)")
    inp = decode_inputs(wl, steps=n_sets)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    return dict(wl=wl, n_sets=n_sets, tok=[dev(inp[n]) for n in ("q", "k", "v", "beta", "log_a")],
                S=torch.from_numpy(inp["S0"]).cuda(),
                o=torch.empty((wl.N, wl.H, wl.d_v), dtype=torch.bfloat16, device="cuda"))


def bench_decode(prep, args, log):
    import gated_delta_rule_21_amd as gdr
    wl, n_sets, (q, k, v, beta, log_a), S, o = prep["wl"], prep["n_sets"], prep["tok"], prep["S"], prep["o"]

    def step(s):
        j = s % n_sets
        gdr.recurrent_step(q[j], k[j], v[j], beta[j], log_a[j], S, o=o)

    warmup = max(args.warmup, 100)
    ms = time_calls(step, warmup, args.decode_steps)
    nbytes = decode_bytes(wl)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"decode: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s")
    return {"value": round(gbs, 1), "unit": "GB/s", "us_per_step": round(ms * 1e3, 2),
            "tokens_per_s": round(wl.N / (ms * 1e-3), 1), "steps": args.decode_steps, "warmup_steps": warmup,
            "workload": wl.name, "bytes_per_step": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic("decode_step_n256h32d128_counters.md", DECODE_SOURCES)}}


def precond_bytes(B: int, T: int, H: int, d_k: int, esz: int, apf: bool) -> int:
    """Bytes of one preconditioner scan: k, beta (and r) read once, d0 read, kw and
    d_T written once."""
    ntok = B * T * H
    return ntok * (2 * d_k * esz + esz * (2 if apf else 1)) + 2 * B * H * d_k * 4


def precond_bwd_bytes(B: int, T: int, H: int, d_k: int, esz: int, apf: bool) -> int:
    """Bytes of one scan backward if every input were read once and every output
    written once: k, dkw, beta (and r) read, d0 and dd_T read; dk, dbeta (and dr)
    written, dd0 written.  The workspace (each token's preconditioner, written by
    the forward sweep and read back by the reverse) is not counted."""
    ntok = B * T * H
    return ntok * (3 * d_k * esz + esz * (4 if apf else 2)) + 3 * B * H * d_k * 4


def prepare_precond(wl, log):
    import torch
    from workloads import precond_factors
    log("generating the scan's retention and starting preconditioner")
    f = precond_factors(wl)
    return dict(r=torch.from_numpy(f["r"]).to(torch.bfloat16).cuda(), d0=torch.from_numpy(f["d0"]).cuda())


def bench_precond(prep, args, log, wl, k, beta):
    """The preconditioner scan (with forgetting) over the keys of the chunk workload."""
    import torch
    import gated_delta_rule_21_amd as gdr
    from workloads import PRECOND_ETA
    r, d0 = prep["r"], prep["d0"]
    kw = torch.empty_like(k)
    dT = torch.empty_like(d0)
    ms = time_calls(lambda i: gdr.precond_scan(k, beta, PRECOND_ETA, r, d0, kw=kw, d_T=dT), args.warmup, args.steps)
    nbytes = precond_bytes(wl.B, wl.T, wl.H, wl.d_k, 2, True)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"preconditioner scan: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    # its backward (the gradients of <dkw, kw> + <dd_T, d_T> in k, beta, r and d0),
    # with seeded N(0, 1) output gradients generated on the GPU before the timing
    gen = torch.Generator(device="cuda").manual_seed(5)
    dkw = torch.randn(k.shape, generator=gen, device="cuda").to(k.dtype)
    dd_T = torch.randn(d0.shape, generator=gen, device="cuda")
    ws = torch.empty(gdr.precond_scan_bwd_workspace_size(wl.B, wl.T, wl.H, wl.d_k), dtype=torch.uint8, device="cuda")
    bms = time_calls(lambda i: gdr.precond_scan_bwd(k, beta, PRECOND_ETA, r, d0, dkw, dd_T, workspace=ws),
                     args.warmup, args.steps)
    del dkw, dd_T, ws
    bbytes = precond_bwd_bytes(wl.B, wl.T, wl.H, wl.d_k, 2, True)
    bgbs = bbytes / (bms * 1e-3) / 1e9
    log(f"preconditioner scan backward: {bms * 1e3:.1f} us")
    return kw, {"workload": "osdn_precond_scan_apf_b%dh%dt%dd%d_bf16" % (wl.B, wl.H, wl.T, wl.d_k),
            "value": round(gbs, 1), "unit": "GB/s", "us_per_launch": round(ms * 1e3, 2),
            "backward_us_per_launch": round(bms * 1e3, 2),
            "backward_roofline": {"bound": "hbm", "achieved": round(bgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(bgbs / HBM_PEAK_GBS, 4), "bytes_per_launch": bbytes,
                                  "traffic": profiled_traffic("precond_scan_bwd_b8h16t8192d128_counters.md",
                                                              PRECOND_SOURCES)},
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
    gate_w = {"none": 0, "scalar": 1, "channel": wl.d_k}[wl.gate]
    state = wl.B * wl.H * wl.d_k * wl.d_v * 4
    rd = ntok * (2 * wl.d_k + 2 * wl.d_v + 1 + gate_w) * esz + state * (2 if with_S0 else 1)
    wr = ntok * (2 * wl.d_k + wl.d_v + 1 + gate_w) * esz + state
    return rd + wr


def bwd_algorithmic(wl, saved: bool = False):
    """Useful flops of the backward per launch: per chunk (C = 64, d = d_k = d_v),
    the chunk-start states 4 C d^2 + C^2 d (K S, T X, K^T Delta), the reverse pass
    6 C d^2 + 3 C^2 d (P, K dS', P^T dO, T^T dDelta, Q^T dO, K^T Z) and the
    per-chunk gradients 10 C d^2 + 11 C^2 d (five state products, eleven 64-row
    products, the masked ones counted at half).  `saved`: the chunk-start states
    come from the training forward and are not counted."""
    C, d = 64, wl.d_k
    per_chunk = 20 * C * d * d + 15 * C * C * d
    if saved:
        per_chunk -= 4 * C * d * d + C * C * d
    return wl.B * wl.H * ((wl.T + C - 1) // C) * per_chunk


def prepare_bwd(wl, log):
    import torch
    import gated_delta_rule_21_amd as gdr
    from workloads import grad_inputs
    log("generating the output gradients")
    g = grad_inputs(wl)
    return dict(dO=torch.from_numpy(g["dO"]).to(torch.bfloat16).cuda(), dS_T=torch.from_numpy(g["dS_T"]).cuda(),
                ws=torch.empty(gdr.chunk_bwd_workspace_size(wl.B, wl.T, wl.H, wl.d_k, wl.d_v, torch.bfloat16,
                                                            wl.gate), dtype=torch.uint8, device="cuda"))


def bench_bwd(prep, args, log, wl, q, k, v, beta, log_a, S0):
    """The backward of the chunk forward over the same workload, with dO ~ N(0, 1)
    and dS_T ~ N(0, 1); the gradients of every input and of S0."""
    import gated_delta_rule_21_amd as gdr
    dO, dS_T, ws = prep["dO"], prep["dS_T"], prep["ws"]
    ms = time_calls(lambda i: gdr.chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T, workspace=ws), args.warmup,
                    args.steps)
    flops = bwd_algorithmic(wl)
    tf = flops / (ms * 1e-3) / 1e12
    log(f"chunk backward: {ms:.3f} ms/step, {tf:.1f} TFLOP/s useful")
    wk_ms = wk_train = None
    import torch
    if wl.gate in ("none", "scalar"):
        # the backward with a separate write key (the preconditioned rule's training
        # step); a copy of k stands for it, since the kernels' work does not depend on
        # its values
        kw = k.clone()
        wk_ms = time_calls(lambda i: gdr.chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T, workspace=ws, kw=kw),
                           args.warmup, args.steps)
        log(f"chunk backward with a write key: {wk_ms:.3f} ms/step")
        # ... and its training path (the forward keeping the chunk-start states)
        o_w = torch.empty_like(v)
        S_w = torch.empty((wl.B, wl.H, wl.d_k, wl.d_v), dtype=torch.float32, device="cuda")
        wf = time_calls(lambda i: gdr.chunk_fwd_save(q, k, v, beta, log_a, S0, kw=kw, o=o_w, S_T=S_w, workspace=ws),
                        args.warmup, args.steps)
        wb = time_calls(lambda i: gdr.chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T, kw=kw, saved=ws), args.warmup,
                        args.steps)
        wk_train = {"forward_ms_per_launch": round(wf, 4), "backward_ms_per_launch": round(wb, 4),
                    "train_step_ms": round(wf + wb, 4),
                    "train_step_tokens_per_s": round(wl.B * wl.T / ((wf + wb) * 1e-3), 1)}
        log(f"write-key training path: forward {wf:.3f} ms, backward {wb:.3f} ms")
        del kw, o_w, S_w
    # the training path: the forward keeps the transform's records and the
    # chunk-start states in the backward's workspace (gdr_chunk_fwd_save) and the
    # backward takes them from there (gdr_chunk_bwd_saved)
    o_s, S_s = torch.empty_like(v), torch.empty((wl.B, wl.H, wl.d_k, wl.d_v), dtype=torch.float32, device="cuda")
    fs_ms = time_calls(lambda i: gdr.chunk_fwd_save(q, k, v, beta, log_a, S0, o=o_s, S_T=S_s, workspace=ws),
                       args.warmup, args.steps)
    bs_ms = time_calls(lambda i: gdr.chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T, saved=ws), args.warmup, args.steps)
    del o_s, S_s
    sflops = bwd_algorithmic(wl, saved=True)
    stf = sflops / (bs_ms * 1e-3) / 1e12
    log(f"training path: forward keeping its states {fs_ms:.3f} ms, backward taking them {bs_ms:.3f} ms "
        f"({stf:.1f} TFLOP/s useful)")
    saved = {"forward_ms_per_launch": round(fs_ms, 4), "backward_ms_per_launch": round(bs_ms, 4),
             "backward_useful_flops_per_launch": sflops,
             "backward_algorithmic_bytes_per_launch": bwd_bytes(wl, False),
             "train_step_ms": round(fs_ms + bs_ms, 4),
             "train_step_tokens_per_s": round(wl.B * wl.T / ((fs_ms + bs_ms) * 1e-3), 1),
             "backward_roofline": {"bound": "mfma", "achieved": round(stf, 2), "peak": BF16_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(stf / BF16_PEAK_TFLOPS, 4),
                                   "traffic": (profiled_traffic("chunk_bwd_saved_gated_b8h16t8192d128_counters.md",
                                                                BWD_SOURCES)
                                               if wl.name == "gated_deltanet_scalar_b8h16t8192d128_bf16" else None)}}
    return {"workload": wl.name + "_backward", "value": round(wl.B * wl.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_launch": round(ms, 4), "useful_flops_per_launch": flops,
            "write_key_ms_per_launch": None if wk_ms is None else round(wk_ms, 4),
            "training_path": saved, "write_key_training_path": wk_train,
            "algorithmic_bytes_per_launch": bwd_bytes(wl, S0 is not None),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": (profiled_traffic("chunk_bwd_gated_b8h16t8192d128_counters.md", BWD_SOURCES)
                                     if wl.name == "gated_deltanet_scalar_b8h16t8192d128_bf16" else None)}}


def bench_bwd_channel(prep, bprep, args, log):
    """The backward on the per-channel workload (B2 H32 T32768 d128, S0 ~ N(0, 0.02^2)):
    the recomputing backward, then the training path (the forward keeping its records
    and chunk-start states, and the backward taking them).  Useful flops as for the
    scalar gate (the per-channel decays inside the products are not counted)."""
    import torch
    import gated_delta_rule_21_amd as gdr
    wl = prep["wl"]
    q, k, v, beta, log_a = prep["sets"][0]["args"]
    S0 = prep["sets"][0]["S0"]
    dO, dS_T, ws = bprep["dO"], bprep["dS_T"], bprep["ws"]
    steps, warmup = max(10, args.steps // 5), max(3, args.warmup // 5)
    ms = time_calls(lambda i: gdr.chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T, workspace=ws), warmup, steps)
    o_s, S_s = torch.empty_like(v), torch.empty((wl.B, wl.H, wl.d_k, wl.d_v), dtype=torch.float32, device="cuda")
    fs = time_calls(lambda i: gdr.chunk_fwd_save(q, k, v, beta, log_a, S0, o=o_s, S_T=S_s, workspace=ws), warmup,
                    steps)
    bs = time_calls(lambda i: gdr.chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T, saved=ws), warmup, steps)
    del o_s, S_s
    flops, sflops = bwd_algorithmic(wl), bwd_algorithmic(wl, saved=True)
    tf, stf = flops / (ms * 1e-3) / 1e12, sflops / (bs * 1e-3) / 1e12
    log(f"per-channel backward: {ms:.3f} ms/step ({tf:.1f} TFLOP/s useful); training path: forward {fs:.3f} ms, "
        f"backward {bs:.3f} ms")
    roof = lambda t: {"bound": "mfma", "achieved": round(t, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(t / BF16_PEAK_TFLOPS, 4), "traffic": None}
    return {"workload": wl.name + "_backward", "value": round(wl.B * wl.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_launch": round(ms, 4), "warmup": warmup, "steps": steps, "useful_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": bwd_bytes(wl, True), "roofline": roof(tf),
            "training_path": {"forward_ms_per_launch": round(fs, 4), "backward_ms_per_launch": round(bs, 4),
                              "train_step_ms": round(fs + bs, 4),
                              "train_step_tokens_per_s": round(wl.B * wl.T / ((fs + bs) * 1e-3), 1),
                              "backward_useful_flops_per_launch": sflops, "backward_roofline": roof(stf)}}


def bench_wkey(args, log, wl, q, k, v, beta, kw, scan_us):
    """Phase 2 of the preconditioned delta rule: the chunk forward with the write
    keys the scan produced (no gate), over the chunk workload's q, k, v, beta."""
    import torch
    import gated_delta_rule_21_amd as gdr
    o = torch.empty_like(v)
    S_T = torch.empty((wl.B, wl.H, wl.d_k, wl.d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdr.chunk_workspace_size(wl.B, wl.T, wl.H, wl.d_k, wl.d_v, torch.bfloat16, "none"),
                     dtype=torch.uint8, device="cuda")
    ms = time_calls(lambda i: gdr.chunk_fwd(q, k, v, beta, None, None, o=o, S_T=S_T, workspace=ws, kw=kw),
                    args.warmup, args.steps)
    nbytes, _ = chunk_algorithmic(wl.replace(gate="none"), with_S0=False)
    nbytes += wl.B * wl.T * wl.H * wl.d_k * 2          # the write keys
    gbs = nbytes / (ms * 1e-3) / 1e9
    total_ms = ms + scan_us * 1e-3
    log(f"write-key forward: {ms * 1e3:.1f} us, {gbs:.0f} GB/s; scan + forward {total_ms * 1e3:.1f} us")
    return {"workload": "osdn_two_phase_b%dh%dt%dd%d_bf16" % (wl.B, wl.H, wl.T, wl.d_k),
            "forward_us": round(ms * 1e3, 2), "scan_us": scan_us,
            "tokens_per_s": round(wl.B * wl.T / (total_ms * 1e-3), 1),
            "forward_roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(gbs / HBM_PEAK_GBS, 4),
                                 "traffic": profiled_traffic("chunk_fwd_wkey_b8h16t8192d128_counters.md", CHUNK_SOURCES)
                                 if (wl.B, wl.T, wl.H, wl.d_k) == (8, 8192, 16, 128) else None},
            "forward_bytes_per_launch": nbytes}


def handoff_lengths(n_seq: int = 32, lo: int = 128, hi: int = 8192, seed: int = 6):
    """Prompt lengths of the serving mix: log-uniform on [lo, hi], seeded."""
    import numpy as np
    rs = np.random.RandomState(seed)
    return [int(round(x)) for x in np.exp(rs.uniform(np.log(lo), np.log(hi), size=n_seq))]


def prepare_handoff(log, n_sets: int = 16):
    import numpy as np
    import torch
    import gated_delta_rule_21_amd as gdr
    from workloads import Workload, chunk_inputs
    lens = handoff_lengths()
    N, H, dk, dv, total = len(lens), 16, 128, 128, int(sum(lens))
    log(f"generating the handoff mix ({N} prompts, {total} tokens)")
    inp = chunk_inputs(Workload("handoff_prefill", B=1, T=total, H=H, d_k=dk, d_v=dv, io="bf16", gate="scalar",
                                s0_std=0.0, seed=6))
    tok = chunk_inputs(Workload("handoff_tokens", B=N, T=n_sets, H=H, d_k=dk, d_v=dv, io="bf16", gate="scalar",
                                s0_std=0.0, seed=7))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()
    return dict(lens=lens, N=N, H=H, dk=dk, dv=dv, total=total, n_sets=n_sets,
                args=[dev(inp[n]) for n in ("q", "k", "v", "beta", "log_a")],
                tok=[[dev(tok[n][:, j]) for j in range(n_sets)] for n in ("q", "k", "v", "beta", "log_a")],
                cu=torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda"),
                o=torch.empty((1, total, H, dv), dtype=torch.bfloat16, device="cuda"),
                S=torch.empty((N, H, dk, dv), dtype=torch.float32, device="cuda"),
                od=torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda"),
                ws=torch.empty(gdr.chunk_varlen_workspace_size(total, N, H, dk, dv, torch.bfloat16, "scalar"),
                               dtype=torch.uint8, device="cuda"))


def bench_handoff(prep, log):
    """Packed prefill of a batch of prompts of mixed lengths, then decode steps on the
    states it hands over (the serving steps on either side of the chunk forward)."""
    import torch
    import gated_delta_rule_21_amd as gdr
    P = prep
    N, H, dk, dv, total, n_sets, lens = P["N"], P["H"], P["dk"], P["dv"], P["total"], P["n_sets"], P["lens"]
    q, k, v, beta, log_a = P["args"]
    tq, tk, tv, tb, tl = P["tok"]
    cu, o, S, od, ws = P["cu"], P["o"], P["S"], P["od"], P["ws"]
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
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--chunk-config", type=int, default=3, choices=(1, 2, 3, 4),
                    help="headline chunk-forward workload (3 = the gated workload of the headline metric)")
    ap.add_argument("--no-configs", action="store_true", help="skip the other chunk-forward workloads")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-handoff", action="store_true",
                    help="skip the packed-prefill -> decode handoff leg")
    ap.add_argument("--no-precond", action="store_true", help="skip the preconditioner-scan leg")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-T", type=int, default=8192)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB streaming copy first (for scaling HBM byte counters)")
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--cpu-b", default="", help=argparse.SUPPRESS)
    ap.add_argument("--cpu-h", default="", help=argparse.SUPPRESS)
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    if args.cpu_baseline_child:
        cpu_baseline_child(args.cpu_T, [int(x) for x in args.cpu_b.split(",")],
                           [int(x) for x in args.cpu_h.split(",")])
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the library has no multi-GPU path (a sharding design is described with the kernels).", file=sys.stderr)
        sys.exit(2)

    log = (lambda *a: None) if args.quiet else (lambda *a: print("[bench]", *a, file=sys.stderr, flush=True))
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import gated_delta_rule_21_amd as gdr
    gdr.load()

    # ---- every input to the GPU first ----
    head = prepare_chunk(args.chunk_config, 1, log)
    wl = head["wl"]
    others = {} if args.no_configs else {c: prepare_chunk(c, 1 if c == 4 else 3, log)
                                         for c in (1, 2, 3, 4) if c != args.chunk_config}
    dec_prep = None if args.no_decode else prepare_decode(log)
    hand_prep = None if args.no_handoff else prepare_handoff(log)
    gated_bf16 = wl.io == "bf16" and wl.gate != "channel"
    pre_prep = None if args.no_precond or wl.io != "bf16" else prepare_precond(wl, log)
    bwd_prep = None if args.no_bwd or wl.io != "bf16" else prepare_bwd(wl, log)
    chan_bwd_prep = None if args.no_bwd or 4 not in others else prepare_bwd(others[4]["wl"], log)
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(log)

    # ---- legs back to back; the headline forward last ----
    configs = {str(c): bench_chunk(p, args.warmup, args.steps, log, f"config {c}") for c, p in sorted(others.items())}
    bwd_chan = None if chan_bwd_prep is None else bench_bwd_channel(others[4], chan_bwd_prep, args, log)
    if chan_bwd_prep is not None:
        chan_bwd_prep.clear()
    for p in others.values():
        p.clear()
    decode = None if dec_prep is None else bench_decode(dec_prep, args, log)
    handoff = None if hand_prep is None else bench_handoff(hand_prep, log)
    q, k, v, beta, log_a = head["sets"][0]["args"]
    S0 = head["sets"][0]["S0"]
    precond = osdn = None
    if pre_prep is not None:
        kw, precond = bench_precond(pre_prep, args, log, wl, k, beta)
        if gated_bf16:
            osdn = bench_wkey(args, log, wl, q, k, v, beta, kw, precond["us_per_launch"])
        del kw
    bwd = None if bwd_prep is None else bench_bwd(bwd_prep, args, log, wl, q, k, v, beta, log_a, S0)
    rec = bench_chunk(head, args.warmup, args.steps, log, "headline")
    ms = rec["ms_per_call"]
    if bwd is not None:
        # forward then the recomputing backward; the training path's own figure is in
        # bwd["training_path"]
        bwd["train_step_ms"] = round(ms + bwd["ms_per_launch"], 4)
        bwd["train_step_tokens_per_s"] = round(wl.B * wl.T / ((ms + bwd["ms_per_launch"]) * 1e-3), 1)
    del q, k, v, beta, log_a, S0, head
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_T, log)

    line = {
        "metric": "tokens/s + % MFMA peak, gated delta-rule chunk fwd T=8192 d=128; decode GB/s",
        "value": rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.io,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": wl.H, "d_k": wl.d_k, "d_v": wl.d_v,
                   "chunk": wl.chunk, "gate": wl.gate, "io": wl.io, "state": "fp32",
                   "S0": "N(0, %g^2)" % wl.s0_std if wl.s0_std > 0 else "zero",
                   "global_batch": wl.B, "seq_len": wl.T, "parallelism": "none (1 GPU)"},
        "tflops_useful": rec["tflops_useful"],
        "mfma_frac_useful": rec["mfma_frac_useful"],
        "roofline": rec["roofline"],
        "algorithmic_bytes_per_launch": rec["algorithmic_bytes_per_launch"],
        "useful_flops_per_launch": rec["useful_flops_per_launch"],
        "configs": configs,
        "decode": decode,
        "handoff": handoff,
        "precond_scan": precond,
        "osdn": osdn,
        "backward": bwd,
        "backward_channel": bwd_chan,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
