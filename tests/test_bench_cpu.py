"""The benchmark's command-line contract, on the CPU: it measures one GPU only and
refuses more; without a GPU it stops with a message instead of falling back; and its
algorithmic byte and flop counts are the closed forms its documentation states."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_no_gpu_no_fallback():
    import torch
    if torch.cuda.is_available():
        return
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 1 and "needs a GPU" in r.stderr and r.stdout == ""


def test_algorithmic_counts():
    from workloads import CONFIGS
    wl = CONFIGS[3]                                 # B8 H16 T8192 d128, bf16, scalar gate
    ntok = wl.B * wl.T * wl.H
    nbytes, flops = bench.chunk_algorithmic(wl, with_S0=False)
    # q, k, v, beta, log_a read; o written; S_T written (fp32)
    assert nbytes == ntok * (128 + 128 + 128 + 1 + 1) * 2 + ntok * 128 * 2 + wl.B * wl.H * 128 * 128 * 4
    C, d = 64, 128
    per_chunk = C * (C - 1) * d + C ** 3 / 3 + C * (C + 1) * 4 * d + 6 * C * d * d
    assert flops == per_chunk * (wl.T // C) * wl.B * wl.H
    state = wl.B * wl.H * d * d * 4
    assert bench.bwd_bytes(wl, with_S0=False) == (ntok * (4 * d + 2) * 2 + state) + (ntok * (3 * d + 2) * 2 + state)
    assert bench.bwd_algorithmic(wl) == wl.B * wl.H * (wl.T // C) * (20 * C * d * d + 15 * C * C * d)
