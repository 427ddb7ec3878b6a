"""The fp64 oracle over every (b, h) slice of a full-size workload, split over host
processes, compared with GPU results element by element.

The GPU results are set as module globals before the worker pool is forked, so
each worker reads its slices from the parent's memory; each worker regenerates
its slices' inputs from the seeded generator, runs the oracle on them, and returns
sums of squared differences and of squared references per slice.  The whole-tensor
relative L2 error is the square root of the ratio of the summed sums.  Workers do
not touch the GPU.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import time

import numpy as np

from oracle import forward, recurrent_step
from workloads import decode_slice, slice_inputs

_GPU = {}


def host_procs() -> int:
    """Worker processes: the host cores this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _chunk_group(args):
    wl, b, hs = args
    sl = [slice_inputs(wl, b, h) for h in hs]
    st = lambda n: np.stack([s[n] for s in sl], axis=1)[None]          # [1, T, nh, .]
    la = None if wl.gate == "none" else st("log_a")
    o_ref, S_ref = forward(st("q"), st("k"), st("v"), st("beta"), la, np.stack([s["S0"] for s in sl])[None])
    out = []
    for i, h in enumerate(hs):
        do = _GPU["o"][b, :, h].astype(np.float64) - o_ref[0, :, i]
        dS = _GPU["S"][b, h].astype(np.float64) - S_ref[0, i]
        out.append((b, h, float((do ** 2).sum()), float((o_ref[0, :, i] ** 2).sum()),
                    float((dS ** 2).sum()), float((S_ref[0, i] ** 2).sum())))
    return out


def whole_chunk(wl, o_gpu: np.ndarray, S_gpu: np.ndarray, group: int = 4):
    """Whole-tensor rel-L2 of o and S_T against the oracle, and the worst (b, h) slice
    of each.  o_gpu [B, T, H, d_v], S_gpu [B, H, d_k, d_v] (host arrays)."""
    _GPU["o"], _GPU["S"] = o_gpu, S_gpu
    items = [(wl, b, list(range(h0, min(h0 + group, wl.H)))) for b in range(wl.B) for h0 in range(0, wl.H, group)]
    procs = host_procs()
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(procs, initializer=_init) as pool:
        rows = [r for part in pool.imap_unordered(_chunk_group, items) for r in part]
    secs = time.perf_counter() - t0
    _GPU.clear()
    num_o, den_o, num_S, den_S = (sum(r[i] for r in rows) for i in (2, 3, 4, 5))
    worst_o = max(rows, key=lambda r: r[2] / max(r[3], 1e-300))
    worst_S = max(rows, key=lambda r: r[4] / max(r[5], 1e-300))
    return dict(o=float(np.sqrt(num_o / den_o)), S=float(np.sqrt(num_S / den_S)),
                worst_o=(worst_o[0], worst_o[1], float(np.sqrt(worst_o[2] / worst_o[3]))),
                worst_S=(worst_S[0], worst_S[1], float(np.sqrt(worst_S[4] / worst_S[5]))),
                slices=len(rows), procs=procs, seconds=secs)


def _decode_group(args):
    wl, steps, n0, n1 = args
    sl = [[decode_slice(wl, n, h, steps) for h in range(wl.H)] for n in range(n0, n1)]
    st = lambda name: np.stack([np.stack([s[name] for s in row], axis=1) for row in sl], axis=1)  # [steps, n, H, .]
    q, k, v, beta = st("q"), st("k"), st("v"), st("beta")
    la = None if wl.gate == "none" else st("log_a")
    S = np.stack([np.stack([s["S0"] for s in row]) for row in sl]).astype(np.float64)
    num_o = den_o = 0.0
    for s in range(steps):
        o, S = recurrent_step(S, q[s], k[s], v[s], beta[s], None if la is None else la[s])
        d = _GPU["o"][s, n0:n1].astype(np.float64) - o
        num_o += float((d ** 2).sum())
        den_o += float((o ** 2).sum())
    dS = _GPU["S"][n0:n1].astype(np.float64) - S
    return num_o, den_o, float((dS ** 2).sum()), float((S ** 2).sum())


def whole_decode(wl, steps: int, o_gpu: np.ndarray, S_gpu: np.ndarray, group: int = 16):
    """Rel-L2 of o over all steps and of the state after the last step, every state of
    the decode workload.  o_gpu [steps, N, H, d_v], S_gpu [N, H, d_k, d_v]."""
    _GPU["o"], _GPU["S"] = o_gpu, S_gpu
    items = [(wl, steps, n0, min(n0 + group, wl.N)) for n0 in range(0, wl.N, group)]
    procs = host_procs()
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(procs, initializer=_init) as pool:
        parts = list(pool.imap_unordered(_decode_group, items))
    secs = time.perf_counter() - t0
    _GPU.clear()
    num_o, den_o, num_S, den_S = (sum(p[i] for p in parts) for i in range(4))
    return dict(o=float(np.sqrt(num_o / den_o)), S=float(np.sqrt(num_S / den_S)), procs=procs, seconds=secs)
