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

from oracle import backward, forward, precond_scan, recurrent_step
from oracle.preconditioner import precond_scan_backward
from workloads import decode_slice, grad_slice, precond_slice, slice_inputs

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
    wl, b, hs, form = args
    sl = [slice_inputs(wl, b, h) for h in hs]
    st = lambda n: np.stack([s[n] for s in sl], axis=1)[None]          # [1, T, nh, .]
    la = None if wl.gate == "none" else st("log_a")
    kw = _GPU.get("kw_in")
    kw = None if kw is None else kw[b:b + 1, :, hs[0]:hs[-1] + 1]
    o_ref, S_ref = forward(st("q"), st("k"), st("v"), st("beta"), la, np.stack([s["S0"] for s in sl])[None], kw=kw,
                           form=form)
    out = []
    for i, h in enumerate(hs):
        do = _GPU["o"][b, :, h].astype(np.float64) - o_ref[0, :, i]
        dS = _GPU["S"][b, h].astype(np.float64) - S_ref[0, i]
        out.append((b, h, float((do ** 2).sum()), float((o_ref[0, :, i] ** 2).sum()),
                    float((dS ** 2).sum()), float((S_ref[0, i] ** 2).sum())))
    return out


def whole_chunk(wl, o_gpu: np.ndarray, S_gpu: np.ndarray, group: int = 4, kw: np.ndarray = None,
                form: str = "page"):
    """Whole-tensor rel-L2 of o and S_T against the oracle, and the worst (b, h) slice
    of each.  o_gpu [B, T, H, d_v], S_gpu [B, H, d_k, d_v] (host arrays); kw the
    write key [B, T, H, d_k] the GPU was given (host), or None; form the gate's
    placement the GPU ran ("page" or "literal")."""
    _GPU["o"], _GPU["S"] = o_gpu, S_gpu
    if kw is not None:
        _GPU["kw_in"] = kw
    items = [(wl, b, list(range(h0, min(h0 + group, wl.H))), form) for b in range(wl.B)
             for h0 in range(0, wl.H, group)]
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


# ---- gradients and the preconditioner scan: one (b, h) slice per task ------------------

def _sums(got: np.ndarray, ref: np.ndarray):
    """(sum of squared differences, sum of squared references) in fp64."""
    r = np.asarray(ref, dtype=np.float64)
    d = np.asarray(got, dtype=np.float64) - r
    return float((d * d).sum()), float((r * r).sum())


def _per_slice(b: int, h: int, got: dict, ref: dict, per_head: tuple):
    """Per-name sums of one (b, h) slice; names in per_head are [B, H, ...] tensors,
    the rest [B, T, H, ...]."""
    out = {}
    for n, g in got.items():
        if n in per_head:
            out[n] = _sums(g[b, h], ref[n][0, 0])
        else:
            out[n] = _sums(g[b, :, h], ref[n][0, :, 0])
    return [(b, h, out)]


def _bwd_slice(args):
    wl, b, h = args
    s = slice_inputs(wl, b, h)
    s.update(grad_slice(wl, b, h))
    e = lambda a: None if a is None else a[None, :, None]
    kw = _GPU.get("kw_in")
    ref = backward(e(s["q"]), e(s["k"]), e(s["v"]), e(s["beta"]), e(s["log_a"]), s["S0"][None, None], e(s["dO"]),
                   s["dS_T"][None, None], kw=None if kw is None else kw[b:b + 1, :, h:h + 1])
    return _per_slice(b, h, _GPU["out"], ref, ("dS0",))


def _scan_slice(args):
    wl, b, h, eta = args
    s = precond_slice(wl, b, h)
    kw, d_T = precond_scan(s["k"][None, :, None], s["beta"][None, :, None], eta, s["r"][None, :, None],
                           s["d0"][None, None])
    return _per_slice(b, h, _GPU["out"], {"kw": kw, "d_T": d_T}, ("d_T",))


def _scan_bwd_slice(args):
    wl, b, h, eta = args
    s = precond_slice(wl, b, h)
    ref = precond_scan_backward(s["k"][None, :, None], s["beta"][None, :, None], eta, s["r"][None, :, None],
                                s["d0"][None, None], _GPU["dkw_in"][b:b + 1, :, h:h + 1],
                                _GPU["ddT_in"][b:b + 1, h:h + 1])
    return _per_slice(b, h, _GPU["out"], ref, ("dd0",))


def _whole(worker, items, out: dict, extra: dict):
    """Run worker over items on host processes; whole-tensor rel-L2 per output name and
    the worst (b, h, rel-L2) slice of each."""
    out = {n: a for n, a in out.items() if a is not None}
    _GPU["out"] = out
    _GPU.update(extra)
    procs = host_procs()
    t0 = time.perf_counter()
    try:
        with mp.get_context("fork").Pool(procs, initializer=_init) as pool:
            rows = [r for part in pool.imap_unordered(worker, items) for r in part]
    finally:
        _GPU.clear()
    secs = time.perf_counter() - t0
    rel, worst = {}, {}
    for n in out:
        num = sum(r[2][n][0] for r in rows)
        den = sum(r[2][n][1] for r in rows)
        rel[n] = float(np.sqrt(num / den)) if den > 0 else float(np.sqrt(num))
        w = max(rows, key=lambda r: r[2][n][0] / max(r[2][n][1], 1e-300))
        worst[n] = (w[0], w[1], float(np.sqrt(w[2][n][0] / max(w[2][n][1], 1e-300))))
    return dict(rel=rel, worst=worst, slices=len(rows), procs=procs, seconds=secs)


def whole_backward(wl, grads: dict, kw: np.ndarray = None):
    """Every (b, h) slice of the chunk forward's gradients against the backward oracle.
    grads: name -> host array as the GPU returned it (dq, dk, dv, dbeta, dlog_a
    [B, T, H, ...], dS0 [B, H, d_k, d_v], dkw with a write key); kw the write key
    the GPU was given (host), or None."""
    items = [(wl, b, h) for b in range(wl.B) for h in range(wl.H)]
    return _whole(_bwd_slice, items, grads, {} if kw is None else {"kw_in": kw})


def whole_scan(wl, eta: float, kw_gpu: np.ndarray, dT_gpu: np.ndarray):
    """Every (b, h) slice of the preconditioner scan (write keys and final
    preconditioner) against the scan oracle."""
    items = [(wl, b, h, eta) for b in range(wl.B) for h in range(wl.H)]
    return _whole(_scan_slice, items, {"kw": kw_gpu, "d_T": dT_gpu}, {})


def whole_scan_backward(wl, eta: float, dkw: np.ndarray, dd_T: np.ndarray, grads: dict):
    """Every (b, h) slice of the scan's gradients (dk, dbeta, dr [B, T, H, ...], dd0
    [B, H, d_k]) against the scan's reverse-mode oracle, for the given incoming
    gradients dkw [B, T, H, d_k] and dd_T [B, H, d_k]."""
    items = [(wl, b, h, eta) for b in range(wl.B) for h in range(wl.H)]
    return _whole(_scan_bwd_slice, items, grads, {"dkw_in": dkw, "ddT_in": dd_T})


def _packed_seq(i):
    inp, cu = _GPU["inp"], _GPU["cu"]
    lo, hi = int(cu[i]), int(cu[i + 1])
    sl = lambda a: None if a is None else np.ascontiguousarray(a[:, lo:hi])
    o_ref, S_ref = forward(*(sl(inp[n]) for n in ("q", "k", "v", "beta", "log_a")), _GPU["S0"][i:i + 1])
    o_sums = _sums(_GPU["out"]["o"][:, lo:hi], o_ref)
    S_sums = _sums(_GPU["out"]["S"][i], S_ref[0])
    return i, o_sums, S_sums, S_ref[0]


def whole_packed(inp: dict, cu: np.ndarray, S0: np.ndarray, o_gpu: np.ndarray, S_gpu: np.ndarray):
    """Packed sequences ([1, T, H, .] inputs, offsets cu) against the oracle run on each
    sequence alone, sequences dealt to host processes.  Returns the rel-L2 of the whole
    o and of the whole S_T, the worst sequence's S_T rel-L2, and the oracle's final
    states [n_seq, H, d_k, d_v] (fp64)."""
    n_seq = len(cu) - 1
    _GPU.update(inp=inp, cu=cu, S0=S0, out={"o": o_gpu, "S": S_gpu})
    procs = host_procs()
    t0 = time.perf_counter()
    try:
        with mp.get_context("fork").Pool(procs, initializer=_init) as pool:
            rows = sorted(pool.imap_unordered(_packed_seq, range(n_seq)), key=lambda r: r[0])
    finally:
        _GPU.clear()
    num_o, den_o = sum(r[1][0] for r in rows), sum(r[1][1] for r in rows)
    num_S, den_S = sum(r[2][0] for r in rows), sum(r[2][1] for r in rows)
    worst = max(float(np.sqrt(r[2][0] / max(r[2][1], 1e-300))) for r in rows)
    return dict(o=float(np.sqrt(num_o / den_o)), S=float(np.sqrt(num_S / den_S)), worst_S=worst,
                S_ref=np.stack([r[3] for r in rows]), procs=procs, seconds=time.perf_counter() - t0)


def assert_whole(label: str, r: dict, tol: float) -> str:
    """Print and report the whole-tensor numbers of r (from whole_backward, whole_scan
    or whole_scan_backward); every name's whole-tensor rel-L2 and its worst (b, h)
    slice must be within tol (NaN fails)."""
    from tests.report import report
    parts = "  ".join(f"{n} {v:.3e}" for n, v in r["rel"].items())
    wn, (wb, wh, wv) = max(r["worst"].items(), key=lambda kv: kv[1][2])
    line = (f"{label}: whole-tensor rel_l2 {parts}; worst slice {wn} (b={wb}, h={wh}) {wv:.3e}; "
            f"{r['slices']} slices on {r['procs']} processes in {r['seconds']:.1f} s")
    print("  " + line, flush=True)
    report(line)
    bad = {n: v for n, v in r["rel"].items() if not v <= tol}
    bad.update({f"{n}[b={w[0]},h={w[1]}]": w[2] for n, w in r["worst"].items() if not w[2] <= tol})
    assert not bad, f"{label}: above {tol}: {bad}"
    return line
