"""The parallel whole-tensor comparison against the oracle (host processes) agrees
with the single-process oracle: zero error for the oracle's own result, and the
relative L2 of a known perturbation."""

import numpy as np

from oracle import backward, forward, precond_scan, recurrent_step, rel_l2
from oracle.preconditioner import precond_scan_backward
from tests.parallel_oracle import whole_backward, whole_chunk, whole_decode, whole_scan, whole_scan_backward
from workloads import DECODE_CONFIG, Workload, chunk_inputs, decode_inputs, grad_inputs, precond_inputs


def test_whole_chunk_matches_single_process():
    wl = Workload("par", B=2, T=70, H=3, d_k=16, d_v=8, io="bf16", gate="channel", s0_std=0.02, seed=3)
    inp = chunk_inputs(wl)
    o, S = forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_a"], inp["S0"])
    r = whole_chunk(wl, o, S, group=2)
    assert r["o"] < 1e-13 and r["S"] < 1e-13 and r["slices"] == 6
    o2 = o.copy()
    o2[1, :, 2] *= 1.01                         # one slice off by 1 %
    r = whole_chunk(wl, o2, S * 1.001, group=2)
    assert abs(r["o"] - rel_l2(o2, o)) < 1e-12 and abs(r["S"] - 1e-3) < 1e-9
    assert r["worst_o"][:2] == (1, 2) and abs(r["worst_o"][2] - 0.01) < 1e-9


def test_whole_decode_matches_single_process():
    wl = DECODE_CONFIG.replace(N=5, H=2, d_k=16, d_v=8, steps=7)
    inp = decode_inputs(wl)
    S = inp["S0"].astype(np.float64)
    o_all = np.empty((7, 5, 2, 8))
    for s in range(7):
        o_all[s], S = recurrent_step(S, inp["q"][s], inp["k"][s], inp["v"][s], inp["beta"][s], inp["log_a"][s])
    r = whole_decode(wl, 7, o_all, S, group=2)
    assert r["o"] < 1e-13 and r["S"] < 1e-13
    r = whole_decode(wl, 7, o_all * 1.02, S, group=3)
    assert abs(r["o"] - 0.02) < 1e-9


def test_whole_chunk_with_write_key():
    wl = Workload("par_kw", B=2, T=40, H=2, d_k=16, d_v=8, io="bf16", gate="scalar", s0_std=0.1, seed=5)
    inp = chunk_inputs(wl)
    kw = inp["k"] * np.random.default_rng(1).uniform(0.5, 1.5, inp["k"].shape)
    o, S = forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_a"], inp["S0"], kw=kw)
    r = whole_chunk(wl, o, S, group=1, kw=kw)
    assert r["o"] < 1e-13 and r["S"] < 1e-13
    r = whole_chunk(wl, o, S, group=1)          # the plain forward differs from the write-key one
    assert r["o"] > 1e-3


def _grads(wl, kw=None):
    x = chunk_inputs(wl)
    x.update(grad_inputs(wl))
    return backward(x["q"], x["k"], x["v"], x["beta"], x["log_a"], x["S0"], x["dO"], x["dS_T"], kw=kw)


def test_whole_backward_matches_single_process():
    wl = Workload("par_bwd", B=2, T=70, H=3, d_k=16, d_v=8, io="bf16", gate="channel", s0_std=0.1, seed=7)
    g = _grads(wl)
    r = whole_backward(wl, g)
    assert r["slices"] == 6 and max(r["rel"].values()) < 1e-13, r["rel"]
    g2 = {n: (None if a is None else a.copy()) for n, a in g.items()}
    g2["dk"][0, :, 1] *= 1.03                   # one slice of dk off by 3 %
    g2["dS0"] *= 1.002
    r = whole_backward(wl, g2)
    assert abs(r["rel"]["dk"] - rel_l2(g2["dk"], g["dk"])) < 1e-12
    assert r["worst"]["dk"][:2] == (0, 1) and abs(r["worst"]["dk"][2] - 0.03) < 1e-9
    assert abs(r["rel"]["dS0"] - 2e-3) < 1e-9 and r["rel"]["dq"] < 1e-13


def test_whole_backward_with_write_key():
    wl = Workload("par_bwd_kw", B=1, T=50, H=2, d_k=16, d_v=8, io="bf16", gate="scalar", s0_std=0.1, seed=9)
    x = chunk_inputs(wl)
    kw = x["k"] * np.random.default_rng(2).uniform(0.5, 1.5, x["k"].shape)
    g = _grads(wl, kw=kw)
    assert "dkw" in g
    r = whole_backward(wl, g, kw=kw)
    assert max(r["rel"].values()) < 1e-13, r["rel"]


def test_whole_scan_and_its_backward():
    wl = Workload("par_scan", B=2, T=90, H=2, d_k=16, d_v=16, io="bf16", gate="scalar", s0_std=0.0, seed=11)
    x = precond_inputs(wl)
    kw, d_T = precond_scan(x["k"], x["beta"], 0.5, x["r"], x["d0"])
    r = whole_scan(wl, 0.5, kw, d_T)
    assert r["slices"] == 4 and max(r["rel"].values()) < 1e-13, r["rel"]
    r = whole_scan(wl, 0.5, kw * 1.01, d_T)
    assert abs(r["rel"]["kw"] - 0.01) < 1e-9
    rng = np.random.default_rng(3)
    dkw, dd_T = rng.standard_normal(kw.shape), rng.standard_normal(d_T.shape)
    g = precond_scan_backward(x["k"], x["beta"], 0.5, x["r"], x["d0"], dkw, dd_T)
    r = whole_scan_backward(wl, 0.5, dkw, dd_T, g)
    assert max(r["rel"].values()) < 1e-13, r["rel"]
    g["dr"] = g["dr"] * 1.05
    r = whole_scan_backward(wl, 0.5, dkw, dd_T, g)
    assert abs(r["rel"]["dr"] - 0.05) < 1e-9


def test_whole_packed_matches_single_process():
    from tests.parallel_oracle import whole_packed
    lens = [0, 5, 70, 1, 130]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    wl = Workload("par_packed", B=1, T=int(cu[-1]), H=2, d_k=16, d_v=8, io="bf16", gate="scalar", s0_std=0.0, seed=13)
    inp = chunk_inputs(wl)
    S0 = np.random.default_rng(4).standard_normal((len(lens), 2, 16, 8)) * 0.1
    o = np.zeros(inp["v"].shape)
    S = np.zeros(S0.shape)
    for i in range(len(lens)):
        lo, hi = int(cu[i]), int(cu[i + 1])
        sl = lambda a: None if a is None else a[:, lo:hi]
        oi, Si = forward(*(sl(inp[n]) for n in ("q", "k", "v", "beta", "log_a")), S0[i:i + 1])
        o[:, lo:hi], S[i] = oi, Si[0]
    r = whole_packed(inp, cu, S0, o, S)
    assert r["o"] < 1e-13 and r["S"] < 1e-13 and r["worst_S"] < 1e-13
    assert np.array_equal(r["S_ref"], S)
    S2 = S.copy()
    S2[3] *= 1.05                               # the one-token sequence's state off by 5 %
    r = whole_packed(inp, cu, S0, o, S2)
    assert abs(r["worst_S"] - 0.05) < 1e-9 and abs(r["S"] - rel_l2(S2, S)) < 1e-12
