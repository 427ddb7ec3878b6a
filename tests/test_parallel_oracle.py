"""The parallel whole-tensor comparison against the oracle (host processes) agrees
with the single-process oracle: zero error for the oracle's own result, and the
relative L2 of a known perturbation."""

import numpy as np

from oracle import forward, recurrent_step, rel_l2
from tests.parallel_oracle import whole_chunk, whole_decode
from workloads import DECODE_CONFIG, Workload, chunk_inputs, decode_inputs


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
