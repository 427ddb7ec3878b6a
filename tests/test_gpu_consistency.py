"""Self-consistency of the GPU path, through the C ABI.

* The chunk forward over T tokens equals T decode steps from the same state: the
  chunkwise form of "Moonshot AI's New Attention Architecture", §3 is the same
  recurrence as the token-by-token update of §2 (the decode step of §1).
* A NaN in one head's inputs stays in that head: (sequence, head) pairs are
  independent recurrences, and nothing else may read them.
"""

import numpy as np
import pytest

from tests.gpu_util import TOL, check, dev, host, need_gpu, say
from workloads import Workload, chunk_inputs

pytestmark = pytest.mark.gpu


def _wl(name, B, T, H, dk, dv, io="bf16", gate="scalar", seed=11):
    return Workload(name, B=B, T=T, H=H, d_k=dk, d_v=dv, io=io, gate=gate, s0_std=0.05, seed=seed)


@pytest.mark.parametrize("io,dk", [("bf16", 128), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("form", ["page", "literal"])
def test_chunk_forward_equals_token_steps(io, dk, gate, form):
    """chunk_fwd over 150 tokens against 150 gdr_recurrent_step calls (state carried
    in place): o of every token and the final state, relative L2 within the I/O
    dtype's tolerance."""
    if io == "f32" and dk == 128 and gate == "channel":
        pytest.skip("the per-channel fp32 chunk forward takes d_k = 64")
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    wl = _wl("steps", 2, 150, 3, dk, 128, io=io, gate=gate, seed=101 + dk)
    inp = chunk_inputs(wl)
    say(f"case chunk vs steps io={io} d_k={dk} gate={gate} form={form}")
    args = {n: dev(inp[n], io) for n in ("q", "k", "v", "beta", "log_a")}
    S0 = torch.from_numpy(inp["S0"]).cuda()
    o_c, S_c = gdr.chunk_fwd(*(args[n] for n in ("q", "k", "v", "beta", "log_a")), S0, form=form)
    S = S0.clone()
    o_s = torch.empty_like(o_c)
    tok = lambda x, t: None if x is None else x[:, t].contiguous()
    for t in range(wl.T):
        o_t, S = gdr.recurrent_step(*(tok(args[n], t) for n in ("q", "k", "v", "beta", "log_a")), S, form=form)
        o_s[:, t] = o_t
    torch.cuda.synchronize()
    check("o: chunk vs steps", host(o_c), host(o_s), TOL[io])
    check("S_T: chunk vs steps", host(S_c), host(S), TOL[io])


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("where", ["k", "v", "log_a", "S0"])
def test_nan_stays_in_its_head(gate, where):
    """A NaN in one (sequence, head)'s k, v, log a or initial state leaves every other
    head's o and S_T bit for bit as without it, and that head's chunks before the NaN."""
    if where == "log_a" and gate == "none":
        pytest.skip("no gate input")
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    wl = _wl("nan", 2, 200, 3, 128, 128, gate=gate, seed=107)
    inp = chunk_inputs(wl)
    say(f"case NaN in {where}, gate={gate}")

    def run(x):
        o, S = gdr.chunk_fwd(*(dev(x[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")),
                             torch.from_numpy(x["S0"]).cuda())
        torch.cuda.synchronize()
        return host(o), host(S)

    o0, S0 = run(inp)
    bad = {n: (None if a is None else a.copy()) for n, a in inp.items()}
    b, h, t = 1, 2, 140
    if where == "S0":
        bad["S0"][b, h, 7, 9] = np.nan
        t = 0
    elif bad[where].ndim == 3:
        bad[where][b, t, h] = np.nan
    else:
        bad[where][b, t, h, 5] = np.nan
    o1, S1 = run(bad)
    keep = np.ones((wl.B, wl.H), bool)
    keep[b, h] = False
    for bb in range(wl.B):
        for hh in range(wl.H):
            if keep[bb, hh]:
                assert np.array_equal(o0[bb, :, hh], o1[bb, :, hh]), f"o of head ({bb}, {hh}) changed"
                assert np.array_equal(S0[bb, hh], S1[bb, hh]), f"S_T of head ({bb}, {hh}) changed"
    first = (t // 64) * 64                      # the chunks before the NaN's chunk are untouched
    assert np.array_equal(o0[b, :first, h], o1[b, :first, h])
    assert not np.isfinite(S1[b, h]).all() or not np.isfinite(o1[b, :, h]).all()
