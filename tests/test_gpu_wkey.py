"""GPU parity of the write-key entry points (gdr_chunk_fwd_wkey,
gdr_recurrent_step_wkey) against the fp64 oracle with the same write keys.

The write key is kw = d * k ("OSDN: Improving Delta Rule with Provable Online
Preconditioning in Linear Attention", §2.1) with a seeded preconditioner d drawn
uniformly from (0.2, 2) per (token, head, channel), rounded to the I/O dtype like
every other input.  Tolerances as for the plain forward and step (relative L2:
2e-2 for bf16 I/O with an fp32 state, 1e-4 for fp32 I/O).
"""

import numpy as np
import pytest

from oracle import forward as oracle_forward, recurrent_step as oracle_step, rel_l2
from tests.gpu_util import TOL, check, dev, host, need_gpu, say
from workloads import CONFIGS, Workload, chunk_inputs
from workloads.inputs import round_to_io

pytestmark = pytest.mark.gpu


def _wkey_inputs(B, T, H, dk, dv, seed, io="bf16", s0=0.02, gate="none"):
    inp = chunk_inputs(Workload("wkey", B=B, T=T, H=H, d_k=dk, d_v=dv, io=io, gate=gate, s0_std=s0, seed=seed))
    d = np.random.default_rng([seed, 7]).uniform(0.2, 2.0, inp["k"].shape)
    inp["kw"] = round_to_io(d * inp["k"], io)
    return inp


@pytest.mark.parametrize("shape", [(2, 200, 3, 128, 128), (1, 130, 2, 64, 128), (1, 65, 2, 128, 64),
                                   (2, 1, 2, 128, 128), (1, 300, 64, 128, 128),
                                   (2, 130, 64, 128, 128)],   # B*H*(d_v/64) = 256: 64-column state tiles
                         ids=lambda s: "B%dT%dH%d_dk%d_dv%d" % s)
def test_write_key_chunk_fwd(shape):
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    B, T, H, dk, dv = shape
    say(f"case write key {shape}")
    inp = _wkey_inputs(B, T, H, dk, dv, seed=101 + T)
    o, S = gdr.chunk_fwd(*(dev(inp[n], "bf16") for n in ("q", "k", "v", "beta")), None,
                         torch.from_numpy(inp["S0"]).cuda(), kw=dev(inp["kw"], "bf16"))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_forward(inp["q"], inp["k"], inp["v"], inp["beta"], None, inp["S0"], kw=inp["kw"])
    check("o", host(o), o_ref, TOL["bf16"])
    check("S_T", host(S), S_ref, TOL["bf16"])


def test_write_key_equal_to_key_is_deltanet():
    """kw = k gives the no-gate forward (OSDN §2.1 with d = 1)."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    inp = _wkey_inputs(2, 150, 2, 128, 128, seed=113)
    args = [dev(inp[n], "bf16") for n in ("q", "k", "v", "beta")]
    S0 = torch.from_numpy(inp["S0"]).cuda()
    o1, S1 = gdr.chunk_fwd(*args, None, S0, kw=args[1])
    o2, S2 = gdr.chunk_fwd(*args, None, S0)
    torch.cuda.synchronize()
    assert rel_l2(host(o1), host(o2)) <= 1e-6 and rel_l2(host(S1), host(S2)) <= 1e-6


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_write_key_decode_step(io):
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    inp = _wkey_inputs(16, 1, 4, 128, 128, seed=127, io=io, s0=0.05)
    st = {n: np.ascontiguousarray(inp[n][:, 0]) for n in ("q", "k", "v", "beta", "kw")}
    S = torch.from_numpy(inp["S0"]).cuda()
    o, S_new = gdr.recurrent_step(*(dev(st[n], io) for n in ("q", "k", "v", "beta")), None, S,
                                  S_new=torch.empty_like(S), kw=dev(st["kw"], io))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_step(inp["S0"], st["q"], st["k"], st["v"], st["beta"], None, kw=st["kw"])
    check("o", host(o), o_ref, TOL[io])
    check("S_new", host(S_new), S_ref, TOL[io])


def test_write_key_prefill_then_decode():
    """The forward's final state continues with write-key decode steps: the same
    as the oracle over the longer sequence."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    inp = _wkey_inputs(2, 133, 2, 128, 128, seed=131)
    T0 = 130
    part = lambda n, sl: np.ascontiguousarray(inp[n][:, sl])
    o, S = gdr.chunk_fwd(*(dev(part(n, slice(0, T0)), "bf16") for n in ("q", "k", "v", "beta")), None,
                         torch.from_numpy(inp["S0"]).cuda(), kw=dev(part("kw", slice(0, T0)), "bf16"))
    outs = []
    for t in range(T0, 133):
        ot, S = gdr.recurrent_step(*(dev(part(n, t), "bf16") for n in ("q", "k", "v", "beta")), None, S,
                                   kw=dev(part("kw", t), "bf16"))
        outs.append(host(ot))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_forward(inp["q"], inp["k"], inp["v"], inp["beta"], None, inp["S0"], kw=inp["kw"])
    check("decode o", np.stack(outs, axis=1), o_ref[:, T0:], TOL["bf16"])
    check("S", host(S), S_ref, TOL["bf16"])


# ---- the write key with a gate ("OSDN", §4: the preconditioner on gated backbones) -------
@pytest.mark.parametrize("form", ["page", "literal"])
@pytest.mark.parametrize("gate,shape", [("scalar", (2, 200, 3, 128, 128)), ("scalar", (1, 130, 2, 64, 128)),
                                        ("scalar", (2, 130, 64, 128, 128)), ("channel", (2, 200, 3, 128, 128)),
                                        ("channel", (1, 65, 2, 128, 64)), ("channel", (1, 1, 2, 128, 128))],
                         ids=lambda x: x if isinstance(x, str) else "B%dT%dH%d_dk%d_dv%d" % x)
def test_write_key_chunk_fwd_gated(gate, shape, form):
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    B, T, H, dk, dv = shape
    say(f"case write key, gate={gate}, {shape}, form={form}")
    inp = _wkey_inputs(B, T, H, dk, dv, seed=211 + T + H, gate=gate)
    o, S = gdr.chunk_fwd(*(dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")),
                         torch.from_numpy(inp["S0"]).cuda(), kw=dev(inp["kw"], "bf16"), form=form)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_a"], inp["S0"], kw=inp["kw"],
                                  form=form)
    check("o", host(o), o_ref, TOL["bf16"])
    check("S_T", host(S), S_ref, TOL["bf16"])


def test_write_key_channel_gate_fast_forgetting():
    """A per-channel block past the transform's split range with a write key: the
    generic kernel pairs k with kw as the split-factor transform does."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    inp = _wkey_inputs(1, 200, 2, 128, 128, seed=223, gate="channel")
    inp["log_a"][0, 70:95, 1, 20:60] = -6.0
    o, S = gdr.chunk_fwd(*(dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")),
                         torch.from_numpy(inp["S0"]).cuda(), kw=dev(inp["kw"], "bf16"))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_a"], inp["S0"], kw=inp["kw"])
    check("o", host(o), o_ref, TOL["bf16"])
    check("S_T", host(S), S_ref, TOL["bf16"])


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("form", ["page", "literal"])
def test_write_key_decode_step_gated(io, gate, form):
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    inp = _wkey_inputs(16, 1, 4, 128, 128, seed=227, io=io, s0=0.05, gate=gate)
    st = {n: np.ascontiguousarray(inp[n][:, 0]) for n in ("q", "k", "v", "beta", "kw", "log_a")}
    S = torch.from_numpy(inp["S0"]).cuda()
    o, S_new = gdr.recurrent_step(*(dev(st[n], io) for n in ("q", "k", "v", "beta", "log_a")), S,
                                  S_new=torch.empty_like(S), kw=dev(st["kw"], io), form=form)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_step(inp["S0"], st["q"], st["k"], st["v"], st["beta"], st["log_a"], kw=st["kw"], form=form)
    check("o", host(o), o_ref, TOL[io])
    check("S_new", host(S_new), S_ref, TOL[io])


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_write_key_gated_prefill_then_decode(gate):
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    inp = _wkey_inputs(2, 133, 2, 128, 128, seed=229, gate=gate)
    T0 = 130
    part = lambda n, sl: np.ascontiguousarray(inp[n][:, sl])
    o, S = gdr.chunk_fwd(*(dev(part(n, slice(0, T0)), "bf16") for n in ("q", "k", "v", "beta", "log_a")),
                         torch.from_numpy(inp["S0"]).cuda(), kw=dev(part("kw", slice(0, T0)), "bf16"))
    outs = [host(o)]
    for t in range(T0, 133):
        ot, S = gdr.recurrent_step(*(dev(part(n, t), "bf16") for n in ("q", "k", "v", "beta", "log_a")), S,
                                   kw=dev(part("kw", t), "bf16"))
        outs.append(host(ot)[:, None])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_a"], inp["S0"], kw=inp["kw"])
    check("o (prefill and decode)", np.concatenate(outs, axis=1), o_ref, TOL["bf16"])
    check("S", host(S), S_ref, TOL["bf16"])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [3, 4])
def test_write_key_full_size_whole_tensor(cfg):
    """The write-key forward over a gated workload at full size: B8 H16 T8192 d128
    with the scalar gate (the launch the benchmark's write-key training path times)
    and B2 H32 T32768 d128 with the per-channel gate; every (b, h) slice against the
    oracle with the same write keys (host processes in parallel): whole-tensor
    relative L2 of o and S_T, and that of the worst slice, within the bf16 tolerance."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    from tests.parallel_oracle import whole_chunk
    from tests.report import report
    wl = CONFIGS[cfg]
    say(f"full-size write-key forward {wl.name}: generating inputs")
    inp = chunk_inputs(wl)
    d = np.random.default_rng([wl.seed, 7]).uniform(0.2, 2.0, inp["k"].shape)
    kw_h = round_to_io(d * inp["k"], "bf16")
    del d
    args = [dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")]
    S0 = torch.from_numpy(inp["S0"]).cuda()
    del inp
    say("  running GPU")
    o, S = gdr.chunk_fwd(*args, S0, kw=dev(kw_h, "bf16"))
    torch.cuda.synchronize()
    o_h, S_h = o.float().cpu().numpy(), S.cpu().numpy()
    del o, S, args, S0
    assert np.isfinite(o_h).all() and np.isfinite(S_h).all()
    say("  oracle on every slice")
    r = whole_chunk(wl, o_h, S_h, group=2 if cfg == 4 else 4, kw=kw_h)
    line = (f"write-key forward {wl.name}: whole-tensor rel_l2 o {r['o']:.3e}  S_T {r['S']:.3e}; worst (b, h, rel_l2) "
            f"o ({r['worst_o'][0]}, {r['worst_o'][1]}, {r['worst_o'][2]:.3e})  S_T ({r['worst_S'][0]}, "
            f"{r['worst_S'][1]}, {r['worst_S'][2]:.3e}); {r['slices']} slices on {r['procs']} processes in "
            f"{r['seconds']:.1f} s")
    say("  " + line)
    report(line)
    assert r["o"] <= TOL["bf16"] and r["S"] <= TOL["bf16"]
    assert r["worst_o"][2] <= TOL["bf16"] and r["worst_S"][2] <= TOL["bf16"]
