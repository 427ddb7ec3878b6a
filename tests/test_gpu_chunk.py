"""GPU parity of gdr_chunk_fwd against the fp64 token-by-token oracle.

Tolerances (relative L2 over the tensor): 1e-4 for fp32 I/O, 2e-2 for bf16 I/O
with an fp32 state, on both the output o and the final state S_T.
"""

import zlib

import numpy as np
import pytest

from tests.gpu_util import TOL, check, gpu_chunk, need_gpu, oracle_chunk, say
from workloads import CONFIGS, Workload, chunk_inputs, slice_inputs

pytestmark = pytest.mark.gpu


def _wl(name, B, T, H, dk, dv, io="bf16", gate="scalar", s0=0.02, seed=11):
    return Workload(name, B=B, T=T, H=H, d_k=dk, d_v=dv, io=io, gate=gate, s0_std=s0, seed=seed)


def _run(wl, form="page"):
    need_gpu()
    say(f"case {wl} form={form}")
    inp = chunk_inputs(wl)
    o, S = gpu_chunk(inp, wl.io, form)
    o_ref, S_ref = oracle_chunk(inp, form)
    check("o", o, o_ref, TOL[wl.io])
    check("S_T", S, S_ref, TOL[wl.io])
    return inp, o, S


def test_config1_deltanet_fp32():
    """DeltaNet, B1 H1 T256 d64, fp32 I/O (the small workload, whole tensor)."""
    _run(CONFIGS[1])


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("shape", [(2, 200, 3, 128, 128), (1, 130, 2, 64, 128), (1, 77, 2, 128, 64),
                                   (2, 64, 2, 64, 64)], ids=lambda s: "B%dT%dH%d_dk%d_dv%d" % s)
def test_bf16_gates_and_shapes(gate, shape):
    B, T, H, dk, dv = shape
    _run(_wl("small", B, T, H, dk, dv, gate=gate, seed=zlib.crc32(repr((gate, shape)).encode()) % 1000))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_literal_ordering(gate):
    _run(_wl("literal", 2, 150, 2, 128, 128, gate=gate, seed=5), form="literal")


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 129])
def test_sequence_lengths(T):
    _run(_wl("lens", 2, T, 2, 128, 128, gate="channel", seed=17 + T))


def test_four_wave_tiles():
    """B*H*(d_v/64) >= 256 selects 64-column tiles (4 waves per workgroup)."""
    _run(_wl("wide", 1, 130, 128, 128, 128, gate="scalar", seed=23))


def test_fp32_channel_gate():
    _run(_wl("f32ch", 2, 150, 2, 64, 128, io="f32", gate="channel", seed=29))


def test_zero_initial_state_pointer():
    need_gpu()
    wl = _wl("nos0", 1, 100, 2, 128, 128, gate="scalar", s0=0.0, seed=31)
    inp = chunk_inputs(wl)
    o, S = gpu_chunk(inp, "bf16", with_S0=False)
    o_ref, S_ref = oracle_chunk(inp, with_S0=False)
    check("o", o, o_ref, TOL["bf16"])
    check("S_T", S, S_ref, TOL["bf16"])


def test_bitwise_determinism():
    need_gpu()
    inp = chunk_inputs(_wl("det", 2, 300, 3, 128, 128, gate="channel", seed=37))
    a = gpu_chunk(inp, "bf16")
    b = gpu_chunk(inp, "bf16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_split_sequence_handoff():
    """S_T of the first part, passed as S0 of the second, reproduces the oracle."""
    need_gpu()
    import torch
    from tests.gpu_util import dev, host
    import gated_delta_rule_21_amd as gdr
    wl = _wl("split", 1, 300, 2, 128, 128, gate="scalar", seed=41)
    inp = chunk_inputs(wl)
    T1 = 100
    part = lambda a, s: None if a is None else np.ascontiguousarray(a[:, s])
    S0 = torch.from_numpy(inp["S0"]).cuda()
    o1, S1 = gdr.chunk_fwd(*(dev(part(inp[n], slice(0, T1)), "bf16") for n in ("q", "k", "v", "beta", "log_a")), S0)
    o2, S2 = gdr.chunk_fwd(*(dev(part(inp[n], slice(T1, None)), "bf16") for n in ("q", "k", "v", "beta", "log_a")), S1)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_chunk(inp)
    check("o", np.concatenate([host(o1), host(o2)], axis=1), o_ref, TOL["bf16"])
    check("S_T", host(S2), S_ref, TOL["bf16"])


def test_state_updated_in_place():
    need_gpu()
    import torch
    from tests.gpu_util import dev, host
    import gated_delta_rule_21_amd as gdr
    inp = chunk_inputs(_wl("inplace", 1, 90, 2, 128, 128, gate="channel", seed=43))
    S = torch.from_numpy(inp["S0"]).cuda()
    o, S_out = gdr.chunk_fwd(*(dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")), S, S_T=S)
    torch.cuda.synchronize()
    assert S_out.data_ptr() == S.data_ptr()
    o_ref, S_ref = oracle_chunk(inp)
    check("o", host(o), o_ref, TOL["bf16"])
    check("S_T", host(S), S_ref, TOL["bf16"])


def test_caller_workspace_reused_and_dirty():
    """A caller workspace full of NaN bit patterns is overwritten before use, and
    one workspace serves calls of different sizes and gates in a row."""
    need_gpu()
    import torch
    from tests.gpu_util import dev, host
    import gated_delta_rule_21_amd as gdr
    big = gdr.chunk_workspace_size(2, 260, 3, 128, 128, torch.bfloat16, "channel")
    ws = torch.full((big,), 0xFF, dtype=torch.uint8, device="cuda")
    for name, shape, gate, seed in (("ws1", (2, 260, 3, 128, 128), "channel", 47),
                                    ("ws2", (1, 70, 2, 64, 128), "scalar", 53)):
        inp = chunk_inputs(_wl(name, *shape, gate=gate, seed=seed))
        S0 = torch.from_numpy(inp["S0"]).cuda()
        o, S = gdr.chunk_fwd(*(dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")), S0, workspace=ws)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle_chunk(inp)
        check(f"{name} o", host(o), o_ref, TOL["bf16"])
        check(f"{name} S_T", host(S), S_ref, TOL["bf16"])
    with pytest.raises(gdr.GdrError):
        inp = chunk_inputs(_wl("ws3", 2, 260, 4, 128, 128, gate="channel", seed=59))  # needs more than `big`
        gdr.chunk_fwd(*(dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")), None, workspace=ws)


# ---- full-size workloads: whole-tensor run on the GPU, sampled (b, h) slices
#      checked against the oracle one slice at a time -----------------------------
def _sampled(cfg):
    need_gpu()
    import torch
    from tests.gpu_util import dev, host
    from oracle import forward
    import gated_delta_rule_21_amd as gdr
    wl = CONFIGS[cfg]
    say(f"full workload {wl.name}: generating inputs")
    inp = chunk_inputs(wl)
    S0 = torch.from_numpy(inp["S0"]).cuda()
    args = [dev(inp[n], wl.io) for n in ("q", "k", "v", "beta", "log_a")]
    del inp
    say("  running GPU")
    o, S = gdr.chunk_fwd(*args, S0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(S).all())
    samples = [(0, 0), (wl.B - 1, wl.H - 1), (wl.B // 2, wl.H // 3)]
    errs_o, errs_S = [], []
    for b, h in samples:
        s = slice_inputs(wl, b, h)
        e = lambda x: None if x is None else x[None, :, None]
        o_ref, S_ref = forward(e(s["q"]), e(s["k"]), e(s["v"]), e(s["beta"]), e(s["log_a"]), s["S0"][None, None])
        errs_o.append(check(f"o[b={b},h={h}]", host(o[b, :, h]), o_ref[0, :, 0], TOL[wl.io]))
        errs_S.append(check(f"S_T[b={b},h={h}]", host(S[b, h]), S_ref[0, 0], TOL[wl.io]))
    say(f"  max rel_l2 o {max(errs_o):.3e}  S_T {max(errs_S):.3e}")


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_workload_sampled(cfg):
    _sampled(cfg)
