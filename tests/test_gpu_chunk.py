"""GPU parity of gdr_chunk_fwd against the fp64 token-by-token oracle.

Tolerances (relative L2 over the tensor): 1e-4 for fp32 I/O, 2e-2 for bf16 I/O
with an fp32 state, on both the output o and the final state S_T.
"""

import zlib

import numpy as np
import pytest

from tests.gpu_util import TOL, check, gpu_chunk, need_gpu, oracle_chunk, say
from tests.report import report
from workloads import CONFIGS, Workload, chunk_inputs

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
    need_gpu()
    wl = CONFIGS[1]
    inp = chunk_inputs(wl)
    o, S = gpu_chunk(inp, wl.io)
    o_ref, S_ref = oracle_chunk(inp)
    e_o, e_s = check("o", o, o_ref, TOL["f32"]), check("S_T", S, S_ref, TOL["f32"])
    report(f"{wl.name}: whole-tensor rel_l2 o {e_o:.3e}  S_T {e_s:.3e}")


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


@pytest.mark.parametrize("gate,form", [("none", "page"), ("scalar", "page"), ("scalar", "literal")])
@pytest.mark.parametrize("shape", [(2, 200, 3, 128, 128), (1, 130, 2, 128, 64), (1, 1, 2, 128, 128)],
                         ids=lambda s: "B%dT%dH%d_dk%d_dv%d" % s)
def test_fp32_dk128(gate, form, shape):
    """fp32 I/O at d_k = 128 (no gate or a scalar gate): the transform through LDS and
    the single-buffered fp32 state pass."""
    B, T, H, dk, dv = shape
    _run(_wl("f32d128", B, T, H, dk, dv, io="f32", gate=gate, seed=37 + T + dv), form=form)


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


# ---- full-size workloads in the benchmarked launch, every (b, h) slice against the oracle ----
@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,form", [(2, "page"), (3, "page"), (4, "page"), (3, "literal"), (4, "literal")])
def test_full_workload_whole_tensor(cfg, form):
    """The whole o and S_T of the full-size workload against the fp64 oracle run on
    every (b, h) slice (host processes in parallel): whole-tensor relative L2 within
    the bf16 tolerance, and the worst slice reported.  The gated workloads also run
    in the literal form (the gate read after the erase)."""
    _whole_forward(CONFIGS[cfg], form, group=2 if cfg == 4 else 4)


@pytest.mark.timeout(900)
def test_longest_sequence_the_offsets_allow():
    """The longest sequence the kernels' 32-bit per-sequence byte offsets allow at H16
    d128 bf16: T = 524,287 tokens, so that T*H*d*2 = 2^31 - 4096 bytes (one token more
    is refused, see the ABI tests), with a ragged last chunk, a scalar gate and an
    initial state; the whole o and S_T against the oracle run on every head."""
    wl = Workload("max_span_b1h16t524287d128_bf16", B=1, T=524287, H=16, d_k=128, d_v=128, io="bf16",
                  gate="scalar", s0_std=0.02, seed=31)
    _whole_forward(wl, "page", group=1)


def _whole_forward(wl, form, group):
    need_gpu()
    import torch
    from tests.gpu_util import dev
    from tests.parallel_oracle import whole_chunk
    import gated_delta_rule_21_amd as gdr
    say(f"full workload {wl.name}: generating inputs")
    inp = chunk_inputs(wl)
    S0 = torch.from_numpy(inp["S0"]).cuda()
    args = [dev(inp[n], wl.io) for n in ("q", "k", "v", "beta", "log_a")]
    del inp
    say("  running GPU")
    o, S = gdr.chunk_fwd(*args, S0, form=form)
    torch.cuda.synchronize()
    o_h, S_h = o.float().cpu().numpy(), S.cpu().numpy()
    del o, S, args, S0
    assert np.isfinite(o_h).all() and np.isfinite(S_h).all()
    say("  oracle on every slice")
    r = whole_chunk(wl, o_h, S_h, group=group, form=form)
    name = wl.name + ("" if form == "page" else " (literal form)")
    line = (f"{name}: whole-tensor rel_l2 o {r['o']:.3e}  S_T {r['S']:.3e}; worst (b, h, rel_l2) o "
            f"({r['worst_o'][0]}, {r['worst_o'][1]}, {r['worst_o'][2]:.3e})  S_T ({r['worst_S'][0]}, {r['worst_S'][1]}, "
            f"{r['worst_S'][2]:.3e}); {r['slices']} slices on {r['procs']} processes in {r['seconds']:.1f} s")
    say("  " + line)
    report(line)
    assert r["o"] <= TOL[wl.io] and r["S"] <= TOL[wl.io]
    assert r["worst_o"][2] <= TOL[wl.io] and r["worst_S"][2] <= TOL[wl.io]


# ---- gates and beta at the edges of their range -----------------------------------------
def _edge(inp, io="bf16", form="page"):
    o, S = gpu_chunk(inp, io, form)
    o_ref, S_ref = oracle_chunk(inp, form)
    check("o", o, o_ref, TOL[io])
    check("S_T", S, S_ref, TOL[io])
    return o, S


@pytest.mark.parametrize("form", ["page", "literal"])
def test_channel_gate_fast_forgetting(form):
    """log a = -6 on 16 channels for 20 tokens (a 16-token block decays by e^-90 in
    those channels, past the transform's split), beside channels at the workload's
    rates; only some chunks and heads take the generic transform."""
    need_gpu()
    inp = chunk_inputs(_wl("fast", 2, 300, 3, 128, 128, gate="channel", seed=61))
    la = inp["log_a"]
    la[0, 20:40, 1, :16] = -6.0                 # chunk 0, head 1
    la[1, 150:175, 0, 100:] = -6.0              # chunk 2, head 0
    la[1, 260:262, 2, 5] = -70.0                # one token per channel past the literal form's bound
    say(f"case fast-forgetting per-channel gate form={form}")
    _edge(inp, form=form)


def test_channel_gate_fast_forgetting_fp32():
    need_gpu()
    inp = chunk_inputs(_wl("fast32", 1, 200, 2, 64, 128, io="f32", gate="channel", seed=67))
    inp["log_a"][0, 70:100, 1, 3:40] = -7.0
    say("case fast-forgetting per-channel gate, fp32 I/O")
    _edge(inp, io="f32")


def test_channel_gate_packed_fast_forgetting():
    """Packed sequences with a block past the split's range in one sequence."""
    need_gpu()
    import torch
    from tests.gpu_util import dev, host
    import gated_delta_rule_21_amd as gdr
    from oracle import forward
    lens = [70, 0, 150, 33]
    wl = _wl("packfast", 1, sum(lens), 2, 128, 128, gate="channel", seed=71)
    inp = chunk_inputs(wl)
    inp["log_a"][0, 80:110, 1, 10:30] = -6.0    # inside the third sequence (tokens 70..219)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    S0 = np.random.default_rng(3).normal(0, 0.02, (len(lens), 2, 128, 128)).astype(np.float32)
    say("case packed sequences, fast-forgetting per-channel gate")
    o, S = gdr.chunk_fwd_varlen(*(dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")), cu,
                                torch.from_numpy(S0).cuda())
    torch.cuda.synchronize()
    o, S = host(o), host(S)
    t0 = 0
    for i, L in enumerate(lens):
        sl = lambda a: a[:, t0:t0 + L]
        o_ref, S_ref = forward(*(sl(inp[n]) for n in ("q", "k", "v", "beta", "log_a")), S0[i:i + 1])
        if L:
            check(f"o[seq {i}]", o[:, t0:t0 + L], o_ref, TOL["bf16"])
        check(f"S_T[seq {i}]", S[i:i + 1], S_ref, TOL["bf16"])
        t0 += L


@pytest.mark.parametrize("form", ["page", "literal"])
def test_scalar_gate_strong(form):
    """A scalar log a = -20 on a few tokens inside chunks (the state is all but erased)."""
    need_gpu()
    inp = chunk_inputs(_wl("strong", 2, 200, 2, 128, 128, gate="scalar", seed=73))
    inp["log_a"][0, 30:33, 0] = -20.0
    inp["log_a"][1, 100, 1] = -20.0
    inp["log_a"][1, 64, 0] = -20.0              # on a chunk's first row
    say(f"case strong scalar gate form={form}")
    _edge(inp, form=form)


@pytest.mark.parametrize("io,dk", [("f32", 64), ("bf16", 128)])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_exact_recall_nonunit_keys(io, dk, gate):
    """Keys of norm 0.5..2 with beta = 1/||k||^2 and q = k: the delta rule stores each
    value exactly (S_t^T k_t = v_t under any gate, decay before the erase), so o = v.
    fp32 I/O holds that to the rounding of beta; bf16 to the rounding of beta and o."""
    need_gpu()
    wl = _wl("recall", 2, 150, 2, dk, 128, io=io, gate=gate, seed=79)
    inp = chunk_inputs(wl)
    rng = np.random.default_rng(5)
    from workloads import round_to_io
    k = inp["k"].astype(np.float64) * rng.uniform(0.5, 2.0, inp["k"].shape[:-1] + (1,))
    inp["k"] = round_to_io(k, io)
    inp["q"] = inp["k"].copy()
    inp["beta"] = round_to_io(1.0 / (inp["k"].astype(np.float64) ** 2).sum(-1), io)
    say(f"case exact recall io={io} d_k={dk} gate={gate}")
    o, _ = _edge(inp, io=io)
    tol = 1e-4 if io == "f32" else 2e-2
    check("o vs v (recall)", o, inp["v"].astype(np.float64), tol)


@pytest.mark.parametrize("beta", [0.0, 1.5])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_beta_outside_unit_interval(beta, gate):
    """beta = 0 (no update: the state only decays) and beta = 1.5 (the erase overshoots).
    With beta = 0 the final state is S0 times the whole decay; the gate is scaled by
    0.05 there so that it stays within fp32's range (e^-5 rather than e^-98)."""
    need_gpu()
    from workloads import round_to_io
    inp = chunk_inputs(_wl("beta", 1, 140, 2, 128, 128, gate=gate, seed=83))
    inp["beta"][:] = beta
    if beta == 0.0 and inp["log_a"] is not None:
        inp["log_a"] = round_to_io(0.05 * inp["log_a"].astype(np.float64), "bf16")
    say(f"case beta={beta} gate={gate}")
    _edge(inp)
