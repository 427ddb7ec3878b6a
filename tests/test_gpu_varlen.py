"""GPU parity of gdr_chunk_fwd_varlen (variable-length sequences packed along T)
against the fp64 oracle run on each sequence alone, and the prefill -> decode
handoff (the packed forward's final states feed gdr_recurrent_step).

A sequence boundary restarts the recurrence from that sequence's own initial
state, so each packed sequence must match the oracle of that sequence alone
(tolerance as for gdr_chunk_fwd: relative L2 2e-2 for bf16 I/O), and must equal
bit for bit what gdr_chunk_fwd gives for the sequence on its own.
"""

import numpy as np
import pytest

from oracle import forward as oracle_forward, recurrent_step as oracle_step, rel_l2
from tests.gpu_util import TOL, check, dev, host, need_gpu, say
from workloads import Workload, chunk_inputs

pytestmark = pytest.mark.gpu

LENS = [0, 1, 63, 64, 65, 130, 200, 7]          # empty, single token, around a chunk, several chunks


def _inputs(lens, H, dk, dv, gate, seed):
    """Packed tokens of all sequences ([1, sum(lens), H, .]) and one initial state per sequence."""
    T = int(sum(lens))
    inp = chunk_inputs(Workload("varlen", B=1, T=T, H=H, d_k=dk, d_v=dv, io="bf16", gate=gate, s0_std=0.0,
                                seed=seed))
    S0 = chunk_inputs(Workload("varlen_s0", B=len(lens), T=1, H=H, d_k=dk, d_v=dv, io="bf16", gate=gate,
                               s0_std=0.02, seed=seed + 1))["S0"]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return inp, S0, cu


def _seq(a, lo, hi):
    return None if a is None else np.ascontiguousarray(a[:, lo:hi])


def _oracle(inp, S0, cu, form="page"):
    N = len(cu) - 1
    o = np.zeros(inp["v"].shape)
    S = np.zeros(S0.shape)
    for i in range(N):
        lo, hi = int(cu[i]), int(cu[i + 1])
        oi, Si = oracle_forward(*(_seq(inp[n], lo, hi) for n in ("q", "k", "v", "beta", "log_a")), S0[i:i + 1],
                                form=form)
        o[:, lo:hi] = oi
        S[i] = Si[0]
    return o, S


def _gpu(inp, S0, cu, form="page"):
    import torch
    import gated_delta_rule_21_amd as gdr
    o, S = gdr.chunk_fwd_varlen(*(dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")),
                                torch.from_numpy(cu).cuda(), torch.from_numpy(S0).cuda(), form=form)
    torch.cuda.synchronize()
    return o, S


def _check_each(o, S, o_ref, S_ref, cu):
    check("o", host(o), o_ref, TOL["bf16"])
    check("S_T", host(S), S_ref, TOL["bf16"])
    Sh = host(S)
    for i in range(len(cu) - 1):            # every sequence on its own, short ones included
        e = rel_l2(Sh[i], S_ref[i])
        assert e <= TOL["bf16"], f"sequence {i} (length {cu[i + 1] - cu[i]}): S_T rel_l2 {e:.3e}"


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("dk", [128, 64])
def test_varlen_matches_oracle_per_sequence(gate, dk):
    need_gpu()
    say(f"case varlen gate={gate} d_k={dk} lens={LENS}")
    inp, S0, cu = _inputs(LENS, 2, dk, 128, gate, seed=61 + dk + len(gate))
    o, S = _gpu(inp, S0, cu)
    o_ref, S_ref = _oracle(inp, S0, cu)
    _check_each(o, S, o_ref, S_ref, cu)


def test_varlen_literal_ordering():
    need_gpu()
    inp, S0, cu = _inputs(LENS, 2, 128, 128, "channel", seed=71)
    o, S = _gpu(inp, S0, cu, form="literal")
    o_ref, S_ref = _oracle(inp, S0, cu, form="literal")
    _check_each(o, S, o_ref, S_ref, cu)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_varlen_equals_separate_calls(gate):
    """Each packed sequence gives bit for bit what gdr_chunk_fwd gives on it alone."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    inp, S0, cu = _inputs(LENS, 2, 128, 128, gate, seed=73)
    o, S = _gpu(inp, S0, cu)
    o, S = o.cpu(), S.cpu()
    for i in range(len(cu) - 1):
        lo, hi = int(cu[i]), int(cu[i + 1])
        if hi == lo:
            assert torch.equal(S[i], torch.from_numpy(S0[i])), f"empty sequence {i}: S_T != S0"
            continue
        oi, Si = gdr.chunk_fwd(*(dev(_seq(inp[n], lo, hi), "bf16") for n in ("q", "k", "v", "beta", "log_a")),
                               torch.from_numpy(S0[i:i + 1]).cuda())
        torch.cuda.synchronize()
        assert torch.equal(o[:, lo:hi], oi.cpu()), f"sequence {i}: o differs"
        assert torch.equal(S[i:i + 1], Si.cpu()), f"sequence {i}: S_T differs"


def test_varlen_many_sequences_wide():
    """More workgroups than CUs (4 x 64 heads x 2 tiles), lengths from 1 to 300."""
    need_gpu()
    rs = np.random.RandomState(5)
    lens = [int(x) for x in rs.randint(1, 300, size=4)]
    inp, S0, cu = _inputs(lens, 64, 128, 128, "scalar", seed=79)
    o, S = _gpu(inp, S0, cu)
    o_ref, S_ref = _oracle(inp, S0, cu)
    _check_each(o, S, o_ref, S_ref, cu)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_prefill_then_decode_handoff(gate):
    """Packed prefill, then one decode token per sequence from the prefill's final
    states, equals the oracle over each sequence plus that token."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    lens = [1, 64, 65, 200]
    N, H, dk, dv = len(lens), 2, 128, 128
    inp, S0, cu = _inputs(lens, H, dk, dv, gate, seed=83)
    tok = chunk_inputs(Workload("next", B=N, T=1, H=H, d_k=dk, d_v=dv, io="bf16", gate=gate, s0_std=0.0, seed=89))
    _, S = _gpu(inp, S0, cu)
    step = {n: (None if tok[n] is None else np.ascontiguousarray(tok[n][:, 0])) for n in ("q", "k", "v", "beta", "log_a")}
    o_dec, S_dec = gdr.recurrent_step(*(dev(step[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")), S)
    torch.cuda.synchronize()
    _, S_pre = _oracle(inp, S0, cu)
    o_ref, S_ref = oracle_step(S_pre, step["q"], step["k"], step["v"], step["beta"], step["log_a"])
    check("decode o", host(o_dec), o_ref, TOL["bf16"])
    check("decode S", host(S_dec), S_ref, TOL["bf16"])


def test_varlen_order_longest_first():
    """The state pass takes packed sequences longest first: the order it leaves at
    the end of the caller's workspace is a permutation sorted by length, ties by
    index; with N * H not a multiple of 8 (the non-interleaved block mapping)."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    lens = [5, 300, 64, 300, 0, 17, 129]
    N, H = len(lens), 3
    inp, S0, cu = _inputs(lens, H, 128, 128, "scalar", seed=97)
    size = gdr.chunk_varlen_workspace_size(int(sum(lens)), N, H, 128, 128, torch.bfloat16, "scalar")
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    o, S = gdr.chunk_fwd_varlen(*(dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")),
                                torch.from_numpy(cu).cuda(), torch.from_numpy(S0).cuda(), workspace=ws)
    torch.cuda.synchronize()
    tail = (N * 4 + 15) // 16 * 16
    order = ws[size - tail:size - tail + 4 * N].cpu().view(torch.int32).numpy()
    want = sorted(range(N), key=lambda i: (-lens[i], i))
    assert list(order) == want, (list(order), want)
    o_ref, S_ref = _oracle(inp, S0, cu)
    _check_each(o, S, o_ref, S_ref, cu)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n_seq", [16384, 16385])
def test_varlen_order_at_its_limit(n_seq):
    """The rank kernel orders up to 16,384 packed sequences longest first and leaves
    the identity order above that; either way every sequence (lengths 0 to 3 tokens)
    matches the oracle run on it alone."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    lens = [int(x) for x in np.random.RandomState(n_seq).randint(0, 4, size=n_seq)]
    N, H, T = n_seq, 2, int(sum(lens))
    say(f"case {N} packed sequences, {T} tokens")
    inp, S0, cu = _inputs(lens, H, 64, 64, "scalar", seed=131)
    size = gdr.chunk_varlen_workspace_size(T, N, H, 64, 64, torch.bfloat16, "scalar")
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    o, S = gdr.chunk_fwd_varlen(*(dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")),
                                torch.from_numpy(cu).cuda(), torch.from_numpy(S0).cuda(), workspace=ws)
    torch.cuda.synchronize()
    tail = (N * 4 + 15) // 16 * 16
    order = ws[size - tail:size - tail + 4 * N].cpu().view(torch.int32).numpy()
    want = sorted(range(N), key=lambda i: (-lens[i], i)) if N <= 16384 else list(range(N))
    assert list(order) == want
    o_ref, S_ref = _oracle(inp, S0, cu)
    _check_each(o, S, o_ref, S_ref, cu)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_varlen_write_key(gate):
    """gdr_chunk_fwd_varlen_wkey: each packed sequence against the write-key oracle of
    that sequence alone, and bit for bit against gdr_chunk_fwd_wkey on it."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    say(f"case varlen write key gate={gate} lens={LENS}")
    inp, S0, cu = _inputs(LENS, 2, 128, 128, gate, seed=91 + len(gate))
    rng = np.random.default_rng(92)
    from workloads import round_to_io
    kw = round_to_io(inp["k"].astype(np.float64) * rng.uniform(0.2, 2.0, inp["k"].shape), "bf16")
    args = [dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")]
    o, S = gdr.chunk_fwd_varlen(*args, torch.from_numpy(cu).cuda(), torch.from_numpy(S0).cuda(), kw=dev(kw, "bf16"))
    torch.cuda.synchronize()
    o_h, S_h = host(o), host(S)
    o_ref = np.zeros(inp["v"].shape)
    S_ref = np.zeros(S0.shape)
    for i in range(len(cu) - 1):
        lo, hi = int(cu[i]), int(cu[i + 1])
        oi, Si = oracle_forward(*(_seq(inp[n], lo, hi) for n in ("q", "k", "v", "beta", "log_a")), S0[i:i + 1],
                                kw=_seq(kw, lo, hi))
        o_ref[:, lo:hi] = oi
        S_ref[i] = Si[0]
        if hi > lo:
            a = [dev(_seq(inp[n], lo, hi), "bf16") for n in ("q", "k", "v", "beta", "log_a")]
            oa, Sa = gdr.chunk_fwd(*a, torch.from_numpy(S0[i:i + 1]).cuda(), kw=dev(_seq(kw, lo, hi), "bf16"))
            torch.cuda.synchronize()
            assert np.array_equal(host(oa), o_h[:, lo:hi]), f"sequence {i}: o differs from the call on it alone"
            assert np.array_equal(host(Sa)[0], S_h[i]), f"sequence {i}: S_T differs from the call on it alone"
    check("o", o_h, o_ref, TOL["bf16"])
    check("S_T", S_h, S_ref, TOL["bf16"])


@pytest.mark.parametrize("gate,dk", [("none", 64), ("scalar", 64), ("channel", 64), ("none", 128), ("scalar", 128)])
def test_varlen_fp32(gate, dk):
    """fp32 I/O over packed sequences: each sequence against the oracle of that sequence
    alone (1e-4) and bit for bit against gdr_chunk_fwd on it."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    say(f"case varlen fp32 gate={gate} d_k={dk} lens={LENS}")
    T = int(sum(LENS))
    inp = chunk_inputs(Workload("varlen32", B=1, T=T, H=2, d_k=dk, d_v=64, io="f32", gate=gate, s0_std=0.0,
                                seed=111 + dk + len(gate)))
    S0 = chunk_inputs(Workload("varlen32_s0", B=len(LENS), T=1, H=2, d_k=dk, d_v=64, io="f32", gate=gate,
                               s0_std=0.02, seed=112))["S0"]
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int32)
    args = [dev(inp[n], "f32") for n in ("q", "k", "v", "beta", "log_a")]
    o, S = gdr.chunk_fwd_varlen(*args, torch.from_numpy(cu).cuda(), torch.from_numpy(S0).cuda())
    torch.cuda.synchronize()
    o_h, S_h = host(o), host(S)
    o_ref, S_ref = _oracle(inp, S0, cu)
    check("o", o_h, o_ref, TOL["f32"])
    check("S_T", S_h, S_ref, TOL["f32"])
    for i in range(len(cu) - 1):
        lo, hi = int(cu[i]), int(cu[i + 1])
        if hi == lo:
            assert np.array_equal(S_h[i], S0[i].astype(np.float64)), f"empty sequence {i}: S_T != S0"
            continue
        a = [dev(_seq(inp[n], lo, hi), "f32") for n in ("q", "k", "v", "beta", "log_a")]
        oa, Sa = gdr.chunk_fwd(*a, torch.from_numpy(S0[i:i + 1]).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(host(oa), o_h[:, lo:hi]), f"sequence {i}: o differs from the call on it alone"
        assert np.array_equal(host(Sa)[0], S_h[i]), f"sequence {i}: S_T differs from the call on it alone"


@pytest.mark.timeout(600)
def test_serving_mix_full_size_whole():
    """The benchmark's serving mix at full size, in the launch it times: 32 prompts of
    log-uniform lengths in [128, 8192] (H16 d128, scalar gate, no initial state)
    through the packed forward, then 16 decode steps on the states it hands over.
    o over every packed token, S_T of every sequence, every decode output and the
    final states against the oracle, whole tensors."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    from bench import handoff_lengths
    from tests.report import report
    lens = handoff_lengths()
    N, H, dk, dv, T, steps = len(lens), 16, 128, 128, int(sum(lens)), 16
    say(f"serving mix: {N} prompts, {T} tokens")
    inp = chunk_inputs(Workload("handoff_prefill", B=1, T=T, H=H, d_k=dk, d_v=dv, io="bf16", gate="scalar",
                                s0_std=0.0, seed=6))
    tok = chunk_inputs(Workload("handoff_tokens", B=N, T=steps, H=H, d_k=dk, d_v=dv, io="bf16", gate="scalar",
                                s0_std=0.0, seed=7))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, S = gdr.chunk_fwd_varlen(*(dev(inp[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")),
                                torch.from_numpy(cu).cuda(), None)
    o_pre = host(o)
    S_pre_gpu = host(S)
    dec = []
    for s in range(steps):
        od, S = gdr.recurrent_step(*(dev(np.ascontiguousarray(tok[n][:, s]), "bf16")
                                     for n in ("q", "k", "v", "beta", "log_a")), S)
        dec.append(host(od))
    torch.cuda.synchronize()
    S_dec = host(S)
    say("  oracle on every sequence")
    from tests.parallel_oracle import whole_packed
    r = whole_packed(inp, cu, np.zeros((N, H, dk, dv)), o_pre, S_pre_gpu)
    e_o, e_s, worst = r["o"], r["S"], r["worst_S"]
    say(f"  prefill o {e_o:.3e}  S_T {e_s:.3e}  worst sequence S_T {worst:.3e} ({r['procs']} processes, "
        f"{r['seconds']:.1f} s)")
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"] and worst <= TOL["bf16"], (e_o, e_s, worst)
    Sr = r["S_ref"]
    e_d = 0.0
    for s in range(steps):
        od_ref, Sr = oracle_step(Sr, *(tok[n][:, s] for n in ("q", "k", "v", "beta", "log_a")))
        e_d = max(e_d, check(f"decode o step {s}", dec[s], od_ref, TOL["bf16"]))
    e_f = check("decode S", S_dec, Sr, TOL["bf16"])
    line = (f"serving mix ({N} prompts, {T} tokens, H{H} d{dk}): prefill o {e_o:.3e}  S_T {e_s:.3e} (worst sequence "
            f"{worst:.3e}); {steps} decode steps: worst o {e_d:.3e}, final S {e_f:.3e}")
    say("  " + line)
    report(line)
