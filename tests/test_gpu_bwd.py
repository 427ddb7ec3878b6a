"""GPU parity of gdr_chunk_bwd (the gradients of the chunk forward) against the
fp64 backward oracle.

The pages print no gradients: the oracle is the reverse mode of the token-by-token
recurrence ("Moonshot AI's New Attention Architecture", §2), pinned by finite
differences of the forward oracle; the GPU path takes the same derivatives through
the chunk form of §3.  The loss is L = <dO, o> + <dS_T, S_T>.

Tolerance: relative L2 over each gradient tensor of 2e-2, as for the forward with
bf16 I/O (bf16 products with fp32 accumulation; the per-chunk states are read in
bf16 as the forward's products read them).  Inputs: the forward's workloads, with
dO ~ N(0, 1) and dS_T ~ N(0, 1).
"""

import numpy as np
import pytest

from oracle import backward as oracle_backward
from tests.gpu_util import TOL, check, dev, host, need_gpu, say
from workloads import CONFIGS, Workload, chunk_inputs, grad_inputs

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dlog_a", "dS0")


def _inputs(B, T, H, dk, dv, gate, seed, s0_std=0.5):
    wl = Workload("bwd", B=B, T=T, H=H, d_k=dk, d_v=dv, io="bf16", gate=gate, s0_std=s0_std, seed=seed)
    x = chunk_inputs(wl)
    x.update(grad_inputs(wl))
    return x


def _gpu(x, with_S0=True, with_dST=True, want_dS0=True, in_place=False, form="page"):
    import torch
    import gated_delta_rule_21_amd as gdr
    S0 = torch.from_numpy(x["S0"]).cuda() if with_S0 else None
    dS_T = torch.from_numpy(x["dS_T"]).cuda() if with_dST else None
    g = gdr.chunk_bwd(dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16"), dev(x["beta"], "bf16"),
                      dev(x["log_a"], "bf16"), S0, dev(x["dO"], "bf16"), dS_T, want_dS0=want_dS0 and not in_place,
                      form=form)
    if in_place:
        g = gdr.chunk_bwd(dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16"), dev(x["beta"], "bf16"),
                          dev(x["log_a"], "bf16"), S0, dev(x["dO"], "bf16"), dS_T, want_dS0=False)
        _in_place(x, S0, dS_T)
        g["dS0"] = dS_T
    torch.cuda.synchronize()
    return {n: (host(t) if t is not None else None) for n, t in g.items()}


def _in_place(x, S0, dS_T):
    """dS0 written over dS_T through the C ABI (the binding allocates dS0 itself)."""
    import ctypes
    import torch
    import gated_delta_rule_21_amd as gdr
    from gated_delta_rule_21_amd._lib import GdrDesc, _ptr
    lib = gdr.load()
    q, k, v, beta = (dev(x[n], "bf16") for n in ("q", "k", "v", "beta"))
    log_a, dO = dev(x["log_a"], "bf16"), dev(x["dO"], "bf16")
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    gate = 0 if log_a is None else 1
    desc = GdrDesc(B, T, H, dk, dv, 64, 1, gate, 0)
    need = ctypes.c_size_t(0)
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(need)) == 0
    ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(beta),
            torch.empty_like(log_a) if log_a is not None else None]
    st = lib.gdr_chunk_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_a), _ptr(S0), _ptr(dO),
                           _ptr(dS_T), *[_ptr(t) for t in outs], _ptr(dS_T), _ptr(ws), ws.numel(), None)
    assert st == 0, lib.gdr_last_error().decode()


def _ref(x, with_S0=True, with_dST=True, form="page"):
    return oracle_backward(x["q"], x["k"], x["v"], x["beta"], x["log_a"], x["S0"] if with_S0 else None, x["dO"],
                           x["dS_T"] if with_dST else None, form=form)


def _compare(got, ref, gate, skip=()):
    for n in NAMES:
        if n in skip or (n == "dlog_a" and gate == "none"):
            continue
        check(n, got[n], ref[n], TOL["bf16"])


SHAPES = [(2, 200, 3, 128, 128), (1, 130, 2, 64, 64), (2, 100, 2, 128, 64), (1, 70, 2, 64, 128)]


@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dT%dH%ddk%ddv%d" % s)
def test_bwd_shapes(gate, shape):
    need_gpu()
    say(f"case bwd gate={gate} shape={shape}")
    x = _inputs(*shape, gate, seed=sum(shape) + (gate == "scalar"))
    _compare(_gpu(x), _ref(x), gate)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129])
def test_bwd_lengths(T):
    need_gpu()
    say(f"case bwd T={T}")
    x = _inputs(2, T, 2, 128, 128, "scalar", seed=400 + T)
    _compare(_gpu(x), _ref(x), "scalar")


def test_bwd_without_state_terms():
    """No initial state and no final-state gradient; dS0 not requested."""
    need_gpu()
    x = _inputs(2, 150, 2, 128, 128, "scalar", seed=21)
    got = _gpu(x, with_S0=False, with_dST=False, want_dS0=False)
    assert got["dS0"] is None
    _compare(got, _ref(x, with_S0=False, with_dST=False), "scalar", skip=("dS0",))


def test_bwd_dS0_in_place():
    need_gpu()
    x = _inputs(1, 140, 2, 128, 128, "scalar", seed=23)
    _compare(_gpu(x, in_place=True), _ref(x), "scalar")


def test_bwd_empty_sequence():
    """T = 0: dS0 is the final-state gradient (zero without one)."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    x = _inputs(2, 0, 2, 128, 128, "scalar", seed=25)
    g = gdr.chunk_bwd(dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16"), dev(x["beta"], "bf16"),
                      dev(x["log_a"], "bf16"), torch.from_numpy(x["S0"]).cuda(), dev(x["dO"], "bf16"),
                      torch.from_numpy(x["dS_T"]).cuda())
    g0 = gdr.chunk_bwd(dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16"), dev(x["beta"], "bf16"),
                       dev(x["log_a"], "bf16"), None, dev(x["dO"], "bf16"), None)
    torch.cuda.synchronize()
    assert np.array_equal(host(g["dS0"]), x["dS_T"].astype(np.float64))
    assert not np.any(host(g0["dS0"]))


def test_bwd_strong_forgetting():
    """Gates of log a = -20 inside chunks (decay factors far below the fp32 range
    of e^{-g}): every factor the kernels form is e^{x} with x <= 0."""
    need_gpu()
    x = _inputs(2, 200, 2, 128, 128, "scalar", seed=27)
    x["log_a"][:, 70:75] = -20.0
    x["log_a"][1, 130] = -20.0
    _compare(_gpu(x), _ref(x), "scalar")


def test_bwd_full_size_whole_tensor():
    """The gated B8 H16 T8192 d128 bf16 workload at full size, in the launch
    configuration the benchmark times; every (b, h) slice against the oracle (host
    processes in parallel): each gradient's whole-tensor relative L2, and that of its
    worst slice, within the bf16 tolerance."""
    _full_size_whole_tensor(CONFIGS[3])


def _full_size_whole_tensor(wl):
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    from tests.parallel_oracle import assert_whole, whole_backward
    say(f"full-size backward {wl.name}: generating inputs")
    x = chunk_inputs(wl)
    x.update(grad_inputs(wl))
    args = [dev(x[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")]
    S0 = torch.from_numpy(x["S0"]).cuda()
    dO, dS_T = dev(x["dO"], "bf16"), torch.from_numpy(x["dS_T"]).cuda()
    del x
    say("  running GPU")
    g = gdr.chunk_bwd(*args, S0, dO, dS_T)
    torch.cuda.synchronize()
    for n in NAMES:
        assert bool(torch.isfinite(g[n].float()).all()), n
    grads = {n: g[n].float().cpu().numpy() for n in NAMES}
    del g, args, S0, dO, dS_T
    say("  oracle on every (b, h) slice")
    assert_whole(f"backward {wl.name}", whole_backward(wl, grads), TOL["bf16"])


def test_bwd_deterministic():
    """Two calls on the same inputs give the same bits (no atomics; every sum is
    taken in a fixed order)."""
    need_gpu()
    x = _inputs(2, 300, 3, 128, 128, "scalar", seed=29)
    a, b = _gpu(x), _gpu(x)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


# ---- packed sequences (gdr_chunk_bwd_varlen) ---------------------------------------
LENS = [0, 1, 63, 64, 65, 130, 200, 7]          # empty, single token, around a chunk, several chunks


def _packed(lens, H, dk, dv, gate, seed):
    """Packed tokens and output gradients ([1, sum(lens), H, .]), one S0 and one dS_T per sequence."""
    T = int(sum(lens))
    wl = Workload("bwd_varlen", B=1, T=T, H=H, d_k=dk, d_v=dv, io="bf16", gate=gate, s0_std=0.0, seed=seed)
    x = chunk_inputs(wl)
    x["dO"] = grad_inputs(wl)["dO"]
    per = Workload("bwd_varlen_states", B=len(lens), T=1, H=H, d_k=dk, d_v=dv, io="bf16", gate=gate, s0_std=0.5,
                   seed=seed + 1)
    x["S0"] = chunk_inputs(per)["S0"]
    x["dS_T"] = grad_inputs(per)["dS_T"]
    return x, np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _seq(a, lo, hi):
    return None if a is None else np.ascontiguousarray(a[:, lo:hi])


@pytest.mark.parametrize("gate,dk,dv", [("scalar", 128, 128), ("scalar", 64, 128), ("none", 128, 128),
                                        ("none", 64, 128), ("channel", 128, 128)])
def test_bwd_varlen(gate, dk, dv):
    """The packed backward against the oracle run on each sequence alone (relative
    L2 over all packed tokens, and per sequence on dS0), and bit for bit against
    gdr_chunk_bwd on each sequence alone.  (A per-sequence check of dbeta on a
    one-token sequence would compare a single sum with heavy cancellation.)"""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    say(f"case bwd varlen gate={gate} d_k={dk} d_v={dv} lens={LENS}")
    x, cu = _packed(LENS, 2, dk, dv, gate, seed=71 + dk + len(gate))
    args = [dev(x[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")]
    g = gdr.chunk_bwd(*args, torch.from_numpy(x["S0"]).cuda(), dev(x["dO"], "bf16"),
                      torch.from_numpy(x["dS_T"]).cuda(), cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    got = {n: (host(t) if t is not None else None) for n, t in g.items()}
    names = ["dq", "dk", "dv", "dbeta"] + (["dlog_a"] if gate != "none" else [])
    ref = {n: np.zeros(got[n].shape) for n in names}
    for i in range(len(LENS)):
        lo, hi = int(cu[i]), int(cu[i + 1])
        seq = {n: _seq(x[n], lo, hi) for n in ("q", "k", "v", "beta", "log_a", "dO")}
        r = oracle_backward(seq["q"], seq["k"], seq["v"], seq["beta"], seq["log_a"], x["S0"][i:i + 1], seq["dO"],
                            x["dS_T"][i:i + 1])
        for n in names:
            ref[n][:, lo:hi] = r[n]
        check(f"dS0[seq {i}, T={hi - lo}]", got["dS0"][i:i + 1], r["dS0"], TOL["bf16"])
        if hi > lo:                      # the same sequence through the fixed-length entry point
            one = gdr.chunk_bwd(*(dev(seq[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")),
                                torch.from_numpy(np.ascontiguousarray(x["S0"][i:i + 1])).cuda(), dev(seq["dO"], "bf16"),
                                torch.from_numpy(np.ascontiguousarray(x["dS_T"][i:i + 1])).cuda())
            torch.cuda.synchronize()
            for n in names:
                assert np.array_equal(host(one[n]), got[n][:, lo:hi]), (n, i)
            assert np.array_equal(host(one["dS0"]), got["dS0"][i:i + 1]), ("dS0", i)
        else:
            assert np.array_equal(got["dS0"][i], x["dS_T"][i].astype(np.float64))
    for n in names:
        check(n, got[n], ref[n], TOL["bf16"])


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("packed", [False, True], ids=["batch", "packed"])
def test_autograd_function(packed, gate):
    """chunk_attn (chunk_fwd with chunk_bwd as its torch autograd backward): the .grad
    of every input against the oracle's gradients of <dO, o> + <dS_T, S_T>."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    say(f"case autograd gate={gate} packed={packed}")
    if packed:
        x, cu = _packed([70, 1, 130], 2, 128, 128, gate, seed=31)
        cu_t = torch.from_numpy(cu).cuda()
    else:
        x, cu_t = _inputs(2, 150, 2, 128, 128, gate, seed=31), None
    leaf = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda().requires_grad_(True)
    ins = {n: leaf(x[n], torch.bfloat16) for n in ("q", "k", "v", "beta", "log_a")}
    S0 = leaf(x["S0"], torch.float32)
    o, S_T = gdr.chunk_attn(ins["q"], ins["k"], ins["v"], ins["beta"], ins["log_a"], S0, cu_seqlens=cu_t)
    loss = (o.float() * torch.from_numpy(x["dO"]).cuda()).sum() + (S_T * torch.from_numpy(x["dS_T"]).cuda()).sum()
    loss.backward()
    torch.cuda.synchronize()
    if packed:
        names = ("dq", "dk", "dv", "dbeta", "dlog_a")
        ref = {n: np.zeros(x[n[1:]].shape) for n in names}
        ref["dS0"] = np.zeros(x["S0"].shape)
        for i in range(len(cu) - 1):
            lo, hi = int(cu[i]), int(cu[i + 1])
            seq = {n: _seq(x[n], lo, hi) for n in ("q", "k", "v", "beta", "log_a", "dO")}
            r = oracle_backward(seq["q"], seq["k"], seq["v"], seq["beta"], seq["log_a"], x["S0"][i:i + 1], seq["dO"],
                                x["dS_T"][i:i + 1])
            for n in names:
                ref[n][:, lo:hi] = r[n]
            ref["dS0"][i] = r["dS0"][0]
    else:
        ref = _ref(x)
    for n, t in (("dq", ins["q"]), ("dk", ins["k"]), ("dv", ins["v"]), ("dbeta", ins["beta"]),
                 ("dlog_a", ins["log_a"]), ("dS0", S0)):
        check(n, host(t.grad), ref[n], TOL["bf16"])


@pytest.mark.parametrize("shape", [(2, 200, 3, 128, 128), (1, 130, 2, 64, 128), (2, 65, 2, 128, 64)],
                         ids=lambda s: "B%dT%dH%ddk%ddv%d" % s)
def test_bwd_literal_form(shape):
    """The erase on the undecayed state (GDR_FORM_LITERAL) with a scalar gate: the A
    factor and the residual's decay read g_{r-1}, so the gradient of those terms goes
    to the gate of the token before."""
    need_gpu()
    say(f"case bwd literal shape={shape}")
    x = _inputs(*shape, "scalar", seed=sum(shape) + 5)
    x["log_a"][:, 40:43] = -6.0            # strong gates: the page and literal forms differ clearly
    _compare(_gpu(x, form="literal"), _ref(x, form="literal"), "scalar")


# ---- per-channel gate (d_k = 128) --------------------------------------------------
@pytest.mark.parametrize("form", ["page", "literal"])
@pytest.mark.parametrize("shape", [(2, 200, 3, 128, 128), (2, 100, 2, 128, 64), (1, 64, 2, 128, 128)],
                         ids=lambda s: "B%dT%dH%ddk%ddv%d" % s)
def test_bwd_channel(shape, form):
    """A gate per key channel: the decayed operands inside the d_k sums, and d log a
    per (token, head, channel)."""
    need_gpu()
    say(f"case bwd channel form={form} shape={shape}")
    x = _inputs(*shape, "channel", seed=sum(shape) + 11)
    _compare(_gpu(x, form=form), _ref(x, form=form), "channel")


@pytest.mark.parametrize("T", [1, 63, 65, 129])
def test_bwd_channel_lengths(T):
    need_gpu()
    say(f"case bwd channel T={T}")
    x = _inputs(1, T, 2, 128, 128, "channel", seed=40 + T)
    _compare(_gpu(x), _ref(x), "channel")


def test_bwd_channel_strong_channels():
    """Some channels forget fast (log a = -3 over 12 tokens, 36 inside one 16-row
    block) beside slow ones: the block-split decay factors stay in range."""
    need_gpu()
    x = _inputs(2, 160, 2, 128, 128, "channel", seed=45)
    x["log_a"][:, 20:32, :, :16] = -3.0
    x["log_a"][1, 100:110, 1, 64:] = -3.0
    _compare(_gpu(x), _ref(x), "channel")
    _compare(_gpu(x, form="literal"), _ref(x, form="literal"), "channel")


def test_bwd_channel_deterministic():
    need_gpu()
    x = _inputs(2, 150, 2, 128, 128, "channel", seed=47)
    a, b = _gpu(x), _gpu(x)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.timeout(900)
def test_bwd_channel_full_size_whole_tensor():
    """The per-channel B2 H32 T32768 d128 bf16 workload at full size; every (b, h)
    slice against the oracle, as for the gated workload."""
    _full_size_whole_tensor(CONFIGS[4])