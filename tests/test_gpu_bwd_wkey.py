"""GPU parity of gdr_chunk_bwd_wkey (the gradients of the write-key chunk forward)
against the fp64 backward oracle.

The write key ("OSDN: Improving Delta Rule with Provable Online Preconditioning in
Linear Attention", §2.1) makes the erase read the state along k and the write go
along kw; the oracle (oracle/backward.py, pinned by finite differences through the
write key) returns dk for the read side and dkw for the write side.  The GPU path
takes the same derivatives through the chunk form, the decomposition checked
against the oracle in fp64 by tests/test_chunk_form.py::test_chunk_backward_equals_oracle.

Inputs: the backward tests' workloads, with a write key kw = d * k, d ~ U(0.2, 2)
per (token, head, channel), rounded to bf16 as the OSDN scan would hand it over.
Tolerance: 2e-2 relative L2 over each gradient tensor, as for the bf16 backward.
"""

import numpy as np
import pytest

from oracle import backward as oracle_backward
from tests.gpu_util import TOL, check, dev, host, need_gpu, say
from workloads import CONFIGS, Workload, chunk_inputs, grad_inputs, round_to_io

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dkw", "dv", "dbeta", "dlog_a", "dS0")


def _with_kw(x, seed):
    d = np.random.default_rng(seed).uniform(0.2, 2.0, x["k"].shape)
    x["kw"] = round_to_io(x["k"].astype(np.float64) * d, "bf16")
    return x


def _inputs(B, T, H, dk, dv, gate, seed, s0_std=0.5):
    wl = Workload("bwd_wkey", B=B, T=T, H=H, d_k=dk, d_v=dv, io="bf16", gate=gate, s0_std=s0_std, seed=seed)
    x = chunk_inputs(wl)
    x.update(grad_inputs(wl))
    return _with_kw(x, seed + 1000)


def _gpu(x, form="page", with_S0=True, with_dST=True, kw="kw"):
    import torch
    import gated_delta_rule_21_amd as gdr
    S0 = torch.from_numpy(x["S0"]).cuda() if with_S0 else None
    dS_T = torch.from_numpy(x["dS_T"]).cuda() if with_dST else None
    g = gdr.chunk_bwd(dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16"), dev(x["beta"], "bf16"),
                      dev(x["log_a"], "bf16"), S0, dev(x["dO"], "bf16"), dS_T, form=form,
                      kw=None if kw is None else dev(x[kw], "bf16"))
    torch.cuda.synchronize()
    return {n: (host(t) if t is not None else None) for n, t in g.items()}


def _ref(x, form="page", with_S0=True, with_dST=True):
    return oracle_backward(x["q"], x["k"], x["v"], x["beta"], x["log_a"], x["S0"] if with_S0 else None, x["dO"],
                           x["dS_T"] if with_dST else None, form=form, kw=x["kw"])


def _compare(got, ref, gate):
    worst = 0.0
    for n in NAMES:
        if n == "dlog_a" and gate == "none":
            continue
        worst = max(worst, check(n, got[n], ref[n], TOL["bf16"]))
    return worst


SHAPES = [(2, 200, 3, 128, 128), (1, 130, 2, 64, 64), (2, 100, 2, 128, 64), (1, 70, 2, 64, 128)]


@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dT%dH%ddk%ddv%d" % s)
def test_bwd_wkey_shapes(gate, shape):
    need_gpu()
    say(f"case bwd write key gate={gate} shape={shape}")
    x = _inputs(*shape, gate, seed=sum(shape) + 7 * (gate == "scalar"))
    _compare(_gpu(x), _ref(x), gate)


@pytest.mark.parametrize("shape", [(2, 200, 3, 128, 128), (1, 130, 2, 64, 128)], ids=lambda s: "B%dT%dH%ddk%ddv%d" % s)
def test_bwd_wkey_literal_form(shape):
    need_gpu()
    say(f"case bwd write key, literal form, shape={shape}")
    x = _inputs(*shape, "scalar", seed=61 + sum(shape))
    x["log_a"][:, 40:43] = -8.0               # strong gates inside a chunk
    _compare(_gpu(x, form="literal"), _ref(x, form="literal"), "scalar")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129])
def test_bwd_wkey_lengths(T):
    need_gpu()
    say(f"case bwd write key T={T}")
    x = _inputs(2, T, 2, 128, 128, "scalar", seed=500 + T)
    _compare(_gpu(x), _ref(x), "scalar")


def test_bwd_wkey_without_state_terms():
    need_gpu()
    say("case bwd write key, no S0 and no dS_T")
    x = _inputs(2, 150, 2, 128, 128, "scalar", seed=71)
    got, ref = _gpu(x, with_S0=False, with_dST=False), _ref(x, with_S0=False, with_dST=False)
    for n in ("dq", "dk", "dkw", "dv", "dbeta", "dlog_a", "dS0"):
        check(n, got[n], ref[n], TOL["bf16"])


def test_bwd_wkey_strong_forgetting():
    need_gpu()
    say("case bwd write key, log a = -20 inside chunks")
    x = _inputs(2, 200, 2, 128, 128, "scalar", seed=73)
    x["log_a"][:, 70:75] = -20.0
    x["log_a"][1, 130] = -20.0
    _compare(_gpu(x), _ref(x), "scalar")


@pytest.mark.parametrize("gate", ["scalar", "none"])
def test_bwd_wkey_equal_to_key(gate):
    """kw = k: the read and write sides add up to gdr_chunk_bwd's dk, and every other
    gradient is that of gdr_chunk_bwd."""
    need_gpu()
    say(f"case bwd write key equal to the key, gate={gate}")
    x = _inputs(2, 150, 2, 128, 128, gate, seed=79)
    a = _gpu(x, kw="k")
    b = _gpu(x, kw=None)
    check("dk + dkw vs dk", a["dk"] + a["dkw"], b["dk"], 1e-2)
    for n in ("dq", "dv", "dbeta", "dS0") + (("dlog_a",) if gate == "scalar" else ()):
        check(f"{n} vs the plain backward", a[n], b[n], 1e-2)


def test_bwd_wkey_deterministic():
    need_gpu()
    say("case bwd write key, two calls bit for bit")
    x = _inputs(2, 300, 3, 128, 128, "scalar", seed=83)
    a, b = _gpu(x), _gpu(x)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


def test_bwd_wkey_full_size_whole_tensor():
    """The gated B8 H16 T8192 d128 bf16 workload with a write key at full size; every
    (b, h) slice against the oracle (host processes in parallel): each gradient's
    whole-tensor relative L2, and that of its worst slice, within the bf16 tolerance."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    from tests.parallel_oracle import assert_whole, whole_backward
    wl = CONFIGS[3]
    say(f"full-size write-key backward {wl.name}: generating inputs")
    x = chunk_inputs(wl)
    x.update(grad_inputs(wl))
    _with_kw(x, 9001)
    args = [dev(x[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")]
    kw = dev(x["kw"], "bf16")
    S0 = torch.from_numpy(x["S0"]).cuda()
    dO, dS_T = dev(x["dO"], "bf16"), torch.from_numpy(x["dS_T"]).cuda()
    kw_host = x["kw"]
    del x
    say("  running GPU")
    g = gdr.chunk_bwd(*args, S0, dO, dS_T, kw=kw)
    torch.cuda.synchronize()
    for n in NAMES:
        assert bool(torch.isfinite(g[n].float()).all()), n
    grads = {n: g[n].float().cpu().numpy() for n in NAMES}
    del g, args, kw, S0, dO, dS_T
    say("  oracle on every (b, h) slice")
    assert_whole(f"write-key backward {wl.name}", whole_backward(wl, grads, kw=kw_host), TOL["bf16"])


@pytest.mark.parametrize("gate", ["scalar", "none"])
def test_autograd_function_write_key(gate):
    """chunk_attn with a write key: the .grad of every input, kw included, against the
    oracle's gradients of <dO, o> + <dS_T, S_T>."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    say(f"case autograd with a write key, gate={gate}")
    x = _inputs(2, 150, 2, 128, 128, gate, seed=89)
    leaf = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda().requires_grad_(True)
    ins = {n: leaf(x[n], torch.bfloat16) for n in ("q", "k", "v", "beta", "kw")}
    ins["log_a"] = leaf(x["log_a"], torch.bfloat16) if gate == "scalar" else None
    S0 = leaf(x["S0"], torch.float32)
    o, S_T = gdr.chunk_attn(ins["q"], ins["k"], ins["v"], ins["beta"], ins["log_a"], S0, kw=ins["kw"])
    loss = (o.float() * torch.from_numpy(x["dO"]).cuda()).sum() + (S_T * torch.from_numpy(x["dS_T"]).cuda()).sum()
    loss.backward()
    torch.cuda.synchronize()
    ref = _ref(x)
    for n, t in (("dq", ins["q"]), ("dk", ins["k"]), ("dkw", ins["kw"]), ("dv", ins["v"]), ("dbeta", ins["beta"]),
                 ("dlog_a", ins["log_a"]), ("dS0", S0)):
        if t is None:
            continue
        check(n, host(t.grad), ref[n], TOL["bf16"])


@pytest.mark.parametrize("gate", ["scalar", "none"])
def test_bwd_wkey_varlen(gate):
    """gdr_chunk_bwd_varlen_wkey: packed sequences of lengths 0, 1, 63, 64, 65, 130,
    200, 7 against the oracle per sequence, and bit for bit against the fixed-length
    write-key backward on each sequence alone."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    say(f"case bwd write key, packed sequences, gate={gate}")
    lens = [0, 1, 63, 64, 65, 130, 200, 7]
    T = int(sum(lens))
    wl = Workload("bwd_wkey_varlen", B=1, T=T, H=2, d_k=128, d_v=128, io="bf16", gate=gate, s0_std=0.0, seed=97)
    x = chunk_inputs(wl)
    x["dO"] = grad_inputs(wl)["dO"]
    per = Workload("bwd_wkey_varlen_states", B=len(lens), T=1, H=2, d_k=128, d_v=128, io="bf16", gate=gate,
                   s0_std=0.5, seed=98)
    x["S0"] = chunk_inputs(per)["S0"]
    x["dS_T"] = grad_inputs(per)["dS_T"]
    _with_kw(x, 99)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t = lambda n: dev(x[n], "bf16")
    g = gdr.chunk_bwd(t("q"), t("k"), t("v"), t("beta"), t("log_a"), torch.from_numpy(x["S0"]).cuda(), t("dO"),
                      torch.from_numpy(x["dS_T"]).cuda(), cu_seqlens=torch.from_numpy(cu).cuda(), kw=t("kw"))
    torch.cuda.synchronize()
    gh = {n: host(v) if v is not None else None for n, v in g.items()}
    seq = lambda a, lo, hi: None if a is None else np.ascontiguousarray(a[:, lo:hi])
    names = ("dq", "dk", "dkw", "dv", "dbeta") + (("dlog_a",) if gate == "scalar" else ())
    ref = {n: np.zeros(gh[n].shape) for n in names}
    ref["dS0"] = np.zeros(x["S0"].shape)
    for i in range(len(lens)):
        lo, hi = int(cu[i]), int(cu[i + 1])
        s = {n: seq(x[n], lo, hi) for n in ("q", "k", "kw", "v", "beta", "log_a", "dO")}
        r = oracle_backward(s["q"], s["k"], s["v"], s["beta"], s["log_a"], x["S0"][i:i + 1], s["dO"],
                            x["dS_T"][i:i + 1], kw=s["kw"])
        for n in names:
            ref[n][:, lo:hi] = r[n]
        ref["dS0"][i] = r["dS0"][0]
        if hi > lo:
            a = gdr.chunk_bwd(*(dev(s[n], "bf16") for n in ("q", "k", "v", "beta", "log_a")),
                              torch.from_numpy(x["S0"][i:i + 1]).cuda(), dev(s["dO"], "bf16"),
                              torch.from_numpy(x["dS_T"][i:i + 1]).cuda(), kw=dev(s["kw"], "bf16"))
            torch.cuda.synchronize()
            for n in names:
                assert np.array_equal(host(a[n]), gh[n][:, lo:hi]), f"sequence {i}: {n} differs from the call on it alone"
            assert np.array_equal(host(a["dS0"])[0], gh["dS0"][i]), f"sequence {i}: dS0"
    for n in names + ("dS0",):
        check(n, gh[n], ref[n], TOL["bf16"])
