"""GPU parity of gdr_precond_scan_bwd (the gradients of the preconditioner scan)
against the fp64 oracle, and of both phases of the preconditioned delta rule
trained end to end.

"OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
Attention", §2.2 (phase 1 scans the keys into write keys k~_t = d_t * k_t;
phase 2 is the delta rule with that write key) and §4 (the method is trained):
the gradient of phase 2's write key flows back through the scan.  The oracle
(oracle.preconditioner.precond_scan_backward) is pinned by finite differences of
the forward scan oracle (tests/test_precond_backward_pins.py).

Inputs: the scan's workloads (unit-norm keys, beta in (0, 1), retention
sigmoid(N(0,1) + 3), d0 ~ U(0.5, 1.5)), with dkw ~ N(0, 1) rounded to the I/O
dtype and dd_T ~ N(0, 1).  Tolerances: relative L2 of 1e-4 (fp32 I/O) and 2e-2
(bf16 I/O) over each gradient tensor; the kernel computes in fp32 for both.
"""

import numpy as np
import pytest

from oracle import backward as oracle_backward
from oracle.preconditioner import precond_scan_backward
from tests.gpu_util import TOL, check, dev, host, need_gpu, say
from workloads import Workload, grad_inputs, precond_inputs, round_to_io

pytestmark = pytest.mark.gpu

ETA = 1.0


def _inputs(B, T, H, dk, io, seed, forget=True):
    wl = Workload("scan_bwd", B=B, T=T, H=H, d_k=dk, d_v=dk, io=io, gate="none", s0_std=0.0, seed=seed)
    x = precond_inputs(wl)
    if not forget:
        x["r"] = None
    rng = np.random.default_rng(seed + 7)
    x["dkw"] = round_to_io(rng.standard_normal((B, T, H, dk)), io)
    x["dd_T"] = rng.standard_normal((B, H, dk)).astype(np.float32)
    return x


def _gpu(x, io, eta=ETA, with_d0=True, with_dkw=True, with_ddT=True):
    import torch
    import gated_delta_rule_21_amd as gdr
    d0 = torch.from_numpy(x["d0"]).cuda() if with_d0 else None
    dd_T = torch.from_numpy(x["dd_T"]).cuda() if with_ddT else None
    g = gdr.precond_scan_bwd(dev(x["k"], io), dev(x["beta"], io), eta, dev(x["r"], io), d0,
                             dev(x["dkw"], io) if with_dkw else None, dd_T)
    torch.cuda.synchronize()
    return {n: (host(t) if t is not None else None) for n, t in g.items()}


def _ref(x, eta=ETA, with_d0=True, with_dkw=True, with_ddT=True):
    return precond_scan_backward(x["k"], x["beta"], eta, x["r"], x["d0"] if with_d0 else None,
                                 x["dkw"] if with_dkw else None, x["dd_T"] if with_ddT else None)


def _compare(got, ref, io):
    worst = 0.0
    for n in ("dk", "dbeta", "dr", "dd0"):
        if ref[n] is None:
            assert got[n] is None, n
            continue
        worst = max(worst, check(n, got[n], ref[n], TOL[io]))
    return worst


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("dk", [128, 64])
@pytest.mark.parametrize("forget", [True, False])
@pytest.mark.parametrize("shape", [(2, 150, 3), (1, 70, 2)], ids=lambda s: "B%dT%dH%d" % s)
def test_scan_bwd(io, dk, forget, shape):
    need_gpu()
    B, T, H = shape
    say(f"case scan backward io={io} d_k={dk} forget={forget} shape={shape}")
    x = _inputs(B, T, H, dk, io, seed=T + dk + forget, forget=forget)
    _compare(_gpu(x, io), _ref(x), io)


@pytest.mark.parametrize("T", [0, 1, 15, 16, 17, 33, 64, 200])
def test_scan_bwd_lengths(T):
    need_gpu()
    say(f"case scan backward T={T}")
    x = _inputs(2, T, 2, 128, "bf16", seed=40 + T)
    got = _gpu(x, "bf16")
    if T == 0:
        assert np.array_equal(got["dd0"], x["dd_T"].astype(np.float64))
        return
    _compare(got, _ref(x), "bf16")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_scan_bwd_optional_inputs(io):
    """No d0 (ones), no dkw (zero), no dd_T (zero), each in turn."""
    need_gpu()
    x = _inputs(2, 100, 2, 128, io, seed=51)
    for opt in ({"with_d0": False}, {"with_dkw": False}, {"with_ddT": False}):
        say(f"case scan backward io={io} {opt}")
        _compare(_gpu(x, io, **opt), _ref(x, **opt), io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_scan_bwd_edge_values(io):
    """Zero keys (d passes unchanged), eta in {0.25, 8}, a retention of 1e-3 over a
    run of tokens, a retention of exactly 0 (d restarts from e_t w_t) inside a
    block of 16 tokens and on a block's first token."""
    need_gpu()
    x = _inputs(2, 120, 2, 128, io, seed=53)
    x["k"][0, 10:13, 1] = 0.0
    x["k"][1, 0, 0] = 0.0
    x["r"][:, 60:80] = 1e-3
    x["r"][0, 37, 0] = 0.0
    x["r"][1, 96, 1] = 0.0
    x["r"] = round_to_io(x["r"], io)
    for eta in (0.25, 8.0):
        say(f"case scan backward edge values io={io} eta={eta}")
        _compare(_gpu(x, io, eta=eta), _ref(x, eta=eta), io)


def test_scan_bwd_deterministic():
    need_gpu()
    x = _inputs(2, 200, 3, 128, "bf16", seed=57)
    a, b = _gpu(x, "bf16"), _gpu(x, "bf16")
    for n in ("dk", "dbeta", "dr", "dd0"):
        assert np.array_equal(a[n], b[n]), n


def test_scan_bwd_full_size_whole_tensor():
    """The B8 H16 T8192 d128 bf16 scan with forgetting at full size; every (b, h)
    slice of 8192 tokens against the oracle (host processes in parallel): each
    gradient's whole-tensor relative L2, and that of its worst slice, within the bf16
    tolerance."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    from tests.parallel_oracle import assert_whole, whole_scan_backward
    wl = Workload("scan_bwd_full", B=8, T=8192, H=16, d_k=128, d_v=128, io="bf16", gate="scalar", s0_std=0.0, seed=3)
    say("full-size scan backward: generating inputs")
    x = precond_inputs(wl)
    rng = np.random.default_rng(99)
    dkw = round_to_io(rng.standard_normal(x["k"].shape), "bf16")
    dd_T = rng.standard_normal((wl.B, wl.H, wl.d_k)).astype(np.float32)
    say("  running GPU")
    g = gdr.precond_scan_bwd(dev(x["k"], "bf16"), dev(x["beta"], "bf16"), ETA, dev(x["r"], "bf16"),
                             torch.from_numpy(x["d0"]).cuda(), dev(dkw, "bf16"), torch.from_numpy(dd_T).cuda())
    torch.cuda.synchronize()
    del x
    grads = {n: g[n].float().cpu().numpy() for n in ("dk", "dbeta", "dr", "dd0")}
    for n, a in grads.items():
        assert np.isfinite(a).all(), n
    del g
    say("  oracle on every (b, h) slice")
    assert_whole("scan backward B8 H16 T8192 d128 bf16", whole_scan_backward(wl, ETA, dkw, dd_T, grads), TOL["bf16"])


@pytest.mark.parametrize("gate", ["none", "scalar"])
def test_two_phase_training_gradient(gate):
    """Both phases through torch autograd: kw, d_T = precond_attn(k, beta, eta, r, d0),
    then o, S_T = chunk_attn(q, k, v, beta, log_a, S0, kw=kw); the .grad of every
    input against the oracle's chain rule (the chunk backward with the write key, its
    dkw through the scan backward; k and beta collect both phases' terms)."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    say(f"case two-phase training gradient gate={gate}")
    B, T, H, dk = 2, 150, 2, 128
    wl = Workload("two_phase", B=B, T=T, H=H, d_k=dk, d_v=dk, io="bf16", gate=gate, s0_std=0.5, seed=61)
    from workloads import chunk_inputs
    x = chunk_inputs(wl)
    x.update(grad_inputs(wl))
    x.update(precond_inputs(wl))          # the same k and beta, plus r and d0
    leaf = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda().requires_grad_(True)
    ins = {n: leaf(x[n], torch.bfloat16) for n in ("q", "k", "v", "beta", "r")}
    ins["log_a"] = leaf(x["log_a"], torch.bfloat16) if gate == "scalar" else None
    S0, d0 = leaf(x["S0"], torch.float32), leaf(x["d0"], torch.float32)
    kw, d_T = gdr.precond_attn(ins["k"], ins["beta"], ETA, ins["r"], d0)
    o, S_T = gdr.chunk_attn(ins["q"], ins["k"], ins["v"], ins["beta"], ins["log_a"], S0, kw=kw)
    loss = (o.float() * torch.from_numpy(x["dO"]).cuda()).sum() + (S_T * torch.from_numpy(x["dS_T"]).cuda()).sum()
    loss.backward()
    torch.cuda.synchronize()
    # the oracle's chain rule; the write key the forward used is the GPU scan's bf16 output
    kw_h = host(kw.detach())
    g2 = oracle_backward(x["q"], x["k"], x["v"], x["beta"], x["log_a"], x["S0"], x["dO"], x["dS_T"], kw=kw_h)
    g1 = precond_scan_backward(x["k"], x["beta"], ETA, x["r"], x["d0"], g2["dkw"], None)
    ref = dict(dq=g2["dq"], dk=g2["dk"] + g1["dk"], dv=g2["dv"], dbeta=g2["dbeta"] + g1["dbeta"], dr=g1["dr"],
               dd0=g1["dd0"], dS0=g2["dS0"], dlog_a=g2["dlog_a"])
    for n, t in (("dq", ins["q"]), ("dk", ins["k"]), ("dv", ins["v"]), ("dbeta", ins["beta"]), ("dr", ins["r"]),
                 ("dd0", d0), ("dS0", S0), ("dlog_a", ins["log_a"])):
        if t is None:
            continue
        check(n, host(t.grad), ref[n], TOL["bf16"])
