"""GPU parity of gdr_precond_scan (the preconditioner scan that produces the write
keys of the preconditioned delta rule) against the fp64 oracle.

Source: "OSDN: Improving Delta Rule with Provable Online Preconditioning in
Linear Attention", §2.2 (kw_t = d_t * k_t, then one gradient step on the
closed-form surrogate), §2.3 (APF retention r_t on the preconditioner).

Tolerances (relative L2 over the tensor) as for the forward: 2e-2 for bf16 I/O,
1e-4 for fp32 I/O, on the write keys kw and on the final preconditioner d_T.
Inputs: keys and beta of the forward's workloads, retention sigmoid(z + 3),
d0 ~ U(0.5, 1.5), eta = 1 unless a case says otherwise.
"""

import numpy as np
import pytest

from oracle import forward as oracle_forward, precond_scan as oracle_scan, rel_l2
from tests.gpu_util import TOL, check, dev, host, need_gpu, say
from workloads import CONFIGS, PRECOND_ETA, Workload, chunk_inputs, precond_inputs

pytestmark = pytest.mark.gpu


def _inputs(B, T, H, dk, io="bf16", seed=0):
    return precond_inputs(Workload("scan", B=B, T=T, H=H, d_k=dk, d_v=dk, io=io, seed=seed))


def _gpu(inp, io, eta=PRECOND_ETA, apf=True, with_d0=True, in_place=False):
    import torch
    import gated_delta_rule_21_amd as gdr
    d0 = torch.from_numpy(inp["d0"]).cuda() if with_d0 else None
    kw, dT = gdr.precond_scan(dev(inp["k"], io), dev(inp["beta"], io), eta, dev(inp["r"], io) if apf else None, d0,
                              d_T=d0 if in_place else None)
    torch.cuda.synchronize()
    if in_place:
        assert dT.data_ptr() == d0.data_ptr()
    return host(kw), host(dT)


def _ref(inp, eta=PRECOND_ETA, apf=True, with_d0=True):
    return oracle_scan(inp["k"], inp["beta"], eta, inp["r"] if apf else None, inp["d0"] if with_d0 else None)


def _run(inp, io, **kw):
    got = _gpu(inp, io, **kw)
    kw.pop("in_place", None)
    ref = _ref(inp, **kw)
    check("kw", got[0], ref[0], TOL[io])
    check("d_T", got[1], ref[1], TOL[io])
    return got, ref


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("dk", [128, 64])
@pytest.mark.parametrize("apf", [True, False], ids=["apf", "no_apf"])
@pytest.mark.parametrize("shape", [(2, 200, 3), (1, 130, 2)], ids=lambda s: "B%dT%dH%d" % s)
def test_scan_shapes(io, dk, apf, shape):
    need_gpu()
    B, T, H = shape
    say(f"case scan io={io} dk={dk} apf={apf} shape={shape}")
    _run(_inputs(B, T, H, dk, io, seed=T + dk + apf), io, apf=apf)


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 129])
def test_scan_lengths(T):
    need_gpu()
    say(f"case scan T={T}")
    inp = _inputs(2, T, 2, 128, seed=300 + T)
    got, ref = _run(inp, "bf16")
    if T == 0:
        assert np.array_equal(got[1], inp["d0"].astype(np.float64))


def test_scan_default_start_and_in_place():
    need_gpu()
    inp = _inputs(1, 150, 2, 128, seed=7)
    _run(inp, "bf16", with_d0=False)     # d0 = ones
    _run(inp, "bf16", in_place=True)     # d_T written over d0


def test_scan_zero_keys_and_extreme_retention():
    """A zero key adds nothing (the surrogate is undefined there); a retention of
    1 is no forgetting; a retention of 1e-3 forgets almost everything at once."""
    need_gpu()
    inp = _inputs(2, 140, 2, 128, seed=9)
    inp["k"][:, [0, 5, 64, 100]] = 0.0
    inp["r"][0] = 1.0
    inp["r"][1, 30:40] = np.float32(0.00099945068359375)   # bf16-exact
    _run(inp, "bf16")
    _run(inp, "f32")


@pytest.mark.parametrize("eta", [0.25, 8.0])
def test_scan_step_sizes(eta):
    need_gpu()
    inp = _inputs(1, 200, 3, 128, seed=11)
    _run(inp, "bf16", eta=eta)
    _run(inp, "f32", eta=eta)


def test_scan_deterministic():
    need_gpu()
    inp = _inputs(2, 300, 3, 128, seed=13)
    a = _gpu(inp, "bf16")
    b = _gpu(inp, "bf16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_two_phase_preconditioned_forward():
    """Phase 1 (the scan) then phase 2 (the forward with the write keys) on the
    GPU against both phases in the oracle (OSDN §2.2: the two-phase execution)."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    wl = Workload("twophase", B=2, T=300, H=3, d_k=128, d_v=128, io="bf16", gate="none", s0_std=0.02, seed=17)
    inp = chunk_inputs(wl)
    pin = precond_inputs(wl)
    k, beta = dev(inp["k"], "bf16"), dev(inp["beta"], "bf16")
    kw, _ = gdr.precond_scan(k, beta, PRECOND_ETA, dev(pin["r"], "bf16"), torch.from_numpy(pin["d0"]).cuda())
    o, S = gdr.chunk_fwd(dev(inp["q"], "bf16"), k, dev(inp["v"], "bf16"), beta, None,
                         torch.from_numpy(inp["S0"]).cuda(), kw=kw)
    torch.cuda.synchronize()
    kw_ref, _ = oracle_scan(inp["k"], inp["beta"], PRECOND_ETA, pin["r"], pin["d0"])
    o_ref, S_ref = oracle_forward(inp["q"], inp["k"], inp["v"], inp["beta"], None, inp["S0"], kw=kw_ref)
    check("o", host(o), o_ref, TOL["bf16"])
    check("S_T", host(S), S_ref, TOL["bf16"])


def test_full_size_scan_whole_tensor():
    """The scan over the keys of the B8 H16 T8192 d128 bf16 workload, in the
    launch configuration the benchmark times; every (b, h) slice against the oracle
    (host processes in parallel): whole-tensor relative L2 of the write keys and
    the final preconditioner, and that of the worst slice, within the bf16 tolerance."""
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    from tests.parallel_oracle import assert_whole, whole_scan
    wl = CONFIGS[3]
    say(f"full-size scan {wl.name}: generating inputs")
    inp = precond_inputs(wl)
    args = [dev(inp["k"], "bf16"), dev(inp["beta"], "bf16"), PRECOND_ETA, dev(inp["r"], "bf16"),
            torch.from_numpy(inp["d0"]).cuda()]
    del inp
    say("  running GPU")
    kw, dT = gdr.precond_scan(*args)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(kw.float()).all()) and bool(torch.isfinite(dT).all())
    kw_h, dT_h = kw.float().cpu().numpy(), dT.cpu().numpy()
    del kw, dT, args
    say("  oracle on every (b, h) slice")
    assert_whole(f"preconditioner scan {wl.name}", whole_scan(wl, PRECOND_ETA, kw_h, dT_h), TOL["bf16"])


def test_scan_strong_forgetting_within_a_chunk():
    """Twenty tokens of retention 1e-3 inside one chunk (a total log-retention
    near -140, below which the chunkwise kernel forms every decay factor with its
    own exponential instead of factoring it)."""
    need_gpu()
    inp = _inputs(2, 200, 2, 128, seed=19)
    inp["r"][:, 70:90] = np.float32(0.00099945068359375)    # bf16-exact
    inp["r"][1, 140:150] = np.float32(0.00099945068359375)
    _run(inp, "bf16")
    _run(inp, "f32")
