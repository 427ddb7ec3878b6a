"""gdr_chunk_fwd_noalloc (scratch in the library's static device array) against
gdr_chunk_fwd (caller workspace), through the C ABI: the same kernels, so the same
bits; two calls in a row, the second smaller, each also within the bf16 tolerance
of the oracle.  A forward whose records exceed the static array is refused."""

import numpy as np
import pytest

from tests.gpu_util import TOL, check, dev, host, need_gpu, oracle_chunk, say
from workloads import CONFIGS, Workload, chunk_inputs

pytestmark = pytest.mark.gpu


def _pair(inp, io="bf16", form="page"):
    import torch
    import gated_delta_rule_21_amd as gdr
    args = [dev(inp[n], io) for n in ("q", "k", "v", "beta", "log_a")]
    S0 = torch.from_numpy(inp["S0"]).cuda()
    o_n, S_n = gdr.chunk_fwd_noalloc(*args, S0, form=form)
    o_w, S_w = gdr.chunk_fwd(*args, S0, form=form)
    torch.cuda.synchronize()
    return host(o_n), host(S_n), host(o_w), host(S_w)


def test_noalloc_two_calls_second_smaller():
    need_gpu()
    cases = [Workload("na1", B=2, T=300, H=3, d_k=128, d_v=128, io="bf16", gate="channel", s0_std=0.02, seed=201),
             Workload("na2", B=1, T=70, H=2, d_k=64, d_v=128, io="bf16", gate="scalar", s0_std=0.02, seed=202)]
    for wl in cases:
        say(f"case {wl}")
        inp = chunk_inputs(wl)
        o_n, S_n, o_w, S_w = _pair(inp)
        assert np.array_equal(o_n, o_w) and np.array_equal(S_n, S_w), "no-alloc result differs from gdr_chunk_fwd"
        o_ref, S_ref = oracle_chunk(inp)
        check("o (no-alloc)", o_n, o_ref, TOL["bf16"])
        check("S_T (no-alloc)", S_n, S_ref, TOL["bf16"])


def test_noalloc_headline_workload():
    """B8 H16 T8192 d128 with a scalar gate: 16384 records, 193 MB of the static array."""
    need_gpu()
    wl = CONFIGS[3]
    say(f"case {wl.name}")
    inp = chunk_inputs(wl)
    o_n, S_n, o_w, S_w = _pair(inp)
    assert np.array_equal(o_n, o_w) and np.array_equal(S_n, S_w)


def test_noalloc_refuses_more_than_the_static_array():
    need_gpu()
    import torch
    import gated_delta_rule_21_amd as gdr
    from gated_delta_rule_21_amd._lib import GDR_ERR_WORKSPACE
    B, T, H = 1, 64 * 4406, 1                     # 4406 per-channel records of 60928 B > 256 MiB
    x = torch.zeros((B, T, H, 128), dtype=torch.bfloat16, device="cuda")
    beta = torch.zeros((B, T, H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdr.GdrError) as e:
        gdr.chunk_fwd_noalloc(x, x, x, beta, x)
    assert e.value.status == GDR_ERR_WORKSPACE and "static scratch" in str(e.value)
