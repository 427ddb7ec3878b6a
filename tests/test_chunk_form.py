"""The chunk equations (as read) reproduce the token-by-token oracle in fp64."""

import numpy as np
import pytest

from oracle import forward
from tests.chunk_form import chunk_forward


def _inputs(seed, B, T, H, dk, dv, gate):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    x = rng.standard_normal((B, T, H) if gate == "scalar" else (B, T, H, dk))
    log_a = None if gate == "none" else -np.logaddexp(0, x)
    S0 = 0.1 * rng.standard_normal((B, H, dk, dv))
    return q, k, v, beta, log_a, S0


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("form", ["page", "literal"])
@pytest.mark.parametrize("C", [1, 2, 8, 16, 64])
def test_chunk_form_equals_oracle(gate, form, C):
    q, k, v, beta, log_a, S0 = _inputs(C, 1, 131, 2, 12, 7, gate)
    o_ref, S_ref = forward(q, k, v, beta, log_a, S0, form=form)
    o, S = chunk_forward(q, k, v, beta, log_a, S0, C, form=form)
    assert np.max(np.abs(o - o_ref)) <= 1e-12 * max(1, np.max(np.abs(o_ref)))
    assert np.max(np.abs(S - S_ref)) <= 1e-12 * max(1, np.max(np.abs(S_ref)))


@pytest.mark.parametrize("C", [1, 8, 64])
def test_write_key_chunk_form_equals_oracle(C):
    """Write keys kw = d * k (OSDN §2.1) with d in (0.2, 2): the chunk equations with kw
    in the Gram columns, the scores and the state write reproduce the oracle."""
    q, k, v, beta, _, S0 = _inputs(100 + C, 1, 131, 2, 12, 7, "none")
    d = np.random.default_rng(C).uniform(0.2, 2.0, k.shape)
    o_ref, S_ref = forward(q, k, v, beta, None, S0, kw=d * k)
    o, S = chunk_forward(q, k, v, beta, None, S0, C, kw=d * k)
    assert np.max(np.abs(o - o_ref)) <= 1e-12 * max(1, np.max(np.abs(o_ref)))
    assert np.max(np.abs(S - S_ref)) <= 1e-12 * max(1, np.max(np.abs(S_ref)))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("form", ["page", "literal"])
@pytest.mark.parametrize("C", [1, 8, 64])
def test_write_key_chunk_form_with_gates(gate, form, C):
    """The write key under a scalar or per-channel gate (the decay first, the residual
    along k, the write along kw): the chunk equations with kw in the Gram columns, the
    scores and the state write reproduce the oracle."""
    q, k, v, beta, log_a, S0 = _inputs(200 + C, 1, 131, 2, 12, 7, gate)
    d = np.random.default_rng(C + 7).uniform(0.2, 2.0, k.shape)
    o_ref, S_ref = forward(q, k, v, beta, log_a, S0, form=form, kw=d * k)
    o, S = chunk_forward(q, k, v, beta, log_a, S0, C, form=form, kw=d * k)
    assert np.max(np.abs(o - o_ref)) <= 1e-12 * max(1, np.max(np.abs(o_ref)))
    assert np.max(np.abs(S - S_ref)) <= 1e-12 * max(1, np.max(np.abs(S_ref)))


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("form", ["page", "literal"])
@pytest.mark.parametrize("wkey", [False, True])
@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunk_backward_equals_oracle(gate, form, wkey, C):
    """The reverse mode of the chunk equations (the decomposition the GPU backward
    follows) reproduces the oracle's token-by-token reverse mode, with and without a
    separate write key, on a ragged T."""
    from oracle import backward
    from tests.chunk_form import chunk_backward
    q, k, v, beta, log_a, S0 = _inputs(300 + C, 1, 131, 2, 12, 7, gate)
    rng = np.random.default_rng(C + 11)
    kw = rng.uniform(0.2, 2.0, k.shape) * k if wkey else None
    do = rng.standard_normal(v.shape)
    dS_T = rng.standard_normal(S0.shape)
    ref = backward(q, k, v, beta, log_a, S0, do, dS_T, form=form, kw=kw)
    got = chunk_backward(q, k, v, beta, log_a, S0, do, dS_T, C, form=form, kw=kw)
    for name in ("dq", "dk", "dv", "dbeta", "dlog_a", "dS0", "dkw"):
        if ref[name] is None:
            assert got[name] is None, name
            continue
        scale = max(1.0, np.max(np.abs(ref[name])))
        assert np.max(np.abs(got[name] - ref[name])) <= 1e-11 * scale, name
