"""Range of the per-channel gate's factor split, emulated in fp32 on the CPU.

With a gate per key channel the decay between rows r >= j of a chunk,
e^{g_r - g_j} (g the running sum of log a, "Moonshot AI's New Attention
Architecture", §3 with the log-domain gate of §5), sits inside the d_k
contraction of the Gram and score blocks.  The GPU transform splits it at the
first row of each 16-row block: e^{g_r - g_16R} (<= 1) on the row operand and
e^{g_16R - g_j} (>= 1) on the column operand.  These tests emulate that split
in float32 to show where it breaks (the column factor overflows, and inf times
the vanished row factor is NaN), and check the range the library keeps it in:
a chunk in which a channel decays by more than e^-64 inside a block goes to a
generic kernel that takes each decay as one exponential.
"""

import numpy as np

SPLIT_MAX = 64.0            # the library's bound on either factor's exponent


def split_product(g, r, j, R):
    """e^{g_r - g_j} through the 16-row split, in float32 (as the transform forms it)."""
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        row = np.exp(np.float32(g[r] - g[16 * R]), dtype=np.float32)
        col = np.exp(np.float32(g[16 * R] - g[j]), dtype=np.float32)
        return np.float32(row * col)


def needs_generic(log_a_chunk):
    """The transform's test for one channel: some in-block decay (or, literal form,
    the row before a block) beyond e^-SPLIT_MAX."""
    g = np.cumsum(log_a_chunk.astype(np.float64))
    gz = np.concatenate([[0.0], g])
    for R in range(4):
        if g[16 * R] - g[16 * R:16 * R + 16].min() > SPLIT_MAX:
            return True
        if gz[16 * R] - g[16 * R] > SPLIT_MAX:
            return True
    return False


def test_split_overflows_past_fp32_range():
    """log a = -6 over 15 tokens of a block: the column factor is e^90 > fp32 max."""
    la = np.full(64, -0.1)
    la[16:32] = -6.0
    g = np.cumsum(la)
    v = split_product(g, 31, 31, 1)            # the diagonal pair (31, 31): true value 1
    assert not np.isfinite(v)
    with np.errstate(over="ignore"):
        assert np.isinf(np.exp(np.float32(g[16] - g[31]), dtype=np.float32))
    assert needs_generic(la)


def test_split_exact_within_range():
    """Inside the bound both factors are finite and their product is the decay to
    fp32 rounding, for every causal pair of every block."""
    rng = np.random.default_rng(0)
    for per_token in (-0.7, -2.0, -64.0 / 15.0):
        la = per_token * rng.uniform(0.5, 1.0, 64)
        la[16:31] = per_token                   # 15 tokens at the rate: span 15 |rate| <= 64
        g = np.cumsum(la)
        assert not needs_generic(la)
        for R in range(4):
            for r in range(16 * R, 16 * R + 16):
                for j in range(16 * R, r + 1):
                    want = np.exp(g[r] - g[j])
                    got = float(split_product(g, r, j, R))
                    assert np.isfinite(got)
                    assert abs(got - want) <= 4e-6 * max(want, 1e-30) + 1e-37


def test_detector_catches_literal_first_row():
    """Literal form: a block's first row reads e^{g_{16R-1} - g_16R}; one token of
    log a = -70 there is past the bound."""
    la = np.full(64, -0.05)
    la[32] = -70.0
    assert needs_generic(la)


def test_workload_gates_stay_far_inside():
    """The per-channel workload draws log a = -softplus(N(0, 1)); over 2e5 blocks of
    16 tokens the largest in-block decay stays far below the bound."""
    rng = np.random.default_rng(1)
    z = rng.standard_normal((200_000, 16))
    la = -(np.maximum(z, 0) + np.log1p(np.exp(-np.abs(z))))
    span = -la[:, 1:].sum(axis=1)              # g_16R - g_{16R+15}
    assert span.max() < 40.0 < SPLIT_MAX
