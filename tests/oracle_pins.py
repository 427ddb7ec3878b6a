"""Pins for the fp64 oracle: facts the pages and plain mathematics fix, independent
of the oracle's own code.

Each pin takes a `fwd` callable with the oracle's `forward` signature,
    fwd(q, k, v, beta, log_a=None, S0=None, *, form="page", erase=True) -> (o, S_T),
and raises AssertionError when the callable disagrees with the pinned fact.
They run against the real oracle (all must pass) and against deliberately
broken copies of it (each copy must fail at least one pin).

Sources:
  [Moonshot §2]  "Moonshot AI's New Attention Architecture: Key Innovations
                 Explained", §2 Core Operator (linear attention, DeltaNet,
                 scalar-gated and per-channel gated updates; erase-then-write).
  [OSDN §1]      "OSDN: Improving Delta Rule with Provable Online
                 Preconditioning in Linear Attention", Technical Summary §1
                 (delta rule = one gradient step on 0.5*||S k - v||^2).
  [OSDN §3]      same page, §3 Theoretical Guarantees (gated Newton condition
                 beta * <d, k^2> = 1; with d = 1 it reads beta * ||k||^2 = 1).
  [OSDN §2.1-2.2] same page: the right-preconditioned step writes along
                 k~ = d * k (§2.1), and its surrogate
                 h = (f(S_t) - f(S_{t-1})) / ||grad f(S_{t-1})||^2 has the closed
                 form ((1 - beta <d, k^2>)^2 - 1) / (2 ||k||^2) (§2.2).

The write-key pins (WKEY_PINS) take fwd(..., kw=...) with kw the write keys.
"""

from __future__ import annotations

from fractions import Fraction
import math

import numpy as np

RNG_SEED = 1234


def _rng(tag: int) -> np.random.Generator:
    return np.random.default_rng([RNG_SEED, tag])


def _rand_inputs(rng, B=2, T=9, H=2, dk=4, dv=3, gate="none", unit_keys=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    if gate == "none":
        log_a = None
    elif gate == "scalar":
        log_a = -rng.uniform(0.01, 0.7, (B, T, H))
    else:
        log_a = -rng.uniform(0.01, 0.7, (B, T, H, dk))
    S0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, beta, log_a, S0


def _close(x, y, tol=1e-11, what=""):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    err = np.max(np.abs(x - y)) / max(1.0, np.max(np.abs(y)))
    assert err <= tol, f"{what}: scaled max error {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# P-a  beta = 0 and no decay: nothing is written or erased, the state stays S0.
#      [Moonshot §2] DeltaNet update with beta_t = 0.
def pin_a_beta_zero_keeps_state(fwd):
    for gate in ("none", "scalar", "channel"):
        q, k, v, beta, log_a, S0 = _rand_inputs(_rng(1), gate=gate)
        beta = np.zeros_like(beta)
        if log_a is not None:
            log_a = np.zeros_like(log_a)           # a_t = 1
        o, S_T = fwd(q, k, v, beta, log_a, S0)
        _close(S_T, S0, what=f"S_T vs S0 ({gate})")
        _close(o, np.einsum("bhkv,bthk->bthv", S0, q), what=f"o vs S0^T q ({gate})")


# P-b  beta_t ||k_t||^2 = 1 makes the step an exact solve of the regression
#      problem: S_t^T k_t = v_t for every t, with any gate, in the page form.
#      [OSDN §1] one exact gradient step on 0.5*||S k - v||^2; [OSDN §3] gated
#      Newton condition with d = 1; [Moonshot §2] erase-then-write on the decayed
#      state.  The other ordering (erase reads the undecayed state) must NOT have
#      this property once a gate is present, which pins the form switch.
def pin_b_exact_recall_under_newton_step(fwd):
    for gate in ("none", "scalar", "channel"):
        q, k, v, beta, log_a, S0 = _rand_inputs(_rng(2), gate=gate, unit_keys=False, dk=5, dv=3)
        beta = 1.0 / np.sum(k * k, axis=-1)
        o, _ = fwd(k, k, v, beta, log_a, S0)          # query = key reads S_t^T k_t
        _close(o, v, tol=1e-10, what=f"S_t^T k_t vs v_t ({gate})")
        if gate != "none":
            o_lit, _ = fwd(k, k, v, beta, log_a, S0, form="literal")
            dev = np.max(np.abs(o_lit - v))
            assert dev > 1e-3, f"literal form unexpectedly recalls exactly ({gate}, dev {dev:.2e})"


# P-c  Orthonormal keys, beta = 1, S0 = 0: each stored value is retrieved exactly
#      (no gate), or scaled by the product of later decays (scalar gate).
#      [Moonshot §2] DeltaNet and scalar-gated updates.
def pin_c_orthonormal_keys_retrieve_values(fwd):
    rng = _rng(3)
    B, H, dk, dv, T = 1, 2, 6, 4, 5
    for gate in ("none", "scalar"):
        k = np.empty((B, T, H, dk))
        for h in range(H):
            Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
            k[0, :, h] = Qm[:T]
        q = rng.standard_normal((B, T, H, dk))
        v = rng.standard_normal((B, T, H, dv))
        beta = np.ones((B, T, H))
        log_a = None if gate == "none" else -rng.uniform(0.05, 0.6, (B, T, H))
        _, S_T = fwd(q, k, v, beta, log_a, np.zeros((B, H, dk, dv)))
        for h in range(H):
            for j in range(T):
                got = S_T[0, h].T @ k[0, j, h]
                scale = 1.0 if gate == "none" else math.exp(float(np.sum(log_a[0, j + 1:, h])))
                _close(got, scale * v[0, j, h], what=f"retrieval j={j} ({gate})")


# P-d  Without the erase term the recurrence is (gated) causal linear attention:
#      o_r = sum_{j<=r} beta_j <q_r * exp(G_r - G_j), k_j> v_j + (q_r * exp(G_r))^T S0,
#      with G the inclusive running sum of log_a from the first token: a write at
#      j is decayed by a_{j+1..r}.  Without a gate this is tril(Q K^T) diag(beta) V
#      + Q S0, a plain masked matrix product.  [Moonshot §2] write-only linear
#      attention and its gated extension.
def pin_d_no_erase_is_linear_attention(fwd):
    for gate in ("none", "scalar", "channel"):
        q, k, v, beta, log_a, S0 = _rand_inputs(_rng(4), gate=gate, T=7, dk=4, dv=5)
        o, S_T = fwd(q, k, v, beta, log_a, S0, erase=False)
        B, T, H, dk = k.shape
        for b in range(B):
            for h in range(H):
                Q, K, V, be = q[b, :, h], k[b, :, h], v[b, :, h], beta[b, :, h]
                if gate == "none":
                    ref = np.tril(Q @ K.T) @ (be[:, None] * V) + Q @ S0[b, h]
                else:
                    la = log_a[b, :, h]
                    G = np.cumsum(la if gate == "channel" else la[:, None] * np.ones((T, dk)), axis=0)
                    ref = np.zeros((T, v.shape[-1]))
                    for r in range(T):
                        ref[r] = (Q[r] * np.exp(G[r])) @ S0[b, h]
                        for j in range(r + 1):
                            ref[r] += be[j] * np.dot(Q[r] * np.exp(G[r] - G[j]), K[j]) * V[j]
                _close(o[b, :, h], ref, what=f"linear-attention closed form ({gate})")


# P-e  beta = 0 with a gate: the state only decays, S_t = diag(exp(G_t)) S0 and
#      o_t = (exp(G_t) * q_t)^T S0, G inclusive running sum of log_a.
#      [Moonshot §2] gated updates with beta = 0 (pins that token t's own gate
#      applies at step t and that a per-channel gate acts on key channels).
def pin_e_pure_decay(fwd):
    for gate, dk, dv in (("scalar", 4, 6), ("channel", 4, 6), ("channel", 5, 5)):
        q, k, v, beta, log_a, S0 = _rand_inputs(_rng(5), gate=gate, dk=dk, dv=dv)
        beta = np.zeros_like(beta)
        o, S_T = fwd(q, k, v, beta, log_a, S0)
        G = np.cumsum(log_a, axis=1)
        if gate == "scalar":
            G = G[..., None] * np.ones(k.shape[-1])
        ref_o = np.einsum("bthk,bhkv->bthv", q * np.exp(G), S0)
        ref_S = np.exp(G[:, -1])[..., None] * S0
        _close(o, ref_o, what=f"decayed read-out ({gate})")
        _close(S_T, ref_S, what=f"decayed state ({gate})")


# P-f  Exact brute force: with rational inputs, multiply out the transition
#      matrices M_t = (I - beta_t k_t k_t^T) diag(a_t) as explicit d_k x d_k
#      matrices in exact rational arithmetic,
#        S_t = M_t S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t.
#      [Moonshot §2] per-channel gated update in matrix form.
def _frac_matmul(A, B):
    return [[sum((A[i][l] * B[l][j] for l in range(len(B))), Fraction(0)) for j in range(len(B[0]))]
            for i in range(len(A))]


def _exact_run(q, k, v, beta, a, S0):
    dk, dv = len(k[0]), len(v[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(len(k)):
        M = [[(Fraction(1) if i == j else Fraction(0)) - beta[t] * k[t][i] * k[t][j]
              for j in range(dk)] for i in range(dk)]
        M = [[M[i][j] * a[t][j] for j in range(dk)] for i in range(dk)]     # (I - b k k^T) diag(a)
        S = _frac_matmul(M, S)
        S = [[S[i][j] + beta[t] * k[t][i] * v[t][j] for j in range(dv)] for i in range(dk)]
        outs.append([sum((S[i][j] * q[t][i] for i in range(dk)), Fraction(0)) for j in range(dv)])
    return outs, S


def pin_f_exact_rational_brute_force(fwd):
    rng = _rng(6)
    dk, dv, T = 3, 2, 6

    def rat(lo, hi, den=8):
        return Fraction(int(rng.integers(lo * den, hi * den + 1)), den)

    for gate in ("none", "scalar", "channel"):
        q = [[rat(-2, 2) for _ in range(dk)] for _ in range(T)]
        k = [[rat(-1, 1) for _ in range(dk)] for _ in range(T)]
        v = [[rat(-2, 2) for _ in range(dv)] for _ in range(T)]
        beta = [Fraction(int(rng.integers(1, 8)), 8) for _ in range(T)]
        if gate == "none":
            a = [[Fraction(1)] * dk for _ in range(T)]
        elif gate == "scalar":
            a = [[Fraction(int(rng.integers(2, 8)), 8)] * dk for _ in range(T)]
        else:
            a = [[Fraction(int(rng.integers(2, 8)), 8) for _ in range(dk)] for _ in range(T)]
        S0 = [[rat(-1, 1) for _ in range(dv)] for _ in range(dk)]
        outs, S_T = _exact_run(q, k, v, beta, a, S0)

        f = lambda x: np.array(x, dtype=np.float64)
        qa, ka, va = f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None]
        ba = f(beta)[None, :, None]
        if gate == "none":
            la = None
        elif gate == "scalar":
            la = np.log(f([row[0] for row in a]))[None, :, None]
        else:
            la = np.log(f(a))[None, :, None]
        o, S = fwd(qa, ka, va, ba, la, f(S0)[None, None])
        _close(o[0, :, 0], f(outs), tol=1e-12, what=f"exact o ({gate})")
        _close(S[0, 0], f(S_T), tol=1e-12, what=f"exact S_T ({gate})")


# P-g  The map (V, S0) -> (O, S_T) is linear for fixed q, k, beta, a.
#      [Moonshot §2] every update is affine in (S, v) with coefficients set by k, beta, a.
def pin_g_linearity(fwd):
    for gate in ("none", "channel"):
        rng = _rng(7)
        q, k, v1, beta, log_a, S01 = _rand_inputs(rng, gate=gate)
        v2 = rng.standard_normal(v1.shape)
        S02 = rng.standard_normal(S01.shape)
        al = 0.37
        o1, s1 = fwd(q, k, v1, beta, log_a, S01)
        o2, s2 = fwd(q, k, v2, beta, log_a, S02)
        o3, s3 = fwd(q, k, al * v1 + v2, beta, log_a, al * S01 + S02)
        _close(o3, al * o1 + o2, what=f"linearity o ({gate})")
        _close(s3, al * s1 + s2, what=f"linearity S ({gate})")


# P-i  A sequence can be split: running the first T1 tokens and then the rest
#      from the state reached gives the same result as one run.  [Moonshot §1]
#      constant-size state carried from one call to the next.
def pin_i_split_sequence(fwd):
    for gate in ("scalar", "channel"):
        q, k, v, beta, log_a, S0 = _rand_inputs(_rng(8), gate=gate, T=11)
        o, S = fwd(q, k, v, beta, log_a, S0)
        T1 = 4
        la1 = None if log_a is None else log_a[:, :T1]
        la2 = None if log_a is None else log_a[:, T1:]
        oa, Sa = fwd(q[:, :T1], k[:, :T1], v[:, :T1], beta[:, :T1], la1, S0)
        ob, Sb = fwd(q[:, T1:], k[:, T1:], v[:, T1:], beta[:, T1:], la2, Sa)
        _close(np.concatenate([oa, ob], axis=1), o, what=f"split o ({gate})")
        _close(Sb, S, what=f"split S ({gate})")


# P-j  A per-channel gate whose channels are equal is the scalar gate, and a zero
#      log-gate is no gate.  [Moonshot §2] the diagonal gate generalises the scalar one.
def pin_j_gate_special_cases(fwd):
    q, k, v, beta, log_a, S0 = _rand_inputs(_rng(9), gate="scalar")
    o_s, S_s = fwd(q, k, v, beta, log_a, S0)
    o_c, S_c = fwd(q, k, v, beta, np.repeat(log_a[..., None], k.shape[-1], axis=-1), S0)
    _close(o_c, o_s, what="channel==scalar o")
    _close(S_c, S_s, what="channel==scalar S")
    o_n, S_n = fwd(q, k, v, beta, None, S0)
    o_z, S_z = fwd(q, k, v, beta, np.zeros_like(log_a), S0)
    _close(o_z, o_n, what="zero gate o")
    _close(S_z, S_n, what="zero gate S")


# P-l  DeltaNet with unit keys and beta in [0, 1]: I - beta k k^T has spectral
#      norm <= 1, so ||S_T||_F <= ||S0||_F + sum_t beta_t ||v_t||.  [Moonshot §2]
def pin_l_norm_bound(fwd):
    q, k, v, beta, _, S0 = _rand_inputs(_rng(10), T=40, dk=3, dv=3)
    v = 5.0 * v
    _, S_T = fwd(q, k, v, beta, None, S0)
    for b in range(S_T.shape[0]):
        for h in range(S_T.shape[1]):
            lhs = np.linalg.norm(S_T[b, h])
            rhs = np.linalg.norm(S0[b, h]) + np.sum(beta[b, :, h] * np.linalg.norm(v[b, :, h], axis=-1))
            assert lhs <= rhs * (1 + 1e-12), f"norm bound violated {lhs} > {rhs}"
    # and the bound is not vacuous: the erase actually removes old content
    q2, k2, v2, beta2, _, S02 = _rand_inputs(_rng(11), T=40, dk=3, dv=3)
    beta2 = np.ones_like(beta2)
    v2 = np.zeros_like(v2)
    _, S_T2 = fwd(q2, k2, v2, beta2, None, S02)
    assert np.linalg.norm(S_T2) < 0.5 * np.linalg.norm(S02), "erase with v = 0 did not shrink the state"


# ---------------------------------------------------------------------------
# Write-key pins ([OSDN §2.1, §2.2]).
# P-m  One step with write key kw = d * k scales the regression residual
#      v - S^T k by exactly (1 - beta <d, k^2>), and the surrogate
#      h = (f(S_t) - f(S_{t-1})) / ||grad f(S_{t-1})||_F^2, f(S) = 0.5 ||S^T k - v||^2,
#      equals the page's closed form ((1 - beta <d, k^2>)^2 - 1) / (2 ||k||^2)
#      whatever S and v are.  [OSDN §2.2]
def pin_m_write_key_surrogate_closed_form(fwd):
    rng = _rng(31)
    for _ in range(4):
        q, k, v, beta, _, S0 = _rand_inputs(rng, B=2, T=1, H=3, dk=5, dv=4, unit_keys=False)
        d = rng.uniform(0.2, 2.0, k.shape)
        _, S1 = fwd(q, k, v, beta, None, S0, kw=d * k)
        kk, vv, bb, dd = k[:, 0], v[:, 0], beta[:, 0], d[:, 0]
        r0 = vv - np.einsum("bhkv,bhk->bhv", S0, kk)
        r1 = vv - np.einsum("bhkv,bhk->bhv", S1, kk)
        c = 1.0 - bb * np.sum(dd * kk * kk, axis=-1)
        _close(r1, c[..., None] * r0, tol=1e-12, what="write-key residual factor")
        f0, f1 = 0.5 * np.sum(r0 ** 2, -1), 0.5 * np.sum(r1 ** 2, -1)
        grad2 = np.sum(r0 ** 2, -1) * np.sum(kk ** 2, -1)          # ||(S^T k - v) k^T||_F^2
        _close((f1 - f0) / grad2, (c ** 2 - 1.0) / (2.0 * np.sum(kk ** 2, -1)), tol=1e-10,
               what="surrogate h closed form")


# P-n  d = 1 (write key = key) is the plain delta rule, and a write key that is
#      zero writes nothing: the state stays S0 and the outputs read S0.  [OSDN §2.1]
def pin_n_write_key_special_cases(fwd):
    q, k, v, beta, _, S0 = _rand_inputs(_rng(32))
    o, S = fwd(q, k, v, beta, None, S0)
    o1, S1 = fwd(q, k, v, beta, None, S0, kw=k.copy())
    _close(o1, o, what="kw = k: o")
    _close(S1, S, what="kw = k: S")
    o0, S0b = fwd(q, k, v, beta, None, S0, kw=np.zeros_like(k))
    _close(S0b, S0, what="kw = 0: S")
    _close(o0, np.einsum("bhkv,bthk->bthv", S0, q), what="kw = 0: o = S0^T q")


# P-o  Exact rational brute force of the write-key recurrence in matrix form,
#        S_t = (I - beta_t kw_t k_t^T) S_{t-1} + beta_t kw_t v_t^T,   o_t = S_t^T q_t,
#      the key-major transpose of [OSDN §2.1]'s S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) kw_t^T.
def pin_o_write_key_exact_rational(fwd):
    rng = _rng(33)
    dk, dv, T = 3, 2, 6

    def rat(lo, hi, den=8):
        return Fraction(int(rng.integers(lo * den, hi * den + 1)), den)

    q = [[rat(-2, 2) for _ in range(dk)] for _ in range(T)]
    k = [[rat(-1, 1) for _ in range(dk)] for _ in range(T)]
    kw = [[rat(-1, 1) for _ in range(dk)] for _ in range(T)]
    v = [[rat(-2, 2) for _ in range(dv)] for _ in range(T)]
    beta = [Fraction(int(rng.integers(1, 8)), 8) for _ in range(T)]
    S = [[rat(-1, 1) for _ in range(dv)] for _ in range(dk)]
    S0 = [row[:] for row in S]
    outs = []
    for t in range(T):
        M = [[(Fraction(1) if i == j else Fraction(0)) - beta[t] * kw[t][i] * k[t][j] for j in range(dk)]
             for i in range(dk)]
        S = _frac_matmul(M, S)
        S = [[S[i][j] + beta[t] * kw[t][i] * v[t][j] for j in range(dv)] for i in range(dk)]
        outs.append([sum((S[i][j] * q[t][i] for i in range(dk)), Fraction(0)) for j in range(dv)])
    f = lambda x: np.array(x, dtype=np.float64)
    o, S_T = fwd(f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None], f(beta)[None, :, None], None,
                 f(S0)[None, None], kw=f(kw)[None, :, None])
    _close(o[0, :, 0], f(outs), tol=1e-12, what="write-key exact o")
    _close(S_T[0, 0], f(S), tol=1e-12, what="write-key exact S_T")


WKEY_PINS = [
    ("P-m", pin_m_write_key_surrogate_closed_form),
    ("P-n", pin_n_write_key_special_cases),
    ("P-o", pin_o_write_key_exact_rational),
]


PINS = [
    ("P-a", pin_a_beta_zero_keeps_state),
    ("P-b", pin_b_exact_recall_under_newton_step),
    ("P-c", pin_c_orthonormal_keys_retrieve_values),
    ("P-d", pin_d_no_erase_is_linear_attention),
    ("P-e", pin_e_pure_decay),
    ("P-f", pin_f_exact_rational_brute_force),
    ("P-g", pin_g_linearity),
    ("P-i", pin_i_split_sequence),
    ("P-j", pin_j_gate_special_cases),
    ("P-l", pin_l_norm_bound),
]
