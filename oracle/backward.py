"""fp64 oracle of the gradients of the delta-rule recurrence (reverse mode).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The GPU library never
calls it and shares no code with it.

The pages print no gradients; they are the reverse-mode derivatives of the
recurrence the forward oracle follows ("Moonshot AI's New Attention
Architecture", §2: the (gated) delta-rule update; "OSDN: Improving Delta Rule
with Provable Online Preconditioning in Linear Attention", §1: the delta rule
as one online gradient step; §2.1: the write key).  Per (batch, head), token t,
with X the state the erase reads (S~ in the page form, S_{t-1} in the literal
form) and kw the write key (k unless given):

    S~ = D_t S_{t-1},  u = X^T k_t,  delta = beta_t (v_t - u),
    S_t = S~ + kw_t delta^T,  o_t = S_t^T q_t.

For a scalar loss with dL/do_t = do_t and dL/dS_T = dS_T, going from t = T down
to 1 with G the gradient of S_t (dS_T, then the carried gradient):

    G       += q_t do_t^T
    dq_t     = S_t do_t
    d delta  = G^T kw_t;     dkw_t = G delta
    dv_t     = beta_t d delta;   dbeta_t = <d delta, v_t - u>;   du = -beta_t d delta
    dk_t    += X du          (plus dkw_t when the write key is k itself)
    dS~      = G (+ k_t du^T in the page form)
    dS_{t-1} = D_t dS~ (+ k_t du^T in the literal form)
    dlog_a_t = sum over the state of dS~ * S~   (per key channel: over d_v only)

and dS_0 is the gradient carried past token 1.

Parity status: pinned by central finite differences of the forward oracle (an
independent code path) for every input, gate, form and the write key; by the
closed form of the beta = 0 case; and by linearity in (dO, dS_T).
"""

from __future__ import annotations

import numpy as np

from .recurrence import gate_kind

__all__ = ["backward"]


def backward(q, k, v, beta, log_a=None, S0=None, do=None, dS_T=None, *, form="page", kw=None):
    """Gradients of L = sum(do * o) + sum(dS_T * S_T) for the forward oracle's run.

    Layouts as the forward oracle: q, k [B, T, H, d_k]; v, do [B, T, H, d_v];
    beta [B, T, H]; log_a None, [B, T, H] or [B, T, H, d_k]; S0, dS_T None
    (zeros) or [B, H, d_k, d_v]; kw None or [B, T, H, d_k].
    Returns a dict of float64 arrays: dq, dk, dv, dbeta, dlog_a (None without a
    gate), dS0, and dkw (None unless kw is given; then dk excludes the write side).
    """
    if form not in ("page", "literal"):
        raise ValueError(f"unknown form {form!r}")
    f64 = lambda x: None if x is None else np.asarray(x, dtype=np.float64)
    q, k, v, beta, log_a, kw = f64(q), f64(k), f64(v), f64(beta), f64(log_a), f64(kw)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    kind = gate_kind(beta, log_a, k)
    do = np.zeros((B, T, H, dv)) if do is None else f64(do)
    kwr = k if kw is None else kw

    # Forward, keeping every state before its token.
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    S_prev = np.zeros((T, B, H, dk, dv))
    for t in range(T):
        S_prev[t] = S
        Sd = _decay(S, log_a, kind, t)
        X = Sd if form == "page" else S
        u = np.einsum("bhkv,bhk->bhv", X, k[:, t])
        delta = beta[:, t, :, None] * (v[:, t] - u)
        S = Sd + kwr[:, t, :, :, None] * delta[:, :, None, :]

    dq = np.zeros_like(q)
    dkk = np.zeros_like(k)
    dkw = np.zeros_like(k)
    dvv = np.zeros_like(v)
    dbeta = np.zeros_like(beta)
    dlog_a = None if kind == "none" else np.zeros_like(log_a)
    G = np.zeros((B, H, dk, dv)) if dS_T is None else np.array(dS_T, dtype=np.float64, copy=True)
    for t in range(T - 1, -1, -1):
        Sp = S_prev[t]
        Sd = _decay(Sp, log_a, kind, t)
        X = Sd if form == "page" else Sp
        u = np.einsum("bhkv,bhk->bhv", X, k[:, t])
        delta = beta[:, t, :, None] * (v[:, t] - u)
        St = Sd + kwr[:, t, :, :, None] * delta[:, :, None, :]

        G = G + q[:, t, :, :, None] * do[:, t, :, None, :]
        dq[:, t] = np.einsum("bhkv,bhv->bhk", St, do[:, t])
        ddelta = np.einsum("bhkv,bhk->bhv", G, kwr[:, t])
        dkw[:, t] = np.einsum("bhkv,bhv->bhk", G, delta)
        dvv[:, t] = beta[:, t, :, None] * ddelta
        dbeta[:, t] = np.sum(ddelta * (v[:, t] - u), axis=-1)
        du = -beta[:, t, :, None] * ddelta
        dkk[:, t] = np.einsum("bhkv,bhv->bhk", X, du)
        dX = k[:, t, :, :, None] * du[:, :, None, :]
        dSd = G + (dX if form == "page" else 0.0)
        if kind == "scalar":
            dlog_a[:, t] = np.sum(dSd * Sd, axis=(-2, -1))
        elif kind == "channel":
            dlog_a[:, t] = np.sum(dSd * Sd, axis=-1)
        G = _decay(dSd, log_a, kind, t) + (dX if form == "literal" else 0.0)

    if kw is None:
        dkk = dkk + dkw
        dkw_out = None
    else:
        dkw_out = dkw
    return dict(dq=dq, dk=dkk, dv=dvv, dbeta=dbeta, dlog_a=dlog_a, dS0=G, dkw=dkw_out)


def _decay(S, log_a, kind, t):
    """D_t S: rows of S (key channels) scaled by exp(log_a_t)."""
    if kind == "none":
        return S
    a = np.exp(log_a[:, t])
    if kind == "scalar":
        return a[:, :, None, None] * S
    return a[:, :, :, None] * S
