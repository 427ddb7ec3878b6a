"""fp64 token-by-token oracle for the (gated) delta-rule recurrence.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The GPU library never
calls it and shares no code with it.

Sources (web pages; cited by title and section):
  [Moonshot §2]  "Moonshot AI's New Attention Architecture: Key Innovations
                 Explained", section 2 "Core Operator: Fine-Grained Gated Delta
                 Rule" -- the DeltaNet update, its scalar-gated form and its
                 per-channel (diagonal) gated form.
  [OSDN §1]      "OSDN: Improving Delta Rule with Provable Online
                 Preconditioning in Linear Attention", Technical Summary §1
                 "Problem Statement" -- the delta rule as one online gradient
                 step on the per-token regression loss 0.5*||S k - v||^2.
  [OSDN §2.1]    same page, §2.1 "Algebraic Equivalence and Hardware
                 Preservation" -- right-preconditioning that step by
                 diag(d_t) writes along the scaled key k~_t = d_t * k_t while
                 the residual still reads the state along k_t.

What is computed (the plain definition; no chunking, no reordering).  The
state is key-major, S in R^{d_k x d_v}.  For each (batch, head) independently
and each token t = 1..T in order:

    D_t   = diag(exp(log_a_t))          (identity when there is no gate;
                                          exp(log_a_t) * I for a scalar gate)
    S~    = D_t S_{t-1}                 decay first  [Moonshot §2, gated forms]
    delta = beta_t (v_t - S~^T k_t)     residual of the regression step  [OSDN §1]
    S_t   = S~ + k_t delta^T            erase along k_t, then write v_t   [Moonshot §2]
    o_t   = S_t^T q_t                   read-out after token t's own write

Expanded, S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} + beta_t k_t v_t^T, which is
the per-channel gated update of [Moonshot §2] written key-major; with a scalar
gate it is the scalar-gated update there, and with no gate the DeltaNet update.

Readings where the pages are open or disagree (each one is listed, with the
evidence, in the design notes):
  * form="page" (default) puts the decay before the erase, as the two gated
    updates of [Moonshot §2] do.  form="literal" is the other ordering,
    S_t = D_t S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T, where the erase reads
    the undecayed state; the two agree when there is no gate.
  * erase=False drops the erase term: S_t = D_t S_{t-1} + beta_t k_t v_t^T (the
    write-only linear-attention state of [Moonshot §2]).  Used by pins only.
  * No query scaling, no normalisation of q or k inside the operator.
  * kw (optional) is the write key of [OSDN §2.1]: the step becomes
    S_t = S~ + kw_t delta^T with delta still from S~^T k_t, i.e. key-major
    S_t = (I - beta_t kw_t k_t^T) S~ + beta_t kw_t v_t^T.  kw = k is the
    update above.  The pages give it for the ungated delta rule; with a gate the
    decay is applied first as above (a reading, used only if asked for).

Parity status: pinned (see the oracle pin tests): special cases, closed forms,
invariants, an exact-rational brute force of the transition-matrix product,
and a hand-worked example.
"""

from __future__ import annotations

import numpy as np

__all__ = ["gate_kind", "recurrent_step", "forward", "rel_l2"]


def gate_kind(beta: np.ndarray, log_a: np.ndarray | None, k: np.ndarray) -> str:
    """Classify the gate from shapes: 'none', 'scalar' (one value per token and
    head) or 'channel' (one value per token, head and key channel)."""
    if log_a is None:
        return "none"
    if log_a.shape == beta.shape:
        return "scalar"
    if log_a.shape == k.shape:
        return "channel"
    raise ValueError(f"log_a shape {log_a.shape} matches neither beta {beta.shape} nor k {k.shape}")


def recurrent_step(S, q, k, v, beta, log_a=None, *, form="page", erase=True, kw=None):
    """One token of the recurrence for a batch of independent states.

    S: [..., d_k, d_v]; q, k: [..., d_k]; v: [..., d_v]; beta: [...];
    log_a: None, [...] (scalar gate) or [..., d_k] (per key channel);
    kw: None (write along k) or the write key [..., d_k] of [OSDN §2.1].
    Returns (o [..., d_v], S_new [..., d_k, d_v]), all float64.
    """
    if form not in ("page", "literal"):
        raise ValueError(f"unknown form {form!r}")
    S = np.asarray(S, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)

    # Decay D_t applied to the state (rows of S are key channels).
    if log_a is None:
        S_dec = S
    else:
        a = np.exp(np.asarray(log_a, dtype=np.float64))
        if a.shape == beta.shape:            # scalar gate
            S_dec = a[..., None, None] * S
        else:                                # per key channel
            S_dec = a[..., :, None] * S

    if erase:
        # The erase reads the decayed state (page form) or the previous state (literal form).
        S_read = S_dec if form == "page" else S
        pred = np.einsum("...kv,...k->...v", S_read, k)          # S^T k
        delta = beta[..., None] * (v - pred)
    else:
        delta = beta[..., None] * v

    k_write = k if kw is None else np.asarray(kw, dtype=np.float64)
    S_new = S_dec + k_write[..., :, None] * delta[..., None, :]   # + k delta^T (kw delta^T)
    o = np.einsum("...kv,...k->...v", S_new, q)                   # S_t^T q_t
    return o, S_new


def forward(q, k, v, beta, log_a=None, S0=None, *, form="page", erase=True, kw=None):
    """Run the recurrence over a whole sequence.

    Layouts (token-major): q, k [B, T, H, d_k]; v [B, T, H, d_v]; beta [B, T, H];
    log_a None, [B, T, H] or [B, T, H, d_k]; S0 None (zeros) or [B, H, d_k, d_v];
    kw None or the write keys [B, T, H, d_k] ([OSDN §2.1]).
    Returns (o [B, T, H, d_v], S_T [B, H, d_k, d_v]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    if log_a is not None:
        log_a = np.asarray(log_a, dtype=np.float64)
    kind = gate_kind(beta, log_a, k)
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        la = None if kind == "none" else log_a[:, t]
        o[:, t], S = recurrent_step(S, q[:, t], k[:, t], v[:, t], beta[:, t], la,
                                    form=form, erase=erase, kw=None if kw is None else kw[:, t])
    return o, S


def rel_l2(x, ref) -> float:
    """Relative L2 error ||x - ref||_2 / ||ref||_2 over the whole array, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return float(num)
    return float(num / den)
