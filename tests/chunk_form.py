"""fp64 chunkwise form of the recurrence, written from the chunk equations.

Not the oracle: this is the blueprint the GPU kernel follows (its derivation is
checked here against the token-by-token oracle), and a source of per-chunk
intermediates for stage-level debugging.

Source: "Moonshot AI's New Attention Architecture: Key Innovations Explained",
§3 Hardware-Friendly Algorithm (chunk state recurrence with the block decay,
the position-to-chunk-end decay and the correction terms W, U; the output as a
state read plus a causally masked intra-chunk product).  Readings taken where
the printed formulas are garbled: the query is scaled by the decay from the
chunk start to its own position (exp(g_r)), the key in the score by exp(-g_j),
and a write at position j is decayed by a_{j+1..C} (factor exp(g_C - g_j), g
inclusive).

Per chunk of c rows (state S entering the chunk, key-major d_k x d_v):
    g      inclusive running sum of log_a inside the chunk          [c, d_k]
    Kr     K * exp(g)      (read key; exp(g - log_a) for the literal ordering)
    Kb     K * exp(-g)
    A      strict_lower(diag(beta) Kr Kb^T)                          [c, c]
    T      (I + A)^-1
    W      T diag(beta) Kr ;  U = T diag(beta) V
    Delta  U - W S
    O      (Q * exp(g)) S + lower_incl((Q * exp(g)) Kb^T) Delta
    S'     diag(exp(g_c)) S + (K * exp(g_c - g))^T Delta

With a write key kw ("OSDN: Improving Delta Rule with Provable Online
Preconditioning in Linear Attention", §2.1: the write side of the step uses
k~ = d * k, the read side k), the key in the Gram matrix's columns, in the
scores and in the state write becomes kw: Kb = KW * exp(-g) and
S' = diag(exp(g_c)) S + (KW * exp(g_c - g))^T Delta, while Kr (the rows of the
Gram matrix and the read of S) stays K.
"""

import numpy as np


def chunk_forward(q, k, v, beta, log_a, S0, C, form="page", keep=False, kw=None):
    q, k, v, beta = (np.asarray(x, np.float64) for x in (q, k, v, beta))
    kw = k if kw is None else np.asarray(kw, np.float64)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S_out = np.zeros((B, H, dk, dv))
    inter = []
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], np.float64)
            for c0 in range(0, T, C):
                c1 = min(T, c0 + C)
                c = c1 - c0
                K, Q, V, be = k[b, c0:c1, h], q[b, c0:c1, h], v[b, c0:c1, h], beta[b, c0:c1, h]
                KW = kw[b, c0:c1, h]
                if log_a is None:
                    L = np.zeros((c, dk))
                elif np.ndim(log_a) == 3:
                    L = np.repeat(np.asarray(log_a[b, c0:c1, h], np.float64)[:, None], dk, axis=1)
                else:
                    L = np.asarray(log_a[b, c0:c1, h], np.float64)
                g = np.cumsum(L, axis=0)
                g_read = g if form == "page" else g - L
                Kr = K * np.exp(g_read)
                Kb = KW * np.exp(-g)
                A = np.tril(be[:, None] * (Kr @ Kb.T), -1)
                Tm = np.linalg.inv(np.eye(c) + A)
                W = Tm @ (be[:, None] * Kr)
                U = Tm @ (be[:, None] * V)
                D = U - W @ S
                Qh = Q * np.exp(g)
                P = np.tril(Qh @ Kb.T)
                o[b, c0:c1, h] = Qh @ S + P @ D
                if keep and b == 0 and h == 0:
                    inter.append(dict(g=g, A=A, T=Tm, W=W, U=U, Delta=D, P=P, S_in=S.copy()))
                S = np.exp(g[-1])[:, None] * S + (KW * np.exp(g[-1] - g)).T @ D
            S_out[b, h] = S
    return (o, S_out, inter) if keep else (o, S_out)



def chunk_backward(q, k, v, beta, log_a, S0, do, dS_T, C, form="page", kw=None):
    """Gradients of L = <do, o> + <dS_T, S_T> through the chunk form above, in fp64.

    The reverse mode of the per-chunk equations (the blueprint the GPU backward
    follows; checked against the token-by-token reverse mode of the oracle in
    tests/test_chunk_form.py).  Per chunk, with Kr = K e^{g_read}, Kb = KW e^{-g},
    Qh = Q e^{g}, Kd = KW e^{g_c - g}, S the state entering the chunk and dS' the
    gradient of the state leaving it:
        dDelta = P^T dO + Kd dS',     dY = T^T dDelta     (the gradient of diag(beta) X)
        dS     = e^{g_c} dS' + Qh^T dO - Kr^T diag(beta) dY
        dv     = diag(beta) dY,  dA = -strict_lower(dY Delta^T),  dP = lower_incl(dO Delta^T)
        dKr    = diag(beta) dA Kb - diag(beta) dY S^T,   dKb = (diag(beta) dA)^T Kr + dP^T Qh
        dQh    = dO S^T + dP Kb,   dKd = Delta dS'^T
        dk     = e^{g_read} dKr,   dkw = e^{-g} dKb + e^{g_c - g} dKd,   dq = e^{g} dQh
        dbeta  = rowsum(dY * X) + rowsum(dA * Kr Kb^T)
        dg     = Qh * dQh - Kb * dKb - Kd * dKd  (+ Kr * dKr on row r, or on row r - 1
                 in the literal form, where g_read_r = g_{r-1}),  dg_c += sum_r Kd * dKd
                 + e^{g_c} * (dS' * S) summed over d_v,
    the products * summed over d_k for a scalar gate and kept per channel for the
    per-channel gate; d log a_s = sum over r >= s of dg_r inside the chunk.
    Returns dq, dk, dv, dbeta, dlog_a (None without a gate), dS0 and dkw (None
    without a write key; then dk holds both sides).
    """
    q, k, v, beta, do = (np.asarray(x, np.float64) for x in (q, k, v, beta, do))
    kw_given = kw is not None
    kw = k if kw is None else np.asarray(kw, np.float64)
    B, T, H, dk_ = k.shape
    dv_ = v.shape[-1]
    dq, dk, dkw, dv, dbeta = (np.zeros_like(x) for x in (q, k, k, v, beta))
    gate = None if log_a is None else ("scalar" if np.ndim(log_a) == 3 else "channel")
    dla = None if log_a is None else np.zeros(np.shape(log_a))
    dS0 = np.zeros((B, H, dk_, dv_))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk_, dv_)) if S0 is None else np.array(S0[b, h], np.float64)
            saved = []
            for c0 in range(0, T, C):                 # forward, keeping each chunk's state
                c1 = min(T, c0 + C)
                if log_a is None:
                    L = np.zeros((c1 - c0, dk_))
                elif gate == "scalar":
                    L = np.repeat(np.asarray(log_a[b, c0:c1, h], np.float64)[:, None], dk_, axis=1)
                else:
                    L = np.asarray(log_a[b, c0:c1, h], np.float64)
                g = np.cumsum(L, axis=0)
                g_read = g if form == "page" else g - L
                K, Q, V, KW = k[b, c0:c1, h], q[b, c0:c1, h], v[b, c0:c1, h], kw[b, c0:c1, h]
                be = beta[b, c0:c1, h]
                Kr, Kb, Qh, Kd = K * np.exp(g_read), KW * np.exp(-g), Q * np.exp(g), KW * np.exp(g[-1] - g)
                A = np.tril(be[:, None] * (Kr @ Kb.T), -1)
                Tm = np.linalg.inv(np.eye(c1 - c0) + A)
                X = V - Kr @ S
                D = Tm @ (be[:, None] * X)
                P = np.tril(Qh @ Kb.T)
                saved.append((c0, c1, g, g_read, S.copy(), Kr, Kb, Qh, Kd, Tm, X, D, P, be))
                S = np.exp(g[-1])[:, None] * S + Kd.T @ D
            G = np.zeros((dk_, dv_)) if dS_T is None else np.array(dS_T[b, h], np.float64)
            for c0, c1, g, g_read, S, Kr, Kb, Qh, Kd, Tm, X, D, P, be in reversed(saved):
                dO = do[b, c0:c1, h]
                dD = P.T @ dO + Kd @ G
                dY = Tm.T @ dD
                dA = -np.tril(dY @ D.T, -1)
                dP = np.tril(dO @ D.T)
                dKr = be[:, None] * (dA @ Kb) - be[:, None] * (dY @ S.T)
                dKb = (be[:, None] * dA).T @ Kr + dP.T @ Qh
                dQh = dO @ S.T + dP @ Kb
                dKd = D @ G.T
                dq[b, c0:c1, h] = dQh * np.exp(g)
                dk[b, c0:c1, h] = dKr * np.exp(g_read)
                dkw[b, c0:c1, h] = dKb * np.exp(-g) + dKd * np.exp(g[-1] - g)
                dv[b, c0:c1, h] = be[:, None] * dY
                dbeta[b, c0:c1, h] = np.sum(dY * X, axis=1) + np.sum(dA * (Kr @ Kb.T), axis=1)
                if dla is not None:
                    dg = Qh * dQh - Kb * dKb - Kd * dKd          # [c, d_k]: per channel
                    dgr = Kr * dKr
                    if form == "page":
                        dg = dg + dgr
                    else:
                        dg[:-1] += dgr[1:]                      # g_read_r = g_{r-1}; row 0 reads 0
                    dg[-1] += np.sum(Kd * dKd, axis=0) + np.exp(g[-1]) * np.sum(G * S, axis=1)
                    suffix = np.cumsum(dg[::-1], axis=0)[::-1]
                    dla[b, c0:c1, h] = suffix.sum(axis=1) if gate == "scalar" else suffix
                G = np.exp(g[-1])[:, None] * G + Qh.T @ dO - Kr.T @ (be[:, None] * dY)
            dS0[b, h] = G
    if not kw_given:
        dk, dkw = dk + dkw, None
    return dict(dq=dq, dk=dk, dv=dv, dbeta=dbeta, dlog_a=dla, dS0=dS0, dkw=dkw)
