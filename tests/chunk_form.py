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
