"""fp64 oracle of the preconditioner scan of the preconditioned delta rule.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The GPU library never
calls it and shares no code with it.

Source: "OSDN: Improving Delta Rule with Provable Online Preconditioning in
Linear Attention" (web page), Technical Summary:
  §2.1  the right-preconditioned step writes along k~_t = d_t * k_t;
  §2.2  d_t is learned by online gradient descent on the surrogate
            h_t(d) = ((1 - beta_t <d, k_t^2>)^2 - 1) / (2 ||k_t||^2),
        which depends on k_t and beta_t only (phase 1: a scan over the keys
        producing the k~_t; phase 2: the delta rule with k~ as the write key);
  §2.3  adaptive preconditioner forgetting (APF): a per-token, per-head
        retention r_t applied to the preconditioner only.

What is computed, for each (batch, head) independently, token by token:

    kw_t    = d_t * k_t                               write key of token t
    grad_t  = -beta_t (1 - beta_t <d_t, k_t^2>) k_t^2 / ||k_t||^2     (the gradient of h_t at d_t)
    d_{t+1} = r_t d_t - eta grad_t                    (r_t = 1 without APF)

Readings where the page is open or garbled (listed with the evidence in the
design notes):
  * the write key of token t uses the preconditioner before token t's update
    (phase 1 produces k~_t and then updates d_t);
  * the step is a descent step, d - eta grad; the page prints "+ eta grad" in
    the APF update, which would ascend the surrogate;
  * the bar over d in the APF update is not specified (no projection is taken);
  * d starts at d_0 (ones unless given) and eta is a scalar hyper-parameter.
  * A zero key (||k_t|| = 0) leaves d unchanged (the surrogate is not defined).

Parity status: pinned (the surrogate's gradient against finite differences of
the page's closed form, descent on h, special cases, the Newton fixed point);
the scan's reverse mode (precond_scan_backward) against central finite
differences of precond_scan, its eta = 0 closed form and linearity in the
incoming gradients.
"""

from __future__ import annotations

import numpy as np

__all__ = ["surrogate", "surrogate_grad", "precond_scan", "precond_scan_backward"]


def surrogate(d, k, beta):
    """h(d) = ((1 - beta <d, k^2>)^2 - 1) / (2 ||k||^2)   [OSDN §2.2], over [..., d_k]."""
    d, k, beta = (np.asarray(x, dtype=np.float64) for x in (d, k, beta))
    x = np.sum(d * k * k, axis=-1)
    return ((1.0 - beta * x) ** 2 - 1.0) / (2.0 * np.sum(k * k, axis=-1))


def surrogate_grad(d, k, beta):
    """Gradient of h in d: -beta (1 - beta <d, k^2>) k^2 / ||k||^2 (zero for a zero key)."""
    d, k, beta = (np.asarray(x, dtype=np.float64) for x in (d, k, beta))
    k2 = k * k
    n2 = np.sum(k2, axis=-1)
    x = np.sum(d * k2, axis=-1)
    scale = np.where(n2 > 0, -beta * (1.0 - beta * x) / np.where(n2 > 0, n2, 1.0), 0.0)
    return scale[..., None] * k2


def precond_scan(k, beta, eta, r=None, d0=None):
    """Phase 1 over whole sequences.

    k [B, T, H, d_k]; beta [B, T, H]; eta scalar; r None (no forgetting) or
    [B, T, H]; d0 None (ones) or [B, H, d_k].
    Returns (kw [B, T, H, d_k], d_T [B, H, d_k]) in float64.
    """
    k = np.asarray(k, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, dk = k.shape
    d = np.ones((B, H, dk)) if d0 is None else np.array(d0, dtype=np.float64, copy=True)
    kw = np.zeros_like(k)
    for t in range(T):
        kw[:, t] = d * k[:, t]
        g = surrogate_grad(d, k[:, t], beta[:, t])
        rt = 1.0 if r is None else np.asarray(r[:, t], dtype=np.float64)[..., None]
        d = rt * d - eta * g
    return kw, d


def precond_scan_backward(k, beta, eta, r=None, d0=None, dkw=None, dd_T=None):
    """Reverse mode of precond_scan: the gradients of L = <dkw, kw> + <dd_T, d_T>.

    The pages print no gradients (the preconditioned rule is trained, "OSDN", §2.2
    and §4); these are the derivatives of the scan above taken token by token in
    reverse.  With w_t = k_t^2, n_t = ||k_t||^2, x_t = <d_t, w_t> and
    c_t = eta beta_t (1 - beta_t x_t) / n_t (so d_{t+1} = r_t d_t + c_t w_t), and D the
    gradient of d carried from the end (D_T = dd_T):

        u_t      = <D_{t+1}, w_t>
        dr_t     = <D_{t+1}, d_t>
        dbeta_t  = u_t eta (1 - 2 beta_t x_t) / n_t
        dw_t     = c_t D_{t+1} - u_t (eta beta_t^2 / n_t) d_t - u_t c_t / n_t
        dk_t     = dkw_t * d_t + 2 k_t * dw_t
        D_t      = r_t D_{t+1} - u_t (eta beta_t^2 / n_t) w_t + dkw_t * k_t

    and dd0 = D_0.  A zero key adds nothing through c_t (its gradient is dkw_t * d_t).
    Shapes as precond_scan; dkw None (zeros) or [B, T, H, d_k], dd_T None (zeros) or
    [B, H, d_k].  Returns a dict of float64 arrays: dk, dbeta, dr (None when r is
    None), dd0.
    """
    k = np.asarray(k, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, dk = k.shape
    d = np.ones((B, H, dk)) if d0 is None else np.array(d0, dtype=np.float64, copy=True)
    ds = np.zeros((T, B, H, dk))
    for t in range(T):                         # the forward, keeping d before every token
        ds[t] = d
        g = surrogate_grad(d, k[:, t], beta[:, t])
        rt = 1.0 if r is None else np.asarray(r[:, t], dtype=np.float64)[..., None]
        d = rt * d - eta * g
    dkw = np.zeros_like(k) if dkw is None else np.asarray(dkw, dtype=np.float64)
    D = np.zeros((B, H, dk)) if dd_T is None else np.array(dd_T, dtype=np.float64, copy=True)
    g_k = np.zeros_like(k)
    g_beta = np.zeros_like(beta)
    g_r = None if r is None else np.zeros(np.shape(r))
    for t in range(T - 1, -1, -1):
        dt, kt, bt = ds[t], k[:, t], beta[:, t]
        w = kt * kt
        n = np.sum(w, axis=-1)
        nz = n > 0
        n1 = np.where(nz, n, 1.0)
        x = np.sum(dt * w, axis=-1)
        c = np.where(nz, eta * bt * (1.0 - bt * x) / n1, 0.0)
        u = np.sum(D * w, axis=-1)
        rho = np.where(nz, eta * bt * bt / n1, 0.0)
        rt = 1.0 if r is None else np.asarray(r[:, t], dtype=np.float64)[..., None]
        if g_r is not None:
            g_r[:, t] = np.sum(D * dt, axis=-1)
        g_beta[:, t] = np.where(nz, u * eta * (1.0 - 2.0 * bt * x) / n1, 0.0)
        dw = c[..., None] * D - (u * rho)[..., None] * dt - np.where(nz, u * c / n1, 0.0)[..., None]
        g_k[:, t] = dkw[:, t] * dt + 2.0 * kt * dw
        D = rt * D - (u * rho)[..., None] * w + dkw[:, t] * kt
    return dict(dk=g_k, dbeta=g_beta, dr=g_r, dd0=D)
