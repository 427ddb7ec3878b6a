"""Pins for the reverse mode of the preconditioner-scan oracle (CPU only), and
planted mistakes that each must fail at least one pin.

The scan is phase 1 of the preconditioned delta rule ("OSDN: Improving Delta Rule
with Provable Online Preconditioning in Linear Attention", §2.2 with the
retention of §2.3); the method is trained (§2.2, §4), and the pages print no
gradients.  The pins check oracle.precond_scan_backward against what it does not
share: central finite differences of oracle.precond_scan, the closed form of the
eta = 0 case (the preconditioner then only decays), and linearity in the incoming
gradients.
"""

import numpy as np
import pytest

from oracle import precond_scan
from oracle.preconditioner import precond_scan_backward


def _inputs(seed, B=2, T=9, H=2, dk=5, forget=True):
    rng = np.random.default_rng([131, seed])
    x = dict(k=rng.standard_normal((B, T, H, dk)), beta=rng.uniform(0.1, 0.9, (B, T, H)),
             r=rng.uniform(0.5, 1.0, (B, T, H)) if forget else None, d0=rng.uniform(0.3, 1.5, (B, H, dk)),
             dkw=rng.standard_normal((B, T, H, dk)), dd_T=rng.standard_normal((B, H, dk)))
    return x


def _loss(x, eta):
    kw, dT = precond_scan(x["k"], x["beta"], eta, x["r"], x["d0"])
    return float(np.sum(x["dkw"] * kw) + np.sum(x["dd_T"] * dT))


# P-y  every gradient agrees with central finite differences of the scan oracle's
#      loss <dkw, kw> + <dd_T, d_T> along random directions
def pin_y_finite_differences(bwd):
    for seed, eta, forget in ((1, 0.7, True), (2, 2.0, True), (3, 0.5, False)):
        x = _inputs(seed, forget=forget)
        g = bwd(x["k"], x["beta"], eta, x["r"], x["d0"], x["dkw"], x["dd_T"])
        rng = np.random.default_rng(seed)
        names = [("k", "dk"), ("beta", "dbeta"), ("d0", "dd0")] + ([("r", "dr")] if forget else [])
        eps = 1e-6
        for name, gname in names:
            d = rng.standard_normal(x[name].shape)
            xp, xm = dict(x), dict(x)
            xp[name] = x[name] + eps * d
            xm[name] = x[name] - eps * d
            fd = (_loss(xp, eta) - _loss(xm, eta)) / (2 * eps)
            an = float(np.sum(g[gname] * d))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), f"{gname} (eta {eta}): finite difference {fd} vs {an}"
        if not forget:
            assert g["dr"] is None


# P-z  eta = 0: d_t = P_t d0 with P_t the product of the retentions before token t,
#      so the loss is sum_t P_t <dkw_t * k_t, d0> + P_T <dd_T, d0>; written out here
#      in closed form, independently of the reverse loop
def pin_z_no_step(bwd):
    x = _inputs(4)
    k, r, d0, dkw, ddT = x["k"], x["r"], x["d0"], x["dkw"], x["dd_T"]
    B, T, H, dk = k.shape
    P = np.concatenate([np.ones((B, 1, H)), np.cumprod(r, axis=1)], axis=1)     # P_0 .. P_T
    g = bwd(k, x["beta"], 0.0, r, d0, dkw, ddT)
    dk_ref = dkw * (P[:, :T, :, None] * d0[:, None])
    dd0_ref = np.sum(P[:, :T, :, None] * dkw * k, axis=1) + P[:, T, :, None] * ddT
    a = np.sum(dkw * k * d0[:, None], axis=-1)                                      # <dkw_t * k_t, d0>
    aT = np.sum(ddT * d0, axis=-1)
    dr_ref = np.zeros_like(r)
    for j in range(T):
        dr_ref[:, j] = (np.sum(P[:, j + 1:T] * a[:, j + 1:T], axis=1) + P[:, T] * aT) / r[:, j]
    assert np.allclose(g["dk"], dk_ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dd0"], dd0_ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dr"], dr_ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dbeta"], 0.0, atol=1e-15)


# P-aa  linear in the incoming gradients (dkw, dd_T)
def pin_aa_linearity(bwd):
    x = _inputs(5)
    y = _inputs(6)
    a, b = 0.7, -1.3
    g1 = bwd(x["k"], x["beta"], 1.0, x["r"], x["d0"], x["dkw"], x["dd_T"])
    g2 = bwd(x["k"], x["beta"], 1.0, x["r"], x["d0"], y["dkw"], y["dd_T"])
    g3 = bwd(x["k"], x["beta"], 1.0, x["r"], x["d0"], a * x["dkw"] + b * y["dkw"], a * x["dd_T"] + b * y["dd_T"])
    for n in ("dk", "dbeta", "dr", "dd0"):
        assert np.allclose(g3[n], a * g1[n] + b * g2[n], rtol=1e-10, atol=1e-12), n


BWD_PINS = [("P-y", pin_y_finite_differences), ("P-z", pin_z_no_step), ("P-aa", pin_aa_linearity)]


@pytest.mark.parametrize("name,pin", BWD_PINS, ids=[n for n, _ in BWD_PINS])
def test_precond_backward_pin(name, pin):
    pin(precond_scan_backward)


def test_zero_key_passes_only_the_write_key_gradient():
    """A token with a zero key leaves d unchanged (the surrogate is undefined there):
    its gradient is dkw_t * d_t, and it passes nothing to beta."""
    x = _inputs(8)
    x["k"][0, 3, 1] = 0.0
    g = precond_scan_backward(x["k"], x["beta"], 1.0, x["r"], x["d0"], x["dkw"], x["dd_T"])
    kw, _ = precond_scan(x["k"][:, :3], x["beta"][:, :3], 1.0, x["r"][:, :3], x["d0"])
    _, d3 = precond_scan(x["k"][:, :3], x["beta"][:, :3], 1.0, x["r"][:, :3], x["d0"])
    assert np.allclose(g["dk"][0, 3, 1], x["dkw"][0, 3, 1] * d3[0, 1], rtol=1e-12)
    assert g["dbeta"][0, 3, 1] == 0.0


def _mutant(mutation):
    """A copy of the reverse loop with one plausible mistake planted."""
    def bwd(k, beta, eta, r=None, d0=None, dkw=None, dd_T=None):
        B, T, H, dk = k.shape
        d = np.ones((B, H, dk)) if d0 is None else np.array(d0, float)
        ds = []
        for t in range(T):
            ds.append(d)
            w = k[:, t] ** 2
            n = w.sum(-1)
            c = eta * beta[:, t] * (1 - beta[:, t] * (d * w).sum(-1)) / n
            rt = 1.0 if r is None else r[:, t][..., None]
            d = rt * d + c[..., None] * w
        D = np.array(dd_T, float)
        out = dict(dk=np.zeros_like(k), dbeta=np.zeros_like(beta), dr=None if r is None else np.zeros_like(r))
        for t in range(T - 1, -1, -1):
            dt, kt, bt = ds[t], k[:, t], beta[:, t]
            w = kt * kt
            n = w.sum(-1)
            x = (dt * w).sum(-1)
            c = eta * bt * (1 - bt * x) / n
            u = (D * w).sum(-1)
            rho = eta * bt * bt / n
            rt = 1.0 if r is None else r[:, t][..., None]
            if r is not None:
                out["dr"][:, t] = ((rt * D) if mutation == "dr_after_retention" else D).__mul__(dt).sum(-1)
            out["dbeta"][:, t] = u * eta * ((1 - bt * x) if mutation == "dbeta_once" else (1 - 2 * bt * x)) / n
            dw = c[..., None] * D - (u * rho)[..., None] * dt
            if mutation != "no_norm_term":
                dw = dw - (u * c / n)[..., None]
            out["dk"][:, t] = dkw[:, t] * dt + (1.0 if mutation == "dk_factor_one" else 2.0) * kt * dw
            carry = -(u * rho)[..., None] * w
            if mutation == "carry_sign":
                carry = -carry
            D = rt * D + carry + (0.0 if mutation == "no_key_write" else dkw[:, t] * kt)
        out["dd0"] = D
        return out
    return bwd


@pytest.mark.parametrize("mutation", ["dr_after_retention", "dbeta_once", "no_norm_term", "dk_factor_one",
                                      "carry_sign", "no_key_write"])
def test_precond_backward_mutant_is_caught(mutation):
    bwd = _mutant(mutation)
    caught = []
    for name, pin in BWD_PINS:
        try:
            pin(bwd)
        except AssertionError:
            caught.append(name)
    assert caught, f"mutation {mutation!r} passed every pin"


def test_unmutated_precond_backward_copy_passes():
    bwd = _mutant("none")
    for name, pin in BWD_PINS:
        pin(bwd)
