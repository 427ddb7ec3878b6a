"""Pins for the preconditioner-scan oracle (CPU only), and planted mistakes that
each must fail at least one pin.

Source: "OSDN: Improving Delta Rule with Provable Online Preconditioning in
Linear Attention", §2.2 (the surrogate h_t and its closed form; phase 1 scans the
keys, producing k~_t = d_t * k_t and updating d_t by online gradient descent on
h_t), §2.3 (APF: a retention r_t on the preconditioner), §3 (gated Newton
condition beta <d, k^2> = 1).
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import forward, precond_scan, surrogate, surrogate_grad


def _keys(seed, B=2, T=7, H=3, dk=5):
    rng = np.random.default_rng([77, seed])
    k = rng.standard_normal((B, T, H, dk))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    r = rng.uniform(0.5, 1.0, (B, T, H))
    d0 = rng.uniform(0.3, 1.5, (B, H, dk))
    return k, beta, r, d0


def _h_page(d, k, beta):
    """The page's closed form, typed independently of the oracle module."""
    x = (d * k * k).sum(-1)
    return ((1 - beta * x) ** 2 - 1) / (2 * (k * k).sum(-1))


# P-p  the gradient used by the scan is the derivative of the page's closed form
def pin_p_gradient_matches_closed_form(scan, grad):
    k, beta, _, d0 = _keys(1)
    kk, bb = k[:, 0], beta[:, 0]
    g = grad(d0, kk, bb)
    eps = 1e-6
    for i in range(kk.shape[-1]):
        e = np.zeros(kk.shape[-1]); e[i] = eps
        fd = (_h_page(d0 + e, kk, bb) - _h_page(d0 - e, kk, bb)) / (2 * eps)
        assert np.max(np.abs(fd - g[..., i])) < 1e-8, f"gradient component {i}"


# P-q  h is the normalised loss change of one write-key step of the delta rule
#      (its definition in §2.2), whatever the state and the value are
def pin_q_surrogate_is_loss_change(scan, grad):
    rng = np.random.default_rng(5)
    k, beta, _, d0 = _keys(2, T=1)
    S = rng.standard_normal((2, 3, 5, 4))
    v = rng.standard_normal((2, 1, 3, 4))
    q = rng.standard_normal((2, 1, 3, 5))
    _, S1 = forward(q, k, v, beta, None, S, kw=d0[:, None] * k)
    r0 = v[:, 0] - np.einsum("bhkv,bhk->bhv", S, k[:, 0])
    r1 = v[:, 0] - np.einsum("bhkv,bhk->bhv", S1, k[:, 0])
    h = (0.5 * (r1 ** 2).sum(-1) - 0.5 * (r0 ** 2).sum(-1)) / ((r0 ** 2).sum(-1) * (k[:, 0] ** 2).sum(-1))
    assert np.max(np.abs(h - surrogate(d0, k[:, 0], beta[:, 0]))) < 1e-10


# P-r  a small step of the scan lowers the surrogate of that token (descent)
def pin_r_descent(scan, grad):
    k, beta, _, d0 = _keys(3, T=1)
    kw, d1 = scan(k, beta, 1e-3, None, d0)
    g = grad(d0, k[:, 0], beta[:, 0])
    moving = (g ** 2).sum(-1) > 1e-12
    before = _h_page(d0, k[:, 0], beta[:, 0])
    after = _h_page(d1, k[:, 0], beta[:, 0])
    assert np.all(after[moving] < before[moving]), "the step did not lower h"
    assert np.allclose(kw[:, 0], d0 * k[:, 0]), "the write key of token t uses d_t"


# P-s  special cases: eta = 0 keeps d (write keys d0 * k); full forgetting (r = 0)
#      with eta = 0 zeroes d after the first token
def pin_s_special_cases(scan, grad):
    k, beta, r, d0 = _keys(4)
    kw, dT = scan(k, beta, 0.0, None, d0)
    assert np.allclose(dT, d0) and np.allclose(kw, d0[:, None] * k)
    kw0, dT0 = scan(k, beta, 0.0, np.zeros_like(r), d0)
    assert np.allclose(kw0[:, 0], d0 * k[:, 0]) and np.allclose(kw0[:, 1:], 0.0) and np.allclose(dT0, 0.0)


# P-t  the gated Newton condition (§3) beta <d, k^2> = 1 is a fixed point: a
#      repeated key with that beta leaves d unchanged
def pin_t_newton_fixed_point(scan, grad):
    k, _, _, d0 = _keys(5, T=1)
    kk = np.repeat(k, 6, axis=1)
    beta = 1.0 / (d0 * k[:, 0] ** 2).sum(-1)
    b6 = np.repeat(beta[:, None], 6, axis=1)
    _, dT = scan(kk, b6, 0.3, None, d0)
    assert np.allclose(dT, d0, atol=1e-12)


# P-u  exact rational run: d_{t+1} = r_t d_t + eta beta_t (1 - beta_t <d_t, k_t^2>) k_t^2 / ||k_t||^2,
#      kw_t = d_t * k_t (descent on the closed form, written out)
def pin_u_exact_rational(scan, grad):
    rng = np.random.default_rng(9)
    T, dk = 5, 3
    F = lambda a, den=8: Fraction(int(a), den)
    k = [[F(rng.integers(-8, 9)) for _ in range(dk)] for _ in range(T)]
    k = [row if any(row) else [F(1)] + row[1:] for row in k]
    beta = [F(rng.integers(1, 8)) for _ in range(T)]
    r = [F(rng.integers(4, 9)) for _ in range(T)]
    eta = Fraction(1, 4)
    d = [F(rng.integers(4, 12)) for _ in range(dk)]
    d0 = d[:]
    kws = []
    for t in range(T):
        kws.append([d[i] * k[t][i] for i in range(dk)])
        n2 = sum(x * x for x in k[t])
        x = sum(d[i] * k[t][i] ** 2 for i in range(dk))
        d = [r[t] * d[i] + eta * beta[t] * (1 - beta[t] * x) * k[t][i] ** 2 / n2 for i in range(dk)]
    f = lambda a: np.array(a, dtype=np.float64)
    kw, dT = scan(f(k)[None, :, None], f(beta)[None, :, None], float(eta), f(r)[None, :, None], f(d0)[None, None])
    assert np.max(np.abs(kw[0, :, 0] - f(kws))) < 1e-12 * max(1, np.max(np.abs(f(kws))))
    assert np.max(np.abs(dT[0, 0] - f(d))) < 1e-12 * max(1, np.max(np.abs(f(d))))


PRECOND_PINS = [("P-p", pin_p_gradient_matches_closed_form), ("P-q", pin_q_surrogate_is_loss_change),
                ("P-r", pin_r_descent), ("P-s", pin_s_special_cases), ("P-t", pin_t_newton_fixed_point),
                ("P-u", pin_u_exact_rational)]


@pytest.mark.parametrize("name,pin", PRECOND_PINS, ids=[n for n, _ in PRECOND_PINS])
def test_precond_pin(name, pin):
    pin(precond_scan, surrogate_grad)


def _mutant(mutation):
    def grad(d, k, beta):
        k2 = k * k
        n2 = k2.sum(-1)
        x = (d * k2).sum(-1)
        if mutation == "no_norm":
            n2 = np.ones_like(n2)
        if mutation == "beta_once":
            return (-beta * (1 - x) / n2)[..., None] * k2
        return (-beta * (1 - beta * x) / n2)[..., None] * k2

    def scan(k, beta, eta, r=None, d0=None):
        B, T, H, dk = k.shape
        d = np.ones((B, H, dk)) if d0 is None else np.array(d0, float)
        kw = np.zeros_like(k)
        for t in range(T):
            g = grad(d, k[:, t], beta[:, t])
            rt = 1.0 if r is None else r[:, t][..., None]
            d_new = (rt * d + eta * g) if mutation == "ascent" else (rt * (d - eta * g) if mutation == "retain_step" else rt * d - eta * g)
            kw[:, t] = (d_new if mutation == "updated_key" else d) * k[:, t]
            d = d_new
        return kw, d
    return scan, grad


@pytest.mark.parametrize("mutation", ["ascent", "updated_key", "no_norm", "beta_once", "retain_step"])
def test_precond_mutant_is_caught(mutation):
    scan, grad = _mutant(mutation)
    caught = []
    for name, pin in PRECOND_PINS:
        try:
            pin(scan, grad)
        except AssertionError:
            caught.append(name)
    assert caught, f"mutation {mutation!r} passed every pin"


def test_unmutated_precond_copy_passes():
    scan, grad = _mutant("none")
    for name, pin in PRECOND_PINS:
        pin(scan, grad)
