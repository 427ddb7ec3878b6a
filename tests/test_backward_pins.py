"""Pins for the backward oracle (CPU only), and planted mistakes that each must
fail at least one pin.

The gradients are the reverse-mode derivatives of the recurrence of "Moonshot
AI's New Attention Architecture", §2 (decay, erase, write) and of the write-key
step of "OSDN: Improving Delta Rule with Provable Online Preconditioning in
Linear Attention", §2.1.  The pins check them against things the backward code
does not share: central finite differences of the forward oracle, the closed
form of the beta = 0 case, and linearity in the output gradients.
"""

import numpy as np
import pytest

from oracle import backward, forward

GATES = ["none", "scalar", "channel"]


def _inputs(seed, gate, B=2, T=5, H=2, dk=4, dv=3, wkey=False):
    rng = np.random.default_rng([91, seed])
    x = dict(q=rng.standard_normal((B, T, H, dk)), k=rng.standard_normal((B, T, H, dk)) / 2,
             v=rng.standard_normal((B, T, H, dv)), beta=rng.uniform(0.1, 0.9, (B, T, H)),
             S0=rng.standard_normal((B, H, dk, dv)), do=rng.standard_normal((B, T, H, dv)),
             dS_T=rng.standard_normal((B, H, dk, dv)))
    x["log_a"] = {"none": None, "scalar": -rng.uniform(0.05, 1.0, (B, T, H)),
                  "channel": -rng.uniform(0.05, 1.0, (B, T, H, dk))}[gate]
    x["kw"] = rng.uniform(0.3, 1.7, (B, T, H, dk)) * x["k"] if wkey else None
    return x


def _loss(x, form):
    o, S = forward(x["q"], x["k"], x["v"], x["beta"], x["log_a"], x["S0"], form=form, kw=x["kw"])
    return float(np.sum(x["do"] * o) + np.sum(x["dS_T"] * S))


# P-v  every gradient agrees with central finite differences of the forward
#      oracle's loss along random directions (the forward code is not shared)
def pin_v_finite_differences(bwd, gate, form, wkey):
    x = _inputs(7 + GATES.index(gate) + 3 * wkey, gate, wkey=wkey)
    g = bwd(x["q"], x["k"], x["v"], x["beta"], x["log_a"], x["S0"], x["do"], x["dS_T"], form=form, kw=x["kw"])
    rng = np.random.default_rng(5)
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"), ("S0", "dS0")]
    if gate != "none":
        names.append(("log_a", "dlog_a"))
    if wkey:
        names.append(("kw", "dkw"))
    eps = 1e-6
    for name, gname in names:
        d = rng.standard_normal(x[name].shape)
        xp, xm = dict(x), dict(x)
        xp[name] = x[name] + eps * d
        xm[name] = x[name] - eps * d
        fd = (_loss(xp, form) - _loss(xm, form)) / (2 * eps)
        an = float(np.sum(g[gname] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), f"{gname}: finite difference {fd} vs {an}"


# P-w  beta = 0, no gate: every state is S0, so dq_t = S0 do_t, dS0 = dS_T + sum_t
#      q_t do_t^T, dk = dv = 0 and dbeta_t = <G_t^T k_t, v_t - S0^T k_t> with
#      G_t = dS_T + sum_{s >= t} q_s do_s^T
def pin_w_beta_zero(bwd, gate, form, wkey):
    x = _inputs(11, "none")
    x["beta"] = np.zeros_like(x["beta"])
    g = bwd(x["q"], x["k"], x["v"], x["beta"], None, x["S0"], x["do"], x["dS_T"], form=form)
    B, T, H, dk = x["k"].shape
    for b in range(B):
        for h in range(H):
            S0 = x["S0"][b, h]
            G = x["dS_T"][b, h].copy()
            for t in range(T - 1, -1, -1):
                q, k, v, do = x["q"][b, t, h], x["k"][b, t, h], x["v"][b, t, h], x["do"][b, t, h]
                G = G + np.outer(q, do)
                assert np.allclose(g["dq"][b, t, h], S0 @ do, atol=1e-12)
                assert np.allclose(g["dbeta"][b, t, h], (G.T @ k) @ (v - S0.T @ k), atol=1e-12)
            assert np.allclose(g["dS0"][b, h], G, atol=1e-12)
    assert np.max(np.abs(g["dk"])) < 1e-12 and np.max(np.abs(g["dv"])) < 1e-12


# P-x  the gradients are linear in (dO, dS_T)
def pin_x_linear_in_output_gradients(bwd, gate, form, wkey):
    x = _inputs(13, gate, wkey=wkey)
    y = _inputs(17, gate, wkey=wkey)
    run = lambda do, dS: bwd(x["q"], x["k"], x["v"], x["beta"], x["log_a"], x["S0"], do, dS, form=form, kw=x["kw"])
    g1, g2 = run(x["do"], x["dS_T"]), run(y["do"], y["dS_T"])
    g12 = run(2.0 * x["do"] + y["do"], 2.0 * x["dS_T"] + y["dS_T"])
    for n in g1:
        if g1[n] is not None:
            assert np.allclose(g12[n], 2.0 * g1[n] + g2[n], atol=1e-10), n


BACKWARD_PINS = [("P-v", pin_v_finite_differences), ("P-w", pin_w_beta_zero),
                 ("P-x", pin_x_linear_in_output_gradients)]
CASES = [(g, f, w) for g in GATES for f in ("page", "literal") for w in (False, True) if not (w and g != "none")]


@pytest.mark.parametrize("name,pin", BACKWARD_PINS, ids=[n for n, _ in BACKWARD_PINS])
@pytest.mark.parametrize("gate,form,wkey", CASES, ids=[f"{g}-{f}{'-wkey' if w else ''}" for g, f, w in CASES])
def test_backward_pin(name, pin, gate, form, wkey):
    pin(backward, gate, form, wkey)


def _mutant(mutation):
    """The backward oracle with one planted mistake (a copy, on the CPU)."""
    import sys
    import oracle  # noqa: F401  (loads the submodule; the package exports a function of the same name)
    src = open(sys.modules["oracle.backward"].__file__).read()
    edits = {
        "no_erase_grad": ("dSd = G + (dX if form == \"page\" else 0.0)", "dSd = G"),
        "erase_grad_sign": ("du = -beta[:, t, :, None] * ddelta", "du = beta[:, t, :, None] * ddelta"),
        "no_decay_on_carry": ("G = _decay(dSd, log_a, kind, t) + (dX if form == \"literal\" else 0.0)",
                              "G = dSd + (dX if form == \"literal\" else 0.0)"),
        "gate_grad_from_new_state": ("dlog_a[:, t] = np.sum(dSd * Sd, axis=(-2, -1))",
                                     "dlog_a[:, t] = np.sum(dSd * St, axis=(-2, -1))"),
        "dq_from_old_state": ("dq[:, t] = np.einsum(\"bhkv,bhv->bhk\", St, do[:, t])",
                              "dq[:, t] = np.einsum(\"bhkv,bhv->bhk\", Sp, do[:, t])"),
        "dbeta_without_prediction": ("dbeta[:, t] = np.sum(ddelta * (v[:, t] - u), axis=-1)",
                                     "dbeta[:, t] = np.sum(ddelta * v[:, t], axis=-1)"),
    }
    old, new = edits[mutation]
    assert src.count(old) == 1, mutation
    ns = {"__name__": "backward_mutant"}
    exec(compile(src.replace(old, new).replace("from .recurrence import gate_kind",
                                               "from oracle.recurrence import gate_kind"), "mutant", "exec"), ns)
    return ns["backward"]


@pytest.mark.parametrize("mutation", ["no_erase_grad", "erase_grad_sign", "no_decay_on_carry",
                                      "gate_grad_from_new_state", "dq_from_old_state", "dbeta_without_prediction"])
def test_backward_mutant_is_caught(mutation):
    bwd = _mutant(mutation)
    caught = []
    for gate, form, wkey in CASES:
        for name, pin in BACKWARD_PINS:
            try:
                pin(bwd, gate, form, wkey)
            except AssertionError:
                caught.append((name, gate, form))
    assert caught, f"mutation {mutation!r} passed every pin"
