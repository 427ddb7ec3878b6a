"""Each plausible mistake planted in a copy of the oracle must fail at least one pin.

The mutants re-implement the recurrence step with one deliberate error each;
the real oracle is untouched.  This shows the pins constrain every term.
"""

import numpy as np
import pytest

from tests.oracle_pins import PINS


def _make_forward(mutation):
    def step(S, q, k, v, beta, log_a, form, erase):
        if log_a is None:
            a = None
        else:
            a = np.exp(log_a) if mutation != "gate_linearised" else 1.0 + log_a
            if mutation == "gate_on_values" and a.shape != beta.shape:
                a_mat = a[..., None, :]                        # scales value columns
            elif a.shape == beta.shape:
                a_mat = a[..., None, None]
            else:
                a_mat = a[..., :, None]
        S_dec = S if a is None else (S if mutation == "decay_after_write" else a_mat * S)
        if form == "literal" or mutation == "literal_default":
            S_read = S
        else:
            S_read = S_dec
        if mutation == "transposed_read":
            pred = np.einsum("...kv,...v->...k", S_read, k)
        else:
            pred = np.einsum("...kv,...k->...v", S_read, k)
        if not erase or mutation == "no_erase":
            delta = beta[..., None] * v
        elif mutation == "erase_sign":
            delta = beta[..., None] * (v + pred)
        elif mutation == "beta_write_only":
            delta = beta[..., None] * v - pred
        elif mutation == "beta_squared":
            delta = beta[..., None] ** 2 * (v - pred)
        else:
            delta = beta[..., None] * (v - pred)
        S_new = S_dec + k[..., :, None] * delta[..., None, :]
        if mutation == "decay_after_write" and a is not None:
            S_new = a_mat * (S + k[..., :, None] * delta[..., None, :])
        if mutation == "read_before_write":
            o = np.einsum("...kv,...k->...v", S_dec, q)
        elif mutation == "transposed_output":
            o = np.einsum("...kv,...v->...k", S_new, q)
        else:
            o = np.einsum("...kv,...k->...v", S_new, q)
        return o, S_new

    def forward(q, k, v, beta, log_a=None, S0=None, *, form="page", erase=True):
        B, T, H, dk = k.shape
        dv = v.shape[-1]
        S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, float)
        if mutation == "ignore_S0":
            S = np.zeros((B, H, dk, dv))
        o = np.zeros((B, T, H, dv))
        for t in range(T):
            if log_a is None:
                la = None
            elif mutation == "gate_off_by_one":
                la = log_a[:, t - 1] if t > 0 else np.zeros_like(log_a[:, 0])
            else:
                la = log_a[:, t]
            o_t, S = step(S, q[:, t], k[:, t], v[:, t], beta[:, t], la, form, erase)
            if mutation == "transposed_output":
                o[:, t] = o_t[..., :dv] if o_t.shape[-1] >= dv else np.pad(o_t, [(0, 0)] * (o_t.ndim - 1) + [(0, dv - o_t.shape[-1])])
            else:
                o[:, t] = o_t
        return o, S

    return forward


MUTATIONS = ["no_erase", "erase_sign", "transposed_read", "beta_write_only", "beta_squared",
             "decay_after_write", "read_before_write", "transposed_output", "ignore_S0",
             "gate_off_by_one", "gate_linearised", "gate_on_values", "literal_default"]


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_mutant_is_caught(mutation):
    fwd = _make_forward(mutation)
    caught = []
    for name, pin in PINS:
        try:
            pin(fwd)
        except (AssertionError, ValueError, IndexError, np.linalg.LinAlgError):
            caught.append(name)
    assert caught, f"mutation {mutation!r} passed every pin"


def test_unmutated_copy_passes_every_pin():
    fwd = _make_forward("none")
    for name, pin in PINS:
        pin(fwd)


# ---- the write key of the preconditioned step ---------------------------------------------
def _make_wkey_forward(mutation):
    """A copy of the (ungated) write-key recurrence with one deliberate error."""
    def forward(q, k, v, beta, log_a=None, S0=None, *, form="page", erase=True, kw=None):
        assert log_a is None
        B, T, H, dk = k.shape
        dv = v.shape[-1]
        kw = k if kw is None else kw
        S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, float)
        o = np.zeros((B, T, H, dv))
        for t in range(T):
            kr, kwr = k[:, t], kw[:, t]
            if mutation == "erase_reads_write_key":
                kr = kwr
            elif mutation == "keys_swapped":
                kr, kwr = kwr, kr
            elif mutation == "write_along_key":
                kwr = kr
            pred = np.einsum("...kv,...k->...v", S, kr)
            b = beta[:, t][..., None]
            delta = (v[:, t] - pred) if mutation == "no_beta" else b * (v[:, t] - pred)
            S_new = S + kwr[..., :, None] * delta[..., None, :]
            if mutation == "write_key_squared":
                S_new = S + (kwr * kwr / np.where(kr == 0, 1, kr))[..., :, None] * delta[..., None, :]
            o[:, t] = np.einsum("...kv,...k->...v", S if mutation == "read_before_write" else S_new, q[:, t])
            S = S_new
        return o, S

    return forward


WKEY_MUTATIONS = ["erase_reads_write_key", "keys_swapped", "write_along_key", "no_beta",
                  "write_key_squared", "read_before_write"]


@pytest.mark.parametrize("mutation", WKEY_MUTATIONS)
def test_write_key_mutant_is_caught(mutation):
    from tests.oracle_pins import WKEY_PINS
    fwd = _make_wkey_forward(mutation)
    caught = []
    for name, pin in WKEY_PINS:
        try:
            pin(fwd)
        except (AssertionError, ValueError, IndexError, np.linalg.LinAlgError):
            caught.append(name)
    assert caught, f"mutation {mutation!r} passed every write-key pin"


def test_unmutated_write_key_copy_passes():
    from tests.oracle_pins import WKEY_PINS
    fwd = _make_wkey_forward("none")
    for name, pin in WKEY_PINS:
        pin(fwd)
