"""The fp64 oracle against facts fixed by the pages and by mathematics (CPU only)."""

import json
import os

import numpy as np
import pytest

from oracle import forward, recurrent_step, rel_l2
from tests.oracle_pins import PINS, WKEY_PINS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_examples.json")


@pytest.mark.parametrize("name,pin", PINS, ids=[n for n, _ in PINS])
def test_pin(name, pin):
    pin(forward)


@pytest.mark.parametrize("name,pin", WKEY_PINS, ids=[n for n, _ in WKEY_PINS])
def test_write_key_pin(name, pin):
    pin(forward)


def _load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _load_golden(), ids=lambda e: e["name"])
def test_hand_worked_example(ex):
    """Step-by-step hand computations (see the fixture for the worked steps)."""
    k = np.array(ex["k"], float)[None, :, None]
    q = np.array(ex["q"], float)[None, :, None]
    v = np.array(ex["v"], float)[None, :, None]
    beta = np.array(ex["beta"], float)[None, :, None]
    log_a = np.log(np.array(ex["a"], float))[None, :, None]
    S0 = np.array(ex["S0"], float)[None, None]
    o, S = forward(q, k, v, beta, log_a, S0, form=ex["form"])
    np.testing.assert_allclose(o[0, :, 0], np.array(ex["o"], float), rtol=0, atol=1e-13)
    np.testing.assert_allclose(S[0, 0], np.array(ex["S_T"], float), rtol=0, atol=1e-13)


def test_step_matches_forward_of_one_token():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((2, 1, 3, 8)), rng.standard_normal((2, 1, 3, 8))
    v, beta = rng.standard_normal((2, 1, 3, 5)), rng.uniform(0, 1, (2, 1, 3))
    la = -rng.uniform(0, 1, (2, 1, 3, 8))
    S0 = rng.standard_normal((2, 3, 8, 5))
    o, S = forward(q, k, v, beta, la, S0)
    o1, S1 = recurrent_step(S0, q[:, 0], k[:, 0], v[:, 0], beta[:, 0], la[:, 0])
    np.testing.assert_array_equal(o[:, 0], o1)
    np.testing.assert_array_equal(S, S1)


def test_empty_sequence_returns_initial_state():
    S0 = np.arange(24, dtype=float).reshape(1, 2, 3, 4)
    o, S = forward(np.zeros((1, 0, 2, 3)), np.zeros((1, 0, 2, 3)), np.zeros((1, 0, 2, 4)),
                   np.zeros((1, 0, 2)), None, S0)
    assert o.shape == (1, 0, 2, 4)
    np.testing.assert_array_equal(S, S0)


def test_rel_l2():
    assert rel_l2([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert abs(rel_l2([3.0, 5.0], [3.0, 4.0]) - 0.2) < 1e-15
