"""Pins for the fp64 gate-map oracle ("Kimi K3 -- Architecture Notes", section
1.2, table, Kimi K3 row: g = g_min * Sigmoid(e^{A_h} z), g_min = -5; beta is a
sigmoid of its logit), and mutants that the pins must reject.

Every pin is a closed form or an algebraic property of the logistic map that
is independent of how the oracle evaluates it: Sigmoid(0) = 1/2,
Sigmoid(ln 3) = 3/4, the limits at +-infinity, Sigmoid(u) + Sigmoid(-u) = 1,
and the role of A_h as a per-head scale of the logit.
"""
import math

import numpy as np
import pytest

import oracle

TOL = 1e-13


def _gate_cases(rng, T=5, H=3, d=4):
    z = rng.standard_normal((T, H, d)) * 3.0
    A = rng.uniform(-1.0, 1.0, H)
    b = rng.standard_normal((T, H)) * 3.0
    return z, A, b


def pin_zero_logit(gate, rng):
    T, H, d = 3, 2, 5
    la, beta = gate(np.zeros((T, H, d)), rng.uniform(-2, 2, H), np.zeros((T, H)))
    assert np.allclose(la, -2.5, rtol=0, atol=TOL), "z = 0 must give g = g_min / 2 = -2.5"
    assert np.allclose(beta, 0.5, rtol=0, atol=TOL), "beta logit 0 must give beta = 1/2"


def pin_ln3(gate, rng):
    l3 = math.log(3.0)
    z = np.array([l3, -l3, 0.0])[None, None, :]
    la, beta = gate(z, np.zeros(1), np.array([[l3]]))
    assert np.allclose(la[0, 0], [-3.75, -1.25, -2.5], rtol=0, atol=TOL), la   # -5 * (3/4, 1/4, 1/2)
    assert abs(float(beta[0, 0]) - 0.75) <= TOL, beta


def pin_limits_and_range(gate, rng):
    z = np.array([40.0, -40.0])[None, None, :]
    la, _ = gate(z, np.zeros(1), np.zeros((1, 1)))
    assert abs(la[0, 0, 0] + 5.0) <= 1e-12, "z -> +inf must approach g_min = -5"
    assert abs(la[0, 0, 1]) <= 1e-15, "z -> -inf must approach 0"
    z, A, b = _gate_cases(rng)
    la, beta = gate(z, A, b)
    assert (la > -5.0).all() and (la < 0.0).all(), "g must lie in (g_min, 0)"
    assert (beta > 0.0).all() and (beta < 1.0).all(), "beta must lie in (0, 1)"


def pin_symmetry(gate, rng):
    z, A, b = _gate_cases(rng)
    la_p, b_p = gate(z, A, b)
    la_m, b_m = gate(-z, A, -b)
    assert np.allclose(la_p + la_m, -5.0, rtol=0, atol=TOL), "g(z) + g(-z) must equal g_min"
    assert np.allclose(b_p + b_m, 1.0, rtol=0, atol=TOL), "beta(b) + beta(-b) must equal 1"


def pin_head_scale(gate, rng):
    z, A, b = _gate_cases(rng, H=3, d=4)
    la, _ = gate(z, A, b)
    for h in range(A.shape[0]):
        ref, _ = gate(z[:, h:h + 1] * math.exp(A[h]), np.zeros(1), b[:, h:h + 1])
        assert np.allclose(la[:, h:h + 1], ref, rtol=0, atol=TOL), f"A_{h} must scale the logit of head {h} by e^A"


def pin_monotone(gate, rng):
    z = np.linspace(-6, 6, 49)[None, None, :]
    la, _ = gate(z, np.array([0.3]), np.zeros((1, 1)))
    assert (np.diff(la[0, 0]) < 0).all(), "g must decrease as the logit grows"


GATE_PINS = (pin_zero_logit, pin_ln3, pin_limits_and_range, pin_symmetry, pin_head_scale, pin_monotone)


def _run(pin, gate):
    pin(gate, np.random.default_rng(7))


@pytest.mark.parametrize("pin", GATE_PINS, ids=lambda p: p.__name__)
def test_gate_oracle_pin(pin):
    _run(pin, oracle.kda_gate_map)


# ---- mutants: plausible mistakes in a gate map -------------------------------

def _sig(u):
    return 1.0 / (1.0 + np.exp(-u))


def mut_softplus_map(z, A, b):           # the unbounded mapping of the table's first row
    return -np.exp(A)[None, :, None] * np.log1p(np.exp(z)), _sig(b)


def mut_scale_not_exponentiated(z, A, b):
    return -5.0 * _sig(A[None, :, None] * z), _sig(b)


def mut_sign_flip(z, A, b):
    return -5.0 * _sig(-np.exp(A)[None, :, None] * z), _sig(b)


def mut_positive_gmin(z, A, b):
    return 5.0 * _sig(np.exp(A)[None, :, None] * z), _sig(b)


def mut_scale_on_channels(z, A, b):      # A broadcast over the channel axis
    return -5.0 * _sig(np.exp(np.resize(A, z.shape[-1]))[None, None, :] * z), _sig(b)


def mut_beta_raw(z, A, b):
    return -5.0 * _sig(np.exp(A)[None, :, None] * z), np.asarray(b, dtype=np.float64)


def mut_beta_flipped(z, A, b):
    return -5.0 * _sig(np.exp(A)[None, :, None] * z), _sig(-b)


def mut_returns_alpha(z, A, b):
    return np.exp(-5.0 * _sig(np.exp(A)[None, :, None] * z)), _sig(b)


def mut_gmin_halved(z, A, b):
    return -2.5 * _sig(np.exp(A)[None, :, None] * z), _sig(b)


MUTANTS = (mut_softplus_map, mut_scale_not_exponentiated, mut_sign_flip, mut_positive_gmin,
           mut_scale_on_channels, mut_beta_raw, mut_beta_flipped, mut_returns_alpha, mut_gmin_halved)


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_gate_mutant_rejected(mutant):
    caught = 0
    for pin in GATE_PINS:
        try:
            with np.errstate(all="ignore"):
                _run(pin, mutant)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"{mutant.__name__} passed every gate pin"


def test_gated_prefill_is_gate_map_then_recurrence():
    """The composite applies the map per head (A indexed by original head number
    when a head subset is selected) and then the section-1.1 recurrence."""
    rng = np.random.default_rng(3)
    T, H, d = 9, 3, 4
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    z, A, b = _gate_cases(rng, T=T, H=H, d=d)
    o_all, f_all = oracle.kda_prefill_gated(q, k, v, z, A, b)
    o_sub, f_sub = oracle.kda_prefill_gated(q, k, v, z, A, b, heads=[2])
    assert np.allclose(o_sub[:, 0], o_all[:, 2], rtol=0, atol=1e-12)
    assert np.allclose(f_sub[:, 0], f_all[:, 2], rtol=0, atol=1e-12)
