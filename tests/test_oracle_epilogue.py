"""Pins for the fp64 output-epilogue oracle ("Kimi K3 -- Architecture Notes",
section 1.3: y = Sigmoid(W_g x) (.) RMSNorm(o), the norm taken head-wise over
the d_v channels; RMSNorm as on the "MoE RMSNorm" page: the mean of squares
plus epsilon = 1e-5 under the square root, then a per-channel gain), and
mutants that the pins must reject.

Every pin is a hand-worked value or a property that holds whatever way the
oracle evaluates the formula: Sigmoid(0) = 1/2, Sigmoid(ln 3) = 3/4, the unit
root-mean-square of a normalised row, scale invariance, the exact place of
epsilon (a row whose mean square equals epsilon is scaled by 1/sqrt 2), the
independence of heads and tokens, and the gain acting channel by channel.
"""
import math

import numpy as np
import pytest

import oracle

TOL = 1e-13
EPS = 1e-5


def _cases(rng, T=4, H=3, d=8):
    o = rng.standard_normal((T, H, d)) * rng.uniform(0.1, 10.0, (T, H, 1))
    g = rng.standard_normal((T, H, d)) * 3.0
    return o, g


def pin_hand_worked(epi, rng):
    # d = 4, o = (2, 0, 0, 0): mean square 1, so with eps = 0 the row is
    # unchanged; a LayerNorm (mean removed) would give (1.73, -0.58, ...).
    y = epi(np.array([[[2.0, 0.0, 0.0, 0.0]]]), np.array([[[40.0, 0.0, math.log(3.0), -40.0]]]), None, 0.0)
    ref = [2.0 / (1.0 + math.exp(-40.0)), 0.0, 0.0, 0.0]
    assert np.allclose(y[0, 0], ref, rtol=0, atol=TOL), y
    # o = (3, 4): mean square 12.5; gates Sigmoid(0) = 1/2 and Sigmoid(ln 3) = 3/4.
    y = epi(np.array([[[3.0, 4.0]]]), np.array([[[0.0, math.log(3.0)]]]), None, 0.0)
    r = math.sqrt(12.5)
    assert np.allclose(y[0, 0], [0.5 * 3.0 / r, 0.75 * 4.0 / r], rtol=0, atol=TOL), y


def pin_eps_place(epi, rng):
    # Every entry sqrt(eps): mean square eps, so the row is scaled by
    # 1 / sqrt(eps + eps) * sqrt(eps) = 1 / sqrt(2).  Large logits make the gate 1.
    d = 6
    o = np.full((1, 1, d), math.sqrt(EPS))
    y = epi(o, np.full((1, 1, d), 60.0), None, EPS)
    assert np.allclose(y, 1.0 / math.sqrt(2.0), rtol=0, atol=1e-12), y
    # and the default epsilon is 1e-5
    y_def = epi(o, np.full((1, 1, d), 60.0))
    assert np.allclose(y_def, y, rtol=0, atol=TOL), "the default epsilon must be 1e-5"
    # A zero row stays zero (epsilon guards the division).
    assert np.all(epi(np.zeros((1, 1, d)), np.zeros((1, 1, d)), None, EPS) == 0.0)


def pin_half_gate(epi, rng):
    o, _ = _cases(rng)
    y_half = epi(o, np.zeros_like(o), None, 0.0)
    y_one = epi(o, np.full_like(o, 60.0), None, 0.0)
    assert np.allclose(y_half, 0.5 * y_one, rtol=0, atol=1e-12), "Sigmoid(0) must halve the output"


def pin_unit_rms(epi, rng):
    o, _ = _cases(rng)
    y = epi(o, np.full_like(o, 60.0), None, 0.0)
    rms = np.sqrt(np.mean(y * y, axis=-1))
    assert np.allclose(rms, 1.0, rtol=0, atol=1e-12), "a normalised row must have unit RMS"


def pin_scale_invariant(epi, rng):
    o, g = _cases(rng)
    y = epi(o, g, None, 0.0)
    assert np.allclose(epi(37.0 * o, g, None, 0.0), y, rtol=0, atol=1e-12)
    assert np.allclose(epi(-o, g, None, 0.0), -y, rtol=0, atol=1e-12)


def pin_gate_symmetry(epi, rng):
    o, g = _cases(rng)
    s = epi(o, g, None, EPS) + epi(o, -g, None, EPS)
    assert np.allclose(s, epi(o, np.full_like(o, 60.0), None, EPS), rtol=0, atol=1e-12), \
        "Sigmoid(u) + Sigmoid(-u) = 1 must hold channel by channel"


def pin_headwise(epi, rng):
    o, g = _cases(rng, T=3, H=4, d=8)
    y = epi(o, g, None, EPS)
    o2 = o.copy()
    o2[1, 2] *= 100.0         # another token and another head must not move
    o2[2, 0] += 5.0
    y2 = epi(o2, g, None, EPS)
    keep = np.ones((3, 4), bool)
    keep[1, 2] = keep[2, 0] = False
    assert np.allclose(y2[keep], y[keep], rtol=0, atol=TOL), "the norm is per (token, head)"


def pin_weight(epi, rng):
    o, g = _cases(rng)
    d = o.shape[-1]
    w = rng.uniform(-2.0, 2.0, d)
    y = epi(o, g, None, EPS)
    yw = epi(o, g, w, EPS)
    assert np.allclose(yw, y * w, rtol=0, atol=1e-12), "the gain scales each channel"
    e = np.zeros(d)
    e[3] = 1.0
    ye = epi(o, g, e, EPS)
    assert np.allclose(np.delete(ye, 3, axis=-1), 0.0, rtol=0, atol=TOL)
    assert np.allclose(epi(o, g, np.ones(d), EPS), y, rtol=0, atol=TOL), "no gain means a gain of 1"


EPI_PINS = (pin_hand_worked, pin_eps_place, pin_half_gate, pin_unit_rms, pin_scale_invariant,
            pin_gate_symmetry, pin_headwise, pin_weight)


def _oracle(o, g, w=None, eps=EPS):
    return oracle.kda_output_gate_rmsnorm(o, g, w, eps)


@pytest.mark.parametrize("pin", EPI_PINS, ids=lambda p: p.__name__)
def test_epilogue_oracle_pin(pin):
    pin(_oracle, np.random.default_rng(5))


# ---- mutants: plausible mistakes in the epilogue -----------------------------

def _sig(u):
    return 1.0 / (1.0 + np.exp(-u))


def _w(w, d):
    return np.ones(d) if w is None else np.asarray(w, float)


def mut_sum_not_mean(o, g, w=None, eps=EPS):
    return _sig(g) * _w(w, o.shape[-1]) * o / np.sqrt(np.sum(o * o, -1, keepdims=True) + eps)


def mut_eps_outside(o, g, w=None, eps=EPS):
    return _sig(g) * _w(w, o.shape[-1]) * o / (np.sqrt(np.mean(o * o, -1, keepdims=True)) + eps + 1e-300)


def mut_eps_1e6(o, g, w=None, eps=EPS):
    return _sig(g) * _w(w, o.shape[-1]) * o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps / 10.0)


def mut_silu_gate(o, g, w=None, eps=EPS):
    return g * _sig(g) * _w(w, o.shape[-1]) * o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps)


def mut_gate_before_norm(o, g, w=None, eps=EPS):
    x = _sig(g) * o
    return _w(w, o.shape[-1]) * x / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps)


def mut_layernorm(o, g, w=None, eps=EPS):
    c = o - o.mean(-1, keepdims=True)
    return _sig(g) * _w(w, o.shape[-1]) * c / np.sqrt(np.mean(c * c, -1, keepdims=True) + eps)


def mut_norm_over_heads(o, g, w=None, eps=EPS):
    return _sig(g) * _w(w, o.shape[-1]) * o / np.sqrt(np.mean(o * o, axis=(-2, -1), keepdims=True) + eps)


def mut_norm_over_tokens(o, g, w=None, eps=EPS):
    return _sig(g) * _w(w, o.shape[-1]) * o / np.sqrt(np.mean(o * o, axis=(0, -1), keepdims=True) + eps)


def mut_gain_added(o, g, w=None, eps=EPS):
    b = 0.0 if w is None else np.asarray(w, float) - 1.0
    return _sig(g) * (o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps) + b)


def mut_sign_gate(o, g, w=None, eps=EPS):
    return _sig(-g) * _w(w, o.shape[-1]) * o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps)


def mut_rms_not_sqrt(o, g, w=None, eps=EPS):
    return _sig(g) * _w(w, o.shape[-1]) * o / (np.mean(o * o, -1, keepdims=True) + eps)


MUTANTS = (mut_sum_not_mean, mut_eps_outside, mut_eps_1e6, mut_silu_gate, mut_gate_before_norm, mut_layernorm,
           mut_norm_over_heads, mut_norm_over_tokens, mut_gain_added, mut_sign_gate, mut_rms_not_sqrt)


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_epilogue_mutant_rejected(mutant):
    caught = 0
    for pin in EPI_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant, np.random.default_rng(5))
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"{mutant.__name__} passed every epilogue pin"
