"""The time-split algebra of the prefill, checked in fp64 against the oracle's token loop.

"Kimi K3 -- Architecture Notes", section 1.1, defines a recurrence that is affine in the state.  The
step map is S -> A_t S + beta_t k_t v_t^T, with A_t = (I - beta_t k_t k_t^T) Diag(alpha_t).  One
long sequence can therefore be cut into segments p = 0..P-1 that run at the same time:

* segment p runs from a zero state (segment 0 from the true initial state).  That gives its
  outputs o0_t and its end state B_p;
* segment p >= 1 also runs from the identity (d_k value columns) with v = 0.  That gives its
  transition Phi_p, the product of its A_t, as the end state.  It also gives the outputs
  qt_t = Phi_t^T q_t, with Phi_t the product up to and including token t;
* a serial scan over the segments forms the true end states:
  S_end,0 = B_0 and S_end,p = Phi_p S_end,p-1 + B_p;
* segment p >= 1 corrects its outputs with the state it really starts from:
  o_t = o0_t + S_end,p-1^T qt_t.

This file writes the split out with the oracle's own recurrence as the per-segment engine.  It
checks, without any GPU, that:

* the split reproduces the unsplit recurrence to rounding for several segment counts, ragged
  last segments and every decay law;
* the transition-run outputs are Phi_t^T q_t, checked by forming Phi_t token by token;
* four plausible mistakes are caught.

The kernels' split entry points implement these phases.  Nothing here is shared with them.
"""
import numpy as np
import pytest

import oracle
from pins import random_case


def split_model(q, k, v, la, beta, S0, seg_len, mistake=None):
    """Time-split evaluation of one run of tokens (shapes as oracle.kda_recurrence)."""
    T, B, d_k = q.shape
    bounds = [(a, min(a + seg_len, T)) for a in range(0, T, seg_len)] or [(0, 0)]
    o = np.zeros(v.shape)
    B_end, phis, qts = [], [], []
    for p, (a, e) in enumerate(bounds):
        sl = slice(a, e)
        init = S0 if (p == 0 and mistake != "drop_init") else np.zeros_like(S0)
        o[sl], b_end = oracle.kda_recurrence(q[sl], k[sl], v[sl], la[sl], beta[sl], init)
        B_end.append(b_end)
        if p > 0:
            eye = np.broadcast_to(np.eye(d_k), (B, d_k, d_k))
            qt, phi = oracle.kda_recurrence(q[sl], k[sl], np.zeros((e - a, B, d_k)), la[sl], beta[sl], eye)
            phis.append(phi)
            qts.append(qt)
    # Serial scan: true end state of every segment.
    S_end = [B_end[0]]
    for p in range(1, len(bounds)):
        phi = phis[p - 1]
        if mistake == "phi_transposed":
            phi = np.swapaxes(phi, 1, 2)
        S_end.append(np.einsum("bkm,bmv->bkv", phi, S_end[p - 1]) + B_end[p])
    # Correction of segments p >= 1 with the state they start from.
    for p in range(1, len(bounds)):
        a, e = bounds[p]
        S_in = S_end[p - 2] if (mistake == "stale_state" and p >= 2) else S_end[p - 1]
        corr = np.einsum("tbk,bkv->tbv", qts[p - 1], S_in)
        if mistake == "skip_correction":
            corr = 0.0
        o[a:e] += corr
    return o, S_end[-1]


CASES = [
    # (T, seg_len, law)
    (48, 16, "softplus"),
    (100, 16, "uniform53"),
    (100, 33, "zero"),
    (130, 64, "softplus"),
    (64, 64, "softplus"),       # one segment: the split is the plain run
    (7, 64, "zero"),            # fewer tokens than one segment
]


@pytest.mark.parametrize("T,seg_len,law", CASES)
def test_split_reproduces_the_recurrence(T, seg_len, law):
    rng = np.random.default_rng(T * 7 + seg_len)
    q, k, v, la, b, S0 = random_case(rng, T, 3, 8, 5, la_law=law)
    o_ref, S_ref = oracle.kda_recurrence(q, k, v, la, b, S0)
    o, S = split_model(q, k, v, la, b, S0, seg_len)
    scale_o, scale_S = np.abs(o_ref).max(), np.abs(S_ref).max()
    assert np.abs(o - o_ref).max() <= 1e-12 * max(scale_o, 1.0)
    assert np.abs(S - S_ref).max() <= 1e-12 * max(scale_S, 1.0)


def test_transition_outputs_are_phi_t_transposed_q():
    """The identity run with v = 0 outputs Phi_t^T q_t, with Phi_t = A_t ... A_1 formed here
    directly from the step matrices A_t = (I - beta_t k_t k_t^T) Diag(alpha_t)."""
    rng = np.random.default_rng(3)
    T, B, d = 20, 2, 6
    q, k, _, la, b, _ = random_case(rng, T, B, d, d, la_law="softplus")
    eye = np.broadcast_to(np.eye(d), (B, d, d))
    qt, phi_T = oracle.kda_recurrence(q, k, np.zeros((T, B, d)), la, b, eye)
    for bb in range(B):
        phi = np.eye(d)
        for t in range(T):
            A = (np.eye(d) - b[t, bb] * np.outer(k[t, bb], k[t, bb])) @ np.diag(np.exp(la[t, bb]))
            phi = A @ phi
            assert np.allclose(qt[t, bb], phi.T @ q[t, bb], rtol=1e-12, atol=1e-14)
        assert np.allclose(phi_T[bb], phi, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mistake", ["phi_transposed", "stale_state", "skip_correction", "drop_init"])
def test_split_mistakes_are_caught(mistake):
    rng = np.random.default_rng(11)
    q, k, v, la, b, S0 = random_case(rng, 80, 2, 8, 4, la_law="zero")
    la = la - 0.02      # alpha close to 1: the incoming state matters in every segment
    o_ref, S_ref = oracle.kda_recurrence(q, k, v, la, b, S0)
    o, S = split_model(q, k, v, la, b, S0, 16, mistake=mistake)
    err = max(np.abs(o - o_ref).max() / np.abs(o_ref).max(), np.abs(S - S_ref).max() / np.abs(S_ref).max())
    assert err > 1e-3, f"mistake {mistake} went unnoticed (err {err})"
