"""Pins for the fp64 KDA oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes ``run(q, k, v, log_alpha, beta, S0) -> (o, S_T)``
with the shapes of ``oracle.kda_recurrence`` (q, k, log_alpha [T, B, d_k],
v [T, B, d_v], beta [T, B], S0 [B, d_k, d_v]) and raises AssertionError when
the implementation under test disagrees with the fact.  The test suite runs
them against the oracle (they must pass) and against copies of the oracle
with one planted mistake each (every copy must fail at least one pin).

None of the pins re-types the oracle's update: they check hand-derived
values, invariants, special cases, an explicitly unrolled matrix product, a
different page's formula and algebraic properties.

Sources: "Kimi K3 -- Architecture Notes" section 1.1 (the recurrence, the
ranges of alpha and beta, the fixed-size state) and section 1.2 (decay bound
log alpha >= -5); the Kimi K3 visualiser page, "Kimi Delta Attention (KDA)"
box (its per-head loop, used only where alpha = 1).
"""

from __future__ import annotations

import json
import os

import numpy as np

TOL = 1e-12


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    scale = max(1.0, float(np.abs(b).max()) if b.size else 1.0)
    err = float(np.abs(a - b).max()) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} (scale {scale:.3e})"


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_case(rng, T, B, d_k, d_v, la_law="softplus", beta=None, unit=True):
    q = rng.standard_normal((T, B, d_k))
    k = rng.standard_normal((T, B, d_k))
    if unit:
        q, k = _unit(q), _unit(k)
    v = rng.standard_normal((T, B, d_v))
    if la_law == "softplus":
        la = -np.minimum(np.log1p(np.exp(rng.standard_normal((T, B, d_k)))), 5.0)
    elif la_law == "uniform53":
        la = rng.uniform(-5.0, -3.0, (T, B, d_k))
    elif la_law == "zero":
        la = np.zeros((T, B, d_k))
    else:
        raise ValueError(la_law)
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, B)))) if beta is None else np.full((T, B), float(beta))
    S0 = 0.5 * rng.standard_normal((B, d_k, d_v))
    return q, k, v, la, b, S0


# ---------------------------------------------------------------------------
# 1. A hand-worked two-token example (d_k = d_v = 2), derived on paper from the
#    section-1.1 recurrence (stored with its derivation in
#    golden/hand_two_token.json).  Values chosen so that every intermediate is
#    a short decimal.
#
#    S0 = [[1, 2], [3, 4]]          (rows are the d_k index)
#    t=1: alpha = (1, 1/2), k = (1, 0), beta = 1/2, v = (2, -2), q = (0, 1)
#         Diag(alpha) S0         = [[1, 2], [1.5, 2]]
#         (Diag(alpha) S0)^T k   = (1, 2);  v - that = (1, -4)
#         S1 = [[1, 2], [1.5, 2]] + 1/2 * [[1, -4], [0, 0]] = [[1.5, 0], [1.5, 2]]
#         o1 = S1^T q = (1.5, 2)
#    t=2: alpha = (1/2, 1), k = (0.6, 0.8), beta = 1, v = (1, 1), q = (1, 0)
#         Diag(alpha) S1         = [[0.75, 0], [1.5, 2]]
#         (...)^T k              = (1.65, 1.6);  v - that = (-0.65, -0.6)
#         S2 = [[0.75, 0], [1.5, 2]] + [[-0.39, -0.36], [-0.52, -0.48]]
#            = [[0.36, -0.36], [0.98, 1.52]]
#         o2 = S2^T q = (0.36, -0.36)
# ---------------------------------------------------------------------------
_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
with open(os.path.join(_GOLDEN, "hand_two_token.json")) as _f:
    HAND = json.load(_f)


def pin_hand_example(run):
    h = HAND
    q = np.array(h["q"])[:, None, :]
    k = np.array(h["k"])[:, None, :]
    v = np.array(h["v"])[:, None, :]
    la = np.log(np.array(h["alpha"]))[:, None, :]
    b = np.array(h["beta"])[:, None]
    S0 = np.array(h["S0"])[None]
    o, S = run(q, k, v, la, b, S0)
    _close(o[:, 0], h["o"], 1e-14, "hand example o")
    _close(S[0], h["S2"], 1e-14, "hand example S2")


# ---------------------------------------------------------------------------
# 2. Delta-rule retrieval: beta = 1 and |k| = 1 make the write exact,
#    S_t^T k_t = v_t, whatever alpha and the previous state are.  With q_t = k_t
#    the output must equal v_t at every token.
# ---------------------------------------------------------------------------
def pin_retrieval(run, rng):
    for la_law in ("softplus", "zero"):
        q, k, v, la, b, S0 = random_case(rng, 12, 3, 6, 6, la_law=la_law, beta=1.0)
        o, _ = run(k, k, v, la, b, S0)
        _close(o, v, 1e-12, f"retrieval ({la_law})")
    q, k, v, la, b, S0 = random_case(rng, 9, 2, 4, 7, beta=1.0)
    o, _ = run(k, k, v, la, b, S0)
    _close(o, v, 1e-12, "retrieval (d_k != d_v)")


# ---------------------------------------------------------------------------
# 3. Identity: beta = 0 and alpha = 1 leave the state untouched.
# ---------------------------------------------------------------------------
def pin_identity(run, rng):
    q, k, v, la, b, S0 = random_case(rng, 10, 3, 5, 4, la_law="zero", beta=0.0)
    o, S = run(q, k, v, la, b, S0)
    _close(S, S0, 1e-15, "identity state")
    _close(o, np.einsum("bkv,tbk->tbv", S0, q), 1e-14, "identity output")


# ---------------------------------------------------------------------------
# 4. Pure decay: beta = 0 gives S_t = Diag(exp(sum_{s<=t} log alpha_s)) S0,
#    i.e. channel c of the d_k rows decays by its own cumulative factor.
# ---------------------------------------------------------------------------
def pin_pure_decay(run, rng):
    q, k, v, la, b, S0 = random_case(rng, 11, 2, 5, 3, la_law="softplus", beta=0.0)
    o, S = run(q, k, v, la, b, S0)
    G = np.exp(np.cumsum(la, axis=0))                     # [T, B, d_k]
    _close(S, G[-1][:, :, None] * S0, 1e-13, "pure decay state")
    for t in range(q.shape[0]):
        St = G[t][:, :, None] * S0
        _close(o[t], np.einsum("bkv,bk->bv", St, q[t]), 1e-13, f"pure decay output t={t}")


# ---------------------------------------------------------------------------
# 5. Basis-key overwrite: k_t = e_i and beta = 1 replace row i of the decayed
#    state by v_t; every other row j is only scaled by alpha_j.
# ---------------------------------------------------------------------------
def pin_basis_overwrite(run, rng):
    d_k, d_v = 5, 3
    S = 0.5 * rng.standard_normal((1, d_k, d_v))
    S_run = S.copy()
    for t, i in enumerate([2, 0, 4, 2, 1]):
        k = np.zeros((1, 1, d_k)); k[0, 0, i] = 1.0
        q = _unit(rng.standard_normal((1, 1, d_k)))
        v = rng.standard_normal((1, 1, d_v))
        la = -rng.uniform(0.0, 5.0, (1, 1, d_k))
        b = np.ones((1, 1))
        expect = np.exp(la[0, 0])[:, None] * S[0]
        expect[i] = v[0, 0]
        _, S_run = run(q, k, v, la, b, S_run)
        _close(S_run[0], expect, 1e-14, f"basis overwrite step {t}")
        S = expect[None]


# ---------------------------------------------------------------------------
# 6. Brute force: with explicit d_k x d_k matrices A_t = (I - b_t k_t k_t^T) Diag(alpha_t)
#    the state is the unrolled product  S_t = A_t...A_1 S0 + sum_s A_t...A_{s+1} b_s k_s v_s^T.
#    Built here as full matrix products over every prefix (T <= 8).
# ---------------------------------------------------------------------------
def pin_brute_force(run, rng):
    for (T, d_k, d_v, law) in ((8, 4, 6, "softplus"), (5, 7, 3, "uniform53"), (1, 3, 3, "softplus")):
        q, k, v, la, b, S0 = random_case(rng, T, 2, d_k, d_v, la_law=law)
        o, S = run(q, k, v, la, b, S0)
        for bi in range(2):
            I = np.eye(d_k)
            A = [(I - b[t, bi] * np.outer(k[t, bi], k[t, bi])) @ np.diag(np.exp(la[t, bi])) for t in range(T)]
            for t in range(T):
                St = np.eye(d_k)
                for s in range(t + 1):
                    St = A[s] @ St
                St = St @ S0[bi]
                for s in range(t + 1):
                    Pm = np.eye(d_k)
                    for u in range(s + 1, t + 1):
                        Pm = A[u] @ Pm
                    St = St + Pm @ (b[s, bi] * np.outer(k[s, bi], v[s, bi]))
                _close(o[t, bi], St.T @ q[t, bi], 1e-12, f"brute force o T={T} t={t}")
            _close(S[bi], St, 1e-12, f"brute force S T={T}")


# ---------------------------------------------------------------------------
# 7. Affinity in (S0, v): o and S_T are linear in the pair (S0, v) for fixed
#    q, k, alpha, beta; and running [0, T) equals running [0, t) then [t, T)
#    from the carried state.
# ---------------------------------------------------------------------------
def pin_linearity_and_split(run, rng):
    q, k, v, la, b, S0 = random_case(rng, 20, 2, 6, 5)
    o, S = run(q, k, v, la, b, S0)
    o1, S1 = run(q, k, np.zeros_like(v), la, b, S0)
    o2, S2 = run(q, k, v, la, b, np.zeros_like(S0))
    _close(o, o1 + o2, 1e-12, "linearity o")
    _close(S, S1 + S2, 1e-12, "linearity S")
    oa, Sa = run(q[:7], k[:7], v[:7], la[:7], b[:7], S0)
    ob, Sb = run(q[7:], k[7:], v[7:], la[7:], b[7:], Sa)
    _close(np.concatenate([oa, ob]), o, 1e-12, "split o")
    _close(Sb, S, 1e-12, "split S")


# ---------------------------------------------------------------------------
# 8. Contraction: for beta in [0,1], |k| = 1, alpha in (0,1] the transition
#    (I - b k k^T) Diag(alpha) has spectral norm <= 1, so
#    |S_t|_F <= |S_{t-1}|_F + b_t |v_t|.
# ---------------------------------------------------------------------------
def pin_contraction(run, rng):
    q, k, v, la, b, S0 = random_case(rng, 30, 2, 6, 4, la_law="softplus")
    b[::3] = 1.0
    S = S0
    for t in range(30):
        _, S_new = run(q[t:t + 1], k[t:t + 1], v[t:t + 1], la[t:t + 1], b[t:t + 1], S)
        lhs = np.linalg.norm(S_new, axis=(1, 2))
        rhs = np.linalg.norm(S, axis=(1, 2)) + b[t] * np.linalg.norm(v[t], axis=-1)
        assert np.all(lhs <= rhs * (1 + 1e-12)), f"contraction violated at t={t}"
        S = S_new


# ---------------------------------------------------------------------------
# 9. Cross-page check: the visualiser's per-head loop (conv, gates and
#    normalisation removed) keeps a [d_v, d_k] state W and does
#    W <- W + b (v - W k) k^T, output W q.  With alpha = 1 this is the notes'
#    recurrence with S = W^T.
# ---------------------------------------------------------------------------
def pin_visualiser_alpha1(run, rng):
    q, k, v, la, b, S0 = random_case(rng, 15, 2, 5, 4, la_law="zero")
    o, S = run(q, k, v, la, b, S0)
    for bi in range(2):
        Wm = S0[bi].T.copy()
        for t in range(15):
            Wm = Wm + b[t, bi] * np.outer(v[t, bi] - Wm @ k[t, bi], k[t, bi])
            _close(o[t, bi], Wm @ q[t, bi], 1e-12, f"visualiser loop t={t}")
        _close(S[bi], Wm.T, 1e-12, "visualiser final state")


# ---------------------------------------------------------------------------
# 10. Single-step closed form (the form a one-pass decode kernel evaluates):
#     with a = exp(log_alpha), w = b (v - S0^T (a*k)):
#       S1 = Diag(a) S0 + k w^T,    o1 = S0^T (a*q) + w (k^T q)
# ---------------------------------------------------------------------------
def pin_single_step(run, rng):
    q, k, v, la, b, S0 = random_case(rng, 1, 4, 6, 5, unit=False)
    o, S = run(q, k, v, la, b, S0)
    a = np.exp(la[0])
    w = b[0][:, None] * (v[0] - np.einsum("bkv,bk->bv", S0, a * k[0]))
    S1 = a[:, :, None] * S0 + k[0][:, :, None] * w[:, None, :]
    o1 = np.einsum("bkv,bk->bv", S0, a * q[0]) + w * np.sum(k[0] * q[0], axis=-1, keepdims=True)
    _close(S, S1, 1e-13, "single step S")
    _close(o[0], o1, 1e-13, "single step o")


ALL_PINS = (
    pin_hand_example,
    pin_retrieval,
    pin_identity,
    pin_pure_decay,
    pin_basis_overwrite,
    pin_brute_force,
    pin_linearity_and_split,
    pin_contraction,
    pin_visualiser_alpha1,
    pin_single_step,
)


def run_pin(pin, run, seed=1234):
    rng = np.random.default_rng(seed)
    if pin is pin_hand_example:
        return pin(run)
    return pin(run, rng)
