"""The tile algebra of the chunkwise prefill, checked in fp64 against the oracle's token loop.

"Kimi K3 -- Architecture Notes", section 1.2, evaluates KDA chunk by chunk: the state is carried
serially across chunks and the work inside a chunk is parallel.  It uses 16-token secondary tiles
whose decay factors are taken relative to a reference point inside the tile, so that a lower
bound on log alpha keeps every factor in range.
The prefill kernel carries the state from tile to tile.  For one tile of positions r = 1..L
(L <= 16) starting from state S, with x_r the inclusive prefix sum of log2(alpha) over the tile
(per key channel) and X = x_L:

    P_rs = sum_c q_rc 2^{x_rc} k_sc 2^{-x_sc}   (s <= r)
    M_rs = sum_c k_rc 2^{x_rc} k_sc 2^{-x_sc}   (s <  r)
    A    = (I + Diag(beta) M)^{-1} Diag(beta)
    W    = A (V - (K * 2^x) S)
    O    = (Q * 2^x) S + P W
    S   <- Diag(2^X) S + (K * 2^{X - x})^T W

This file writes that algebra out in plain NumPy (a library solve serves as the triangular
inverse) and checks, without any GPU:

* it reproduces the token recurrence to rounding at the decay floor, under U[-5, -3] and under
  the softplus law, for full and partial tiles and a random initial state (the chunk-algebra
  model of the hot-path scope);
* with log alpha >= -5 no factor of a 16-token tile leaves the normal fp32 range, while a
  64-token span would overflow (the range argument of section 1.2);
* with bf16 inputs and bf16 product operands the error stays well inside the 2e-2 tolerance of
  the bf16 workloads;
* three plausible mistakes in the algebra are caught.

Nothing here is shared with the oracle or the HIP library.
"""
import numpy as np
import pytest

import oracle
from pins import random_case

LOG2E = 1.0 / np.log(2.0)
FLT_MAX_LOG2 = 128.0        # float32 max is just below 2^128
FLT_MIN_NORMAL_LOG2 = -126.0


def bf16(x):
    """Round to the nearest bfloat16 (ties to even), returned as float64."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def tile_model(q, k, v, log_alpha, beta, S0, tile=16, mistake=None, op=None):
    """Tile recurrence over one run of tokens.  Shapes as oracle.kda_recurrence:
    q, k, log_alpha [T, B, d_k]; v [T, B, d_v]; beta [T, B]; S0 [B, d_k, d_v].
    `op` rounds every matrix-product operand (None: exact).
    Returns (o, S_T, widest), widest = the largest |exponent| (base 2) of any tile factor."""
    op = op or (lambda a: a)
    T, B, d_k = q.shape
    S = np.array(S0, dtype=np.float64)
    o = np.zeros(v.shape)
    widest = 0.0
    for t0 in range(0, T, tile):
        sl = slice(t0, min(t0 + tile, T))
        L = sl.stop - sl.start
        x = np.cumsum(log_alpha[sl] * LOG2E, axis=0)            # [L, B, d_k], inclusive prefix
        X = x[-1]                                               # [B, d_k]
        widest = max(widest, float(np.abs(x).max()))
        e1 = np.exp2(x)                                         # 2^{x_r}      in (0, 1]
        e2 = np.exp2(X[None] - x)                               # 2^{X - x_r}  in (0, 1]
        if mistake == "suffix_includes_r":
            e2 = np.exp2(X[None] - x + log_alpha[sl] * LOG2E)
        col = np.exp2(-x)                                       # 2^{-x_s}     in [1, ...)
        Qe1, Ke1, Ke2, Kb = op(q[sl] * e1), op(k[sl] * e1), op(k[sl] * e2), op(k[sl] * col)
        P = np.einsum("rbc,sbc->brs", Qe1, Kb)
        M = np.einsum("rbc,sbc->brs", Ke1, Kb)
        lower_incl = np.tril(np.ones((L, L)))
        strict = np.tril(np.ones((L, L)), -1)
        P = P * (strict if mistake == "P_strict" else lower_incl)
        M = M * strict
        b = beta[sl].T                                          # [B, L]
        lhs = np.eye(L)[None] + b[:, :, None] * M
        A = op(np.linalg.solve(lhs, np.eye(L)[None].repeat(B, 0)) * b[:, None, :])
        P = op(P)
        if mistake == "decay_after_update":
            S = np.exp2(X)[:, :, None] * S
        Sop = op(S)                                             # the state as a product operand
        U = op(v[sl] - np.einsum("rbc,bcv->rbv", Ke1, Sop))
        W = op(np.einsum("brs,sbv->rbv", A, U))
        o[sl] = np.einsum("rbc,bcv->rbv", Qe1, Sop) + np.einsum("brs,sbv->rbv", P, W)
        if mistake == "decay_after_update":
            S = S + np.einsum("rbc,rbv->bcv", Ke2, W)
        else:
            S = np.exp2(X)[:, :, None] * S + np.einsum("rbc,rbv->bcv", Ke2, W)
    return o, S, widest


def _case(seed, T, la_law, B=3, d_k=16, d_v=8):
    """Unit q, k, Gaussian v, sigmoid beta and a random initial state; log alpha from one of the
    workloads' laws, or the floor -5 everywhere."""
    rng = np.random.default_rng(seed)
    q, k, v, la, beta, S0 = random_case(rng, T, B, d_k, d_v, la_law="zero" if la_law == "floor" else la_law)
    if la_law == "floor":
        la = np.full_like(la, -5.0)
    return q, k, v, la, beta, S0


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


@pytest.mark.parametrize("la_law", ["floor", "uniform53", "softplus"])
@pytest.mark.parametrize("T", [1, 7, 16, 37, 64, 100])
def test_tile_algebra_reproduces_the_token_recurrence(la_law, T):
    q, k, v, la, beta, S0 = _case(7 + T, T, la_law)
    o_ref, S_ref = oracle.kda_recurrence(q, k, v, la, beta, S0)
    o, S, _ = tile_model(q, k, v, la, beta, S0)
    assert _rel(o, o_ref) < 1e-10 and _rel(S, S_ref) < 1e-10


def test_decay_floor_keeps_tile_factors_in_fp32_range():
    # log alpha >= -5 everywhere, and exactly -5 (the floor) in the worst case
    q, k, v, la, beta, S0 = _case(3, 64, "floor")
    assert np.all(la >= -5.0)
    _, _, widest = tile_model(q, k, v, la, beta, S0)
    bound = 16 * 5.0 * LOG2E                   # e^{80} = 2^{115.4}
    assert widest <= bound + 1e-9
    assert bound < FLT_MAX_LOG2 and -bound > FLT_MIN_NORMAL_LOG2
    # the same factors over a whole 64-token chunk would not fit: e^{320} overflows fp32
    assert 64 * 5.0 * LOG2E > FLT_MAX_LOG2
    _, _, widest64 = tile_model(q, k, v, la, beta, S0, tile=64)
    assert widest64 > FLT_MAX_LOG2


@pytest.mark.parametrize("la_law", ["uniform53", "softplus"])
def test_bf16_operands_stay_within_the_tolerance(la_law):
    """bf16 inputs and bf16 product operands (the scaled q and k rows, P, A, the state as an
    operand, U and W) with an fp32-or-better state: the error the bf16 workloads' 2e-2
    tolerance has to absorb, at the workloads' d = 128 over 1024 tokens."""
    rng = np.random.default_rng(5)
    T, B, d = 1024, 2, 128
    q, k, v, la, beta, S0 = random_case(rng, T, B, d, d, la_law=la_law)
    q, k, v = bf16(q), bf16(k), bf16(v)
    S0 = 0.02 * rng.standard_normal((B, d, d))
    o_ref, S_ref = oracle.kda_recurrence(q, k, v, la, beta, S0)
    o, S, _ = tile_model(q, k, v, la, beta, S0, op=bf16)
    eo, es = _rel(bf16(o), o_ref), _rel(S, S_ref)
    assert eo < 2e-2 and es < 2e-2, (eo, es)
    assert eo > 1e-4          # the rounding is really applied


@pytest.mark.parametrize("mistake", ["P_strict", "suffix_includes_r", "decay_after_update"])
def test_planted_mistakes_are_caught(mistake):
    q, k, v, la, beta, S0 = _case(11, 37, "softplus")
    o_ref, S_ref = oracle.kda_recurrence(q, k, v, la, beta, S0)
    o, S, _ = tile_model(q, k, v, la, beta, S0, mistake=mistake)
    assert max(_rel(o, o_ref), _rel(S, S_ref)) > 1e-3
