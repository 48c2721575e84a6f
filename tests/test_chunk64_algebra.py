"""The chunk algebra of the bf16 prefill kernel (the state advances once per 64-token chunk),
checked in fp64 against the oracle's token loop.

"Kimi K3 -- Architecture Notes", section 1.2, evaluates KDA chunk by chunk: the state is carried
serially across chunks and the work inside a chunk is parallel, with 16-token secondary tiles whose
decay factors are taken relative to a reference point so that the lower bound on log alpha keeps
every factor in range.  The bf16 kernel uses 64-token chunks of four such tiles.  With x the
inclusive prefix sum of log2(alpha) over a tile, e = 2^x, Gamma_i = 2^{x_last} the decay over
tile i, and per key channel

    D_i = prod_{m<i} Gamma_m,   F_i = prod_{m>=i} Gamma_m,   R_{i'}(j) = K_j 2^{-x_j} prod_{m=j}^{i'-1} Gamma_m,

it forms for one chunk from state S (tiles i, j; rows are tokens):

    P_ij = (Q_i e_i) R_i(j)^T (j < i),   P_ii = (Q_i e_i)(K_i 2^{-x_i})^T (s <= r),   M likewise (s < r)
    A_i  = (I + Diag(beta_i) M_ii)^{-1} Diag(beta_i)
    W_i  = A_i (V_i - (K_i e_i D_i) S - sum_{j<i} M_ij W_j)
    O_i  = (Q_i e_i D_i) S + sum_{j<=i} P_ij W_j
    S   <- Diag(F_0) S + sum_i (K_i 2^{-x_i} F_i)^T W_i

This file writes exactly that out in plain NumPy (a library solve serves as each tile's inverse)
and checks, without any GPU:

* it reproduces the token recurrence to rounding under every decay law of the workloads, for
  full and partial chunks and a random initial state;
* with log alpha >= -5 every factor stays inside the normal fp32 range: the tile-relative row
  factors and the diagonal column factors within 2^{+-115.4}, and every chunk-referenced factor
  at most 1 (a factor below the range can only stand for a product that small);
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
FLT_MAX_LOG2 = 128.0
FLT_MIN_NORMAL_LOG2 = -126.0


def bf16(x):
    """Round to the nearest bfloat16 (ties to even), returned as float64."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def chunk_model(q, k, v, log_alpha, beta, S0, op=None, mistake=None):
    """The chunk algebra over one run of tokens (shapes as oracle.kda_recurrence).  `op` rounds
    every matrix-product operand (None: exact).  Returns (o, S_T, ranges) where ranges records
    the largest base-2 exponent of the tile-relative factors and the largest magnitude of the
    chunk-referenced ones."""
    op = op or (lambda a: a)
    T, B, d_k = q.shape
    d_v = v.shape[2]
    C, L = 64, 16
    Tp = -(-T // C) * C
    pad = lambda a: np.concatenate([a, np.zeros((Tp - T,) + a.shape[1:])]) if Tp > T else a
    q, k, v, la, beta = (pad(np.asarray(a, np.float64)) for a in (q, k, v, log_alpha, beta))
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((Tp, B, d_v))
    ranges = {"tile_exp": 0.0, "chunk_factor": 0.0}
    eye = np.eye(L)[None].repeat(B, 0)
    for c0 in range(0, Tp, C):
        t = [slice(c0 + L * i, c0 + L * (i + 1)) for i in range(4)]
        x = [np.cumsum(la[t[i]] * LOG2E, axis=0) for i in range(4)]     # [16, B, d_k]
        ranges["tile_exp"] = max(ranges["tile_exp"], max(float(np.abs(xi).max()) for xi in x))
        e = [np.exp2(xi) for xi in x]
        G = [ei[-1] for ei in e]                                         # [B, d_k] tile decays
        D = [np.prod(G[:i], axis=0) if i else np.ones_like(G[0]) for i in range(4)]
        F = [np.prod(G[i:], axis=0) for i in range(4)]
        if mistake == "D_includes_own_tile":
            D = [np.prod(G[:i + 1], axis=0) for i in range(4)]
        QL = [q[t[i]] * e[i] for i in range(4)]
        KL = [k[t[i]] * e[i] for i in range(4)]
        KB = [k[t[i]] * np.exp2(-x[i]) for i in range(4)]

        def R(ip, j):
            span = G[j:ip] if mistake != "R_without_gap" else G[j:j + 1]
            return KB[j] * np.prod(span, axis=0)

        Qc = [QL[i] * D[i] for i in range(4)]
        K1c = [KL[i] * D[i] for i in range(4)]
        K2c = [KB[i] * F[i] for i in range(4)]
        for a in Qc + K1c + K2c + [R(ip, j) for ip in range(4) for j in range(ip)]:
            ranges["chunk_factor"] = max(ranges["chunk_factor"], float(np.abs(a).max()))
        gram = lambda X, Y: np.einsum("rbc,sbc->brs", op(X), op(Y))      # [B, 16 r, 16 s]
        incl, strict = np.tril(np.ones((L, L))), np.tril(np.ones((L, L)), -1)
        P = {(i, i): gram(QL[i], KB[i]) * incl for i in range(4)}
        M = {(i, i): gram(KL[i], KB[i]) * strict for i in range(4)}
        for i in range(4):
            for j in range(i):
                P[i, j] = gram(QL[i], R(i, j))
                M[i, j] = gram(KL[i], R(i, j))
        A = []
        for i in range(4):
            b = beta[t[i]].T                                             # [B, 16]
            A.append(op(np.linalg.solve(eye + b[:, :, None] * M[i, i], eye) * b[:, None, :]))
        Sop = op(S)
        W = []
        for i in range(4):
            Z = v[t[i]] - np.einsum("rbc,bcv->rbv", op(K1c[i]), Sop)
            if mistake != "drop_cross_M":
                for j in range(i):
                    Z = Z - np.einsum("brs,sbv->rbv", op(M[i, j]), W[j])
            W.append(op(np.einsum("brs,sbv->rbv", A[i], op(Z))))
        for i in range(4):
            oi = np.einsum("rbc,bcv->rbv", op(Qc[i]), Sop)
            for j in range(i + 1):
                oi = oi + np.einsum("brs,sbv->rbv", op(P[i, j]), W[j])
            o[t[i]] = oi
        S = F[0][:, :, None] * S + sum(np.einsum("rbc,rbv->bcv", op(K2c[i]), W[i]) for i in range(4))
    return o[:T], S, ranges


def _case(seed, T, la_law, B=2, d_k=16, d_v=8):
    rng = np.random.default_rng(seed)
    q, k, v, la, beta, S0 = random_case(rng, T, B, d_k, d_v, la_law="zero" if la_law == "floor" else la_law)
    if la_law == "floor":
        la = np.full_like(la, -5.0)
    return q, k, v, la, beta, S0


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


@pytest.mark.parametrize("la_law", ["floor", "uniform53", "softplus", "zero"])
@pytest.mark.parametrize("T", [1, 7, 16, 37, 64, 65, 100, 150, 257])
def test_chunk_algebra_reproduces_the_token_recurrence(la_law, T):
    q, k, v, la, beta, S0 = _case(3 + T, T, la_law)
    o_ref, S_ref = oracle.kda_recurrence(q, k, v, la, beta, S0)
    o, S, _ = chunk_model(q, k, v, la, beta, S0)
    assert _rel(o, o_ref) < 1e-10 and _rel(S, S_ref) < 1e-10


def test_decay_floor_keeps_every_factor_in_fp32_range():
    q, k, v, la, beta, S0 = _case(4, 192, "floor")
    _, _, ranges = chunk_model(q, k, v, la, beta, S0)
    bound = 16 * 5.0 * LOG2E                     # e^{80} = 2^{115.4}: a whole tile at the floor
    assert ranges["tile_exp"] <= bound + 1e-9
    assert bound < FLT_MAX_LOG2 and -bound > FLT_MIN_NORMAL_LOG2
    # the chunk-referenced factors (unit keys and queries) never exceed 1
    assert ranges["chunk_factor"] <= 1.0 + 1e-12


@pytest.mark.parametrize("la_law", ["uniform53", "softplus"])
def test_bf16_operands_stay_within_the_tolerance(la_law):
    """bf16 inputs and bf16 product operands with an fp64 state: the error the 2e-2 tolerance of
    the bf16 workloads has to absorb, at d = 128 over 1024 tokens."""
    rng = np.random.default_rng(6)
    T, B, d = 1024, 2, 128
    q, k, v, la, beta, S0 = random_case(rng, T, B, d, d, la_law=la_law)
    q, k, v = bf16(q), bf16(k), bf16(v)
    S0 = 0.02 * rng.standard_normal((B, d, d))
    o_ref, S_ref = oracle.kda_recurrence(q, k, v, la, beta, S0)
    o, S, _ = chunk_model(q, k, v, la, beta, S0, op=bf16)
    eo, es = _rel(bf16(o), o_ref), _rel(S, S_ref)
    assert eo < 2e-2 and es < 2e-2, (eo, es)
    assert eo > 1e-4          # the rounding is really applied


@pytest.mark.parametrize("mistake", ["D_includes_own_tile", "R_without_gap", "drop_cross_M"])
def test_planted_mistakes_are_caught(mistake):
    q, k, v, la, beta, S0 = _case(12, 150, "softplus")
    o_ref, S_ref = oracle.kda_recurrence(q, k, v, la, beta, S0)
    o, S, _ = chunk_model(q, k, v, la, beta, S0, mistake=mistake)
    assert max(_rel(o, o_ref), _rel(S, S_ref)) > 1e-3
