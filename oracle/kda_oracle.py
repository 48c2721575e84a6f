"""Plain fp64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

What it computes
----------------
"Kimi K3 -- Architecture Notes", section 1.1 (Kimi Delta Attention), defines one
head of KDA as the recurrence

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t = S_t^T q_t

with the state S in R^{d_k x d_v} (constant in size, per the same section), alpha_t a
per-channel retention factor in (0,1)^{d_k} and beta_t a scalar write strength.
The oracle evaluates that definition literally, one token at a time, in fp64,
with alpha_t = exp(log_alpha_t) (the same notes, section 1.2, parameterise the
decay through its logarithm g = log alpha).  The loop is vectorised only over
independent (sequence, head) pairs; there is no chunking, blocking or
reordering of the token loop.

Readings of the pages taken here (each is listed with its reason in the design
notes of the repository):

* The notes' form (decay applied before the delta correction) is used, not the
  visualiser page's variant that forms the correction from the undecayed state;
  the two agree exactly when alpha = 1.
* alpha scales the d_k rows of S (the notes give alpha in (0,1)^{d_k} and
  S in R^{d_k x d_v}).
* No 1/sqrt(d_k) output scale: the notes write o_t = S_t^T q_t.
* The closed ranges log_alpha in [-5, 0] and beta in [0, 1] are accepted; the
  oracle itself is exact for any finite inputs.

Array conventions (all arguments are NumPy arrays; any float dtype is upcast
exactly to float64 before use):

    q, k          [T, H, d_k]      token-major, heads in the middle
    v             [T, H, d_v]
    log_alpha     [T, H, d_k]
    beta          [T, H]
    init_state    [N, H, d_k, d_v] or None (zeros)
    cu_seqlens    [N + 1] int, cu[0] = 0, non-decreasing, cu[N] = T; or None
                  meaning one sequence covering all T tokens

Parity unpinned: nothing in this file.  Every function is pinned by the
``-m "not gpu"`` tests against closed forms, invariants and brute force.
"""

from __future__ import annotations

import numpy as np

__all__ = ["kda_prefill", "kda_decode_step", "kda_recurrence"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kda_recurrence(q, k, v, log_alpha, beta, S0):
    """Run the section-1.1 recurrence over one run of tokens.

    q, k: [T, B, d_k]; v: [T, B, d_v]; log_alpha: [T, B, d_k]; beta: [T, B];
    S0: [B, d_k, d_v].  B is any number of independent (sequence, head) pairs.
    Returns (o [T, B, d_v], S_T [B, d_k, d_v]) in float64.

    Per token t and pair b:
        D   = Diag(exp(log_alpha_t))           retention, acts on the d_k rows
        S'  = D S_{t-1}
        S_t = (I - beta_t k_t k_t^T) S' + beta_t k_t v_t^T
            = S' + beta_t k_t (v_t - S'^T k_t)^T
        o_t = S_t^T q_t
    """
    q, k, v, la, b = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(beta)
    S = _f64(S0).copy()
    T = q.shape[0]
    o = np.zeros(v.shape, dtype=np.float64)
    for t in range(T):
        S = np.exp(la[t])[:, :, None] * S                      # Diag(alpha_t) S_{t-1}
        pred = np.einsum("bkv,bk->bv", S, k[t])                 # (Diag(alpha_t) S_{t-1})^T k_t
        S = S + b[t][:, None, None] * (k[t][:, :, None] * (v[t] - pred)[:, None, :])
        o[t] = np.einsum("bkv,bk->bv", S, q[t])                 # S_t^T q_t
    return o, S


def kda_prefill(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, heads=None):
    """KDA over a packed batch of sequences (prefill).

    Returns (o [T, H', d_v], final_state [N, H', d_k, d_v]) in float64, where
    H' = H, or len(heads) when ``heads`` selects a subset of head indices (the
    other heads are independent and are simply not computed).

    Sequence n owns tokens [cu[n], cu[n+1]); it starts from init_state[n]
    (zeros when init_state is None) and its state after its last token is
    final_state[n].  A zero-length sequence returns its initial state.
    """
    q = np.asarray(q)
    T, H, d_k = q.shape
    d_v = np.asarray(v).shape[2]
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    hs = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    Hs = hs.shape[0]
    if init_state is None:
        S0_all = np.zeros((N, Hs, d_k, d_v))
    else:
        S0_all = _f64(init_state)[:, hs]
    o = np.zeros((T, Hs, d_v))
    final = np.zeros((N, Hs, d_k, d_v))
    for n in range(N):
        a, e = int(cu[n]), int(cu[n + 1])
        sl = slice(a, e)
        o_n, S_n = kda_recurrence(
            np.asarray(q)[sl][:, hs], np.asarray(k)[sl][:, hs], np.asarray(v)[sl][:, hs],
            np.asarray(log_alpha)[sl][:, hs], np.asarray(beta)[sl][:, hs], S0_all[n])
        o[sl] = o_n
        final[n] = S_n
    return o, final


def kda_decode_step(q, k, v, log_alpha, beta, state):
    """One decode step: every (sequence, head) pair advances by one token.

    q, k, log_alpha: [N, H, d_k]; v: [N, H, d_v]; beta: [N, H];
    state: [N, H, d_k, d_v].  Returns (o [N, H, d_v], new_state) in float64;
    the input state array is not modified.  This is the same recurrence body
    as ``kda_recurrence`` applied to a single token.
    """
    q = _f64(q)
    N, H, d_k = q.shape
    d_v = np.asarray(v).shape[2]
    B = N * H
    o, S = kda_recurrence(
        q.reshape(1, B, d_k), _f64(k).reshape(1, B, d_k), _f64(v).reshape(1, B, d_v),
        _f64(log_alpha).reshape(1, B, d_k), _f64(beta).reshape(1, B),
        _f64(state).reshape(B, d_k, d_v))
    return o.reshape(N, H, d_v), S.reshape(N, H, d_k, d_v)
