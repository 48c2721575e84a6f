"""Plain fp64 CPU oracle for the KDA input prologue.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

What it computes
----------------
"Kimi K3 -- Architecture Notes", section 1.1: the q, k and v projections each
pass a short convolution and then Swish, and q and k are then L2-normalised.
The "Kimi K3" visualiser page (tools/llm-vis), in its "Kimi Delta Attention
(KDA)" box, gives the convolution's width (4) and calls it a short convolution
over q/k/v that supplies local context before the update.  Per head and channel c (a depthwise, causal
convolution; the newest input meets the last tap):

    conv(x)_t[c] = sum_{j=0}^{K-1} w[c, j] * x_{t-(K-1)+j}[c],    K = 4,
    swish(u)     = u * Sigmoid(u),
    l2(u)        = u / sqrt(sum_c u[c]^2 + eps),
    q = l2(swish(conv(x_q))),  k = l2(swish(conv(x_k))),  v = swish(conv(x_v)).

Inputs before a sequence's first token are the K-1 entries of a convolution
state (the last K-1 inputs of the previous segment, oldest first), or zeros
when none is given; the final state of a sequence is the last K-1 entries of
its state followed by its inputs.  This is what lets prefill resume and
decode advance one token at a time.

Readings taken (listed with their reasons in the design notes): the notes'
order (Swish, then the L2 norm) where the listing in the visualiser page's KDA
box applies the norm first and leaves v without Swish; no convolution bias; eps = 1e-6 inside
the root of the L2 norm; per-head channel order q (d_k), k (d_k), v (d_v) in
the packed weights and state.

Array conventions (NumPy arrays, upcast exactly to float64):

    x_q, x_k     [T, H, d_k]            x_v  [T, H, d_v]
    conv_w       [H, 2 d_k + d_v, K]    (q channels, then k, then v, per head)
    conv_state   [N, K-1, H, 2 d_k + d_v] or None (zeros)
    cu_seqlens   [N + 1] or None (one sequence)

Parity unpinned: nothing in this file.  Pinned by the ``-m "not gpu"`` tests
against single-tap weights (identity and a pure delay), the impulse response,
split-and-resume through the state, isolation of packed sequences, closed
forms of Swish, unit norm, the place of eps and a hand-worked example of the
order of Swish and the norm.
"""

from __future__ import annotations

import numpy as np

__all__ = ["CONV_K", "L2_EPS", "short_conv", "swish", "l2_normalize", "kda_prologue"]

CONV_K = 4
L2_EPS = 1e-6


def _bounds(T, cu_seqlens):
    if cu_seqlens is None:
        return [(0, T)]
    cu = [int(c) for c in np.asarray(cu_seqlens)]
    return [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def short_conv(x, w, conv_state=None, cu_seqlens=None):
    """Depthwise causal convolution per (head, channel).

    x [T, H, C], w [H, C, K], conv_state [N, K-1, H, C] or None.
    Returns (y [T, H, C], final state [N, K-1, H, C]), in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, H, C = x.shape
    K = w.shape[-1]
    seqs = _bounds(T, cu_seqlens)
    N = len(seqs)
    if conv_state is None:
        state = np.zeros((N, K - 1, H, C))
    else:
        state = np.asarray(conv_state, dtype=np.float64)
    y = np.zeros_like(x)
    final = np.zeros((N, K - 1, H, C))
    for n, (a, b) in enumerate(seqs):
        # the sequence's inputs preceded by its K-1 state entries, oldest first
        ext = np.concatenate([state[n], x[a:b]], axis=0)          # [K-1 + L, H, C]
        for t in range(b - a):
            acc = np.zeros((H, C))
            for j in range(K):
                acc += w[:, :, j] * ext[t + j]                    # ext[t + K-1] is x_t
            y[a + t] = acc
        final[n] = ext[ext.shape[0] - (K - 1):]
    return y, final


def swish(u):
    """u * Sigmoid(u), evaluated stably in float64."""
    u = np.asarray(u, dtype=np.float64)
    e = np.exp(-np.abs(u))
    sig = np.where(u >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return u * sig


def l2_normalize(u, eps=L2_EPS):
    """u / sqrt(sum(u^2) + eps) over the last axis."""
    u = np.asarray(u, dtype=np.float64)
    return u / np.sqrt(np.sum(u * u, axis=-1, keepdims=True) + float(eps))


def kda_prologue(x_q, x_k, x_v, conv_w, conv_state=None, cu_seqlens=None, eps=L2_EPS):
    """q, k, v of the recurrence from the three projection outputs.

    Returns (q [T, H, d_k], k [T, H, d_k], v [T, H, d_v], final conv state
    [N, K-1, H, 2 d_k + d_v]), in float64.
    """
    x_q = np.asarray(x_q, dtype=np.float64)
    x_k = np.asarray(x_k, dtype=np.float64)
    x_v = np.asarray(x_v, dtype=np.float64)
    d_k = x_q.shape[-1]
    x = np.concatenate([x_q, x_k, x_v], axis=-1)                  # per-head channel order q, k, v
    y, final = short_conv(x, conv_w, conv_state, cu_seqlens)
    a = swish(y)
    q = l2_normalize(a[..., :d_k], eps)
    k = l2_normalize(a[..., d_k:2 * d_k], eps)
    v = a[..., 2 * d_k:]
    return q, k, v, final
