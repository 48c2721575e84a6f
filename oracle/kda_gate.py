"""Plain fp64 CPU oracle for the lower-bounded KDA gate map.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

What it computes
----------------
"Kimi K3 -- Architecture Notes", section 1.2 (the lower-bounded decay), table,
Kimi K3 row: the per-step log-decay of key channel c of head h is obtained
from a decay logit z by

    g = g_min * Sigmoid(exp(A_h) * z),        g_min = -5 (fixed),

so that alpha = exp(g) lies in (exp(g_min), 1).  A_h is a per-head log-scale
(a learned parameter, initialised to 0, same section).  The write strength is
a sigmoid of its own logit (section 1.1 gives beta in (0,1); the reference
listing of the Kimi K3 visualiser page, "Kimi Delta Attention (KDA)" box,
forms it as the sigmoid of a projection).

The projections that produce the logits (W_alpha k + b_alpha, W_beta k) lie
outside this path: the logits are inputs.

Array conventions (NumPy arrays, upcast exactly to float64):

    g_logits      [T, H, d_k]     decay logits z
    a_log         [H]             per-head log-scale A_h
    beta_logits   [T, H]          write-strength logits

``kda_prefill_gated`` / ``kda_decode_step_gated`` apply the map and then the
recurrence of ``kda_oracle`` (section 1.1) unchanged.

Parity unpinned: nothing in this file.  The map is pinned by the
``-m "not gpu"`` tests against its closed forms (z = 0, z = ln 3, the limits
z -> +-inf), the symmetry Sigmoid(u) + Sigmoid(-u) = 1 and the scaling role of
A_h.
"""

from __future__ import annotations

import numpy as np

from .kda_oracle import kda_decode_step, kda_prefill

__all__ = ["G_MIN", "kda_gate_map", "kda_prefill_gated", "kda_decode_step_gated"]

G_MIN = -5.0


def _sigmoid(u):
    """Logistic function, evaluated without overflow for either sign of u."""
    u = np.asarray(u, dtype=np.float64)
    e = np.exp(-np.abs(u))
    return np.where(u >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def kda_gate_map(g_logits, a_log, beta_logits):
    """Returns (log_alpha [T, H, d_k], beta [T, H]) in float64.

    log_alpha = g_min * Sigmoid(exp(A_h) * z) per section 1.2's table (Kimi K3
    row); beta = Sigmoid(beta logit).
    """
    z = np.asarray(g_logits, dtype=np.float64)
    A = np.asarray(a_log, dtype=np.float64)
    scale = np.exp(A)[None, :, None]            # exp(A_h), one per head
    log_alpha = G_MIN * _sigmoid(scale * z)
    beta = _sigmoid(np.asarray(beta_logits, dtype=np.float64))
    return log_alpha, beta


def kda_prefill_gated(q, k, v, g_logits, a_log, beta_logits, init_state=None, cu_seqlens=None, heads=None):
    """KDA prefill with the decay and write strength given as logits.

    ``heads`` selects a subset of heads as in ``kda_prefill``; ``a_log`` is
    always indexed by the original head numbers.
    """
    la, b = kda_gate_map(g_logits, a_log, beta_logits)
    return kda_prefill(q, k, v, la, b, init_state, cu_seqlens, heads=heads)


def kda_decode_step_gated(q, k, v, g_logits, a_log, beta_logits, state):
    """One decode step with the decay and write strength given as logits."""
    la, b = kda_gate_map(g_logits, a_log, beta_logits)
    return kda_decode_step(q, k, v, la, b, state)
