"""Plain fp64 CPU oracle for the KDA output epilogue.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

What it computes
----------------
"Kimi K3 -- Architecture Notes", section 1.3 (full-rank output gate): the
recurrent output o of each head is normalised head-wise with RMSNorm and
multiplied element-wise by a sigmoid gate computed from the layer input,

    y = Sigmoid(W_g x) (.) RMSNorm(o),

before the output projection W_o (which, like W_g x, lies outside this path:
the gate logits are an input).  RMSNorm over the d_v channels of one
(token, head), with the conventions of the same pages' RMSNorm module
(epsilon 1e-5 inside the square root, fp32 or wider accumulation, a learned
per-channel weight):

    RMSNorm(o)_c = w_c * o_c / sqrt(mean_c'(o_c'^2) + eps).

Readings taken (listed with their reasons in the design notes): one weight
vector w [d_v] shared by the heads (the norm is head-wise over d_v), and w = 1
when no weight is given.

Array conventions (NumPy arrays, upcast exactly to float64):

    o             [T, H, d_v]   recurrent output
    gate_logits   [T, H, d_v]   W_g x, reshaped per head
    weight        [d_v] or None

Parity unpinned: nothing in this file.  Pinned by the ``-m "not gpu"`` tests
against a hand-worked example, Sigmoid(0) = 1/2, scale invariance of the norm,
the unit root-mean-square of its output and the role of the weight.
"""

from __future__ import annotations

import numpy as np

__all__ = ["RMS_EPS", "kda_output_gate_rmsnorm"]

RMS_EPS = 1e-5


def _sigmoid(u):
    e = np.exp(-np.abs(u))
    return np.where(u >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def kda_output_gate_rmsnorm(o, gate_logits, weight=None, eps=RMS_EPS):
    """y = Sigmoid(gate_logits) * RMSNorm(o) over the last axis, in float64."""
    o = np.asarray(o, dtype=np.float64)
    g = np.asarray(gate_logits, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    normed = o / np.sqrt(ms + float(eps))
    if weight is not None:
        normed = normed * np.asarray(weight, dtype=np.float64)
    return _sigmoid(g) * normed
