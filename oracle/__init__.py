"""fp64 CPU oracle for Kimi Delta Attention -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The HIP library never does.
"""
from .kda_epilogue import RMS_EPS, kda_output_gate_rmsnorm
from .kda_gate import G_MIN, kda_decode_step_gated, kda_gate_map, kda_prefill_gated
from .kda_prologue import CONV_K, L2_EPS, kda_prologue, l2_normalize, short_conv, swish
from .kda_oracle import kda_decode_step, kda_prefill, kda_recurrence

__all__ = ["kda_prefill", "kda_decode_step", "kda_recurrence",
           "G_MIN", "kda_gate_map", "kda_prefill_gated", "kda_decode_step_gated",
           "RMS_EPS", "kda_output_gate_rmsnorm",
           "CONV_K", "L2_EPS", "short_conv", "swish", "l2_normalize", "kda_prologue"]
