"""MI355X (gfx950) Kimi Delta Attention: chunkwise prefill, decode and the
output epilogue.

The computation lives in libkda.so (hand-written HIP kernels behind the C ABI
of include/kda.h).  This package only marshals torch tensors into that ABI.
"""
from ._lib import (RMS_EPS, KDAError, kda_chunk_prefill, kda_chunk_prefill_gated,
                   kda_chunk_prefill_gated_epilogue, kda_decode_step, kda_decode_step_gated,
                   kda_decode_step_gated_epilogue, kda_output_gate_rmsnorm, kda_short_conv_prologue, kda_decode_step_fused, load,
                   kda_chunk_prefill_split, kda_chunk_prefill_gated_split, split_segments,
                   split_workspace_bytes, wait_giveups, kda_chunk_prefill_split_noalloc, SPLIT_SCRATCH_BYTES)

__all__ = ["kda_chunk_prefill", "kda_decode_step", "kda_chunk_prefill_gated", "kda_decode_step_gated",
           "kda_output_gate_rmsnorm", "kda_chunk_prefill_gated_epilogue", "kda_decode_step_gated_epilogue",
           "kda_short_conv_prologue", "kda_decode_step_fused", "kda_chunk_prefill_split",
           "kda_chunk_prefill_gated_split", "split_segments", "split_workspace_bytes", "RMS_EPS", "load", "KDAError",
           "wait_giveups", "kda_chunk_prefill_split_noalloc", "SPLIT_SCRATCH_BYTES"]
