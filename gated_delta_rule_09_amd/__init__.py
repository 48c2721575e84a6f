"""MI355X (gfx950) Kimi Delta Attention: chunkwise prefill and decode.

The computation lives in libkda.so (hand-written HIP kernels behind the C ABI
of include/kda.h).  This package only marshals torch tensors into that ABI.
"""
from ._lib import (KDAError, kda_chunk_prefill, kda_chunk_prefill_gated, kda_decode_step,
                   kda_decode_step_gated, load)

__all__ = ["kda_chunk_prefill", "kda_decode_step", "kda_chunk_prefill_gated", "kda_decode_step_gated",
           "load", "KDAError"]
