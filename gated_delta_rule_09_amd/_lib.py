"""ctypes binding of libkda.so.

Marshalling only: tensors are checked for device, dtype, shape and layout,
outputs are allocated with torch when the caller does not pass them, and the
C entry points of the same names are called with raw device pointers and the
caller's current HIP stream.  Every step of the computation runs in the HIP
kernels; there is no fallback of any kind.  When the library is missing or
cannot be loaded, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK = 0
KDA_F32 = 0
KDA_BF16 = 1
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
           4: "KDA_ERR_ALIGN", 5: "KDA_ERR_NO_DEVICE", 6: "KDA_ERR_HIP", 7: "KDA_ERR_VALUE"}
ABI_VERSION = 4
RMS_EPS = 1e-5      # epsilon of the model's RMSNorm
SPLIT_SCRATCH_BYTES = 64 << 20   # KDA_SPLIT_SCRATCH_BYTES: the no-alloc split's scratch per device

# Every symbol include/kda.h declares, with its ctypes signature.
_VP, _I32, _I64, _F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
SIGNATURES = {
    "kda_abi_version": (ctypes.c_int, []),
    "kda_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kda_last_error": (ctypes.c_char_p, []),
    "kda_wait_giveups": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), _I32, _VP]),
    "kda_chunk_prefill": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                          _I32, _I64, _I32, _I32, _I32, ctypes.c_int,
                                          _VP, _VP, _VP]),
    "kda_decode_step": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP,
                                        _I32, _I32, _I32, _I32, ctypes.c_int, _VP, _VP]),
    "kda_chunk_prefill_gated": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                                _I32, _I64, _I32, _I32, _I32, ctypes.c_int,
                                                _VP, _VP, _VP]),
    "kda_decode_step_gated": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                              _I32, _I32, _I32, _I32, ctypes.c_int, _VP, _VP]),
    "kda_output_gate_rmsnorm": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I32, _F32, ctypes.c_int, _VP, _VP]),
    "kda_chunk_prefill_gated_epilogue": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _F32, _VP, _VP,
                                                         _I32, _I64, _I32, _I32, _I32, ctypes.c_int,
                                                         _VP, _VP, _VP]),
    "kda_decode_step_gated_epilogue": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _F32, _VP,
                                                       _I32, _I32, _I32, _I32, ctypes.c_int, _VP, _VP]),
    "kda_short_conv_prologue": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I32,
                                                ctypes.c_int, _VP, _VP, _VP, _VP, _VP]),
    "kda_decode_step_fused": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _F32, _VP,
                                              _I32, _I32, _I32, _I32, ctypes.c_int, _VP, _VP]),
    "kda_chunk_prefill_split": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I32, _I32, _I32, ctypes.c_int,
                                                _I32, _VP, ctypes.c_size_t, _VP, _VP, _VP]),
    "kda_chunk_prefill_gated_split": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I32, _I32, _I32,
                                                      ctypes.c_int, _I32, _VP, ctypes.c_size_t, _VP, _VP, _VP]),
    "kda_split_workspace_bytes": (ctypes.c_size_t, [_I64, _I32, _I32, _I32, ctypes.c_int, _I32]),
    "kda_chunk_prefill_split_noalloc": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I32, _I32, _I32,
                                                        ctypes.c_int, _I32, _VP, _VP, _VP]),
    "kda_split_segments": (_I32, [_I64, _I32, _I32, _I32, _I32]),
}

_lib = None


class KDAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = _lib
        detail = ""
        if lib is not None:
            detail = lib.kda_status_string(status).decode()
            last = lib.kda_last_error().decode()
            if last:
                detail += f" ({last})"
        super().__init__(f"{fn} returned {_STATUS.get(status, status)}: {detail}")
        self.status = status


def load(path: Optional[str] = None):
    """Load libkda.so (once) and declare its signatures.  Raises if it is absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run `python -m gated_delta_rule_09_amd.build` first")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.kda_abi_version() != ABI_VERSION:
        raise RuntimeError("libkda ABI version mismatch")
    if path is None:
        _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {dt}")


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def kda_chunk_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      log_alpha: torch.Tensor, beta: torch.Tensor,
                      init_state: Optional[torch.Tensor] = None,
                      cu_seqlens: Optional[torch.Tensor] = None,
                      o: Optional[torch.Tensor] = None,
                      final_state: Optional[torch.Tensor] = None,
                      output_final_state: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA prefill; see include/kda.h.  Returns (o, final_state)."""
    lib = load()
    T, H, d_k = q.shape
    d_v = v.shape[2]
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    _check(q, "q", (T, H, d_k), dt, dev)
    _check(k, "k", (T, H, d_k), dt, dev)
    _check(v, "v", (T, H, d_v), dt, dev)
    _check(log_alpha, "log_alpha", (T, H, d_k), torch.float32, dev)
    _check(beta, "beta", (T, H), torch.float32, dev)
    if init_state is not None:
        _check(init_state, "init_state", (N, H, d_k, d_v), torch.float32, dev)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if o is None:
        o = torch.empty((T, H, d_v), dtype=dt, device=dev)
    _check(o, "o", (T, H, d_v), dt, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, d_k, d_v), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (N, H, d_k, d_v), torch.float32, dev)
    st = lib.kda_chunk_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                               _ptr(init_state), _ptr(cu_seqlens), N, T, H, d_k, d_v, code,
                               _ptr(o), _ptr(final_state), _stream_handle(dev))
    if st != KDA_OK:
        raise KDAError("kda_chunk_prefill", st)
    return o, final_state


def kda_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    log_alpha: torch.Tensor, beta: torch.Tensor, state: torch.Tensor,
                    o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One KDA decode step; ``state`` is updated in place.  Returns o [N, H, d_v]."""
    lib = load()
    N, H, d_k = q.shape
    d_v = v.shape[2]
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    _check(q, "q", (N, H, d_k), dt, dev)
    _check(k, "k", (N, H, d_k), dt, dev)
    _check(v, "v", (N, H, d_v), dt, dev)
    _check(log_alpha, "log_alpha", (N, H, d_k), torch.float32, dev)
    _check(beta, "beta", (N, H), torch.float32, dev)
    _check(state, "state", (N, H, d_k, d_v), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, d_v), dtype=dt, device=dev)
    _check(o, "o", (N, H, d_v), dt, dev)
    st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(state),
                             N, H, d_k, d_v, code, _ptr(o), _stream_handle(dev))
    if st != KDA_OK:
        raise KDAError("kda_decode_step", st)
    return o


def kda_chunk_prefill_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            g_logits: torch.Tensor, a_log: torch.Tensor, beta_logits: torch.Tensor,
                            init_state: Optional[torch.Tensor] = None,
                            cu_seqlens: Optional[torch.Tensor] = None,
                            o: Optional[torch.Tensor] = None,
                            final_state: Optional[torch.Tensor] = None,
                            output_final_state: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA prefill from decay / write-strength logits (see include/kda.h,
    kda_chunk_prefill_gated).  Returns (o, final_state)."""
    lib = load()
    T, H, d_k = q.shape
    d_v = v.shape[2]
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    _check(q, "q", (T, H, d_k), dt, dev)
    _check(k, "k", (T, H, d_k), dt, dev)
    _check(v, "v", (T, H, d_v), dt, dev)
    _check(g_logits, "g_logits", (T, H, d_k), dt, dev)
    _check(a_log, "a_log", (H,), torch.float32, dev)
    _check(beta_logits, "beta_logits", (T, H), torch.float32, dev)
    if init_state is not None:
        _check(init_state, "init_state", (N, H, d_k, d_v), torch.float32, dev)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if o is None:
        o = torch.empty((T, H, d_v), dtype=dt, device=dev)
    _check(o, "o", (T, H, d_v), dt, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, d_k, d_v), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (N, H, d_k, d_v), torch.float32, dev)
    st = lib.kda_chunk_prefill_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g_logits), _ptr(a_log), _ptr(beta_logits),
                                     _ptr(init_state), _ptr(cu_seqlens), N, T, H, d_k, d_v, code,
                                     _ptr(o), _ptr(final_state), _stream_handle(dev))
    if st != KDA_OK:
        raise KDAError("kda_chunk_prefill_gated", st)
    return o, final_state


def split_segments(total_T: int, H: int, d_k: int, d_v: int, num_cus: Optional[int] = None,
                   device: Optional[torch.device] = None) -> int:
    """Segment count for the time-split prefill (include/kda.h, kda_split_segments).
    num_cus defaults to the compute units of ``device`` (the current device)."""
    lib = load()
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(device or torch.cuda.current_device()).multi_processor_count
    return int(lib.kda_split_segments(int(total_T), int(H), int(d_k), int(d_v), int(num_cus)))


def split_workspace_bytes(total_T: int, H: int, d_k: int, d_v: int, dtype: torch.dtype, segments: int) -> int:
    """Workspace bytes of a time-split prefill (include/kda.h, kda_split_workspace_bytes)."""
    return int(load().kda_split_workspace_bytes(int(total_T), int(H), int(d_k), int(d_v), _dtype_code(dtype),
                                                int(segments)))


def _split_call(name: str, q, k, v, decay, decay_dtype, a_log, beta, init_state, segments, workspace, o,
                final_state, output_final_state, noalloc=False):
    lib = load()
    T, H, d_k = q.shape
    d_v = v.shape[2]
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    _check(q, "q", (T, H, d_k), dt, dev)
    _check(k, "k", (T, H, d_k), dt, dev)
    _check(v, "v", (T, H, d_v), dt, dev)
    _check(decay, "decay", (T, H, d_k), decay_dtype, dev)
    if a_log is not None:
        _check(a_log, "a_log", (H,), torch.float32, dev)
    _check(beta, "beta", (T, H), torch.float32, dev)
    if init_state is not None:
        _check(init_state, "init_state", (1, H, d_k, d_v), torch.float32, dev)
    if segments is None:
        segments = split_segments(T, H, d_k, d_v, device=dev)
    if o is None:
        o = torch.empty((T, H, d_v), dtype=dt, device=dev)
    _check(o, "o", (T, H, d_v), dt, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((1, H, d_k, d_v), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (1, H, d_k, d_v), torch.float32, dev)
    need = int(lib.kda_split_workspace_bytes(T, H, d_k, d_v, code, int(segments)))
    if noalloc:
        st = getattr(lib, name)(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(beta), _ptr(init_state), T, H, d_k,
                                d_v, code, int(segments), _ptr(o), _ptr(final_state), _stream_handle(dev))
        if st != KDA_OK:
            raise KDAError(name, st)
        return o, final_state
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is not None and workspace.device != dev:
        raise ValueError(f"workspace is on {workspace.device}, expected {dev}")
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(decay)]
    if a_log is not None:
        args.append(_ptr(a_log))
    args += [_ptr(beta), _ptr(init_state), T, H, d_k, d_v, code, int(segments), _ptr(workspace), ws_bytes,
             _ptr(o), _ptr(final_state), _stream_handle(dev)]
    st = getattr(lib, name)(*args)
    if st != KDA_OK:
        raise KDAError(name, st)
    return o, final_state


def kda_chunk_prefill_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            log_alpha: torch.Tensor, beta: torch.Tensor,
                            init_state: Optional[torch.Tensor] = None,
                            segments: Optional[int] = None,
                            workspace: Optional[torch.Tensor] = None,
                            o: Optional[torch.Tensor] = None,
                            final_state: Optional[torch.Tensor] = None,
                            output_final_state: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Prefill of one sequence split in time (include/kda.h, kda_chunk_prefill_split).
    segments=None asks the library's cost model for the device; the workspace is
    allocated here unless given (a device tensor of at least split_workspace_bytes
    bytes).  Returns (o, final_state) with final_state [1, H, d_k, d_v]."""
    return _split_call("kda_chunk_prefill_split", q, k, v, log_alpha, torch.float32, None, beta, init_state,
                       segments, workspace, o, final_state, output_final_state)


def kda_chunk_prefill_split_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                    log_alpha: torch.Tensor, beta: torch.Tensor,
                                    init_state: Optional[torch.Tensor] = None,
                                    segments: Optional[int] = None,
                                    o: Optional[torch.Tensor] = None,
                                    final_state: Optional[torch.Tensor] = None,
                                    output_final_state: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The time-split prefill on the library's own scratch (include/kda.h,
    kda_chunk_prefill_split_noalloc): the C call allocates nothing.  Pass o and
    final_state to keep this wrapper from allocating them."""
    return _split_call("kda_chunk_prefill_split_noalloc", q, k, v, log_alpha, torch.float32, None, beta, init_state,
                       segments, None, o, final_state, output_final_state, noalloc=True)


def kda_chunk_prefill_gated_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                  g_logits: torch.Tensor, a_log: torch.Tensor, beta_logits: torch.Tensor,
                                  init_state: Optional[torch.Tensor] = None,
                                  segments: Optional[int] = None,
                                  workspace: Optional[torch.Tensor] = None,
                                  o: Optional[torch.Tensor] = None,
                                  final_state: Optional[torch.Tensor] = None,
                                  output_final_state: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated prefill of one sequence split in time (include/kda.h, kda_chunk_prefill_gated_split)."""
    return _split_call("kda_chunk_prefill_gated_split", q, k, v, g_logits, q.dtype, a_log, beta_logits, init_state,
                       segments, workspace, o, final_state, output_final_state)


def kda_decode_step_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          g_logits: torch.Tensor, a_log: torch.Tensor, beta_logits: torch.Tensor,
                          state: torch.Tensor, o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One KDA decode step from decay / write-strength logits; ``state`` is updated
    in place.  Returns o [N, H, d_v]."""
    lib = load()
    N, H, d_k = q.shape
    d_v = v.shape[2]
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    _check(q, "q", (N, H, d_k), dt, dev)
    _check(k, "k", (N, H, d_k), dt, dev)
    _check(v, "v", (N, H, d_v), dt, dev)
    _check(g_logits, "g_logits", (N, H, d_k), dt, dev)
    _check(a_log, "a_log", (H,), torch.float32, dev)
    _check(beta_logits, "beta_logits", (N, H), torch.float32, dev)
    _check(state, "state", (N, H, d_k, d_v), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, d_v), dtype=dt, device=dev)
    _check(o, "o", (N, H, d_v), dt, dev)
    st = lib.kda_decode_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g_logits), _ptr(a_log), _ptr(beta_logits),
                                   _ptr(state), N, H, d_k, d_v, code, _ptr(o), _stream_handle(dev))
    if st != KDA_OK:
        raise KDAError("kda_decode_step_gated", st)
    return o


def _check_epilogue_args(out_gate: torch.Tensor, norm_weight: Optional[torch.Tensor], shape, dt, dev):
    _check(out_gate, "out_gate_logits", shape, dt, dev)
    if norm_weight is not None:
        _check(norm_weight, "norm_weight", (shape[-1],), torch.float32, dev)


def kda_output_gate_rmsnorm(o: torch.Tensor, gate_logits: torch.Tensor,
                            norm_weight: Optional[torch.Tensor] = None, eps: float = RMS_EPS,
                            y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Output epilogue y = Sigmoid(gate_logits) * w * o / sqrt(mean(o^2) + eps) over
    the last axis (see include/kda.h).  ``y`` may be ``o`` or ``gate_logits``."""
    lib = load()
    dev, dt = o.device, o.dtype
    code = _dtype_code(dt)
    if o.dim() < 1:
        raise ValueError("o must have a channel axis")
    d_v = o.shape[-1]
    _check(o, "o", o.shape, dt, dev)
    _check_epilogue_args(gate_logits, norm_weight, o.shape, dt, dev)
    if y is None:
        y = torch.empty_like(o)
    _check(y, "y", o.shape, dt, dev)
    rows = o.numel() // d_v if d_v else 0
    st = lib.kda_output_gate_rmsnorm(_ptr(o), _ptr(gate_logits), _ptr(norm_weight), rows, d_v, float(eps), code,
                                     _ptr(y), _stream_handle(dev))
    if st != KDA_OK:
        raise KDAError("kda_output_gate_rmsnorm", st)
    return y


def kda_chunk_prefill_gated_epilogue(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                     g_logits: torch.Tensor, a_log: torch.Tensor, beta_logits: torch.Tensor,
                                     out_gate_logits: torch.Tensor, norm_weight: Optional[torch.Tensor] = None,
                                     eps: float = RMS_EPS,
                                     init_state: Optional[torch.Tensor] = None,
                                     cu_seqlens: Optional[torch.Tensor] = None,
                                     y: Optional[torch.Tensor] = None,
                                     final_state: Optional[torch.Tensor] = None,
                                     output_final_state: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated chunkwise prefill followed by the output epilogue (see include/kda.h,
    kda_chunk_prefill_gated_epilogue).  Returns (y, final_state)."""
    lib = load()
    T, H, d_k = q.shape
    d_v = v.shape[2]
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    _check(q, "q", (T, H, d_k), dt, dev)
    _check(k, "k", (T, H, d_k), dt, dev)
    _check(v, "v", (T, H, d_v), dt, dev)
    _check(g_logits, "g_logits", (T, H, d_k), dt, dev)
    _check(a_log, "a_log", (H,), torch.float32, dev)
    _check(beta_logits, "beta_logits", (T, H), torch.float32, dev)
    _check_epilogue_args(out_gate_logits, norm_weight, (T, H, d_v), dt, dev)
    if init_state is not None:
        _check(init_state, "init_state", (N, H, d_k, d_v), torch.float32, dev)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if y is None:
        y = torch.empty((T, H, d_v), dtype=dt, device=dev)
    _check(y, "y", (T, H, d_v), dt, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, d_k, d_v), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (N, H, d_k, d_v), torch.float32, dev)
    st = lib.kda_chunk_prefill_gated_epilogue(_ptr(q), _ptr(k), _ptr(v), _ptr(g_logits), _ptr(a_log),
                                              _ptr(beta_logits), _ptr(out_gate_logits), _ptr(norm_weight),
                                              float(eps), _ptr(init_state), _ptr(cu_seqlens), N, T, H, d_k, d_v,
                                              code, _ptr(y), _ptr(final_state), _stream_handle(dev))
    if st != KDA_OK:
        raise KDAError("kda_chunk_prefill_gated_epilogue", st)
    return y, final_state


def kda_decode_step_gated_epilogue(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                   g_logits: torch.Tensor, a_log: torch.Tensor, beta_logits: torch.Tensor,
                                   out_gate_logits: torch.Tensor, state: torch.Tensor,
                                   norm_weight: Optional[torch.Tensor] = None, eps: float = RMS_EPS,
                                   y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One gated decode step with the output epilogue fused; ``state`` is updated
    in place.  Returns y [N, H, d_v]."""
    lib = load()
    N, H, d_k = q.shape
    d_v = v.shape[2]
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    _check(q, "q", (N, H, d_k), dt, dev)
    _check(k, "k", (N, H, d_k), dt, dev)
    _check(v, "v", (N, H, d_v), dt, dev)
    _check(g_logits, "g_logits", (N, H, d_k), dt, dev)
    _check(a_log, "a_log", (H,), torch.float32, dev)
    _check(beta_logits, "beta_logits", (N, H), torch.float32, dev)
    _check_epilogue_args(out_gate_logits, norm_weight, (N, H, d_v), dt, dev)
    _check(state, "state", (N, H, d_k, d_v), torch.float32, dev)
    if y is None:
        y = torch.empty((N, H, d_v), dtype=dt, device=dev)
    _check(y, "y", (N, H, d_v), dt, dev)
    st = lib.kda_decode_step_gated_epilogue(_ptr(q), _ptr(k), _ptr(v), _ptr(g_logits), _ptr(a_log),
                                            _ptr(beta_logits), _ptr(out_gate_logits), _ptr(norm_weight),
                                            float(eps), _ptr(state), N, H, d_k, d_v, code, _ptr(y),
                                            _stream_handle(dev))
    if st != KDA_OK:
        raise KDAError("kda_decode_step_gated_epilogue", st)
    return y


def kda_short_conv_prologue(x_q: torch.Tensor, x_k: torch.Tensor, x_v: torch.Tensor, conv_w: torch.Tensor,
                            conv_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
                            q: Optional[torch.Tensor] = None, k: Optional[torch.Tensor] = None,
                            v: Optional[torch.Tensor] = None, conv_state_out: Optional[torch.Tensor] = None,
                            output_conv_state: bool = True):
    """Short convolution, Swish and the L2 norm of q and k (see include/kda.h,
    kda_short_conv_prologue).  Returns (q, k, v, conv_state_out)."""
    lib = load()
    T, H, d_k = x_q.shape
    d_v = x_v.shape[2]
    dev, dt = x_q.device, x_q.dtype
    code = _dtype_code(dt)
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    C = 2 * d_k + d_v
    _check(x_q, "x_q", (T, H, d_k), dt, dev)
    _check(x_k, "x_k", (T, H, d_k), dt, dev)
    _check(x_v, "x_v", (T, H, d_v), dt, dev)
    _check(conv_w, "conv_w", (H, C, 4), torch.float32, dev)
    if conv_state is not None:
        _check(conv_state, "conv_state", (N, 3, H, C), dt, dev)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    q = torch.empty_like(x_q) if q is None else q
    k = torch.empty_like(x_k) if k is None else k
    v = torch.empty_like(x_v) if v is None else v
    _check(q, "q", (T, H, d_k), dt, dev)
    _check(k, "k", (T, H, d_k), dt, dev)
    _check(v, "v", (T, H, d_v), dt, dev)
    if output_conv_state and conv_state_out is None:
        conv_state_out = torch.empty((N, 3, H, C), dtype=dt, device=dev)
    if conv_state_out is not None:
        _check(conv_state_out, "conv_state_out", (N, 3, H, C), dt, dev)
    st = lib.kda_short_conv_prologue(_ptr(x_q), _ptr(x_k), _ptr(x_v), _ptr(conv_w), _ptr(conv_state),
                                     _ptr(cu_seqlens), N, T, H, d_k, d_v, code, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(conv_state_out), _stream_handle(dev))
    if st != KDA_OK:
        raise KDAError("kda_short_conv_prologue", st)
    return q, k, v, conv_state_out


def kda_decode_step_fused(x_q: torch.Tensor, x_k: torch.Tensor, x_v: torch.Tensor, conv_w: torch.Tensor,
                          conv_state: torch.Tensor, g_logits: torch.Tensor, a_log: torch.Tensor,
                          beta_logits: torch.Tensor, out_gate_logits: torch.Tensor, state: torch.Tensor,
                          norm_weight: Optional[torch.Tensor] = None, eps: float = RMS_EPS,
                          y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One whole decode step (prologue, gate maps, recurrence, epilogue) in one
    kernel; ``conv_state`` and ``state`` are updated in place.  Returns y [N, H, d_v]."""
    lib = load()
    N, H, d_k = x_q.shape
    d_v = x_v.shape[2]
    dev, dt = x_q.device, x_q.dtype
    code = _dtype_code(dt)
    C = 2 * d_k + d_v
    _check(x_q, "x_q", (N, H, d_k), dt, dev)
    _check(x_k, "x_k", (N, H, d_k), dt, dev)
    _check(x_v, "x_v", (N, H, d_v), dt, dev)
    _check(conv_w, "conv_w", (H, C, 4), torch.float32, dev)
    _check(conv_state, "conv_state", (N, 3, H, C), dt, dev)
    _check(g_logits, "g_logits", (N, H, d_k), dt, dev)
    _check(a_log, "a_log", (H,), torch.float32, dev)
    _check(beta_logits, "beta_logits", (N, H), torch.float32, dev)
    _check_epilogue_args(out_gate_logits, norm_weight, (N, H, d_v), dt, dev)
    _check(state, "state", (N, H, d_k, d_v), torch.float32, dev)
    if y is None:
        y = torch.empty((N, H, d_v), dtype=dt, device=dev)
    _check(y, "y", (N, H, d_v), dt, dev)
    st = lib.kda_decode_step_fused(_ptr(x_q), _ptr(x_k), _ptr(x_v), _ptr(conv_w), _ptr(conv_state), _ptr(g_logits),
                                   _ptr(a_log), _ptr(beta_logits), _ptr(out_gate_logits), _ptr(norm_weight),
                                   float(eps), _ptr(state), N, H, d_k, d_v, code, _ptr(y), _stream_handle(dev))
    if st != KDA_OK:
        raise KDAError("kda_decode_step_fused", st)
    return y


def wait_giveups(reset: bool = True, device=None) -> int:
    """Count of bounded in-kernel waits that ran out on the device since the
    last reset (0 when every wait ended normally); synchronises the current
    stream."""
    lib = load()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    n = ctypes.c_uint32(0)
    with torch.cuda.device(dev):
        st = lib.kda_wait_giveups(ctypes.byref(n), 1 if reset else 0, _stream_handle(dev))
    if st != KDA_OK:
        raise KDAError("kda_wait_giveups", st)
    return int(n.value)
