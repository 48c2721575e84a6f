"""Seeded synthetic inputs for KDA prefill and decode.

This module only draws random tensors with fixed laws and shapes.  It holds
none of the recurrence's arithmetic, and both the HIP path's tests/benchmark
and the fp64 oracle receive exactly the tensors it returns.

Laws (one per workload; draws happen in the fixed order q, k, v, beta logits,
log-alpha noise, initial state):

* q, k ~ N(0, 1), each token-head vector scaled to unit L2 norm in fp32, then
  cast to the working dtype (bf16 keeps the norm within about 2^-8 of 1).
* v ~ N(0, 1), cast to the working dtype.
* beta = sigmoid(N(0, 1)), fp32.
* log_alpha, fp32, per (token, head, channel), one of
    "softplus":  -min(softplus(N(0, 1)), 5)    values in [-5, 0)
    "uniform53": U[-5, -3]                     pushed towards the -5 floor
    "zero":      0                             no decay (alpha = 1)
    "floor":     -5                            every channel at the floor
* initial state ~ N(0, 0.02) (standard deviation 0.02), fp32, or zeros.
* packed lengths: integers uniform on {lo, ..., hi}.

Large tensors are drawn on the target device with a seeded torch generator so
that 64K- and 1M-token workloads do not pass through host memory.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

LOG_ALPHA_LAWS = ("softplus", "uniform53", "zero", "floor")

# Workloads, named by what they are.
WORKLOADS = {
    "tiny_fp32": dict(lengths=[256], H=2, d=64, dtype="f32", la_law="softplus", init="zeros", seed=0),
    "bf16_4k": dict(lengths=[4096], H=96, d=128, dtype="bf16", la_law="softplus", init="normal", seed=1),
    "varlen16": dict(lengths="uniform16_1k_8k", H=96, d=128, dtype="bf16", la_law="softplus", init="normal", seed=2),
    "long_64k": dict(lengths=[65536], H=96, d=128, dtype="bf16", la_law="uniform53", init="normal", seed=3),
    "long_1m": dict(lengths=[1048576], H=96, d=128, dtype="bf16", la_law="uniform53", init="normal", seed=3),
}
DECODE_WORKLOAD = dict(N=512, H=96, d=128, dtype="bf16", la_law="softplus", seed=4, steps=100)


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def varlen_lengths(seed: int, count: int = 16, lo: int = 1024, hi: int = 8192) -> list:
    """Sequence lengths uniform on the integers {lo, ..., hi} (inclusive)."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, size=count)]


def workload_lengths(name: str) -> list:
    spec = WORKLOADS[name]
    if spec["lengths"] == "uniform16_1k_8k":
        return varlen_lengths(spec["seed"])
    return list(spec["lengths"])


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def _log_alpha(shape, law: str, g: torch.Generator, device) -> torch.Tensor:
    if law == "softplus":
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return -torch.clamp(torch.nn.functional.softplus(z), max=5.0)
    if law == "uniform53":
        u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        return -5.0 + 2.0 * u
    if law == "zero":
        return torch.zeros(shape, device=device, dtype=torch.float32)
    if law == "floor":
        return torch.full(shape, -5.0, device=device, dtype=torch.float32)
    raise ValueError(f"unknown log-alpha law {law!r}")


@dataclass
class PrefillInputs:
    q: torch.Tensor            # [T, H, d_k]  dtype
    k: torch.Tensor            # [T, H, d_k]  dtype
    v: torch.Tensor            # [T, H, d_v]  dtype
    log_alpha: torch.Tensor    # [T, H, d_k]  fp32
    beta: torch.Tensor         # [T, H]       fp32
    init_state: Optional[torch.Tensor]   # [N, H, d_k, d_v] fp32 or None
    cu_seqlens: Optional[torch.Tensor]   # [N + 1] int32 or None
    lengths: list

    @property
    def N(self) -> int:
        return len(self.lengths)


def prefill_inputs(lengths: Sequence[int], H: int, d: int, dtype: str = "bf16",
                   la_law: str = "softplus", init: str = "normal", seed: int = 0,
                   device="cpu", d_v: Optional[int] = None, packed: Optional[bool] = None,
                   slab: int = 65536) -> PrefillInputs:
    """Draw one packed prefill batch.

    ``packed`` controls whether ``cu_seqlens`` is returned (defaults to True
    when there is more than one sequence).  Tensors are drawn in token slabs
    of ``slab`` tokens to bound temporary memory on very long inputs.
    """
    d_k = d
    d_v = d if d_v is None else d_v
    lengths = [int(x) for x in lengths]
    T = int(sum(lengths))
    dt = torch_dtype(dtype)
    g = _generator(seed, device)
    q = torch.empty((T, H, d_k), dtype=dt, device=device)
    k = torch.empty((T, H, d_k), dtype=dt, device=device)
    v = torch.empty((T, H, d_v), dtype=dt, device=device)
    beta = torch.empty((T, H), dtype=torch.float32, device=device)
    la = torch.empty((T, H, d_k), dtype=torch.float32, device=device)
    for t0 in range(0, T, slab):
        t1 = min(T, t0 + slab)
        n = t1 - t0
        q[t0:t1] = _unit_rows(torch.randn((n, H, d_k), generator=g, device=device)).to(dt)
        k[t0:t1] = _unit_rows(torch.randn((n, H, d_k), generator=g, device=device)).to(dt)
        v[t0:t1] = torch.randn((n, H, d_v), generator=g, device=device).to(dt)
        beta[t0:t1] = torch.sigmoid(torch.randn((n, H), generator=g, device=device))
        la[t0:t1] = _log_alpha((n, H, d_k), la_law, g, device)
    N = len(lengths)
    if init == "normal":
        init_state = 0.02 * torch.randn((N, H, d_k, d_v), generator=g, device=device)
    elif init == "zeros":
        init_state = None
    else:
        raise ValueError(f"unknown init law {init!r}")
    if packed is None:
        packed = N > 1
    cu = None
    if packed:
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device=device)
    return PrefillInputs(q, k, v, la, beta, init_state, cu, lengths)


def workload_inputs(name: str, device="cpu", **overrides) -> PrefillInputs:
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    lengths = workload_lengths(name) if "lengths" not in overrides else overrides["lengths"]
    return prefill_inputs(lengths, spec["H"], spec["d"], spec["dtype"], spec["la_law"],
                          spec["init"], spec["seed"], device=device)


def decode_state(N: int, H: int, d: int, seed: int, device="cpu", d_v: Optional[int] = None) -> torch.Tensor:
    """Initial decode state [N, H, d_k, d_v] ~ N(0, 0.02), fp32."""
    d_v = d if d_v is None else d_v
    g = _generator(seed, device)
    return 0.02 * torch.randn((N, H, d, d_v), generator=g, device=device)


def decode_inputs(N: int, H: int, d: int, dtype: str = "bf16", la_law: str = "softplus",
                  seed: int = 4, step: int = 0, device="cpu", d_v: Optional[int] = None) -> dict:
    """Per-step decode inputs: q, k [N, H, d_k], v [N, H, d_v], log_alpha [N, H, d_k], beta [N, H]."""
    d_v = d if d_v is None else d_v
    dt = torch_dtype(dtype)
    g = _generator(seed * 1_000_003 + 7919 * (step + 1), device)
    q = _unit_rows(torch.randn((N, H, d), generator=g, device=device)).to(dt)
    k = _unit_rows(torch.randn((N, H, d), generator=g, device=device)).to(dt)
    v = torch.randn((N, H, d_v), generator=g, device=device).to(dt)
    beta = torch.sigmoid(torch.randn((N, H), generator=g, device=device))
    la = _log_alpha((N, H, d), la_law, g, device)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta)


def to_numpy(x: Optional[torch.Tensor]):
    """Exact host copy: bf16 is widened to fp32 (exactly), fp32 is copied as is."""
    if x is None:
        return None
    x = x.detach().to("cpu")
    if x.dtype == torch.bfloat16:
        x = x.float()
    return x.numpy()


# ---- logit inputs of the gated entry points ---------------------------------
# Recipe: q, k, v and the initial state as above; decay logits z ~ N(0, 2^2)
# in the element type of q (a wide spread, so that g = -5 Sigmoid(e^A z) spans
# nearly all of (-5, 0)); per-head log-scales A_h ~ U[-1, 1]; write-strength
# logits b ~ N(0, 1) in fp32 (Sigmoid(b) has the law of beta above).

@dataclass
class GatedInputs:
    q: torch.Tensor            # [T, H, d_k]  dtype
    k: torch.Tensor            # [T, H, d_k]  dtype
    v: torch.Tensor            # [T, H, d_v]  dtype
    g_logits: torch.Tensor     # [T, H, d_k]  dtype
    a_log: torch.Tensor        # [H]          fp32
    beta_logits: torch.Tensor  # [T, H]       fp32
    init_state: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    lengths: list


def gated_inputs(lengths: Sequence[int], H: int, d: int, dtype: str = "bf16", init: str = "normal",
                 seed: int = 0, device="cpu", d_v: Optional[int] = None, packed: Optional[bool] = None,
                 slab: int = 65536) -> GatedInputs:
    """Draw one packed prefill batch for the gated entry points (recipe above)."""
    base = prefill_inputs(lengths, H, d, dtype=dtype, la_law="zero", init=init, seed=seed, device=device,
                          d_v=d_v, packed=packed, slab=slab)
    T = int(sum(int(x) for x in lengths))
    dt = torch_dtype(dtype)
    g = _generator(seed * 7 + 101, device)
    z = torch.empty((T, H, d), dtype=dt, device=device)
    b = torch.empty((T, H), dtype=torch.float32, device=device)
    for t0 in range(0, T, slab):
        t1 = min(T, t0 + slab)
        z[t0:t1] = (2.0 * torch.randn((t1 - t0, H, d), generator=g, device=device)).to(dt)
        b[t0:t1] = torch.randn((t1 - t0, H), generator=g, device=device)
    a = 2.0 * torch.rand((H,), generator=g, device=device) - 1.0
    return GatedInputs(base.q, base.k, base.v, z, a, b, base.init_state, base.cu_seqlens, base.lengths)


def decode_gated_inputs(N: int, H: int, d: int, dtype: str = "bf16", seed: int = 4, step: int = 0,
                        device="cpu", d_v: Optional[int] = None) -> dict:
    """Per-step decode inputs of the gated entry point: q, k, v, g_logits, beta_logits
    (recipe above); a_log is drawn from ``seed`` alone, so it is the same every step."""
    base = decode_inputs(N, H, d, dtype=dtype, la_law="zero", seed=seed, step=step, device=device, d_v=d_v)
    dt = torch_dtype(dtype)
    g = _generator(seed * 1_000_033 + 104729 * (step + 1), device)
    z = (2.0 * torch.randn((N, H, d), generator=g, device=device)).to(dt)
    b = torch.randn((N, H), generator=g, device=device)
    ga = _generator(seed * 7 + 101, device)
    a = 2.0 * torch.rand((H,), generator=ga, device=device) - 1.0
    return dict(q=base["q"], k=base["k"], v=base["v"], g_logits=z, a_log=a, beta_logits=b)


# ---- inputs of the output epilogue ------------------------------------------
# Recipe: the output o ~ N(0, 1) per channel times a per-row scale 10^U[-3, 1]
# (rows from 1e-3, where the mean square is a tenth of epsilon = 1e-5 and the
# epsilon term dominates, to 10), in the working dtype; gate logits
# W_g x ~ N(0, 2^2) in the working dtype (Sigmoid spans nearly all of (0, 1));
# the RMSNorm gain w ~ U[0.5, 1.5], fp32, one per channel.

def epilogue_inputs(shape: Sequence[int], dtype: str = "bf16", seed: int = 0, device="cpu",
                    slab_rows: int = 1 << 22) -> dict:
    """o, gate logits [*shape] and gain [shape[-1]] for the output epilogue (recipe above)."""
    shape = tuple(int(s) for s in shape)
    d = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    dt = torch_dtype(dtype)
    g = _generator(seed * 31 + 977, device)
    o = torch.empty((rows, d), dtype=dt, device=device)
    gl = torch.empty((rows, d), dtype=dt, device=device)
    for r0 in range(0, rows, slab_rows):
        r1 = min(rows, r0 + slab_rows)
        scale = 10.0 ** (4.0 * torch.rand((r1 - r0, 1), generator=g, device=device) - 3.0)
        o[r0:r1] = (torch.randn((r1 - r0, d), generator=g, device=device) * scale).to(dt)
        gl[r0:r1] = (2.0 * torch.randn((r1 - r0, d), generator=g, device=device)).to(dt)
    w = 0.5 + torch.rand((d,), generator=g, device=device)
    return dict(o=o.view(shape), gate=gl.view(shape), weight=w)


def out_gate_inputs(shape: Sequence[int], dtype: str = "bf16", seed: int = 0, step: int = 0, device="cpu") -> dict:
    """Gate logits [*shape] and gain [shape[-1]] for the fused epilogue entry points
    (laws of the recipe above; the gain depends on ``seed`` only)."""
    shape = tuple(int(s) for s in shape)
    dt = torch_dtype(dtype)
    g = _generator(seed * 31 + 983 + 7919 * step, device)
    gl = (2.0 * torch.randn(shape, generator=g, device=device)).to(dt)
    gw = _generator(seed * 31 + 991, device)
    w = 0.5 + torch.rand((shape[-1],), generator=gw, device=device)
    return dict(gate=gl, weight=w)


# ---- inputs of the input prologue -------------------------------------------
# Recipe: projection outputs x_q, x_k, x_v ~ N(0, 1) in the working dtype;
# convolution taps ~ U[-1/2, 1/2] fp32 (the default bound 1/sqrt(fan-in) of a
# width-4 depthwise convolution); initial convolution state ~ N(0, 1) in the
# working dtype (earlier projection outputs), or none.

def prologue_inputs(lengths: Sequence[int], H: int, d: int, dtype: str = "bf16", seed: int = 0, device="cpu",
                    d_v: Optional[int] = None, state: bool = True, packed: Optional[bool] = None,
                    slab: int = 65536) -> dict:
    """x_q, x_k, x_v, conv_w, conv_state, cu_seqlens for the prologue (recipe above)."""
    d_v = d if d_v is None else d_v
    lengths = [int(x) for x in lengths]
    T, N = sum(lengths), len(lengths)
    dt = torch_dtype(dtype)
    g = _generator(seed * 53 + 1201, device)
    xs = []
    for dd in (d, d, d_v):
        x = torch.empty((T, H, dd), dtype=dt, device=device)
        for t0 in range(0, T, slab):
            t1 = min(T, t0 + slab)
            x[t0:t1] = torch.randn((t1 - t0, H, dd), generator=g, device=device).to(dt)
        xs.append(x)
    C = 2 * d + d_v
    w = torch.rand((H, C, 4), generator=g, device=device) - 0.5
    st = torch.randn((N, 3, H, C), generator=g, device=device).to(dt) if state else None
    if packed is None:
        packed = N > 1
    cu = None
    if packed:
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device=device)
    return dict(x_q=xs[0], x_k=xs[1], x_v=xs[2], conv_w=w, conv_state=st, cu_seqlens=cu, lengths=lengths)


def decode_prologue_inputs(N: int, H: int, d: int, dtype: str = "bf16", seed: int = 0, step: int = 0, device="cpu",
                           d_v: Optional[int] = None) -> dict:
    """Per-step projection outputs x_q, x_k, x_v [N, H, .] (laws of the prologue
    recipe), and, from ``seed`` alone, the taps [H, C, 4] and the initial
    convolution state [N, 3, H, C]."""
    d_v = d if d_v is None else d_v
    dt = torch_dtype(dtype)
    g = _generator(seed * 53 + 1301 + 7717 * (step + 1), device)
    xs = [torch.randn((N, H, dd), generator=g, device=device).to(dt) for dd in (d, d, d_v)]
    C = 2 * d + d_v
    gp = _generator(seed * 53 + 1303, device)
    w = torch.rand((H, C, 4), generator=gp, device=device) - 0.5
    st = torch.randn((N, 3, H, C), generator=gp, device=device).to(dt)
    return dict(x_q=xs[0], x_k=xs[1], x_v=xs[2], conv_w=w, conv_state=st)
