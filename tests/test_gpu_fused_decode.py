"""Parity of the whole fused decode step (input prologue of section 1.1, gate
maps of section 1.2, the recurrence, output epilogue of section 1.3 of
"Kimi K3 -- Architecture Notes", one kernel) with the fp64 oracles composed
in that order (MI355X)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import RMS_EPS, kda_decode_step_fused

pytestmark = pytest.mark.gpu


def oracle_step(xq, xk, xv, w, cst, z, A, b, og, gain, S):
    """One token per sequence: prologue (each sequence of length 1 with its own
    state), gated decode, epilogue.  Arrays are [1 or N, H, .] host copies."""
    N = xq.shape[0]
    cu = np.arange(N + 1, dtype=np.int64)
    q, k, v, cst_new = oracle.kda_prologue(xq, xk, xv, w, cst, cu)
    o, S_new = oracle.kda_decode_step_gated(q, k, v, z, A, b, S)
    return oracle.kda_output_gate_rmsnorm(o, og, gain, RMS_EPS), S_new, cst_new


def row_check(y, y_ref, dtype, what):
    y = np.asarray(y, np.float64)
    nr = np.linalg.norm(y - y_ref, axis=-1) / np.linalg.norm(y_ref, axis=-1)
    announce(f"  {what}: y norm-wise rel err {rel_err(y, y_ref):.3e}, worst row rel err {nr.max():.3e}")
    assert np.isfinite(y).all()
    assert nr.max() <= TOL[dtype], f"{what}: a row of y beyond {TOL[dtype]}"


@pytest.mark.parametrize("dtype,d,d_v", [("bf16", 128, 128), ("f32", 64, 128), ("bf16", 128, 64), ("f32", 64, 64)])
def test_fused_decode_steps(dtype, d, d_v):
    N, H, steps = 6, 3, 12
    announce(f"fused decode N={N} H={H} d_k={d} d_v={d_v} {dtype}, {steps} steps")
    state = ki.decode_state(N, H, d, seed=70, device=device(), d_v=d_v)
    S_ref = host(state).astype(np.float64)
    p0 = ki.decode_prologue_inputs(N, H, d, dtype, seed=70, step=0, device=device(), d_v=d_v)
    cst = p0["conv_state"].clone()
    cst_ref = host(cst)
    for step in range(steps):
        p = ki.decode_prologue_inputs(N, H, d, dtype, seed=70, step=step, device=device(), d_v=d_v)
        g = ki.decode_gated_inputs(N, H, d, dtype=dtype, seed=70, step=step, device=device(), d_v=d_v)
        og = ki.out_gate_inputs((N, H, d_v), dtype, seed=70, step=step, device=device())
        gain = og["weight"] if step % 3 else None
        y = kda_decode_step_fused(p["x_q"], p["x_k"], p["x_v"], p["conv_w"], cst, g["g_logits"], g["a_log"],
                                  g["beta_logits"], og["gate"], state, norm_weight=gain)
        torch.cuda.synchronize()
        y_ref, S_ref, cst_ref = oracle_step(host(p["x_q"]), host(p["x_k"]), host(p["x_v"]), host(p["conv_w"]),
                                            cst_ref, host(g["g_logits"]), host(g["a_log"]), host(g["beta_logits"]),
                                            host(og["gate"]), None if gain is None else host(gain), S_ref)
        row_check(host(y), y_ref, dtype, f"step {step}")
        assert np.array_equal(host(cst), cst_ref), f"step {step}: the convolution state must be an exact shift"
    es = rel_err(host(state), S_ref)
    announce(f"  state rel err after {steps} steps {es:.3e}")
    assert es <= TOL[dtype]


def test_fused_decode_full_shape_sampled_pairs():
    """512 sequences x 96 heads, 3 steps; 64 seeded (sequence, head) pairs are
    followed by the oracle, each as its own one-head problem."""
    N, H, d = 512, 96, 128
    announce(f"fused decode full shape N={N} H={H}")
    state = ki.decode_state(N, H, d, seed=71, device=device())
    flat = np.random.default_rng(71).choice(N * H, 64, replace=False)
    ns, hs = torch.tensor(flat // H, device=device()), torch.tensor(flat % H, device=device())
    hh = flat % H
    S_ref = host(state[ns, hs]).astype(np.float64)[None]
    cst = ki.decode_prologue_inputs(N, H, d, "bf16", seed=71, step=0, device=device())["conv_state"].clone()
    cst_ref = host(cst[ns, :, hs]).transpose(1, 0, 2)[None]           # [1, 3, 64, C]
    for step in range(3):
        p = ki.decode_prologue_inputs(N, H, d, "bf16", seed=71, step=step, device=device())
        g = ki.decode_gated_inputs(N, H, d, "bf16", seed=71, step=step, device=device())
        og = ki.out_gate_inputs((N, H, d), "bf16", seed=71, step=step, device=device())
        y = kda_decode_step_fused(p["x_q"], p["x_k"], p["x_v"], p["conv_w"], cst, g["g_logits"], g["a_log"],
                                  g["beta_logits"], og["gate"], state, norm_weight=og["weight"])
        sel = lambda t: host(t[ns, hs])[None]
        y_ref, S_ref, cst_ref = oracle_step(sel(p["x_q"]), sel(p["x_k"]), sel(p["x_v"]), host(p["conv_w"])[hh],
                                            cst_ref, sel(g["g_logits"]), host(g["a_log"])[hh],
                                            sel(g["beta_logits"]), sel(og["gate"]), host(og["weight"]), S_ref)
        row_check(sel(y), y_ref, "bf16", f"step {step}")
        assert np.array_equal(host(cst[ns, :, hs]).transpose(1, 0, 2)[None], cst_ref)
    torch.cuda.synchronize()
    es = rel_err(host(state[ns, hs])[None], S_ref)
    announce(f"  state rel err {es:.3e}")
    assert es <= TOL["bf16"]
