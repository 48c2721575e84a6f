"""Parity of the gated HIP entry points (decay and write strength given as
logits, mapped in-kernel by the lower-bounded decay of the architecture
notes, section 1.2) with the fp64 oracle (MI355X)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import kda_chunk_prefill_gated, kda_decode_step_gated

pytestmark = pytest.mark.gpu


def check_prefill(x, dtype, heads=None, what=""):
    tol = TOL[dtype]
    announce(f"gated prefill {what}: lengths={x.lengths[:4]}{'...' if len(x.lengths) > 4 else ''} "
             f"H={x.q.shape[1]} d_k={x.q.shape[2]} d_v={x.v.shape[2]} {dtype}")
    o, fin = kda_chunk_prefill_gated(x.q, x.k, x.v, x.g_logits, x.a_log, x.beta_logits, x.init_state,
                                     x.cu_seqlens)
    torch.cuda.synchronize()
    hs = slice(None) if heads is None else list(heads)
    o_ref, f_ref = oracle.kda_prefill_gated(host(x.q), host(x.k), host(x.v), host(x.g_logits), host(x.a_log),
                                            host(x.beta_logits), host(x.init_state), host(x.cu_seqlens),
                                            heads=heads)
    eo = rel_err(host(o)[:, hs], o_ref)
    ef = rel_err(host(fin)[:, hs], f_ref)
    announce(f"  rel err o={eo:.3e} final={ef:.3e} (tol {tol})")
    assert np.isfinite(host(o)).all() and np.isfinite(host(fin)).all()
    assert eo <= tol, f"o rel err {eo}"
    assert ef <= tol, f"final state rel err {ef}"


def test_gated_tiny_fp32():
    x = ki.gated_inputs([256], H=2, d=64, dtype="f32", init="zeros", seed=10, device=device())
    check_prefill(x, "f32", what="tiny fp32")


def check_all_heads(x, what):
    """Every head of a large bf16 workload against the oracle, fanned out over
    child processes (one slice of heads each)."""
    import oracle_pool
    announce(f"gated prefill {what}: {sum(x.lengths)} tokens, H={x.q.shape[1]}, all heads")
    o, fin = kda_chunk_prefill_gated(x.q, x.k, x.v, x.g_logits, x.a_log, x.beta_logits, x.init_state,
                                     x.cu_seqlens)
    torch.cuda.synchronize()
    r = oracle_pool.prefill(x.q, x.k, x.v, x.g_logits, x.beta_logits, x.init_state, x.cu_seqlens, a_log=x.a_log,
                            o_gpu=o, fin_gpu=fin, progress=announce)
    announce(f"  rel err o={r['rel_o']:.3e} final={r['rel_f']:.3e} over {r['heads']} heads "
             f"({r['seconds']:.1f} s in {r['workers']} processes; tol {TOL['bf16']})")
    assert r["finite"]
    assert r["rel_o"] <= TOL["bf16"] and r["rel_f"] <= TOL["bf16"]


def test_gated_bf16_4k_all_heads():
    x = ki.gated_inputs([4096], H=96, d=128, dtype="bf16", seed=11, device=device())
    check_all_heads(x, "bf16 4K")


@pytest.mark.parametrize("lengths", [[1], [37], [65], [128 + 17], [5, 0, 70, 1, 33]])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("f32", 128)])
def test_gated_ragged_lengths(lengths, dtype, d):
    x = ki.gated_inputs(lengths, H=3, d=d, dtype=dtype, seed=sum(lengths) + 12,
                        device=device(), packed=len(lengths) > 1)
    check_prefill(x, dtype, what=f"ragged {lengths}")


@pytest.mark.timeout(600)
def test_gated_varlen_all_heads():
    x = ki.gated_inputs(ki.workload_lengths("varlen16"), H=96, d=128, dtype="bf16", seed=13, device=device())
    check_all_heads(x, "packed varlen")


@pytest.mark.timeout(600)
def test_gated_long_64k_all_heads():
    x = ki.gated_inputs([65536], H=96, d=128, dtype="bf16", seed=14, device=device())
    check_all_heads(x, "64K")


@pytest.mark.parametrize("dtype,d,d_v", [("bf16", 128, 128), ("f32", 64, 128), ("bf16", 128, 64)])
def test_gated_decode_steps(dtype, d, d_v):
    N, H, steps = 6, 3, 12
    announce(f"gated decode N={N} H={H} d_k={d} d_v={d_v} {dtype}, {steps} steps")
    state = ki.decode_state(N, H, d, seed=15, device=device(), d_v=d_v)
    ref = host(state).astype(np.float64)
    worst_o = 0.0
    for step in range(steps):
        x = ki.decode_gated_inputs(N, H, d, dtype=dtype, seed=15, step=step, device=device(), d_v=d_v)
        o = kda_decode_step_gated(x["q"], x["k"], x["v"], x["g_logits"], x["a_log"], x["beta_logits"], state)
        torch.cuda.synchronize()
        o_ref, ref = oracle.kda_decode_step_gated(host(x["q"]), host(x["k"]), host(x["v"]), host(x["g_logits"]),
                                                  host(x["a_log"]), host(x["beta_logits"]), ref)
        worst_o = max(worst_o, rel_err(host(o), o_ref))
    es = rel_err(host(state), ref)
    announce(f"  rel err o (worst step)={worst_o:.3e} state={es:.3e}")
    assert worst_o <= TOL[dtype] and es <= TOL[dtype]
