"""Parity of the time-split prefill (kda_chunk_prefill_split and its gated form) with the fp64
oracle (MI355X).  The split runs segments of one sequence at once and joins them through the
segment transitions.  Its result must be the unsplit recurrence's, to the tolerances of the
workloads (1e-4 fp32, 2e-2 bf16)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import (kda_chunk_prefill, kda_chunk_prefill_gated, kda_chunk_prefill_gated_split,
                                     kda_chunk_prefill_split, kda_decode_step, split_segments,
                                     split_workspace_bytes)

pytestmark = pytest.mark.gpu


def _check(o, fin, o_ref, f_ref, dtype, what, heads=None):
    hs = slice(None) if heads is None else list(heads)
    eo = rel_err(host(o)[:, hs], o_ref)
    ef = rel_err(host(fin)[:, hs], f_ref)
    announce(f"  {what}: rel err o={eo:.3e} final={ef:.3e} (tol {TOL[dtype]})")
    assert np.isfinite(host(o)).all() and np.isfinite(host(fin)).all()
    assert eo <= TOL[dtype], f"o rel err {eo}"
    assert ef <= TOL[dtype], f"final state rel err {ef}"


SHAPES = [
    # T, segments, dtype, d_k, d_v, log-decay law, initial state
    (300, 2, "bf16", 128, 128, "softplus", "normal"),
    (1000, 3, "bf16", 128, 128, "zero", "normal"),
    (1030, 5, "bf16", 64, 64, "uniform53", "normal"),
    (777, 4, "bf16", 128, 64, "zero", "normal"),      # d_v != d_k: the two segment runs are two launches
    (777, 4, "bf16", 64, 128, "softplus", "zeros"),
    (500, 3, "f32", 64, 64, "zero", "normal"),
    (640, 10, "f32", 64, 128, "floor", "normal"),
    (4096, 64, "bf16", 128, 128, "zero", "normal"),    # 64 segments of one chunk
]


@pytest.mark.parametrize("T,segments,dtype,d_k,d_v,law,init", SHAPES)
def test_split_matches_oracle(T, segments, dtype, d_k, d_v, law, init):
    x = ki.prefill_inputs([T], H=3, d=d_k, d_v=d_v, dtype=dtype, la_law=law, init=init, seed=T + segments,
                          device=device())
    announce(f"split prefill T={T} segments={segments} {dtype} d_k={d_k} d_v={d_v} law={law} init={init}")
    o, fin = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=segments)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.kda_prefill(host(x.q), host(x.k), host(x.v), host(x.log_alpha), host(x.beta),
                                      host(x.init_state))
    _check(o, fin, o_ref, f_ref, dtype, "split")


def test_split_keeps_the_carried_state_exact_when_nothing_decays():
    """alpha = 1 and small beta: the state that enters each later segment dominates its outputs,
    so a wrong transition, scan or correction would show at once."""
    x = ki.prefill_inputs([2000], H=2, d=128, dtype="bf16", la_law="zero", init="normal", seed=21, device=device())
    x.beta.mul_(0.05)
    x.init_state.mul_(20.0)
    announce("split prefill, alpha = 1, beta <= 0.05, large initial state, 6 segments")
    o, fin = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=6)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.kda_prefill(host(x.q), host(x.k), host(x.v), host(x.log_alpha), host(x.beta),
                                      host(x.init_state))
    _check(o, fin, o_ref, f_ref, "bf16", "alpha = 1")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_gated_split_matches_oracle(dtype, d):
    x = ki.gated_inputs([900], 3, d, dtype=dtype, init="normal", seed=22, device=device(), d_v=d)
    announce(f"gated split prefill T=900 segments=4 {dtype} d={d}")
    o, fin = kda_chunk_prefill_gated_split(x.q, x.k, x.v, x.g_logits, x.a_log, x.beta_logits, x.init_state,
                                           segments=4)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.kda_prefill_gated(host(x.q), host(x.k), host(x.v), host(x.g_logits), host(x.a_log),
                                            host(x.beta_logits), host(x.init_state))
    _check(o, fin, o_ref, f_ref, dtype, "gated split")


@pytest.mark.parametrize("T,segments", [(700, 1), (64, 8), (40, 3)])
def test_one_segment_is_the_plain_prefill_bit_for_bit(T, segments):
    x = ki.prefill_inputs([T], H=2, d=128, dtype="bf16", seed=23, device=device())
    announce(f"split prefill T={T} segments={segments}: one segment used")
    assert split_workspace_bytes(T, 2, 128, 128, torch.bfloat16, segments) == 0
    o1, f1 = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=segments)
    o2, f2 = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_split_aliasing_skipping_and_workspace_reuse():
    """final_state may alias init_state; output_final_state=False skips it; one workspace serves
    two calls in a row, the second smaller, and a workspace full of garbage changes nothing."""
    x = ki.prefill_inputs([1500], H=2, d=128, dtype="bf16", init="normal", seed=24, device=device())
    ws = torch.full((split_workspace_bytes(1500, 2, 128, 128, torch.bfloat16, 5),), 0xFF, dtype=torch.uint8,
                    device=device())
    announce("split prefill aliasing / workspace reuse")
    o1, f1 = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=5, workspace=ws)
    alias = x.init_state.clone()
    o2, f2 = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, alias, segments=5, workspace=ws,
                                     final_state=alias)
    o3, f3 = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=5, workspace=ws,
                                     output_final_state=False)
    torch.cuda.synchronize()
    assert f3 is None
    assert torch.equal(o1, o2) and torch.equal(o1, o3) and torch.equal(f1, alias)
    y = ki.prefill_inputs([400], H=2, d=128, dtype="bf16", init="normal", seed=25, device=device())
    o4, f4 = kda_chunk_prefill_split(y.q, y.k, y.v, y.log_alpha, y.beta, y.init_state, segments=3, workspace=ws)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.kda_prefill(host(y.q), host(y.k), host(y.v), host(y.log_alpha), host(y.beta),
                                      host(y.init_state))
    _check(o4, f4, o_ref, f_ref, "bf16", "second call on the same workspace")


def test_split_is_deterministic():
    x = ki.prefill_inputs([3000], H=2, d=128, dtype="bf16", init="normal", seed=26, device=device())
    a = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=7)
    b = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=7)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _pool_check(x, o, fin, what, a_log=None):
    """Every head against the fp64 oracle, fanned out over child processes."""
    import oracle_pool
    decay, beta = (x.log_alpha, x.beta) if a_log is None else (x.g_logits, x.beta_logits)
    r = oracle_pool.prefill(x.q, x.k, x.v, decay, beta, x.init_state, None, a_log=a_log, o_gpu=o, fin_gpu=fin,
                            progress=announce)
    announce(f"  {what}: rel err o={r['rel_o']:.3e} final={r['rel_f']:.3e} over {r['heads']} heads "
             f"({r['seconds']:.1f} s in {r['workers']} processes; tol {TOL['bf16']})")
    assert r["finite"]
    assert r["rel_o"] <= TOL["bf16"] and r["rel_f"] <= TOL["bf16"]


def test_split_at_full_length_twelve_heads():
    """One GPU's share of a 96-head layer split 8 ways (H = 12), T = 65,536, d = 128, bf16, with the
    library's own segment count.  Checked against the fp64 oracle and against the unsplit kernel
    on every head."""
    T, H = 65536, 12
    x = ki.prefill_inputs([T], H=H, d=128, dtype="bf16", init="normal", seed=27, device=device())
    seg = split_segments(T, H, 128, 128)
    announce(f"split prefill T={T} H={H}: {seg} segments")
    assert seg > 1
    o, fin = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=seg)
    o_plain, f_plain = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state)
    torch.cuda.synchronize()
    assert rel_err(host(o), host(o_plain)) <= TOL["bf16"]
    assert rel_err(host(fin), host(f_plain)) <= TOL["bf16"]
    _pool_check(x, o, fin, "all heads")


@pytest.mark.parametrize("gated,d_v", [(True, 128), (False, 64)])
def test_split_at_full_length_gated_and_mixed_widths(gated, d_v):
    """T = 65,536, H = 12 with the library's segment count: the gated split, and d_v = 64 < d_k
    (the segment runs and the transition runs are then two launches).  Against the unsplit
    kernel and the fp64 oracle on every head."""
    T, H, d = 65536, 12, 128
    seg = split_segments(T, H, d, d_v)
    announce(f"split prefill T={T} H={H} d_k={d} d_v={d_v} gated={gated}: {seg} segments")
    if gated:
        x = ki.gated_inputs([T], H, d, dtype="bf16", init="normal", seed=28, device=device(), d_v=d_v)
        o, fin = kda_chunk_prefill_gated_split(x.q, x.k, x.v, x.g_logits, x.a_log, x.beta_logits, x.init_state,
                                               segments=seg)
        o_plain, f_plain = kda_chunk_prefill_gated(x.q, x.k, x.v, x.g_logits, x.a_log, x.beta_logits, x.init_state)
    else:
        x = ki.prefill_inputs([T], H=H, d=d, d_v=d_v, dtype="bf16", init="normal", seed=28, device=device())
        o, fin = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=seg)
        o_plain, f_plain = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state)
    torch.cuda.synchronize()
    assert seg > 1
    assert rel_err(host(o), host(o_plain)) <= TOL["bf16"]
    assert rel_err(host(fin), host(f_plain)) <= TOL["bf16"]
    _pool_check(x, o, fin, "all heads", a_log=x.a_log if gated else None)


def test_split_state_continues_into_decode():
    """A split prefill of T - 5 tokens followed by 5 decode steps from its final state gives the
    last 5 outputs and the final state of the whole run (fp64 oracle over all T tokens)."""
    T, H = 2053, 2
    x = ki.prefill_inputs([T], H=H, d=128, dtype="bf16", init="normal", seed=29, device=device())
    announce(f"split prefill of {T - 5} tokens (4 segments) + 5 decode steps vs the oracle over {T}")
    t = T - 5
    _, state = kda_chunk_prefill_split(x.q[:t].clone(), x.k[:t].clone(), x.v[:t].clone(), x.log_alpha[:t].clone(),
                                       x.beta[:t].clone(), x.init_state, segments=4)
    outs = []
    for s_ in range(t, T):
        sl = lambda a: a[s_:s_ + 1].clone()
        outs.append(kda_decode_step(sl(x.q), sl(x.k), sl(x.v), sl(x.log_alpha), sl(x.beta), state))
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.kda_prefill(host(x.q), host(x.k), host(x.v), host(x.log_alpha), host(x.beta),
                                      host(x.init_state))
    eo = rel_err(host(torch.cat(outs)), o_ref[t:])
    es = rel_err(host(state), f_ref)
    announce(f"  tail o={eo:.3e} state={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
