"""Parity of the HIP chunkwise prefill with the fp64 oracle (MI355X)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import KDAError, kda_chunk_prefill, wait_giveups

pytestmark = pytest.mark.gpu


def run_and_check(x, dtype, heads=None, tol=None, what=""):
    tol = TOL[dtype] if tol is None else tol
    announce(f"prefill {what}: lengths={x.lengths[:4]}{'...' if len(x.lengths) > 4 else ''} "
             f"H={x.q.shape[1]} d_k={x.q.shape[2]} d_v={x.v.shape[2]} {dtype}")
    o, fin = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens)
    torch.cuda.synchronize()
    hs = slice(None) if heads is None else list(heads)
    o_ref, f_ref = oracle.kda_prefill(host(x.q), host(x.k), host(x.v), host(x.log_alpha), host(x.beta),
                                      host(x.init_state), host(x.cu_seqlens), heads=heads)
    eo = rel_err(host(o)[:, hs], o_ref)
    ef = rel_err(host(fin)[:, hs], f_ref)
    announce(f"  rel err o={eo:.3e} final={ef:.3e} (tol {tol})")
    assert np.isfinite(host(o)).all() and np.isfinite(host(fin)).all()
    assert eo <= tol, f"o rel err {eo}"
    assert ef <= tol, f"final state rel err {ef}"
    return o, fin


def test_tiny_fp32_workload():
    x = ki.workload_inputs("tiny_fp32", device=device())
    run_and_check(x, "f32", what="tiny fp32 (T=256, H=2, d=64)")


def check_all_heads(x, o, fin, dtype, what, heads=None):
    """Every head (or `heads`) of a large workload against the oracle, fanned out
    over child processes (one slice of heads each)."""
    import oracle_pool
    n = len(heads) if heads is not None else x.q.shape[1]
    announce(f"  oracle on {n} heads in up to {oracle_pool.host_cores()} processes ({what})")
    r = oracle_pool.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens, o_gpu=o, fin_gpu=fin,
                            heads=heads, progress=announce)
    announce(f"  rel err o={r['rel_o']:.3e} final={r['rel_f']:.3e} over {r['heads']} heads "
             f"({r['seconds']:.1f} s in {r['workers']} processes; tol {TOL[dtype]})")
    assert r["finite"]
    assert r["rel_o"] <= TOL[dtype], f"o rel err {r['rel_o']}"
    assert r["rel_f"] <= TOL[dtype], f"final state rel err {r['rel_f']}"


def test_bf16_4k_workload_all_heads():
    """The 4K single-sequence workload (H = 96, d = 128, bf16), every head."""
    x = ki.workload_inputs("bf16_4k", device=device())
    announce("prefill bf16 4K (H=96, d=128), all heads")
    o, fin = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens)
    torch.cuda.synchronize()
    check_all_heads(x, o, fin, "bf16", "bf16 4K")


@pytest.mark.timeout(600)
def test_varlen_workload_all_heads():
    """The packed workload (16 sequences of U{1K..8K} tokens, H = 96, d = 128, bf16),
    every head of every sequence, with its own initial and final state."""
    x = ki.workload_inputs("varlen16", device=device())
    announce(f"prefill packed varlen 16 x U{{1K..8K}}: {sum(x.lengths)} tokens, H=96, all heads")
    o, fin = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens)
    torch.cuda.synchronize()
    check_all_heads(x, o, fin, "bf16", "packed varlen")


@pytest.mark.timeout(600)
def test_long_64k_workload_all_heads():
    """The benchmarked workload (one sequence of 65,536 tokens, H = 96, d = 128, bf16,
    log alpha ~ U[-5, -3]), every head, in the launch bench.py times."""
    x = ki.workload_inputs("long_64k", device=device())
    announce("prefill long 64K (H=96, d=128, log alpha ~ U[-5,-3]), all heads")
    o, fin = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, None)
    torch.cuda.synchronize()
    assert wait_giveups() == 0
    check_all_heads(x, o, fin, "bf16", "long 64K")


@pytest.mark.timeout(900)
def test_long_1m_capacity_four_heads():
    """Capacity run: one sequence of 1,048,576 tokens, H=96, d=128 (about 155 GB of device
    memory), checked against the fp64 oracle on 4 sampled heads, one child process each."""
    x = ki.workload_inputs("long_1m", device=device())
    announce("prefill capacity run T=1,048,576 H=96 d=128 bf16 (log alpha ~ U[-5,-3])")
    o, fin = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, None)
    torch.cuda.synchronize()
    assert wait_giveups() == 0
    heads = sorted(np.random.default_rng(5).choice(96, 4, replace=False).tolist())
    check_all_heads(x, o, fin, "bf16", "1M", heads=heads)


@pytest.mark.parametrize("lengths", [[1], [37], [100], [64], [65], [128 + 17], [1, 1, 1], [5, 0, 70, 1, 33]])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_lengths(lengths, dtype):
    x = ki.prefill_inputs(lengths, H=3, d=64 if dtype == "f32" else 128, dtype=dtype, seed=sum(lengths) + 7,
                          device=device(), packed=len(lengths) > 1)
    run_and_check(x, dtype, what=f"ragged {lengths}")


@pytest.mark.parametrize("d_k,d_v,dtype", [(64, 64, "bf16"), (64, 128, "bf16"), (128, 64, "bf16"),
                                           (64, 128, "f32"), (128, 128, "f32"), (128, 64, "f32")])
def test_head_dims(d_k, d_v, dtype):
    x = ki.prefill_inputs([200, 64], H=2, d=d_k, d_v=d_v, dtype=dtype, seed=d_k + d_v, device=device())
    run_and_check(x, dtype, what=f"d_k={d_k} d_v={d_v}")


@pytest.mark.parametrize("la_law", ["floor", "zero", "uniform53"])
def test_decay_extremes(la_law):
    x = ki.prefill_inputs([300], H=2, d=128, dtype="bf16", la_law=la_law, seed=5, device=device())
    run_and_check(x, "bf16", what=f"log alpha law {la_law}")


@pytest.mark.parametrize("b", [0.0, 1.0])
def test_beta_extremes(b):
    x = ki.prefill_inputs([150], H=2, d=128, dtype="bf16", seed=6, device=device())
    x.beta.fill_(b)
    if b == 0.0:
        # beta = 0 is pure decay, S_T = Diag(exp(sum log alpha)) S_0.  Under the
        # softplus law 150 tokens decay by about e^-120, below fp32's range, so a
        # milder decay keeps the reference representable.
        x.log_alpha.mul_(0.05)
    run_and_check(x, "bf16", what=f"beta = {b}")


def test_retrieval_invariant_through_the_kernel():
    """alpha = 1, beta = 1, q = k (unit, fp32): every output equals its value row."""
    x = ki.prefill_inputs([130], H=2, d=64, dtype="f32", la_law="zero", seed=8, device=device())
    x.beta.fill_(1.0)
    o, _ = kda_chunk_prefill(x.k, x.k, x.v, x.log_alpha, x.beta, x.init_state)
    torch.cuda.synchronize()
    assert rel_err(host(o), host(x.v)) <= 1e-4


def test_split_and_resume_matches_one_pass():
    x = ki.prefill_inputs([333], H=2, d=128, dtype="bf16", seed=9, device=device())
    o, fin = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state)
    t = 150
    oa, fa = kda_chunk_prefill(x.q[:t], x.k[:t], x.v[:t], x.log_alpha[:t], x.beta[:t], x.init_state)
    ob, fb = kda_chunk_prefill(x.q[t:], x.k[t:], x.v[t:], x.log_alpha[t:], x.beta[t:], fa)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.kda_prefill(host(x.q), host(x.k), host(x.v), host(x.log_alpha), host(x.beta),
                                      host(x.init_state))
    assert rel_err(np.concatenate([host(oa), host(ob)]), o_ref) <= 2e-2
    assert rel_err(host(fb), f_ref) <= 2e-2
    assert rel_err(host(fb), host(fin)) <= 2e-2


def test_final_state_may_alias_init_state_and_may_be_skipped():
    x = ki.prefill_inputs([90, 40], H=2, d=128, dtype="bf16", seed=10, device=device())
    init = x.init_state.clone()
    o1, f1 = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, init, x.cu_seqlens)
    alias = init.clone()
    o2, f2 = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, alias, x.cu_seqlens, final_state=alias)
    o3, f3 = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, init, x.cu_seqlens, output_final_state=False)
    torch.cuda.synchronize()
    assert f3 is None
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
    assert torch.equal(f1, alias)


def test_zero_tokens_copies_initial_state():
    x = ki.prefill_inputs([0, 0], H=2, d=64, dtype="bf16", seed=11, device=device())
    o, fin = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(fin, x.init_state)


def test_bitwise_deterministic():
    x = ki.prefill_inputs([700], H=4, d=128, dtype="bf16", seed=12, device=device())
    o1, f1 = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state)
    o2, f2 = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_binding_rejects_wrong_dtype():
    x = ki.prefill_inputs([16], H=1, d=64, dtype="bf16", seed=13, device=device())
    with pytest.raises(TypeError):
        kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha.double(), x.beta)
    with pytest.raises((KDAError, ValueError)):
        kda_chunk_prefill(x.q, x.k, x.v[:, :, :32].contiguous(), x.log_alpha, x.beta)   # d_v = 32


@pytest.mark.parametrize("lengths", [[1], [37], [65], [145], [5, 0, 70, 1, 33]])
@pytest.mark.parametrize("d_v", [64, 128])
@pytest.mark.parametrize("la_law", ["floor", "zero"])
def test_fp32_dk128(lengths, d_v, la_law):
    """fp32 inputs with d_k = 128 (one LDS buffer, the two roles taking turns):
    ragged and packed lengths, both value widths, log alpha at -5 and at 0,
    within the fp32 tolerance of 1e-4."""
    x = ki.prefill_inputs(lengths, H=3, d=128, d_v=d_v, dtype="f32", la_law=la_law, seed=sum(lengths) + d_v,
                          device=device(), packed=len(lengths) > 1)
    run_and_check(x, "f32", what=f"fp32 d_k=128 d_v={d_v} log alpha {la_law}")
