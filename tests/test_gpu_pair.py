"""The two prefill kernels against the fp64 oracle and against each other.

bf16 prefills with d_k = d_v = 128 run as a producer/state pair of workgroups
when the whole grid fits the device at once (N x H <= 128 on 256 CUs), and as
the single-workgroup kernel otherwise or when the pair is switched off.  The
pair performs the same operations in the same order, split over two
workgroups, so the two kernels must agree bit for bit; each is also held to
the oracle's tolerance.  prefill_pair_launches() shows which kernel ran.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import (kda_chunk_prefill, kda_chunk_prefill_gated, prefill_pair_launches,
                                     prefill_pair_mode, wait_giveups)

pytestmark = pytest.mark.gpu


def both_kernels(call):
    """(pair result, single-workgroup result, whether the pair kernel ran)."""
    old = prefill_pair_mode(1)
    try:
        n0 = prefill_pair_launches()
        a = call()
        torch.cuda.synchronize()
        ran = prefill_pair_launches() - n0
        prefill_pair_mode(0)
        n1 = prefill_pair_launches()
        b = call()
        torch.cuda.synchronize()
        assert prefill_pair_launches() == n1, "the pair kernel ran while switched off"
    finally:
        prefill_pair_mode(old)
    assert wait_giveups() == 0
    return a, b, ran == 1


def check(res, ref, what):
    (o, f), (o_ref, f_ref) = res, ref
    eo, ef = rel_err(host(o), o_ref), rel_err(host(f), f_ref)
    announce(f"  {what}: rel err o={eo:.3e} final={ef:.3e} (tol {TOL['bf16']})")
    assert np.isfinite(host(o)).all() and np.isfinite(host(f)).all()
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


CASES = [([1], 2), ([37], 3), ([64], 2), ([65], 2), ([145], 4), ([5, 0, 70, 1, 33], 3), ([1000], 16),
         ([4096], 8), ([300, 700], 64), ([130], 128)]


@pytest.mark.parametrize("lengths,H", CASES)
def test_pair_kernel_matches_oracle_and_single_kernel(lengths, H):
    x = ki.prefill_inputs(lengths, H=H, d=128, dtype="bf16", la_law="floor" if H == 3 else "softplus",
                          seed=71 + H, device=device())
    announce(f"pair vs single prefill: lengths={lengths} H={H} d=128 bf16")
    call = lambda: kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens)
    pair, single, ran = both_kernels(call)
    assert ran, "the pair kernel did not run for a grid that fits the device"
    ref = oracle.kda_prefill(host(x.q), host(x.k), host(x.v), host(x.log_alpha), host(x.beta),
                             host(x.init_state), host(x.cu_seqlens))
    check(pair, ref, "pair")
    check(single, ref, "single")
    assert torch.equal(pair[0], single[0]) and torch.equal(pair[1], single[1]), \
        "the two kernels differ (they perform the same operations in the same order)"


@pytest.mark.parametrize("lengths,H", [([1], 2), ([65], 3), ([5, 0, 70, 1, 33], 2), ([2000], 8)])
def test_pair_kernel_gated(lengths, H):
    x = ki.gated_inputs(lengths, H=H, d=128, dtype="bf16", seed=91 + H, device=device())
    announce(f"pair vs single gated prefill: lengths={lengths} H={H} d=128 bf16")
    call = lambda: kda_chunk_prefill_gated(x.q, x.k, x.v, x.g_logits, x.a_log, x.beta_logits, x.init_state,
                                          x.cu_seqlens)
    pair, single, ran = both_kernels(call)
    assert ran
    ref = oracle.kda_prefill_gated(host(x.q), host(x.k), host(x.v), host(x.g_logits), host(x.a_log),
                                   host(x.beta_logits), host(x.init_state), host(x.cu_seqlens))
    check(pair, ref, "pair")
    check(single, ref, "single")
    assert torch.equal(pair[0], single[0]) and torch.equal(pair[1], single[1])


def test_grid_beyond_the_device_runs_the_single_kernel():
    """129 (sequence, head) pairs need 272 workgroups: more than 256 CUs hold at
    once, so the call runs the single-workgroup kernel (still exact)."""
    x = ki.prefill_inputs([70], H=129, d=128, dtype="bf16", seed=5, device=device())
    announce("prefill H=129 (grid larger than the device): single-workgroup kernel")
    n0 = prefill_pair_launches()
    o, f = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens)
    torch.cuda.synchronize()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    if 16 * ((129 + 7) // 8) > n_cu:
        assert prefill_pair_launches() == n0
    ref = oracle.kda_prefill(host(x.q), host(x.k), host(x.v), host(x.log_alpha), host(x.beta),
                             host(x.init_state), None)
    check((o, f), ref, "H=129")


def test_pair_kernel_repeated_launches_and_aliasing():
    """Many launches on one stream share the ring (the epoch tells them apart);
    a final state may alias the initial state."""
    x = ki.prefill_inputs([333], H=4, d=128, dtype="bf16", seed=8, device=device())
    announce("pair prefill: 20 launches on one stream, then in place")
    outs = [kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, None) for _ in range(20)]
    torch.cuda.synchronize()
    for o, f in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(f, outs[0][1])
    st = x.init_state.clone()
    o2, f2 = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, st, None, final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o2, outs[0][0]) and torch.equal(st, outs[0][1])
    assert wait_giveups() == 0
