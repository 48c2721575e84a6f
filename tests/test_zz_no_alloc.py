"""The allocation-free time split (kda_chunk_prefill_split_noalloc, on the
library's own scratch) against the entry point that takes a workspace, through
the C ABI: two calls in a row on the same scratch, the second smaller, each
bit-identical to the workspace entry point's result (the same kernels run on
the same inputs) and within the bf16 tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import (SPLIT_SCRATCH_BYTES, KDAError, kda_chunk_prefill_split,
                                     kda_chunk_prefill_split_noalloc, split_workspace_bytes)

pytestmark = pytest.mark.gpu


def _one(T, H, d_k, d_v, segments, seed, dtype="bf16"):
    x = ki.prefill_inputs([T], H=H, d=d_k, d_v=d_v, dtype=dtype, seed=seed, device=device())
    need = split_workspace_bytes(T, H, d_k, d_v, x.q.dtype, segments)
    announce(f"no-alloc split T={T} H={H} d_k={d_k} d_v={d_v} {dtype} segments={segments}: "
             f"{need} of {SPLIT_SCRATCH_BYTES} scratch bytes")
    assert 0 < need <= SPLIT_SCRATCH_BYTES
    o_ws, f_ws = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=segments)
    o = torch.empty_like(o_ws)
    fin = torch.empty_like(f_ws)
    kda_chunk_prefill_split_noalloc(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=segments, o=o,
                                    final_state=fin)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ws) and torch.equal(fin, f_ws), "differs from the workspace entry point"
    o_ref, f_ref = oracle.kda_prefill(host(x.q), host(x.k), host(x.v), host(x.log_alpha), host(x.beta),
                                      host(x.init_state))
    eo, ef = rel_err(host(o), o_ref), rel_err(host(fin), f_ref)
    announce(f"  bit-identical to the workspace entry point; rel err o={eo:.3e} final={ef:.3e}")
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


def test_noalloc_split_two_calls_second_smaller():
    _one(4096, 4, 128, 128, 4, seed=81)
    _one(1000, 2, 128, 64, 3, seed=82)


def test_noalloc_split_fp32_and_one_segment():
    _one(700, 2, 64, 64, 5, seed=83, dtype="f32")
    # one segment is the plain prefill: no scratch is used
    x = ki.prefill_inputs([300], H=2, d=64, dtype="bf16", seed=84, device=device())
    o, fin = kda_chunk_prefill_split_noalloc(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=1)
    o1, f1 = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=1)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(fin, f1)


def test_noalloc_split_rejects_a_plan_beyond_the_scratch():
    T, H, d = 65536, 12, 128
    x = ki.prefill_inputs([T], H=H, d=d, dtype="bf16", seed=85, device=device())
    assert split_workspace_bytes(T, H, d, d, torch.bfloat16, 8) > SPLIT_SCRATCH_BYTES
    with pytest.raises(KDAError, match="KDA_ERR_VALUE"):
        kda_chunk_prefill_split_noalloc(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=8)
