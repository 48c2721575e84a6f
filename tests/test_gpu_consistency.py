"""Consistency of the HIP entry points with each other (MI355X), independent of the oracle's
arithmetic: a prefill continued by decode steps equals one prefill over all tokens, and a
packed batch equals its sequences launched one by one."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import kda_chunk_prefill, kda_decode_step

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_prefill_then_decode_equals_one_prefill(dtype, d):
    """Section 1.1's recurrence carried by the state alone: prefill over the first T - 5 tokens,
    then five single-token decode steps on the returned state, must give the last five outputs
    and the final state of one prefill over all T tokens."""
    T, tail = 133, 5
    announce(f"prefill {T - tail} + {tail} decode steps vs prefill {T}, {dtype} d={d}")
    x = ki.prefill_inputs([T], H=3, d=d, dtype=dtype, la_law="softplus", init="normal", seed=21, device=device())
    o_all, f_all = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state)
    h = T - tail
    # slices are copied: the entry points take 16-byte-aligned buffers
    cp = lambda t: t.clone()
    o_head, state = kda_chunk_prefill(cp(x.q[:h]), cp(x.k[:h]), cp(x.v[:h]), cp(x.log_alpha[:h]), cp(x.beta[:h]),
                                      x.init_state)
    outs = []
    for t in range(h, T):
        sl = slice(t, t + 1)
        outs.append(kda_decode_step(cp(x.q[sl]), cp(x.k[sl]), cp(x.v[sl]), cp(x.log_alpha[sl]), cp(x.beta[sl]),
                                    state))
    torch.cuda.synchronize()
    tol = TOL[dtype]
    eo = rel_err(np.concatenate([host(o) for o in outs]), host(o_all)[h:])
    ef = rel_err(host(state), host(f_all))
    eh = rel_err(host(o_head), host(o_all)[:h])
    announce(f"  rel err tail o={eo:.3e} state={ef:.3e} head o={eh:.3e} (tol {tol})")
    assert eo <= tol and ef <= tol and eh <= tol


def test_packed_batch_is_bitwise_equal_to_separate_launches():
    """Every sequence of a packed batch starts its own chunks, so packing changes no arithmetic:
    the outputs and final states are bit for bit those of one launch per sequence."""
    lengths = [70, 5, 130, 64, 1]
    announce(f"packed {lengths} vs one launch per sequence, bf16 d=128")
    x = ki.prefill_inputs(lengths, H=2, d=128, dtype="bf16", seed=22, device=device())
    o, fin = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens)
    cu = host(x.cu_seqlens).astype(np.int64)
    sep_o, sep_f = [], []
    for n in range(len(lengths)):
        a, b = int(cu[n]), int(cu[n + 1])
        cp = lambda t: t[a:b].clone()        # the entry points take 16-byte-aligned buffers
        on, fn = kda_chunk_prefill(cp(x.q), cp(x.k), cp(x.v), cp(x.log_alpha), cp(x.beta),
                                   x.init_state[n:n + 1].clone())
        sep_o.append(on)
        sep_f.append(fn)
    torch.cuda.synchronize()
    assert torch.equal(o, torch.cat(sep_o))
    assert torch.equal(fin, torch.cat(sep_f))
