"""Parity of the HIP decode step with the fp64 oracle (MI355X)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import kda_decode_step

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d_k,d_v", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_steps_small(d_k, d_v, dtype):
    announce(f"decode small d_k={d_k} d_v={d_v} {dtype}")
    N, H = 7, 3
    state = ki.decode_state(N, H, d_k, seed=1, device=device(), d_v=d_v)
    S_ref = host(state).astype(np.float64)
    for step in range(5):
        x = ki.decode_inputs(N, H, d_k, dtype=dtype, seed=2, step=step, device=device(), d_v=d_v)
        o = kda_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], state)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.kda_decode_step(host(x["q"]), host(x["k"]), host(x["v"]), host(x["log_alpha"]),
                                              host(x["beta"]), S_ref)
        assert rel_err(host(o), o_ref) <= TOL[dtype]
    assert rel_err(host(state), S_ref) <= TOL[dtype]


def test_decode_full_workload_100_steps_sampled_pairs():
    """512 sequences x 96 heads, fp32 state (3.2 GB) updated in place for 100
    steps; o at every step and the state after step 100 are compared on 64
    seeded (sequence, head) pairs."""
    w = ki.DECODE_WORKLOAD
    N, H, d = w["N"], w["H"], w["d"]
    announce(f"decode full workload N={N} H={H} d={d} steps={w['steps']}")
    state = ki.decode_state(N, H, d, seed=w["seed"], device=device())
    rng = np.random.default_rng(w["seed"])
    flat = rng.choice(N * H, 64, replace=False)
    ns, hs = torch.tensor(flat // H, device=device()), torch.tensor(flat % H, device=device())
    S_ref = host(state[ns, hs]).astype(np.float64)[None]          # [1, 64, d, d]
    worst = 0.0
    for step in range(w["steps"]):
        x = ki.decode_inputs(N, H, d, dtype=w["dtype"], la_law=w["la_law"], seed=w["seed"], step=step, device=device())
        o = kda_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], state)
        sel = {kk: host(vv[ns, hs])[None] for kk, vv in x.items()}
        o_ref, S_ref = oracle.kda_decode_step(sel["q"], sel["k"], sel["v"], sel["log_alpha"], sel["beta"], S_ref)
        worst = max(worst, rel_err(host(o[ns, hs])[None], o_ref))
    torch.cuda.synchronize()
    es = rel_err(host(state[ns, hs])[None], S_ref)
    announce(f"  worst per-step o rel err {worst:.3e}; state after 100 steps {es:.3e}")
    assert worst <= TOL["bf16"] and es <= TOL["bf16"]
