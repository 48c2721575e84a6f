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


def test_decode_full_workload_100_steps_all_pairs():
    """512 sequences x 96 heads, fp32 state (3.2 GB) updated in place for 100
    steps; o at every step and the state after step 100 are compared with the
    fp64 oracle on every (sequence, head) pair (the oracle runs in child
    processes, 32 sequences each)."""
    import oracle_pool
    w = ki.DECODE_WORKLOAD
    N, H, d = w["N"], w["H"], w["d"]
    announce(f"decode full workload N={N} H={H} d={d} steps={w['steps']}, all pairs")
    state = ki.decode_state(N, H, d, seed=w["seed"], device=device())
    with oracle_pool.DecodeRun(N, H, d, d) as run:
        run.save_state0(state)
        for step in range(w["steps"]):
            x = ki.decode_inputs(N, H, d, dtype=w["dtype"], la_law=w["la_law"], seed=w["seed"], step=step,
                                 device=device())
            o = kda_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], state)
            run.save_step(x, o)
            if step % 25 == 24:
                announce(f"  {step + 1} steps run and saved")
        torch.cuda.synchronize()
        r = run.compare(state, progress=announce)
    announce(f"  oracle {r['seconds']:.1f} s in {r['workers']} processes; worst per-step o rel err "
             f"{r['rel_o']:.3e}; state after 100 steps {r['rel_f']:.3e}")
    assert r["finite"]
    assert r["pair_steps"] == N * H * w["steps"]
    assert r["rel_o"] <= TOL["bf16"] and r["rel_f"] <= TOL["bf16"]
