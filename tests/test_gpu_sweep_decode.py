"""Seeded sweep of the decode entry points over mixed shapes (MI355X).

Each case uses 1 to 300 sequences, 1 to 5 heads, and d_k and d_v each 64 or 128, in both dtypes.
Every log-decay law of the workloads appears, plus the floor -5 and 0. A share of the cases uses
the gated entry point. Each case runs three consecutive steps on one state, and every step's o
and the final state are compared with the fp64 oracle to the workloads' tolerances (1e-4 fp32,
2e-2 bf16)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import kda_decode_step, kda_decode_step_gated

pytestmark = pytest.mark.gpu

CASES = 24
STEPS = 3


def _case(i):
    rng = np.random.default_rng(5000 + i)
    return dict(N=int(rng.integers(1, 301)), H=int(rng.integers(1, 6)), d_k=int(rng.choice([64, 128])),
                d_v=int(rng.choice([64, 128])), dtype="f32" if rng.random() < 0.35 else "bf16",
                la_law=str(rng.choice(list(ki.LOG_ALPHA_LAWS))), gated=bool(rng.random() < 0.35))


@pytest.mark.parametrize("i", range(CASES))
def test_decode_sweep(i):
    c = _case(i)
    announce(f"decode sweep case {i}: {c}")
    N, H, d_k, d_v, dt = c["N"], c["H"], c["d_k"], c["d_v"], c["dtype"]
    state = ki.decode_state(N, H, d_k, seed=6000 + i, device=device(), d_v=d_v)
    S_ref = host(state).astype(np.float64)
    worst = 0.0
    for step in range(STEPS):
        if c["gated"]:
            x = ki.decode_gated_inputs(N, H, d_k, dtype=dt, seed=6000 + i, step=step, device=device(), d_v=d_v)
            o = kda_decode_step_gated(x["q"], x["k"], x["v"], x["g_logits"], x["a_log"], x["beta_logits"], state)
            torch.cuda.synchronize()
            o_ref, S_ref = oracle.kda_decode_step_gated(host(x["q"]), host(x["k"]), host(x["v"]), host(x["g_logits"]),
                                                        host(x["a_log"]), host(x["beta_logits"]), S_ref)
        else:
            x = ki.decode_inputs(N, H, d_k, dtype=dt, la_law=c["la_law"], seed=6000 + i, step=step, device=device(),
                                 d_v=d_v)
            o = kda_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], state)
            torch.cuda.synchronize()
            o_ref, S_ref = oracle.kda_decode_step(host(x["q"]), host(x["k"]), host(x["v"]), host(x["log_alpha"]),
                                                  host(x["beta"]), S_ref)
        assert np.isfinite(host(o)).all()
        worst = max(worst, rel_err(host(o), o_ref))
    es = rel_err(host(state), S_ref)
    announce(f"  worst step o={worst:.3e} state={es:.3e} (tol {TOL[dt]})")
    assert worst <= TOL[dt] and es <= TOL[dt]
