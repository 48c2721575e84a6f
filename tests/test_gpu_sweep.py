"""Seeded sweep of the prefill entry points over mixed shapes (MI355X): 1 to 4 packed sequences of
0 to 300 tokens, 1 to 3 heads, d_k and d_v each 64 or 128, both dtypes (fp32 needs d_k = 64),
every log-decay law of the workloads plus the floor -5 and 0, with and without initial states;
the gated entry point on a share of the cases.  Each case is compared with the fp64 oracle to
the workloads' tolerances (1e-4 fp32, 2e-2 bf16)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import kda_chunk_prefill, kda_chunk_prefill_gated

pytestmark = pytest.mark.gpu

CASES = 36


def _case(i):
    rng = np.random.default_rng(1000 + i)
    n_seq = int(rng.integers(1, 5))
    lengths = [int(x) for x in rng.integers(0, 301, size=n_seq)]
    if sum(lengths) == 0:
        lengths[0] = int(rng.integers(1, 301))
    H = int(rng.integers(1, 4))
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    d_k = 64 if dtype == "f32" else int(rng.choice([64, 128]))
    d_v = int(rng.choice([64, 128]))
    la_law = str(rng.choice(list(ki.LOG_ALPHA_LAWS)))
    init = str(rng.choice(["zeros", "normal"]))
    gated = bool(rng.random() < 0.3)
    return dict(lengths=lengths, H=H, dtype=dtype, d_k=d_k, d_v=d_v, la_law=la_law, init=init, gated=gated,
                packed=n_seq > 1 or bool(rng.random() < 0.5))


@pytest.mark.parametrize("i", range(CASES))
def test_prefill_sweep(i):
    c = _case(i)
    announce(f"sweep case {i}: {c}")
    tol = TOL[c["dtype"]]
    if c["gated"]:
        x = ki.gated_inputs(c["lengths"], c["H"], c["d_k"], dtype=c["dtype"], init=c["init"], seed=2000 + i,
                            device=device(), d_v=c["d_v"], packed=c["packed"])
        o, fin = kda_chunk_prefill_gated(x.q, x.k, x.v, x.g_logits, x.a_log, x.beta_logits, x.init_state,
                                         x.cu_seqlens)
        torch.cuda.synchronize()
        o_ref, f_ref = oracle.kda_prefill_gated(host(x.q), host(x.k), host(x.v), host(x.g_logits), host(x.a_log),
                                                host(x.beta_logits), host(x.init_state), host(x.cu_seqlens))
    else:
        x = ki.prefill_inputs(c["lengths"], c["H"], c["d_k"], dtype=c["dtype"], la_law=c["la_law"], init=c["init"],
                              seed=2000 + i, device=device(), d_v=c["d_v"], packed=c["packed"])
        o, fin = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens)
        torch.cuda.synchronize()
        o_ref, f_ref = oracle.kda_prefill(host(x.q), host(x.k), host(x.v), host(x.log_alpha), host(x.beta),
                                          host(x.init_state), host(x.cu_seqlens))
    eo = rel_err(host(o), o_ref) if o_ref.size else 0.0
    ef = rel_err(host(fin), f_ref)
    announce(f"  rel err o={eo:.3e} final={ef:.3e} (tol {tol})")
    assert np.isfinite(host(o)).all() and np.isfinite(host(fin)).all()
    assert eo <= tol and ef <= tol
