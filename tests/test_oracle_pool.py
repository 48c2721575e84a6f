"""The child-process oracle harness that the full-workload GPU parity tests use
(tests/oracle_pool.py) reports what it is given: outputs equal to the oracle's
give errors at rounding level, and an error planted in one pair, one head or
one step is found at its size (CPU only, small shapes)."""
import os

import numpy as np
import torch

import kda_inputs as ki
import oracle
import oracle_pool


def _decode_run(N, H, d, steps, plant=None):
    """Decode steps through DecodeRun with the oracle's own fp32-rounded outputs
    standing in for the GPU's; plant = (step, n, h, col, delta) adds delta to
    one output element."""
    state = ki.decode_state(N, H, d, seed=5)
    S = state.double().numpy()
    o_max = []
    with oracle_pool.DecodeRun(N, H, d, d, workers=3) as run:
        run.save_state0(state)
        for s in range(steps):
            x = ki.decode_inputs(N, H, d, dtype="bf16", seed=6, step=s)
            o, S = oracle.kda_decode_step(*(ki.to_numpy(x[n]) for n in ("q", "k", "v", "log_alpha", "beta")), S)
            o_max.append(float(np.abs(o).max()))
            o32 = torch.from_numpy(o.astype(np.float32))
            if plant is not None and plant[0] == s:
                o32[plant[1], plant[2], plant[3]] += plant[4]
            run.save_step(x, o32)
        r = run.compare(torch.from_numpy(S.astype(np.float32)))
        root = run.root
    return r, root, o_max


def test_decode_run_matches_itself():
    r, root, _ = _decode_run(7, 3, 16, 4)
    assert r["finite"] and r["workers"] == 3 and r["pair_steps"] == 7 * 3 * 4
    assert r["rel_o"] < 1e-6 and r["rel_f"] < 1e-6
    assert not os.path.exists(root)


def test_decode_run_finds_a_planted_error():
    # the planted element sits in the last worker's sequences, in step 2
    r, _, o_max = _decode_run(7, 3, 16, 4, plant=(2, 6, 1, 5, 0.25))
    assert abs(r["rel_o"] - 0.25 / o_max[2]) < 1e-5 and r["rel_f"] < 1e-6


def test_prefill_pool_finds_a_planted_error():
    x = ki.prefill_inputs([40, 25], H=4, d=16, dtype="bf16", la_law="softplus", init="normal", seed=8)
    n = ki.to_numpy
    o, fin = oracle.kda_prefill(n(x.q), n(x.k), n(x.v), n(x.log_alpha), n(x.beta), n(x.init_state),
                                n(x.cu_seqlens))
    o32, f32 = torch.from_numpy(o.astype(np.float32)), torch.from_numpy(fin.astype(np.float32))
    kw = dict(init_state=x.init_state, cu_seqlens=x.cu_seqlens, workers=2)
    r = oracle_pool.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, o_gpu=o32, fin_gpu=f32, **kw)
    assert r["finite"] and r["heads"] == 4 and r["token_heads"] == 65 * 4
    assert r["rel_o"] < 1e-6 and r["rel_f"] < 1e-6
    o32[50, 3, 7] += 0.5
    f32[1, 2, 3, 4] -= 0.5
    r = oracle_pool.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, o_gpu=o32, fin_gpu=f32, **kw)
    assert r["rel_o"] >= 0.5 / float(np.abs(o).max()) - 1e-6
    assert r["rel_f"] >= 0.5 / float(np.abs(fin).max()) - 1e-6
