"""The seeded synthetic inputs follow their stated laws (CPU only)."""
import numpy as np
import torch

import kda_inputs as ki


def test_prefill_inputs_laws_and_determinism():
    a = ki.prefill_inputs([100, 37], H=3, d=16, dtype="bf16", la_law="softplus", init="normal", seed=11)
    b = ki.prefill_inputs([100, 37], H=3, d=16, dtype="bf16", la_law="softplus", init="normal", seed=11)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.log_alpha, b.log_alpha), (a.beta, b.beta), (a.init_state, b.init_state)):
        assert torch.equal(x, y)
    assert a.q.shape == (137, 3, 16) and a.q.dtype == torch.bfloat16
    assert a.log_alpha.dtype == torch.float32 and a.beta.shape == (137, 3)
    assert a.cu_seqlens.tolist() == [0, 100, 137] and a.cu_seqlens.dtype == torch.int32
    n = torch.linalg.vector_norm(a.k.float(), dim=-1)
    assert torch.all((n - 1).abs() < 2 ** -7)
    la = a.log_alpha
    assert float(la.max()) < 0 and float(la.min()) >= -5.0
    assert float(a.beta.min()) > 0 and float(a.beta.max()) < 1
    assert abs(float(a.init_state.std()) - 0.02) < 0.002


def test_log_alpha_laws():
    u = ki.prefill_inputs([512], H=2, d=8, la_law="uniform53", seed=3).log_alpha
    assert float(u.min()) >= -5.0 and float(u.max()) <= -3.0
    z = ki.prefill_inputs([8], H=1, d=4, la_law="zero", seed=3).log_alpha
    assert float(z.abs().max()) == 0.0
    f = ki.prefill_inputs([8], H=1, d=4, la_law="floor", seed=3).log_alpha
    assert torch.all(f == -5.0)


def test_varlen_lengths_range():
    L = ki.varlen_lengths(2)
    assert len(L) == 16 and min(L) >= 1024 and max(L) <= 8192
    assert L == ki.varlen_lengths(2)


def test_decode_inputs_shapes():
    d = ki.decode_inputs(5, 3, 16, seed=4, step=2)
    assert d["q"].shape == (5, 3, 16) and d["beta"].shape == (5, 3)
    s = ki.decode_state(5, 3, 16, seed=4)
    assert s.shape == (5, 3, 16, 16) and s.dtype == torch.float32


def test_to_numpy_is_exact_for_bf16():
    x = torch.randn(1000).to(torch.bfloat16)
    y = ki.to_numpy(x)
    assert y.dtype == np.float32
    assert torch.equal(torch.from_numpy(y).to(torch.bfloat16), x)
