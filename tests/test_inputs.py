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


def test_gated_inputs_laws():
    x = ki.gated_inputs([300], H=4, d=16, dtype="bf16", seed=5)
    y = ki.gated_inputs([300], H=4, d=16, dtype="bf16", seed=5)
    assert torch.equal(x.g_logits, y.g_logits) and torch.equal(x.a_log, y.a_log)
    assert x.g_logits.dtype == torch.bfloat16 and x.g_logits.shape == (300, 4, 16)
    assert abs(float(x.g_logits.float().std()) - 2.0) < 0.2
    assert float(x.a_log.min()) >= -1.0 and float(x.a_log.max()) <= 1.0
    assert x.beta_logits.dtype == torch.float32 and abs(float(x.beta_logits.std()) - 1.0) < 0.15


def test_epilogue_inputs_laws():
    e = ki.epilogue_inputs((400, 3, 64), "bf16", seed=9)
    assert torch.equal(e["o"], ki.epilogue_inputs((400, 3, 64), "bf16", seed=9)["o"])
    assert e["o"].shape == (400, 3, 64) and e["gate"].dtype == torch.bfloat16 and e["weight"].shape == (64,)
    rms = e["o"].float().pow(2).mean(-1).sqrt().flatten()
    assert float(rms.min()) > 1e-4 and float(rms.max()) < 40.0          # row scales 10^U[-3, 1]
    assert float(rms.min()) < 1e-2 and float(rms.max()) > 3.0
    assert abs(float(e["gate"].float().std()) - 2.0) < 0.1
    assert float(e["weight"].min()) >= 0.5 and float(e["weight"].max()) <= 1.5
    g = ki.out_gate_inputs((7, 3, 64), "f32", seed=9, step=1)
    assert g["gate"].dtype == torch.float32 and torch.equal(g["weight"], ki.out_gate_inputs((2, 3, 64), "f32", seed=9)["weight"])


def test_prologue_inputs_laws():
    p = ki.prologue_inputs([5, 0, 9], H=2, d=16, d_v=8, dtype="bf16", seed=3)
    assert p["x_q"].shape == (14, 2, 16) and p["x_v"].shape == (14, 2, 8)
    assert p["conv_w"].shape == (2, 40, 4) and p["conv_w"].dtype == torch.float32
    assert float(p["conv_w"].abs().max()) <= 0.5
    assert p["conv_state"].shape == (3, 3, 2, 40) and p["conv_state"].dtype == torch.bfloat16
    assert p["cu_seqlens"].tolist() == [0, 5, 5, 14]
    assert ki.prologue_inputs([4], H=1, d=16, state=False, seed=3)["conv_state"] is None
    d0 = ki.decode_prologue_inputs(3, 2, 16, "bf16", seed=4, step=0)
    d1 = ki.decode_prologue_inputs(3, 2, 16, "bf16", seed=4, step=1)
    assert torch.equal(d0["conv_w"], d1["conv_w"]) and torch.equal(d0["conv_state"], d1["conv_state"])
    assert not torch.equal(d0["x_q"], d1["x_q"])
