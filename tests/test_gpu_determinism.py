"""Every entry point is bitwise deterministic run to run (MI355X): the same
inputs give the same output bits, whatever the order in which workgroups are
scheduled."""
import pytest
import torch

import kda_inputs as ki
from gpu_util import announce, device
from gated_delta_rule_09_amd import (kda_chunk_prefill_gated, kda_chunk_prefill_gated_epilogue, kda_decode_step,
                                     kda_decode_step_fused, kda_decode_step_gated, kda_output_gate_rmsnorm,
                                     kda_short_conv_prologue)

pytestmark = pytest.mark.gpu


def twice(fn):
    a = fn()
    b = fn()
    torch.cuda.synchronize()
    return a, b


def same(a, b):
    if isinstance(a, (tuple, list)):
        return all(same(x, y) for x, y in zip(a, b))
    return a is None and b is None or torch.equal(a, b)


def test_gated_prefill_and_epilogue_deterministic():
    announce("determinism: gated prefill, gated prefill + epilogue (packed varlen)")
    x = ki.gated_inputs([700, 1, 333, 64], H=8, d=128, dtype="bf16", seed=80, device=device())
    og = ki.out_gate_inputs((sum(x.lengths), 8, 128), "bf16", seed=80, device=device())
    assert same(*twice(lambda: kda_chunk_prefill_gated(x.q, x.k, x.v, x.g_logits, x.a_log, x.beta_logits,
                                                       x.init_state, x.cu_seqlens)))
    assert same(*twice(lambda: kda_chunk_prefill_gated_epilogue(x.q, x.k, x.v, x.g_logits, x.a_log, x.beta_logits,
                                                                og["gate"], og["weight"], init_state=x.init_state,
                                                                cu_seqlens=x.cu_seqlens)))


def test_streaming_kernels_deterministic():
    announce("determinism: epilogue, prologue")
    e = ki.epilogue_inputs((999, 7, 128), "bf16", seed=81, device=device())
    assert same(*twice(lambda: kda_output_gate_rmsnorm(e["o"], e["gate"], e["weight"])))
    p = ki.prologue_inputs([40, 0, 300, 5], H=6, d=128, dtype="bf16", seed=81, device=device())
    assert same(*twice(lambda: kda_short_conv_prologue(p["x_q"], p["x_k"], p["x_v"], p["conv_w"], p["conv_state"],
                                                       p["cu_seqlens"])))


def test_decode_variants_deterministic():
    announce("determinism: decode, gated decode, fused decode step")
    N, H, d = 33, 6, 128
    st = ki.decode_state(N, H, d, seed=82, device=device())
    x = ki.decode_inputs(N, H, d, seed=82, step=0, device=device())
    g = ki.decode_gated_inputs(N, H, d, seed=82, step=0, device=device())
    og = ki.out_gate_inputs((N, H, d), "bf16", seed=82, device=device())
    pr = ki.decode_prologue_inputs(N, H, d, "bf16", seed=82, device=device())

    def run(fn):
        s = st.clone()
        return fn(s), s

    assert same(*twice(lambda: run(lambda s: kda_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], s))))
    assert same(*twice(lambda: run(lambda s: kda_decode_step_gated(g["q"], g["k"], g["v"], g["g_logits"],
                                                                   g["a_log"], g["beta_logits"], s))))

    def fused(s):
        cs = pr["conv_state"].clone()
        y = kda_decode_step_fused(pr["x_q"], pr["x_k"], pr["x_v"], pr["conv_w"], cs, g["g_logits"], g["a_log"],
                                  g["beta_logits"], og["gate"], s, norm_weight=og["weight"])
        return y, cs

    assert same(*twice(lambda: run(fused)))
