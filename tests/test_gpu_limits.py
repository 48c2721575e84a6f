"""Entry points at the edges of their size range (MI355X): many heads, thousands of packed
sequences, a large decode batch, and the time split near the head count its 32-bit offsets
allow.  Outputs are checked against the fp64 oracle on sampled heads or pairs."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import kda_chunk_prefill, kda_chunk_prefill_split, kda_decode_step

pytestmark = pytest.mark.gpu


def _sampled_prefill_check(x, o, fin, heads, tol):
    """Oracle on the sampled heads only (sliced on the device before the copy to the host)."""
    hs = torch.tensor(heads, device=o.device)
    sel = lambda t: None if t is None else host(t.index_select(1, hs))
    o_ref, f_ref = oracle.kda_prefill(sel(x.q), sel(x.k), sel(x.v), sel(x.log_alpha), sel(x.beta),
                                      sel(x.init_state), host(x.cu_seqlens))
    eo = rel_err(sel(o), o_ref)
    ef = rel_err(sel(fin), f_ref)
    announce(f"  sampled heads {heads}: rel err o={eo:.3e} final={ef:.3e} (tol {tol})")
    assert eo <= tol and ef <= tol


def test_prefill_eight_thousand_heads():
    """H = 8192 (16,384 workgroups, the largest per-row strides of the buffer offsets at this T)."""
    H = 8192
    x = ki.prefill_inputs([130], H=H, d=128, dtype="bf16", init="normal", seed=31, device=device())
    announce(f"prefill T=130 H={H} d=128 bf16")
    o, fin = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state)
    torch.cuda.synchronize()
    heads = sorted(np.random.default_rng(31).choice(H, 4, replace=False).tolist()) + [H - 1]
    _sampled_prefill_check(x, o, fin, heads, TOL["bf16"])


def test_prefill_two_thousand_packed_sequences():
    """2000 packed sequences of 0 to 40 tokens (zero-length ones included), H = 2."""
    lengths = np.random.default_rng(32).integers(0, 41, size=2000).tolist()
    x = ki.prefill_inputs(lengths, H=2, d=64, dtype="f32", init="normal", seed=32, device=device(), packed=True)
    announce(f"prefill 2000 packed sequences, {sum(lengths)} tokens, H=2 d=64 fp32")
    o, fin = kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.kda_prefill(host(x.q), host(x.k), host(x.v), host(x.log_alpha), host(x.beta),
                                      host(x.init_state), host(x.cu_seqlens))
    eo, ef = rel_err(host(o), o_ref), rel_err(host(fin), f_ref)
    announce(f"  rel err o={eo:.3e} final={ef:.3e}")
    assert eo <= TOL["f32"] and ef <= TOL["f32"]


def test_decode_large_batch_sampled_pairs():
    """N = 2048 sequences x H = 64 heads (131,072 pairs, 2.1 GB of d = 64 state), one step."""
    N, H, d = 2048, 64, 64
    state = ki.decode_state(N, H, d, seed=33, device=device())
    dx = ki.decode_inputs(N, H, d, dtype="bf16", seed=33, step=0, device=device())
    announce(f"decode N={N} H={H} d={d} bf16")
    rng = np.random.default_rng(33)
    pairs = [(int(n), int(h)) for n, h in zip(rng.integers(0, N, 16), rng.integers(0, H, 16))] + [(N - 1, H - 1)]
    S0 = {p: host(state[p[0], p[1]]).astype(np.float64) for p in pairs}
    o = kda_decode_step(dx["q"], dx["k"], dx["v"], dx["log_alpha"], dx["beta"], state)
    torch.cuda.synchronize()
    worst_o = worst_s = 0.0
    for (n, h) in pairs:
        sl = lambda t: host(t[n:n + 1, h:h + 1])
        o_ref, s_ref = oracle.kda_decode_step(sl(dx["q"]), sl(dx["k"]), sl(dx["v"]), sl(dx["log_alpha"]),
                                              sl(dx["beta"]), S0[(n, h)][None, None])
        worst_o = max(worst_o, rel_err(host(o[n:n + 1, h:h + 1]), o_ref))
        worst_s = max(worst_s, rel_err(host(state[n:n + 1, h:h + 1]), s_ref))
    announce(f"  {len(pairs)} sampled pairs: worst rel err o={worst_o:.3e} state={worst_s:.3e}")
    assert worst_o <= TOL["bf16"] and worst_s <= TOL["bf16"]


def test_split_with_many_heads():
    """The time split at H = 32,000, d = 128 bf16: 512 * H * 128 * 2 bytes = 4.19e9, just under
    the 2^32 of the correction's 32-bit offsets (the host refuses larger H; see the ABI tests)."""
    H = 32000
    x = ki.prefill_inputs([300], H=H, d=128, dtype="bf16", init="normal", seed=34, device=device())
    announce(f"split prefill T=300 H={H} d=128 bf16, 3 segments")
    o, fin = kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, segments=3)
    torch.cuda.synchronize()
    heads = sorted(np.random.default_rng(34).choice(H, 3, replace=False).tolist()) + [H - 1]
    _sampled_prefill_check(x, o, fin, heads, TOL["bf16"])
