"""Parity of the HIP input prologue (ShortConv(4), Swish, L2 norm of q and k;
"Kimi K3 -- Architecture Notes", section 1.1) with the fp64 oracle (MI355X)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from gpu_util import TOL, announce, device, host, rel_err
from gated_delta_rule_09_amd import kda_short_conv_prologue

pytestmark = pytest.mark.gpu

# The inputs are exact in both dtypes; the kernel sums the 4 taps and takes
# Swish and the norm in fp32 (a few ulp of the largest term), then rounds to
# the working dtype (bf16: at most 2^-8 relative).
ELEM_REL = {"f32": 1e-5, "bf16": 2.0 ** -8}
ELEM_ABS = 2e-6


def check(x, dtype, heads=None, what=""):
    announce(f"prologue {what}: lengths={x['lengths'][:5]}{'...' if len(x['lengths']) > 5 else ''} "
             f"H={x['x_q'].shape[1]} d_k={x['x_q'].shape[2]} d_v={x['x_v'].shape[2]} {dtype} "
             f"state={'yes' if x['conv_state'] is not None else 'no'}")
    q, k, v, fin = kda_short_conv_prologue(x["x_q"], x["x_k"], x["x_v"], x["conv_w"], x["conv_state"],
                                           x["cu_seqlens"])
    torch.cuda.synchronize()
    hs = slice(None) if heads is None else torch.tensor(list(heads), device=x["x_q"].device)
    sel = lambda t, ax=1: t if heads is None else t.index_select(ax, hs)    # heads picked on the device
    st = None if x["conv_state"] is None else host(sel(x["conv_state"], 2))
    rq, rk, rv, rfin = oracle.kda_prologue(host(sel(x["x_q"])), host(sel(x["x_k"])), host(sel(x["x_v"])),
                                           host(sel(x["conv_w"], 0)), st, host(x["cu_seqlens"]))
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        g = host(sel(got)).astype(np.float64)
        err = np.abs(g - ref)
        bound = ELEM_REL[dtype] * np.abs(ref) + ELEM_ABS * max(1.0, float(np.abs(ref).max()))
        worst = float((err / bound).max()) if err.size else 0.0
        announce(f"  {name}: norm-wise rel err {rel_err(g, ref) if err.size else 0:.3e}, "
                 f"worst element err / bound {worst:.3f}")
        assert np.isfinite(g).all()
        assert (err <= bound).all(), f"{name} beyond the element-wise bound"
        assert err.size == 0 or rel_err(g, ref) <= TOL[dtype]
    gf = host(sel(fin, 2))
    announce(f"  final conv state: {int((gf != rfin).sum())} mismatches of {gf.size}")
    assert np.array_equal(gf, rfin), "the final convolution state is a copy of inputs and must be exact"
    if heads is None:
        nq = np.linalg.norm(host(q).astype(np.float64), axis=-1)
        assert nq.size == 0 or np.abs(nq - 1).max() < (5e-3 if dtype == "bf16" else 1e-5)
    return q, k, v, fin


@pytest.mark.parametrize("lengths", [[1], [2], [3], [5], [64], [65], [131], [5, 0, 70, 1, 33], [2, 1, 0, 62, 3]])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prologue_ragged(lengths, dtype):
    x = ki.prologue_inputs(lengths, H=5, d=128 if dtype == "bf16" else 64, dtype=dtype, seed=sum(lengths) + 60,
                           device=device(), packed=len(lengths) > 1)
    check(x, dtype, what=f"ragged {lengths}")


@pytest.mark.parametrize("d_k,d_v", [(128, 64), (64, 128), (64, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prologue_head_dims_and_no_state(d_k, d_v, dtype):
    x = ki.prologue_inputs([37, 100], H=7, d=d_k, d_v=d_v, dtype=dtype, seed=61, device=device(), state=False)
    check(x, dtype, what=f"d_k={d_k} d_v={d_v}, zero state")


def test_prologue_split_and_resume_equals_whole():
    """Running a sequence in two calls, the second from the first's final
    state, gives the one-call result bit for bit."""
    x = ki.prologue_inputs([200], H=4, d=128, dtype="bf16", seed=62, device=device())
    q, k, v, fin = check(x, "bf16", what="whole")
    cut = 77
    a = {kk: (vv[:cut] if kk in ("x_q", "x_k", "x_v") else vv) for kk, vv in x.items()}
    a["lengths"] = [cut]
    qa, ka, va, fa = check(a, "bf16", what="first part")
    # the second part starts from the kernel's own state, so it is compared with
    # the whole run (held to the oracle above), not handed to the oracle
    qb, kb, vb, fb = kda_short_conv_prologue(x["x_q"][cut:], x["x_k"][cut:], x["x_v"][cut:], x["conv_w"], fa)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([qa, qb]), q) and torch.equal(torch.cat([ka, kb]), k)
    assert torch.equal(torch.cat([va, vb]), v) and torch.equal(fb, fin)


def test_prologue_varlen_all_heads():
    """The packed workload's shape (16 sequences of U{1K..8K} tokens, H = 96), every
    head, compared in groups of 12 heads to bound the oracle's host memory."""
    x = ki.prologue_inputs(ki.workload_lengths("varlen16"), H=96, d=128, dtype="bf16", seed=63, device=device())
    for g in np.array_split(np.arange(96), 8):
        check(x, "bf16", heads=g, what=f"packed varlen, heads {g[0]}-{g[-1]}")


def test_prologue_long_64k_sampled_heads():
    x = ki.prologue_inputs([65536], H=96, d=128, dtype="bf16", seed=64, device=device())
    check(x, "bf16", heads=np.random.default_rng(64).choice(96, 4, replace=False), what="64K")


def test_prologue_rejects_overlapping_states():
    x = ki.prologue_inputs([10], H=2, d=64, dtype="bf16", seed=65, device=device())
    with pytest.raises(Exception, match="KDA_ERR_VALUE"):
        kda_short_conv_prologue(x["x_q"], x["x_k"], x["x_v"], x["conv_w"], x["conv_state"], None,
                                conv_state_out=x["conv_state"])
