"""Pins for the fp64 input-prologue oracle ("Kimi K3 -- Architecture Notes",
section 1.1: the q/k/v projections pass a short convolution and Swish, then q
and k are L2-normalised; the "Kimi Delta Attention (KDA)" box of the "Kimi K3"
visualiser page: convolution width 4), and
mutants that the pins must reject.

The pins are closed forms and structural facts that hold however the oracle
evaluates the formulas: single-tap weights give the identity and a pure
3-token delay through the state, an impulse returns the taps in reverse
order, a sequence split anywhere and resumed through the state gives the same
result, packed sequences do not see each other, Swish(0) = 0,
Swish(ln 3) = (3/4) ln 3, Swish(u) - Swish(-u) = u, normalised rows have unit
norm, a row of norm sqrt(eps) is scaled by 1/sqrt 2, and the order Swish-then-
norm maps (ln 3, -ln 3) to (3, -1) / sqrt 10 (norm-then-Swish would not).
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest

import oracle

TOL = 1e-12
K = 4


def _rand(rng, T=11, H=2, C=5):
    return rng.standard_normal((T, H, C)), rng.standard_normal((H, C, K)), rng.standard_normal((1, K - 1, H, C))


def pin_identity_tap(impl, rng):
    x, _, st = _rand(rng)
    w = np.zeros((x.shape[1], x.shape[2], K))
    w[..., K - 1] = 1.0
    y, fin = impl.conv(x, w, st)
    assert np.allclose(y, x, rtol=0, atol=TOL), "the last tap meets the current input"
    assert np.allclose(fin[0], x[-(K - 1):], rtol=0, atol=TOL), "the final state holds the last K-1 inputs"


def pin_delay(impl, rng):
    x, _, st = _rand(rng)
    w = np.zeros((x.shape[1], x.shape[2], K))
    w[..., 0] = 1.0
    y, _ = impl.conv(x, w, st)
    assert np.allclose(y[:K - 1], st[0], rtol=0, atol=TOL), "the first outputs come from the state, oldest first"
    assert np.allclose(y[K - 1:], x[:-(K - 1)], rtol=0, atol=TOL), "the first tap delays by K-1 tokens"
    y0, _ = impl.conv(x, w, None)
    assert np.allclose(y0[:K - 1], 0.0, rtol=0, atol=TOL), "no state means zeros before the start"


def pin_impulse(impl, rng):
    T, H, C, t0 = 12, 1, 3, 5
    x = np.zeros((T, H, C))
    x[t0, 0, 1] = 1.0
    w = rng.standard_normal((H, C, K))
    y, _ = impl.conv(x, w)
    for m in range(K):
        assert abs(y[t0 + m, 0, 1] - w[0, 1, K - 1 - m]) <= TOL, "an impulse returns the taps newest first"
    mask = np.ones_like(y, bool)
    mask[t0:t0 + K, 0, 1] = False
    assert np.allclose(y[mask], 0.0, rtol=0, atol=TOL), "the convolution is causal and depthwise"


def pin_split_resume(impl, rng):
    x, w, st = _rand(rng, T=13)
    y, fin = impl.conv(x, w, st)
    for cut in (1, 2, 3, 7):
        ya, fa = impl.conv(x[:cut], w, st)
        yb, fb = impl.conv(x[cut:], w, fa)
        assert np.allclose(np.concatenate([ya, yb]), y, rtol=0, atol=1e-12), f"split at {cut}"
        assert np.allclose(fb, fin, rtol=0, atol=TOL), f"final state after split at {cut}"


def pin_packed(impl, rng):
    x, w, _ = _rand(rng, T=10)
    st = rng.standard_normal((3, K - 1, x.shape[1], x.shape[2]))
    cu = np.array([0, 4, 4, 10])
    y, fin = impl.conv(x, w, st, cu)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        yn, fn = impl.conv(x[a:b], w, st[n:n + 1])
        assert np.allclose(y[a:b], yn, rtol=0, atol=TOL), f"sequence {n} must not see its neighbours"
        assert np.allclose(fin[n], fn[0], rtol=0, atol=TOL)
    assert np.allclose(fin[1], st[1], rtol=0, atol=TOL), "an empty sequence keeps its state"


def _ident_w(H, dk, dv):
    w = np.zeros((H, 2 * dk + dv, K))
    w[..., K - 1] = 1.0
    return w


def pin_swish_closed(impl, rng):
    H, dk, dv = 1, 2, 3
    l3 = math.log(3.0)
    xq = rng.standard_normal((3, H, dk))
    xk = rng.standard_normal((3, H, dk))
    xv = np.array([[[0.0, l3, -l3]], [[1.5, -1.5, 4.0]], [[-2.0, 2.0, 0.5]]])
    _, _, v, _ = impl.prologue(xq, xk, xv, _ident_w(H, dk, dv))
    assert np.allclose(v[0, 0], [0.0, 0.75 * l3, -0.25 * l3], rtol=0, atol=TOL), "v = Swish(conv x_v), not normed"
    assert np.allclose(v[1, 0, 0] - v[1, 0, 1], 1.5, rtol=0, atol=TOL), "Swish(u) - Swish(-u) = u"
    assert np.allclose(v[2, 0, 1] - v[2, 0, 0], 2.0, rtol=0, atol=TOL)


def pin_order_and_norm(impl, rng):
    H, dk, dv = 1, 2, 2
    l3 = math.log(3.0)
    xq = np.array([[[l3, -l3]]])
    xk = np.array([[[-l3, l3]]])
    q, k, _, _ = impl.prologue(xq, xk, np.zeros((1, H, dv)), _ident_w(H, dk, dv), eps=0.0)
    r = math.sqrt(10.0)
    assert np.allclose(q[0, 0], [3.0 / r, -1.0 / r], rtol=0, atol=TOL), "Swish first, then the L2 norm"
    assert np.allclose(k[0, 0], [-1.0 / r, 3.0 / r], rtol=0, atol=TOL)
    xq, xk, xv = (rng.standard_normal((6, 3, 8)) for _ in range(3))
    w = rng.standard_normal((3, 24, K))
    q, k, v, _ = impl.prologue(xq, xk, xv, w, eps=0.0)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=0, atol=1e-12)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=0, atol=1e-12)
    assert not np.allclose(np.linalg.norm(v, axis=-1), 1.0, rtol=0, atol=1e-3), "v is not normalised"


def pin_eps_place(impl, rng):
    eps = oracle.L2_EPS
    u = np.zeros((1, 1, 4))
    u[0, 0, 2] = math.sqrt(eps)
    assert np.allclose(impl.l2(u, eps), u / math.sqrt(2.0 * eps), rtol=0, atol=TOL)
    assert np.allclose(impl.l2(u, eps)[0, 0, 2], 1.0 / math.sqrt(2.0), rtol=0, atol=TOL)
    assert np.allclose(impl.l2(u), impl.l2(u, 1e-6), rtol=0, atol=TOL), "the default eps is 1e-6"
    assert np.all(impl.l2(np.zeros((2, 3)), eps) == 0.0), "a zero row stays zero"


def pin_channel_blocks(impl, rng):
    H, dk, dv, T = 2, 3, 4, 5
    xq, xk, xv = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dv))
    w = np.zeros((H, 2 * dk + dv, K))
    w[:, :dk, K - 1] = 1.0                       # only q's block passes
    q, k, v, fin = impl.prologue(xq, xk, xv, w)
    assert np.allclose(k, 0.0, rtol=0, atol=TOL) and np.allclose(v, 0.0, rtol=0, atol=TOL), \
        "per head the channels are q (d_k), then k (d_k), then v (d_v)"
    assert np.allclose(q, impl.l2(oracle.swish(xq)), rtol=0, atol=1e-12)
    assert np.allclose(fin[0, :, :, dk:2 * dk], xk[-(K - 1):], rtol=0, atol=TOL), "the state packs q, k, v"
    assert np.allclose(fin[0, :, :, 2 * dk:], xv[-(K - 1):], rtol=0, atol=TOL)


PRO_PINS = (pin_identity_tap, pin_delay, pin_impulse, pin_split_resume, pin_packed, pin_swish_closed,
            pin_order_and_norm, pin_eps_place, pin_channel_blocks)

ORACLE = SimpleNamespace(conv=oracle.short_conv, prologue=oracle.kda_prologue, l2=oracle.l2_normalize)


@pytest.mark.parametrize("pin", PRO_PINS, ids=lambda p: p.__name__)
def test_prologue_oracle_pin(pin):
    pin(ORACLE, np.random.default_rng(11))


# ---- mutants: plausible mistakes, planted in a second, flag-driven copy -------

def _sig(u):
    return 1.0 / (1.0 + np.exp(-u))


def make_impl(flip_taps=False, ignore_state=False, leak=False, state_newest_first=False, final_first=False,
              norm_first=False, swish_v=True, norm_v=False, sigmoid_for_swish=False, eps_default=1e-6,
              eps_outside=False, order="qkv", lookahead=False):
    def conv(x, w, conv_state=None, cu_seqlens=None):
        x = np.asarray(x, float)
        T, H, C = x.shape
        cu = [0, T] if cu_seqlens is None else list(np.asarray(cu_seqlens))
        N = len(cu) - 1
        st = np.zeros((N, K - 1, H, C)) if (conv_state is None or ignore_state) else np.asarray(conv_state, float)
        if state_newest_first:
            st = st[:, ::-1]
        y = np.zeros_like(x)
        fin = np.zeros((N, K - 1, H, C))
        carry = None
        for n in range(N):
            a, b = cu[n], cu[n + 1]
            s0 = carry if (leak and carry is not None) else st[n]
            ext = np.concatenate([s0, x[a:b]])
            for t in range(b - a):
                for j in range(K):
                    jj = K - 1 - j if flip_taps else j
                    src = t + j + (1 if lookahead else 0)
                    if src < ext.shape[0]:
                        y[a + t] += w[:, :, jj] * ext[src]
            fin[n] = ext[:K - 1] if final_first else ext[-(K - 1):]
            carry = fin[n]
        return y, fin

    def act(u):
        return _sig(u) if sigmoid_for_swish else u * _sig(u)

    def l2(u, eps=eps_default):
        u = np.asarray(u, float)
        nrm = np.sqrt(np.sum(u * u, -1, keepdims=True))
        return u / (nrm + eps) if eps_outside else u / np.sqrt(nrm * nrm + eps)

    def prologue(xq, xk, xv, w, conv_state=None, cu_seqlens=None, eps=eps_default):
        dk = np.shape(xq)[-1]
        parts = {"q": np.asarray(xq, float), "k": np.asarray(xk, float), "v": np.asarray(xv, float)}
        x = np.concatenate([parts[c] for c in order], -1)
        y, fin = conv(x, w, conv_state, cu_seqlens)
        sizes = {"q": dk, "k": dk, "v": np.shape(xv)[-1]}
        out, o = {}, 0
        for c in order:
            out[c] = y[..., o:o + sizes[c]]
            o += sizes[c]
        def qk(u):
            return act(l2(u, eps)) if norm_first else l2(act(u), eps)
        v = act(out["v"]) if swish_v else out["v"]
        if norm_v:
            v = l2(v, eps)
        return qk(out["q"]), qk(out["k"]), v, fin

    return SimpleNamespace(conv=conv, prologue=prologue, l2=l2)


MUTANTS = {
    "flipped_taps": dict(flip_taps=True),
    "state_ignored": dict(ignore_state=True),
    "state_leaks_across_sequences": dict(leak=True),
    "state_newest_first": dict(state_newest_first=True),
    "final_state_first_inputs": dict(final_first=True),
    "norm_before_swish": dict(norm_first=True),
    "v_without_swish": dict(swish_v=False),
    "v_normalised": dict(norm_v=True),
    "sigmoid_for_swish": dict(sigmoid_for_swish=True),
    "eps_1e5": dict(eps_default=1e-5),
    "eps_outside_root": dict(eps_outside=True),
    "channels_kqv": dict(order="kqv"),
    "one_token_lookahead": dict(lookahead=True),
}


def test_flag_copy_without_flags_passes_every_pin():
    impl = make_impl()
    for pin in PRO_PINS:
        pin(impl, np.random.default_rng(11))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_prologue_mutant_rejected(name):
    impl = make_impl(**MUTANTS[name])
    caught = 0
    for pin in PRO_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl, np.random.default_rng(11))
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"{name} passed every prologue pin"
