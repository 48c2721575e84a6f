"""The fp64 oracle against the facts its pins fix (CPU only)."""
import numpy as np
import pytest

import oracle
from pins import ALL_PINS, run_pin


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    run_pin(pin, oracle.kda_recurrence)


def test_decode_step_matches_single_token_prefill():
    rng = np.random.default_rng(5)
    N, H, d = 3, 2, 6
    q = rng.standard_normal((N, H, d)); k = rng.standard_normal((N, H, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, H, d)); la = -rng.uniform(0, 5, (N, H, d)); b = rng.uniform(0, 1, (N, H))
    S = rng.standard_normal((N, H, d, d))
    S_copy = S.copy()
    o, S1 = oracle.kda_decode_step(q, k, v, la, b, S)
    assert np.array_equal(S, S_copy), "decode must not modify its input"
    # the same token as a length-1 sequence per decode slot, through the packed prefill
    cu = np.arange(N + 1)
    o2, S2 = oracle.kda_prefill(q, k, v, la, b, init_state=S, cu_seqlens=cu)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-14)


def test_packed_sequences_are_independent():
    rng = np.random.default_rng(6)
    lengths = [5, 0, 9, 1, 3]
    T, H, d = sum(lengths), 2, 4
    q = rng.standard_normal((T, H, d)); k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d)); la = -rng.uniform(0, 5, (T, H, d)); b = rng.uniform(0, 1, (T, H))
    init = rng.standard_normal((len(lengths), H, d, d))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, fin = oracle.kda_prefill(q, k, v, la, b, init_state=init, cu_seqlens=cu)
    for n, L in enumerate(lengths):
        sl = slice(cu[n], cu[n + 1])
        o_n, f_n = oracle.kda_prefill(q[sl], k[sl], v[sl], la[sl], b[sl], init_state=init[n:n + 1])
        np.testing.assert_array_equal(o[sl], o_n)
        np.testing.assert_array_equal(fin[n], f_n[0])
    # the zero-length sequence returns its initial state unchanged
    np.testing.assert_array_equal(fin[1], init[1])


def test_head_subset_equals_full_slice():
    rng = np.random.default_rng(7)
    T, H, d = 13, 5, 4
    q = rng.standard_normal((T, H, d)); k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d)); la = -rng.uniform(0, 5, (T, H, d)); b = rng.uniform(0, 1, (T, H))
    init = rng.standard_normal((1, H, d, d))
    o, fin = oracle.kda_prefill(q, k, v, la, b, init_state=init)
    hs = [4, 1]
    o_s, fin_s = oracle.kda_prefill(q, k, v, la, b, init_state=init, heads=hs)
    np.testing.assert_array_equal(o_s, o[:, hs])
    np.testing.assert_array_equal(fin_s, fin[:, hs])


def test_zero_init_equals_explicit_zero_state():
    rng = np.random.default_rng(8)
    T, H, d = 7, 2, 3
    args = [rng.standard_normal((T, H, d)) for _ in range(3)] + [-rng.uniform(0, 5, (T, H, d)), rng.uniform(0, 1, (T, H))]
    o1, f1 = oracle.kda_prefill(*args)
    o2, f2 = oracle.kda_prefill(*args, init_state=np.zeros((1, H, d, d)))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


def test_decay_bound_numbers_from_the_notes():
    """Section 1.2 of the architecture notes: with log alpha >= -5 a 16-token
    tile's cumulative log-decay lies in [-80, 0], so the reciprocal rescale is
    at most e^80, which fp32 and bf16 (same 8-bit exponent) represent; a
    64-token chunk would need e^320, which they do not."""
    assert np.isfinite(np.float32(np.exp(80.0)))
    assert np.float32(np.exp(-80.0)) > 0.0
    with np.errstate(over="ignore"):
        assert not np.isfinite(np.float32(np.exp(320.0)))
    assert abs(np.exp(-5.0) - 6.7e-3) < 1e-4


def test_oracle_regression_fixture():
    """The oracle still reproduces the values its generator script stored."""
    import json, os
    from golden.make_oracle_regression import case
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    with open(os.path.join(here, "oracle_regression.json")) as f:
        ref = json.load(f)
    c = case()
    o, fin = oracle.kda_prefill(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"],
                                init_state=c["init_state"], cu_seqlens=c["cu_seqlens"])
    np.testing.assert_allclose(o, np.array(ref["o"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(fin, np.array(ref["final_state"]), rtol=0, atol=1e-13)
