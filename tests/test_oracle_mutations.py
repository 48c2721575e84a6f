"""Every pin set is only as good as the mistakes it catches.

Each function below is a copy of the oracle's token loop with ONE plausible
mistake planted in it (on the CPU; nothing here touches a GPU).  The test
asserts that at least one pin from ``pins.ALL_PINS`` rejects every mutant, so a
dropped term, a wrong sign, a wrong index or a transposed operand in the oracle
could not pass its own pins.
"""
import numpy as np
import pytest

from pins import ALL_PINS, run_pin


def _loop(q, k, v, la, b, S0, step):
    q, k, v, la, b = (np.asarray(x, dtype=np.float64) for x in (q, k, v, la, b))
    S = np.asarray(S0, dtype=np.float64).copy()
    o = np.zeros(v.shape)
    for t in range(q.shape[0]):
        S, o[t] = step(S, q[t], k[t], v[t], la[t], b[t])
    return o, S


def _mv(S, x):          # S^T x per pair
    return np.einsum("bkv,bk->bv", S, x)


def _outer(x, y):
    return x[:, :, None] * y[:, None, :]


def m_decay_on_value_index(S, q, k, v, la, b):
    S = S * np.exp(la)[:, None, :]              # alpha applied to the d_v columns
    S = S + b[:, None, None] * _outer(k, v - _mv(S, k))
    return S, _mv(S, q)


def m_undecayed_prediction(S, q, k, v, la, b):
    pred = _mv(S, k)                            # error formed before the decay
    S = np.exp(la)[:, :, None] * S
    S = S + b[:, None, None] * _outer(k, v - pred)
    return S, _mv(S, q)


def m_missing_beta(S, q, k, v, la, b):
    S = np.exp(la)[:, :, None] * S
    S = S + _outer(k, v - _mv(S, k))
    return S, _mv(S, q)


def m_wrong_sign(S, q, k, v, la, b):
    S = np.exp(la)[:, :, None] * S
    S = S + b[:, None, None] * _outer(k, v + _mv(S, k))
    return S, _mv(S, q)


def m_transposed_output(S, q, k, v, la, b):
    S = np.exp(la)[:, :, None] * S
    S = S + b[:, None, None] * _outer(k, v - _mv(S, k))
    return S, np.einsum("bkv,bv->bk", S, q)     # S q instead of S^T q


def m_output_before_update(S, q, k, v, la, b):
    S = np.exp(la)[:, :, None] * S
    o = _mv(S, q)
    S = S + b[:, None, None] * _outer(k, v - _mv(S, k))
    return S, o


def m_decay_after_write(S, q, k, v, la, b):
    S = S + b[:, None, None] * _outer(k, v - _mv(S, k))
    S = np.exp(la)[:, :, None] * S
    return S, _mv(S, q)


def m_no_decay(S, q, k, v, la, b):
    S = S + b[:, None, None] * _outer(k, v - _mv(S, k))
    return S, _mv(S, q)


def m_alpha_is_log_alpha(S, q, k, v, la, b):
    S = (1.0 + la)[:, :, None] * S              # first-order exp
    S = S + b[:, None, None] * _outer(k, v - _mv(S, k))
    return S, _mv(S, q)


def m_inverse_decay(S, q, k, v, la, b):
    S = np.exp(-la)[:, :, None] * S
    S = S + b[:, None, None] * _outer(k, v - _mv(S, k))
    return S, _mv(S, q)


def m_query_is_key(S, q, k, v, la, b):
    S = np.exp(la)[:, :, None] * S
    S = S + b[:, None, None] * _outer(k, v - _mv(S, k))
    return S, _mv(S, k)


def m_transposed_write(S, q, k, v, la, b):
    S = np.exp(la)[:, :, None] * S
    S = S + b[:, None, None] * _outer(v - _mv(S, k), k)
    return S, _mv(S, q)


def m_beta_squared(S, q, k, v, la, b):
    S = np.exp(la)[:, :, None] * S
    S = S + (b * b)[:, None, None] * _outer(k, v - _mv(S, k))
    return S, _mv(S, q)


def m_no_delta(S, q, k, v, la, b):
    S = np.exp(la)[:, :, None] * S
    S = S + b[:, None, None] * _outer(k, v)     # plain additive write
    return S, _mv(S, q)


def m_decay_once_per_run(S, q, k, v, la, b, _state={}):
    S = np.exp(la)[:, :, None] ** 0.5 * S       # half the log-decay
    S = S + b[:, None, None] * _outer(k, v - _mv(S, k))
    return S, _mv(S, q)


MUTANTS = [
    m_decay_on_value_index, m_undecayed_prediction, m_missing_beta, m_wrong_sign,
    m_transposed_output, m_output_before_update, m_decay_after_write, m_no_decay,
    m_alpha_is_log_alpha, m_inverse_decay, m_query_is_key, m_transposed_write,
    m_beta_squared, m_no_delta, m_decay_once_per_run,
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_some_pin_rejects_mutant(mutant):
    run = lambda q, k, v, la, b, S0: _loop(q, k, v, la, b, S0, mutant)
    caught = []
    for pin in ALL_PINS:
        try:
            run_pin(pin, run)
        except (AssertionError, ValueError, IndexError) as e:
            caught.append(pin.__name__)
    assert caught, f"no pin rejects {mutant.__name__}"


def test_unmutated_copy_passes_every_pin():
    def step(S, q, k, v, la, b):
        S = np.exp(la)[:, :, None] * S
        S = S + b[:, None, None] * _outer(k, v - _mv(S, k))
        return S, _mv(S, q)
    run = lambda q, k, v, la, b, S0: _loop(q, k, v, la, b, S0, step)
    for pin in ALL_PINS:
        run_pin(pin, run)
