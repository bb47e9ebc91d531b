"""The fp64 recurrent oracle against closed forms, invariants and the chunked
form (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins


def _orc(lib):
    def f(q, k, v, alpha, beta, S0=None, eta=None):
        return oracle.recurrent(q, k, v, alpha, beta, S0=S0, eta=eta, lib=lib)
    return f


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    pin(_orc(oracle_lib))


def test_null_alpha_is_one_and_null_S0_is_zero(oracle_lib):
    r = np.random.default_rng(0)
    q, k = r.standard_normal((2, 1, 2, 9, 4))
    v = r.standard_normal((1, 2, 9, 3))
    beta = r.uniform(0, 1, (1, 2, 9))
    O1, S1 = oracle.recurrent(q, k, v, None, beta, lib=oracle_lib)
    O2, S2 = oracle.recurrent(q, k, v, np.ones_like(beta), beta,
                              S0=np.zeros((1, 2, 3, 4)), lib=oracle_lib)
    assert np.array_equal(O1, O2) and np.array_equal(S1, S2)


def test_heads_independent(oracle_lib):
    """Each (b, h) sequence is independent: running one head alone gives the
    same bits as running it inside the batch."""
    r = np.random.default_rng(1)
    q, k = r.standard_normal((2, 2, 3, 11, 4))
    v = r.standard_normal((2, 3, 11, 5))
    a = r.uniform(0.5, 1, (2, 3, 11))
    b = r.uniform(0, 1, (2, 3, 11))
    O, S = oracle.recurrent(q, k, v, a, b, lib=oracle_lib)
    sl = (slice(1, 2), slice(2, 3))
    O1, S1 = oracle.recurrent(q[sl], k[sl], v[sl], a[sl], b[sl], lib=oracle_lib)
    assert np.array_equal(O[sl], O1) and np.array_equal(S[sl], S1)


def test_bad_arguments_raise(oracle_lib):
    with pytest.raises(ValueError):
        oracle.recurrent(np.zeros((1, 1, 4, 3)), np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 4, 2)),
                         None, np.zeros((1, 1, 4)), lib=oracle_lib)
