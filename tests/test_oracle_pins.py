"""The fp64 oracle against its pins (CPU only)."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@settings(max_examples=150, deadline=None)
@given(D=st.integers(1, 8), L=st.integers(1, 16), chunk=st.integers(1, 17),
       seed=st.integers(0, 2**31 - 1),
       scale=st.floats(0.05, 2.0, allow_nan=False))
def test_onepass_equals_twopass_bruteforce(D, L, chunk, seed, scale):
    """The one-pass expansion vbar(1+rbar) - u equals vbar - C rho."""
    oracle_pins.pin_onepass_equals_twopass(oracle.Oracle(), D=D, L=L,
                                           chunk=chunk, seed=seed, scale=scale)


@settings(max_examples=60, deadline=None)
@given(D=st.integers(1, 6), L=st.integers(1, 12),
       seed=st.integers(0, 2**31 - 1))
def test_explicit_covariance_bruteforce(D, L, seed):
    """Oracle vs a direct numpy outer-product sum on tiny inputs."""
    r = np.random.default_rng(seed)
    q, rho = r.standard_normal(D), r.standard_normal(D)
    K, V = r.standard_normal((L, D)), r.standard_normal((L, D))
    s = 0.7
    z = s * (K @ q)
    p = np.exp(z - z.max())
    p /= p.sum()
    vbar = p @ V
    kbar = p @ K
    C = sum(p[j] * np.outer(V[j] - vbar, K[j] - kbar) for j in range(L))
    expect = vbar - C @ rho
    o = oracle.decode(q[None, None], rho[None, None], K[None, None],
                      V[None, None], scale=s)
    np.testing.assert_allclose(o[0, 0], expect, atol=1e-12, rtol=0)


def test_threads_do_not_change_results():
    r = np.random.default_rng(3)
    B, H, L, D = 3, 4, 33, 8
    q, rho = r.standard_normal((B, H, D)), r.standard_normal((B, H, D))
    k, v = r.standard_normal((B, H, L, D)), r.standard_normal((B, H, L, D))
    a = oracle.decode(q, rho, k, v, threads=1)
    b = oracle.decode(q, rho, k, v, threads=4)
    assert np.array_equal(a, b)


def test_bf16_inputs_are_upcast_exactly():
    import torch
    g = torch.Generator().manual_seed(5)
    x = torch.randn(2, 3, 4, generator=g).to(torch.bfloat16)
    a = oracle._f64(x)
    assert a.dtype == np.float64
    assert np.array_equal(a, x.to(torch.float64).numpy())
