"""The oracle against its pins (CPU only)."""

import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle_pins as P
from oracle import sdpa as O


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


@settings(max_examples=40, deadline=None)
@given(
    B=st.integers(1, 2), Nq=st.integers(1, 6), Nk=st.integers(1, 6), G=st.integers(1, 3),
    Hkv=st.integers(1, 2), d=st.integers(1, 4), causal=st.booleans(),
    scale=st.floats(0.05, 3.0), seed=st.integers(0, 2**31 - 1),
)
def test_random_tiny_vs_brute_force(B, Nq, Nk, G, Hkv, d, causal, scale, seed):
    q, k, v = P.rng_case(seed, B, Nq, Nk, G * Hkv, Hkv, d, std=2.0)
    o_ref, l_ref = P.brute_attention(q, k, v, causal, scale)
    o, l = O.attention(q, k, v, causal, scale)
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(l - l_ref)) <= 1e-12


def test_attention_rows_matches_full():
    q, k, v = P.rng_case(5, 2, 20, 20, 4, 2, 8)
    o, l = O.attention(q, k, v, True, 0.3)
    rows = [0, 7, 19]
    orow, lrow = O.attention_rows(q, k, v, True, 0.3, 1, 3, rows)
    assert np.array_equal(orow, o[1, rows, 3]) and np.array_equal(lrow, l[1, 3, rows])


def test_extreme_scores_stay_finite():
    # scores near 1e3 in magnitude: the max-subtraction keeps exp finite
    q, k, v = P.rng_case(6, 1, 6, 6, 1, 1, 4)
    o, l = O.attention(q * 40.0, k * 40.0, v, False, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    o2, l2 = P.brute_attention(q * 40.0, k * 40.0, v, False, 1.0)
    assert np.max(np.abs(o - o2)) <= 1e-12
    assert np.max(np.abs(l - l2)) <= 1e-9 * np.max(np.abs(l2))


def test_empty_key_set_reading():
    # No visible key (Nk = 0): O = 0 and LSE = -inf, never NaN.
    q = np.ones((1, 2, 1, 3))
    k = np.zeros((1, 0, 1, 3))
    v = np.zeros((1, 0, 1, 3))
    o, l = O.attention(q, k, v, False, 1.0)
    assert np.all(o == 0.0) and np.all(l == -math.inf)
    od, ld = O.decode(q[:, :1], np.zeros((1, 4, 1, 3)), np.zeros((1, 4, 1, 3)), [0], 1.0)
    assert np.all(od == 0.0) and np.all(ld == -math.inf)


def test_kv_head_rejects_indivisible():
    with pytest.raises(ValueError):
        O.kv_head_of(0, 6, 4)
