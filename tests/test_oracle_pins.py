"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.default())


@settings(max_examples=25, deadline=None)
@given(Bsz=st.integers(1, 2), L=st.integers(1, 12), D=st.integers(1, 4), N=st.integers(1, 6),
       seed=st.integers(0, 2**31 - 1), states=st.booleans())
def test_closed_form_random_shapes(Bsz, L, D, N, seed, states):
    pins.pin_closed_form(oracle.default(), seed=seed, shape=(Bsz, L, D, N), states=states)


def test_empty_sequence_keeps_state():
    orc = oracle.default()
    rng = np.random.default_rng(0)
    c = pins.rand_case(rng, 2, 0, 3, 4, states=True)
    y, h, cs = orc.conv_scan_fwd(**c)
    assert y.shape == (2, 0, 3)
    assert np.array_equal(h, c["ssm_state"]) and np.array_equal(cs, c["conv_state"])


def test_oracle_threads_agree():
    orc = oracle.default()
    rng = np.random.default_rng(1)
    c = pins.rand_case(rng, 2, 33, 7, 4, states=True)
    y1, h1, _ = orc.conv_scan_fwd(**c, nthreads=1)
    y4, h4, _ = orc.conv_scan_fwd(**c, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(h1, h4)
