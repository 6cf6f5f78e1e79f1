"""The GPU parity checker's bars on planted errors (CPU only): the state bar
must catch one bad element that the per-head Frobenius ratio alone would
average away, and must pass fp32-level rounding noise."""
import numpy as np
import pytest

from . import parity


def _state(seed=3):
    r = np.random.default_rng(seed)
    return r.normal(0, 0.05, (2, 4, 128, 128))


def test_state_bar_passes_rounding_noise():
    S = _state()
    noisy = S * (1 + np.random.default_rng(4).normal(0, 1e-7, S.shape))
    rep = parity.check_state(noisy.astype(np.float32), S, report=True)
    assert rep["fro"] < 1e-6 and rep["elem_rms"] < 1e-5


def test_state_bar_catches_one_element_off_by_its_low_half():
    # one element of one head wrong by 2^-11 of a large value: the Frobenius
    # ratio stays far under 1e-4, the elementwise bar fails
    S = _state()
    bad = S.copy()
    i = np.unravel_index(np.argmax(np.abs(S[1, 2])), S[1, 2].shape)
    bad[1, 2][i] *= 1 + 2.0 ** -11
    assert parity.rel_fro_per_head(bad, S, axes=(2, 3)).max() < 1e-4
    with pytest.raises(parity.ParityError, match="max\\|dS\\|"):
        parity.check_state(bad, S)


def test_state_bar_catches_non_finite_values():
    S = _state()
    bad = S.copy()
    bad[0, 0, 5, 5] = np.nan
    with pytest.raises(parity.ParityError):
        parity.check_state(bad, S)


def test_o_bar_catches_one_element_off_by_its_low_half():
    r = np.random.default_rng(5)
    o = r.normal(0, 1e-3, (64, 6, 128))
    bad = o.copy()
    bad[10, 3, 7] += 4 * 1e-3 * 2.0 ** -11 * 2
    with pytest.raises(parity.ParityError):
        parity.check_o(bad, o)
