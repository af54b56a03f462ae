"""Pins for the oracle's vocabulary argmax (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import pins


def test_argmax_constructed_ties_and_spikes():
    pins.check_argmax_constructed(oracle.vocab_argmax)


def test_argmax_brute_force_linear_scan():
    pins.check_argmax_brute_force(oracle.vocab_argmax)


def test_argmax_single_column():
    assert list(oracle.vocab_argmax(np.array([[3.0], [-1.0]], dtype=np.float32))) == [0, 0]


def test_argmax_rejects_nan():
    with pytest.raises(ValueError):
        oracle.vocab_argmax(np.array([[0.0, np.nan]], dtype=np.float32))
