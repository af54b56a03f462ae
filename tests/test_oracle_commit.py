"""Pins for the oracle's commit step (CPU)."""
import numpy as np
import pytest

import oracle
from tests import pins


def test_commit_golden():
    pins.check_commit_golden(oracle.commit_accepted)


def test_commit_against_parent_chase():
    pins.check_commit_against_parent_chase(oracle.commit_accepted, oracle.accept_walk)


def test_commit_rejects_bad_paths():
    k = np.zeros((1, 1, 10, 2))
    for L, path in [(3, [0, 1, 2]), (1, [1, 2]), (2, [0, 2, 2]), (1, [0, 9])]:
        pn = np.array([path + [-1] * (5 - len(path))], dtype=np.int32)
        with pytest.raises(ValueError):
            oracle.commit_accepted(k, k, np.array([2]), np.array([L]), pn, 5)
