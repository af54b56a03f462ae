"""Pins for the oracle's paged-cache gather (CPU)."""
import oracle
from tests import pins


def test_gather_pages_round_trip():
    pins.check_gather_pages_round_trip(oracle.gather_pages)


def test_gather_pages_identity():
    pins.check_gather_pages_identity(oracle.gather_pages)
