"""Pins for the oracle's e4m3 quantization of query rows (CPU only):
torch's float8_e4m3fn conversion, constructed ties, and the row recipe's
closed forms (largest magnitude -> 448, zero rows, half-step bound)."""
import oracle
from tests import pins


def test_encode_matches_torch_float8():
    pins.check_e4m3_encode_against_torch(oracle.encode_e4m3)


def test_ties_round_to_even():
    pins.check_e4m3_ties_go_to_even(oracle.encode_e4m3)


def test_row_quantization_recipe():
    pins.check_row_quantization(oracle.quantize_rows_e4m3, oracle.dequantize_rows_e4m3)
