"""Pins for the oracle's low-precision formats (CPU only).  e4m3
quantization of query rows: torch's float8_e4m3fn conversion, constructed
ties, and the row recipe's closed forms (largest magnitude -> 448, zero
rows, half-step bound).  e2m1: the 16 values listed by hand, and the nibble
order against a packer written in the test."""
import oracle
from tests import pins


def test_encode_matches_torch_float8():
    pins.check_e4m3_encode_against_torch(oracle.encode_e4m3)


def test_ties_round_to_even():
    pins.check_e4m3_ties_go_to_even(oracle.encode_e4m3)


def test_row_quantization_recipe():
    pins.check_row_quantization(oracle.quantize_rows_e4m3, oracle.dequantize_rows_e4m3)


def test_e2m1_values():
    pins.check_e2m1_table(oracle.e2m1_decode_table)


def test_e2m1_nibble_order():
    pins.check_e2m1_packing(oracle.decode_e2m1_packed)
