"""Pins of the 8-bit KV cache oracle (CPU only)."""

import oracle_pins as P
from oracle import fp8


def test_e4m3_matches_library_decoding():
    P.pin_e4m3_library(fp8.e4m3_table)


def test_e4m3_closed_forms():
    P.pin_e4m3_closed_forms(fp8.e4m3_value)


def test_fp8_decode_matches_library_attention():
    P.pin_fp8_decode_library(fp8.ref_decode_fp8)


def test_fp8_scale_laws():
    P.pin_fp8_scale_laws(fp8.ref_decode_fp8)
