"""Pins of the producer-step oracle (CPU only)."""

import oracle_pins as P
from oracle import fp8
from oracle import store_kv as SK


def test_round_bf16_library():
    P.pin_round_bf16_library(SK.round_bf16)


def test_e4m3_round_library():
    P.pin_e4m3_round_library(SK.e4m3_round, fp8.e4m3_table)


def test_hadamard():
    P.pin_hadamard(SK.hadamard)


def test_rope():
    P.pin_rope(SK.rope)


def test_rms_norm_library():
    P.pin_rms_norm_library(SK.rms_norm)


def test_scores_invariant_under_hadamard():
    P.pin_store_kv_scores_invariant(SK.ref_store_kv)


def test_composition_closed_forms():
    P.pin_store_kv_composition(SK.ref_store_kv)
