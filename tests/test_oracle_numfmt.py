"""Pins for the oracle's bf16 and E4M3 codecs.

bf16 carries the scales of the int8 card (model table, row "Weights") and the
rotated activations; E4M3 carries the FP8 card's weight codes (model table,
row "Weights"). Pinned against hand-derived values (tests/golden), the
library casts of torch, and round trips over every code.
"""

import json
import os

import numpy as np
import torch

from oracle import numfmt

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_bf16_hand_values():
    case = _load("bf16_rounding.json")
    for row in case["cases"]:
        x = float.fromhex(row["x"])
        want = float.fromhex(row["bf16"]) if row["bf16"] not in ("inf", "-inf") else float(row["bf16"])
        got = float(numfmt.bf16_round(np.array([x]))[0])
        assert got == want, (row, got)


def test_bf16_matches_torch_cast_of_float32():
    # For float32 inputs a single rounding to bf16 is exactly torch's cast.
    rng = np.random.default_rng(7)
    x32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    got = numfmt.bf16_round(x32.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_ties_to_even_against_torch():
    # exact midpoints between neighbouring bf16 values, built from bits
    rng = np.random.default_rng(8)
    hi = rng.integers(0x0080, 0x7F00, 5000).astype(np.uint32)
    bits = (hi << 16) | 0x8000          # exactly half an ulp above a bf16 value
    x32 = bits.view(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    got = numfmt.bf16_round(x32.astype(np.float64))
    assert np.array_equal(got, want)
    # and the result always has an even last significand bit
    assert np.all((numfmt.bf16_to_bits(got) & 1) == 0)


def test_bf16_bits_round_trip():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = numfmt.bf16_from_bits(b)
    finite = np.isfinite(v)
    assert np.array_equal(numfmt.bf16_to_bits(v[finite]), b[finite])
    # every finite bf16 value is a fixed point of the rounding
    assert np.array_equal(numfmt.bf16_round(v[finite]), v[finite])


def test_e4m3_decode_all_codes_against_torch():
    c = np.arange(256, dtype=np.uint8)
    got = numfmt.e4m3_decode(c)
    want = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(got)
    assert np.array_equal(got[ok], want[ok])


def test_e4m3_special_codes():
    case = _load("e4m3_codes.json")
    for row in case["codes"]:
        c = int(row["code"], 16)
        v = numfmt.e4m3_decode(np.array([c], dtype=np.uint8))[0]
        if row["value"] == "nan":
            assert np.isnan(v)
        else:
            assert v == float.fromhex(row["value"]), row


def test_e4m3_encode_round_trip_all_finite_codes():
    c = np.arange(256, dtype=np.uint8)
    v = numfmt.e4m3_decode(c)
    ok = ~np.isnan(v)
    assert np.array_equal(numfmt.e4m3_encode_sat(v[ok]), c[ok])


def test_e4m3_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-12, 6, 100000)))
    x = np.clip(x, -448, 448)
    x32 = x.astype(np.float32)
    want = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = numfmt.e4m3_encode_sat(x32.astype(np.float64))
    # torch keeps the sign of values that round to zero as well
    assert np.array_equal(got, want)


def test_e4m3_midpoints_ties_to_even_against_torch():
    c = np.arange(0, 0x7E, dtype=np.uint8)          # 0 .. 416 (positive finite, below max)
    lo = numfmt.e4m3_decode(c)
    hi = numfmt.e4m3_decode(c + 1)
    mid = (lo + hi) / 2                              # exact in fp64 and in float32
    want = torch.from_numpy(mid.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = numfmt.e4m3_encode_sat(mid)
    assert np.array_equal(got, want)
    assert np.all(got % 2 == 0)                      # the even neighbour wins


def test_e4m3_saturation():
    x = np.array([448.0, 448.5, 463.99, 464.0, 480.0, 1e6, -449.0, -1e30])
    got = numfmt.e4m3_encode_sat(x)
    assert list(got) == [0x7E] * 6 + [0xFE] * 2
