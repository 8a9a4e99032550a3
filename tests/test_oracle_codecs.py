"""Pins of the oracle's storage codecs (bf16 and OCP E4M3FN) against the format
definitions and against torch's CPU casts (a library routine)."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_definition_points():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_definition_points.json")))
    tab = e4m3.decode_table()
    for code, val in g["points"]:
        assert tab[code] == val and np.signbit(tab[code]) == np.signbit(val), code
    for code in g["nan_codes"]:
        assert np.isnan(tab[code])
    assert np.sum(np.isfinite(tab)) == 254
    for case in g["encode_cases"]:
        assert int(e4m3.encode_rne(np.array([case["x"]]))[0]) == case["code"], case


def test_e4m3_table_monotone_and_symmetric():
    tab = e4m3.decode_table()
    pos = tab[:127]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(tab[128:255], -tab[:127])


def test_e4m3_roundtrip_all_finite_codes():
    tab = e4m3.decode_table()
    codes = np.array([c for c in range(256) if np.isfinite(tab[c]) and c != 0x80], np.uint8)
    assert np.array_equal(e4m3.encode_rne(tab[codes]), codes)


def test_e4m3_midpoints_round_to_even():
    tab = e4m3.decode_table()
    for c in range(0, 126):
        mid = 0.5 * (tab[c] + tab[c + 1])
        got = int(e4m3.encode_rne(np.array([mid]))[0])
        even = c if (c & 1) == 0 else c + 1
        assert got == even, (c, mid, got)
        # just inside each side of the midpoint
        lo = np.nextafter(mid, -np.inf)
        hi = np.nextafter(mid, np.inf)
        assert int(e4m3.encode_rne(np.array([lo]))[0]) == c
        assert int(e4m3.encode_rne(np.array([hi]))[0]) == c + 1


def test_e4m3_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 50,
        rng.uniform(-2 ** -5, 2 ** -5, 100000).astype(np.float32),
        np.exp(rng.uniform(-12, 6.1, 100000)).astype(np.float32),
    ])
    x = x[(np.abs(x) < 464) & (x != 0)]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3.encode_rne(x)
    # a magnitude that rounds to zero is +0 in the oracle (torch keeps the sign)
    ref = np.where((ref & 0x7F) == 0, 0, ref)
    assert np.array_equal(got, ref)


def test_e4m3_saturates_and_rejects_nan():
    assert np.all(e4m3.encode_rne(np.array([448.0, 449, 1e30, np.inf])) == 0x7E)
    assert np.all(e4m3.encode_rne(np.array([-448.0, -1e30, -np.inf])) == 0xFE)
    with pytest.raises(ValueError):
        e4m3.encode_rne(np.array([np.nan]))


def test_bf16_decode_points():
    assert bf16.decode(np.array([0x3F80]))[0] == 1.0
    assert bf16.decode(np.array([0xC000]))[0] == -2.0
    assert bf16.decode(np.array([0x0001]))[0] == 2.0 ** -133
    assert bf16.decode(np.array([0x7F7F]))[0] == (2 - 2 ** -7) * 2.0 ** 127


def test_bf16_encode_ties_to_even():
    assert bf16.encode_rne(np.array([1 + 2 ** -8]))[0] == 0x3F80
    assert bf16.encode_rne(np.array([1 + 3 * 2 ** -8]))[0] == 0x3F82
    assert bf16.encode_rne(np.array([-(1 + 2 ** -8 + 2 ** -30)]))[0] == 0xBF81


def test_bf16_encode_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(300000) * 10.0 ** rng.integers(-30, 30, 300000),
                        rng.standard_normal(1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16.encode_rne(x.astype(np.float64)), ref)
    assert np.array_equal(bf16.decode(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                          .to(torch.float64).numpy())
