"""Pins of the oracle's number formats (E4M3, bf16, E8M0) against the format
specifications, brute force and torch's library casts."""

import os

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs
from tests import brute_prologue as brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_e4m3_table_matches_ocp_spec_points():
    tab = oracle.e4m3_decode_table()
    for code, val in _read_rows("e4m3_ocp_values.txt"):
        c = int(code, 16)
        if val == "nan":
            assert np.isnan(tab[c])
        else:
            assert tab[c] == float(val)
            assert np.signbit(tab[c]) == val.startswith("-")


def test_e4m3_table_monotone_and_symmetric():
    tab = oracle.e4m3_decode_table()
    pos = tab[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(tab[0x80:0xFF], -pos)


def _sweep_values():
    tab = oracle.e4m3_decode_table()
    pos = tab[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(1)
    rand = np.exp(rng.uniform(np.log(2.0**-12), np.log(600.0), size=3000))
    extra = np.array([0.0, 2.0**-10, 2.0**-11, 3 * 2.0**-11, 448.0, 450.0, 460.0,
                      463.9, 464.0, 480.0, 1e6, 1e30])
    base = np.concatenate([pos, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                           rand, extra])
    return np.concatenate([base, -base])


def test_e4m3_encode_equals_bruteforce_nearest_even():
    vals = _sweep_values()
    got = oracle.e4m3_encode(vals)
    for v, g in zip(vals, got):
        assert g == brute.e4m3_round(float(v)), (v, g)


def test_e4m3_encode_saturates_and_keeps_sign_of_zero():
    got = oracle.e4m3_encode(np.array([1e9, -1e9, 448.0, 463.99, 464.0, -0.0, -1e-30]))
    assert list(got) == [0x7E, 0xFE, 0x7E, 0x7E, 0x7E, 0x80, 0x80]


def test_e4m3_encode_matches_torch_cast_below_448():
    rng = np.random.default_rng(2)
    v = np.concatenate([
        rng.standard_normal(20000) * 100,
        np.exp(rng.uniform(np.log(2.0**-11), np.log(448.0), size=20000)),
    ]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v.astype(np.float64)), t)


def test_e4m3_decode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_bf16_golden_rows():
    for src, want, *_ in _read_rows("bf16_values.txt"):
        x = np.array([int(src, 16)], np.uint32).view(np.float32)
        assert oracle.f32_to_bf16_bits(x)[0] == int(want, 16), src


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties and near-ties
    bits[:50000] = (bits[:50000] & 0xFFFF0000) | 0x8000
    bits[50000:60000] = (bits[50000:60000] & 0xFFFF0000) | 0x7FFF
    x = bits.view(np.float32)
    keep = ~np.isnan(x)
    x = x[keep]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(x), want)


def test_bf16_nan_stays_nan():
    x = np.array([np.nan, -np.nan], np.float32)
    back = codecs.bf16_bits_to_f32(oracle.f32_to_bf16_bits(x))
    assert np.isnan(back).all()


def test_bf16_matches_bruteforce_nearest_even():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(2000) * 10).astype(np.float32)
    got = oracle.f32_to_bf16_bits(x)
    for v, g in zip(x, got):
        assert g == brute.bf16_round_bits(float(v))


@pytest.mark.parametrize("code,val", [(127, 1.0), (128, 2.0), (126, 0.5), (0, 2.0**-127),
                                      (254, 2.0**127)])
def test_e8m0_decode_points(code, val):
    assert oracle.e8m0_decode(np.array([code]))[0] == val


def test_e8m0_nan_code():
    assert np.isnan(oracle.e8m0_decode(np.array([255]))[0])
