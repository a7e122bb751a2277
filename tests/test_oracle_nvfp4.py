"""Pins of the oracle's NVFP4 cache variant (the epilogue page's
``_nvfp4_quant32`` / ``_nvfp4_quant64`` quantizer and ``_nvfp4_cache_views``
layout), against things other than the oracle itself: exhaustive nearest-even
search over the E2M1 grid, exact rational products, the OCP E2M1 value table,
the page's printed formula for the swizzled scale bytes, closed-form
properties of the group scale, and the separately written scalar statement in
``tests/brute_prologue.py``. Planted mistakes at the end must each fail a pin."""

import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import codecs, prologue
from tests import brute_prologue as brute
from tests.test_oracle_pipeline import TINY_DECODE, TINY_PREFILL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_ocp_values.txt")


def _e2m1_nearest_even(x):
    """Exhaustive search: nearest E2M1 magnitude code to |x| (saturating at 6),
    ties to the code with an even mantissa bit."""
    mag = min(abs(Fraction(x)), Fraction(6))
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
            Fraction(4), Fraction(6)]
    best = min(range(8), key=lambda c: (abs(grid[c] - mag), c % 2))
    return best


def test_e2m1_decode_matches_ocp_table():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    for code, value in rows:
        assert codecs.e2m1_decode(int(code, 16)) == float(value), code


def test_e2m1_encode_equals_bruteforce_nearest_even():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    xs = list(grid) + [(a + b) / 2 for a, b in zip(grid, grid[1:])]
    xs += [np.nextafter(x, np.inf) for x in xs] + [np.nextafter(x, -np.inf) for x in xs if x > 0]
    xs += [6.5, 7.0, 100.0, 1e30, 2.0 ** -30, 0.2499999, 5.0000001]
    xs += list(np.random.default_rng(3).uniform(0, 8, 2000))
    xs = np.array(xs + [-x for x in xs], np.float64)
    got = codecs.e2m1_encode(xs)
    for x, c in zip(xs, got):
        want = _e2m1_nearest_even(x)
        assert (c & 0x7) == want, (x, c, want)
        if want:
            assert bool(c & 0x8) == (x < 0), (x, c)


def test_f32_mul_rz_is_exact_truncation():
    rng = np.random.default_rng(4)
    a = (rng.standard_normal(3000) * 10).astype(np.float32)
    b = (rng.standard_normal(3000) * 0.1).astype(np.float32)
    a[:10] = np.float32(2.8125)  # products that are exact in float32 stay unchanged
    b[:10] = np.float32(0.5)
    got = codecs.f32_mul_rz(a, b)
    for x, y, r in zip(a, b, got):
        p = Fraction(float(x)) * Fraction(float(y))
        assert abs(Fraction(float(r))) <= abs(p)
        assert r == 0 or (r > 0) == (p > 0)
        bits = struct.unpack("<I", struct.pack("<f", float(r)))[0]
        up = struct.unpack("<f", struct.pack("<I", bits + 1))[0]  # next magnitude away from zero
        assert abs(Fraction(up)) > abs(p), (x, y, r)


def _rows(T=64, seed=5, scale=1.0):
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal((T, 128)) * scale).astype(np.float32)
    v[0, :16] = 0.0  # an all-zero group
    v[1, 16:32] = -1e-30  # a group below the scale floor
    return v


@pytest.mark.parametrize("gs", [None, np.float32(1.0 / np.float32(0.37))])
def test_group_scale_puts_the_group_max_on_six(gs):
    # sf = RN_E4M3(amax / 6 * gs) is within half an E4M3 step (2^-4 relative) of
    # amax / 6 * gs, so the group max times the reciprocal lies in
    # [6 / (1 + 2^-4), 6 / (1 - 2^-4)] = [5.65, 6.4]: nearest-even E2M1 gives 6
    # (the midpoint below is 5). Holds where that product is an E4M3 normal.
    v = _rows()
    data, sf = oracle.nvfp4_quantize(v, gs)
    codes = np.stack([data & 0xF, data >> 4], axis=-1).reshape(v.shape[0], 128)
    a = np.abs(v.reshape(-1, 8, 16)).max(axis=2) / 6.0 * (1.0 if gs is None else float(gs))
    normal = (a >= 2.0 ** -6) & (a < 448)
    mags = (codes.reshape(-1, 8, 16) & 0x7).max(axis=2)
    assert normal.sum() > 100
    assert np.all(mags[normal] == 7)
    # groups below the floor take the floor's code 2^-9 (0x01); all-zero groups give zero codes
    assert sf[0, 0] == 0x01 and np.all(codes[0, :16] == 0)
    assert sf[1, 1] == 0x01


def test_elements_round_to_nearest_of_the_truncated_product():
    v = _rows(seed=6)
    data, sf = oracle.nvfp4_quantize(v, None)
    codes = np.stack([data & 0xF, data >> 4], axis=-1).reshape(v.shape[0], 128)
    sfv = codecs.e4m3_decode(sf)
    for t in range(8):
        for g in range(8):
            r = Fraction(float(np.float32(1.0) / np.float32(sfv[t, g])))
            for i in range(16 * g, 16 * g + 16):
                q = Fraction(float(v[t, i])) * r  # exact product, before truncation
                want = _e2m1_nearest_even(float(q))
                got = int(codes[t, i]) & 0x7
                # truncation can only move an exact product down onto a midpoint
                assert got == want or (got == want - 1 and abs(q) > 0), (t, i)


def test_truncated_product_keeps_a_midpoint_on_the_even_code():
    # The page truncates v * r because r = RN(1 / sf) can exceed 1 / sf: a raw
    # value that is exactly a midpoint times sf would otherwise round past it.
    # Find an E4M3 scale whose float32 reciprocal rounds up by more than
    # 0.8 * 2^-24, and put 1.25 * sf (tie between 1 and 1.5: even is 1) in a
    # group whose max is 6 * sf.
    tab = codecs.e4m3_decode_table()
    pick = None
    for c in range(0x30, 0x60):
        s = tab[c]
        r = np.float32(1.0) / np.float32(s)
        if Fraction(float(r)) * Fraction(s) - 1 > Fraction(8, 10) * Fraction(2) ** -24:
            pick = s
            break
    assert pick is not None
    v = np.zeros((1, 128), np.float32)
    v[0, 0] = 6 * pick
    v[0, 1] = 1.25 * pick
    v[0, 2] = -1.25 * pick
    data, sf = oracle.nvfp4_quantize(v, None)
    assert codecs.e4m3_decode(sf[0, 0]) == pick
    assert data[0, 0] >> 4 == 0x2  # element 1: +1.0
    assert data[0, 1] & 0xF == 0xA  # element 2: -1.0


def test_zero_magnitude_codes_are_positive():
    v = np.zeros((1, 128), np.float32)
    v[0, 0] = -6.0
    v[0, 1:16] = -1e-3  # rounds to a zero magnitude
    v[0, 16:32] = -0.0
    data, _ = oracle.nvfp4_quantize(v, None)
    codes = np.stack([data & 0xF, data >> 4], axis=-1).reshape(128)
    assert codes[0] == 0xF
    assert np.all(codes[1:] == 0)


def test_swizzled_scale_offsets_match_the_pages_formula():
    seen = set()
    for t in range(16):
        for g in range(8):
            off = oracle.nvfp4_scale_offset(t, g, True)
            assert off == (t // 4 * 4 + g // 2) * 8 + g % 2 * 4 + t % 4
            seen.add(off)
            assert oracle.nvfp4_scale_offset(t, g, False) == 8 * t + g
    assert seen == set(range(128))


def _check_against_brute(inp, out, mode):
    b = brute.run(inp, mode)
    flat = {k: out[k].reshape(-1) for k in ("kv_cache", "index_cache")}
    written = {k: np.zeros(flat[k].shape, bool) for k in flat}
    for (name, idx), val in b["writes"].items():
        assert flat[name][idx] == val, (name, idx)
        written[name][idx] = True
    for k in flat:  # nothing else changed
        assert np.all(flat[k][~written[k]] == inp[k].reshape(-1)[~written[k]]), k
    slots = np.asarray(inp["slot_mapping"])
    live = int(((slots >= 0) & (slots < 16 * inp["kv_cache"].shape[0])).sum())
    nkv = int(inp["nkv"])
    assert written["kv_cache"].sum() == live * 2 * nkv * 72
    assert written["index_cache"].sum() == live * 72


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_nvfp4_matches_scalar_bruteforce(mode):
    wl = TINY_DECODE if mode == "decode" else TINY_PREFILL
    inp = synth.with_nvfp4_caches(synth.make_workload(wl, seed=31), 0.37, 1.9)
    out = oracle.decode(inp) if mode == "decode" else oracle.prefill(inp)
    _check_against_brute(inp, out, mode)


def test_nvfp4_unit_global_scales_match_scalar_bruteforce():
    inp = synth.with_nvfp4_caches(synth.make_workload(TINY_DECODE, seed=32))
    _check_against_brute(inp, oracle.decode(inp), "decode")


def test_nvfp4_redecode_approximates_the_fp8_path():
    # Decoding the NVFP4 K cache (codes x group scale x global scale) gives the
    # K head to within an E2M1 half step of each group's scale: the same K the
    # FP8 path stores.
    base = synth.make_workload(TINY_DECODE, seed=33)
    gk = 0.5
    inp = synth.with_nvfp4_caches(base, gk, 1.0)
    out = oracle.decode(inp)
    fp8 = oracle.decode(base)
    for s, slot in enumerate(inp["slot_mapping"]):
        if slot < 0:
            continue
        page, t = slot // 16, slot % 16
        sl = out["kv_cache"][page, 0]
        data = sl[t * 64:(t + 1) * 64]
        codes = np.stack([data & 0xF, data >> 4], axis=-1).reshape(128)
        sc = np.array([sl[1024 + 8 * t + g] for g in range(8)])
        k = codecs.e2m1_decode(codes) * np.repeat(codecs.e4m3_decode(sc), 16) * gk
        k_ref = codecs.e4m3_decode(fp8["k_codes"][s, 0]) * float(fp8["k_s"][s, 0])
        # NVFP4 error: at most one E2M1 unit at the group's scale (half the grid
        # spacing of 2 in [4, 6], or saturation from at most 6.4); the FP8
        # path's: half an E4M3 step, 2^-4 of the value, or 2^-10 of the token
        # scale among the subnormals
        unit = np.repeat(codecs.e4m3_decode(sc), 16) * gk
        fp8_err = np.abs(k_ref) * 2.0 ** -4 + 2.0 ** -10 * float(fp8["k_s"][s, 0])
        assert np.all(np.abs(k - k_ref) <= unit + fp8_err + 1e-12)


# ---------------------------------------------------------------- mutations
def _swap_nibbles(v, gs=None):
    data, sf = _orig(v, gs)
    return ((data >> 4) | ((data & 0xF) << 4)).astype(np.uint8), sf


def _scale_times_six(v, gs=None):
    v = np.asarray(v, np.float32)
    data, sf = _orig(v / np.float32(36.0), gs)  # as if amax * 6 instead of / 6
    return data, sf


def _rn_product(a, b):
    return (np.asarray(a, np.float32) * np.asarray(b, np.float32)).astype(np.float32)


def _keep_negative_zero(v, gs=None):
    data, sf = _orig(v, gs)
    v = np.asarray(v, np.float32)
    codes = np.stack([data & 0xF, data >> 4], axis=-1).reshape(v.shape[0], 128)
    codes = np.where((codes == 0) & np.signbit(v), 0x8, codes)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), sf


def _no_swizzle(t, g, swizzled):
    return 8 * t + g


def _group_32(v, gs=None):
    v = np.asarray(v, np.float32)
    data, sf = _orig(v, gs)
    # the scale of each pair of groups taken from the pair's larger max
    pair = np.maximum(sf[:, 0::2], sf[:, 1::2])
    return data, np.repeat(pair, 2, axis=1)


_orig = prologue.nvfp4_quantize

MUTATIONS = {
    "nibble_order": ("nvfp4_quantize", _swap_nibbles),
    "scale_times_six": ("nvfp4_quantize", _scale_times_six),
    "round_nearest_product": ("f32_mul_rz", _rn_product),
    "negative_zero_kept": ("nvfp4_quantize", _keep_negative_zero),
    "v_scales_unswizzled": ("nvfp4_scale_offset", _no_swizzle),
    "group_of_32_scale": ("nvfp4_quantize", _group_32),
}

PINS = [
    test_zero_magnitude_codes_are_positive,
    test_truncated_product_keeps_a_midpoint_on_the_even_code,
    lambda: test_group_scale_puts_the_group_max_on_six(None),
    lambda: test_nvfp4_matches_scalar_bruteforce("decode"),
]


@pytest.mark.parametrize("case", sorted(MUTATIONS))
def test_planted_nvfp4_mistake_is_caught(case, monkeypatch):
    name, fn = MUTATIONS[case]
    for mod in (oracle, prologue, codecs):
        if hasattr(mod, name):
            monkeypatch.setattr(mod, name, fn)
    caught = False
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught = True
            break
    assert caught, f"no pin caught the planted mistake {case!r}"
