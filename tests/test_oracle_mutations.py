"""Planted mistakes in the oracle must make a pin fail.

Each case swaps one oracle function for a plausible wrong version (a flipped
sign, a dropped term, a transposed index, a wrong constant) and runs the pins
that should notice. The oracle itself is restored after each case."""

import numpy as np
import pytest

import oracle
import synth
from oracle import codecs, prologue
from tests import test_oracle_codecs as pins_codecs
from tests import test_oracle_pipeline as pins


def _wrong_rope(yh, g, cos, sin, eps):
    o, n = _orig["head_norm_rope"](yh, g, cos, sin, eps)
    o = o.copy()
    x1, x2 = n[:, :32], n[:, 32:64]
    o[:, :32] = x1 * cos + x2 * sin  # rotation the other way
    o[:, 32:64] = x2 * cos - x1 * sin
    return o, n


def _no_one_plus_g(ar, res, g_in, eps):
    h, acc, xn = _orig["input_norm"](ar, res, g_in, eps)
    g = codecs.bf16_bits_to_f64(g_in)
    return h, acc, xn / (1.0 + g)[None, :]  # plain RMSNorm: gamma ignored


def _rope_partner_off_by_one(yh, g, cos, sin, eps):
    o, n = _orig["head_norm_rope"](yh, g, cos, sin, eps)
    o = o.copy()
    x1, x2 = n[:, :32], np.roll(n[:, 32:64], 1, axis=1)
    o[:, :32] = x1 * cos - x2 * sin
    o[:, 32:64] = x2 * cos + x1 * sin
    return o, n


def _scale_240(xn):
    amax = np.abs(xn).max(axis=1)
    s = np.where(amax == 0, np.float32(1), (amax / 240.0).astype(np.float32)).astype(np.float32)
    return codecs.e4m3_encode(xn / s.astype(np.float64)[:, None]), s


def _ties_away(v):
    v = np.asarray(v, np.float64)
    out = _orig["e4m3_encode"](v)
    # nudge exact midpoints upward before rounding (ties away from zero)
    nudged = _orig["e4m3_encode"](np.nextafter(v, np.where(v < 0, -np.inf, np.inf)))
    tab = codecs.e4m3_decode_table()
    lo = tab[out & 0x7F]
    hi = tab[nudged & 0x7F]
    mid = np.abs(np.abs(v) - (lo + hi) / 2) == 0
    return np.where(mid & (hi != lo), nudged, out).astype(np.uint8)


def _mx_ceil(xn):
    M, K = xn.shape
    blk = xn.reshape(M, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)
    code = np.where(amax == 0, 127, np.clip(ex - 8 + 127, 0, 254))  # ceil, not floor
    X = codecs.e8m0_decode(code)
    return codecs.e4m3_encode(blk / X[:, :, None]).reshape(M, K), code.astype(np.uint8)


def _skip_mx_sat(xn):
    M, K = xn.shape
    blk = xn.reshape(M, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)
    code = np.where(amax == 0, 127, np.clip(ex - 1 - 7 + 127, 0, 254))  # emax 7, not 8
    X = codecs.e8m0_decode(code)
    return codecs.e4m3_encode(blk / X[:, :, None]).reshape(M, K), code.astype(np.uint8)


def _q_inv_f64(o_q, q_fp8_scale):
    x = o_q.astype(np.float32).astype(np.float64) / float(q_fp8_scale)  # true quotient, no float32 product
    return codecs.e4m3_encode(x)


def _q_no_inverse(o_q, q_fp8_scale):
    x = o_q.astype(np.float32) * np.float32(q_fp8_scale)  # multiplied by the scale itself
    return codecs.e4m3_encode(x.astype(np.float64))


def _static_v_dynamic(v, static=False):
    return _orig["_scaled_codes"](v, False)  # the static flag ignored


_orig = {
    "_scaled_codes": prologue._scaled_codes,
    "head_norm_rope": prologue.head_norm_rope,
    "input_norm": prologue.input_norm,
    "quantize_per_token": prologue.quantize_per_token,
    "e4m3_encode": codecs.e4m3_encode,
    "mxfp8_quantize": prologue.mxfp8_quantize,
}

CASES = {
    "rope_direction": ("head_norm_rope", _wrong_rope),
    "rope_partner_index": ("head_norm_rope", _rope_partner_off_by_one),
    "gamma_dropped": ("input_norm", _no_one_plus_g),
    "fp8_max_240": ("quantize_per_token", _scale_240),
    "e4m3_ties_away": ("e4m3_encode", _ties_away),
    "mx_scale_ceil": ("mxfp8_quantize", _mx_ceil),
    "mx_emax_7": ("mxfp8_quantize", _skip_mx_sat),
    "q_fp8_float64_quotient": ("q_fp8_codes", _q_inv_f64),
    "q_fp8_times_scale": ("q_fp8_codes", _q_no_inverse),
    "static_scale_ignored": ("_scaled_codes", _static_v_dynamic),
}

PINS = [
    pins.test_rope_is_complex_multiplication_on_first_64_dims,
    pins.test_rmsnorm_gamma_enters_as_one_plus_g,
    pins.test_per_token_quant_error_and_full_scale_code,
    pins.test_mxfp8_block_properties,
    pins_codecs.test_e4m3_encode_equals_bruteforce_nearest_even,
    pins.test_decode_matches_scalar_bruteforce,
    pins.test_prefill_matches_scalar_bruteforce,
    pins.test_static_scale_equals_dynamic_at_full_scale_rows,
    pins.test_q_fp8_codes_equal_bruteforce_near_midpoints,
    lambda: pins.test_variants_match_scalar_bruteforce("decode"),
]


def _patch(monkeypatch, name, fn):
    for mod in (oracle, prologue, codecs):
        if hasattr(mod, name):
            monkeypatch.setattr(mod, name, fn)


@pytest.mark.parametrize("case", sorted(CASES))
def test_planted_mistake_is_caught(case, monkeypatch):
    name, fn = CASES[case]
    _patch(monkeypatch, name, fn)
    failed = []
    for pin in PINS:  # cheapest first; stop at the first pin that notices
        try:
            pin()
        except AssertionError:
            failed.append(getattr(pin, "__name__", "pin"))
            break
    assert failed, f"no pin caught the planted mistake {case!r}"


def test_unmutated_oracle_passes_same_pins():
    for pin in PINS:
        pin()


def test_cache_layout_transpose_is_caught(monkeypatch):
    # K written dim-major like V (a transposed cache index) must fail the brute force
    orig = prologue._epilogue

    def wrong(y, inp):
        out = orig(y, inp)
        kc = out["k_cache"]
        for s, slot in enumerate(inp["slot_mapping"]):
            if slot < 0:
                continue
            page, t = slot // 16, slot % 16
            for j in range(int(inp["nkv"])):
                kc[page, j].reshape(8, 16, 16)[:, t, :] = 0x7F
                kc[page, j].reshape(128, 16)[:, t] = out["k_codes"][s, j]
        return out

    monkeypatch.setattr(prologue, "_epilogue", wrong)
    inp = synth.make_workload(pins.TINY_DECODE, seed=11)
    with pytest.raises(AssertionError):
        pins._check_against_brute(inp, oracle.decode(inp), "decode")
