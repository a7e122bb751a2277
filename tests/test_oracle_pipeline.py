"""Pins of the oracle's prologue steps: library routines (torch casts and
rms_norm), closed forms (exact integer dot products, RoPE as complex
multiplication), invariants (norm preservation, quantization error bounds, one
write per slot) and a separately written scalar brute force of the whole path."""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import codecs, prologue
from tests import brute_prologue as brute

TINY_DECODE = synth.Workload("tiny", "decode", 3, 128, 1, 64, 2, "random", skip_frac=0.34)
TINY_PREFILL = synth.Workload("tinyp", "prefill", 3, 64, 1, 64, 2, "random", skip_frac=0.34)


def _small(mode="decode", **kw):
    base = dict(name="small", mode=mode, tokens=12, hidden=256, nkv=2, max_pos=512,
                num_pages=4, layout="random")
    base.update(kw)
    return synth.Workload(**base)


# ---------------------------------------------------------------- a1 residual
def test_h_out_matches_torch_bf16_sum():
    inp = synth.make_workload(_small())
    h, acc, _ = oracle.input_norm(inp["ar"], inp["res"], inp["g_in"], inp["eps"])
    ar = torch.from_numpy(inp["ar"].view(np.int16)).view(torch.bfloat16)
    rs = torch.from_numpy(inp["res"].view(np.int16)).view(torch.bfloat16)
    want = (ar.float() + rs.float()).bfloat16().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(h, want)
    assert np.array_equal(acc, (ar.float() + rs.float()).numpy())


# ---------------------------------------------------------------- a2 RMSNorm
def test_rmsnorm_with_zero_gamma_is_torch_rms_norm():
    inp = synth.make_workload(_small())
    g0 = np.zeros_like(inp["g_in"])  # bf16 +0 -> (1 + g) = 1
    _, acc, xn = oracle.input_norm(inp["ar"], inp["res"], g0, inp["eps"])
    eps = float(np.float32(inp["eps"]))
    want = torch.nn.functional.rms_norm(torch.from_numpy(acc.astype(np.float64)),
                                        (acc.shape[1],), eps=eps).numpy()
    np.testing.assert_allclose(xn, want, rtol=1e-14, atol=0)


def test_rmsnorm_output_rms_closed_form():
    inp = synth.make_workload(_small())
    g0 = np.zeros_like(inp["g_in"])
    _, acc, xn = oracle.input_norm(inp["ar"], inp["res"], g0, inp["eps"])
    a = acc.astype(np.float64)
    ms = (a * a).mean(axis=1)
    eps = float(np.float32(inp["eps"]))
    np.testing.assert_allclose(np.sqrt((xn * xn).mean(axis=1)), np.sqrt(ms / (ms + eps)),
                               rtol=1e-13)


def test_rmsnorm_gamma_enters_as_one_plus_g():
    inp = synth.make_workload(_small())
    g0 = np.zeros_like(inp["g_in"])
    _, _, x0 = oracle.input_norm(inp["ar"], inp["res"], g0, inp["eps"])
    _, _, xg = oracle.input_norm(inp["ar"], inp["res"], inp["g_in"], inp["eps"])
    g = codecs.bf16_bits_to_f64(inp["g_in"])
    np.testing.assert_allclose(xg, x0 * (1 + g)[None, :], rtol=1e-15)


# ---------------------------------------------------------------- a3 quantization
def test_per_token_quant_error_and_full_scale_code():
    inp = synth.make_workload(_small(outlier_frac=0.02))
    _, _, xn = oracle.input_norm(inp["ar"], inp["res"], inp["g_in"], inp["eps"])
    x8, s_x = oracle.quantize_per_token(xn)
    q = xn / s_x.astype(np.float64)[:, None]
    deq = oracle.e4m3_decode(x8)
    # half a code step: 2^(E-4) in binade E, 2^-10 in the subnormal range
    e = np.floor(np.log2(np.maximum(np.abs(q), 2.0**-6)))
    assert np.all(np.abs(deq - q) <= 2.0 ** (e - 4) * (1 + 1e-12))
    # the row maximum maps to +-448 (amax / RN(amax/448) rounds to 448)
    assert np.all(np.any((x8 & 0x7F) == 0x7E, axis=1))
    np.testing.assert_allclose(s_x, np.abs(xn).max(axis=1) / 448, rtol=2**-23)


def test_per_token_quant_zero_row_scale_one():
    x8, s_x = oracle.quantize_per_token(np.zeros((2, 64)))
    assert np.all(s_x == 1.0) and np.all((x8 & 0x7F) == 0)


def test_mxfp8_block_properties():
    rng = np.random.default_rng(5)
    xn = rng.standard_normal((5, 256)) * np.exp(rng.uniform(-8, 8, size=(5, 1)))
    xn[0, :32] = 0.0  # an all-zero block
    xq, xs = oracle.mxfp8_quantize(xn)
    assert xs[0, 0] == 127 and np.all((xq[0, :32] & 0x7F) == 0)
    X = oracle.e8m0_decode(xs)
    deq = oracle.e4m3_decode(xq).reshape(5, 8, 32) * X[:, :, None]
    blk = xn.reshape(5, 8, 32)
    for r in range(5):
        for b in range(8):
            if r == 0 and b == 0:
                continue
            amax = np.abs(blk[r, b]).max()
            # OCP MX: X = 2^(floor(log2 amax) - 8)
            assert X[r, b] == 2.0 ** (np.floor(np.log2(amax)) - 8)
            codes = xq.reshape(5, 8, 32)[r, b] & 0x7F
            top = oracle.e4m3_decode(codes.max())
            assert 256 <= top <= 448
            q = blk[r, b] / X[r, b]
            e = np.floor(np.log2(np.maximum(np.abs(q), 2.0**-6)))
            err = np.abs(deq[r, b] / X[r, b] - np.clip(q, -448, 448))
            assert np.all(err <= 2.0 ** (e - 4) * (1 + 1e-12))


# ---------------------------------------------------------------- a4 projection
def test_decode_projection_equals_exact_integer_dot():
    inp = synth.make_workload(_small(hidden=1024))
    _, _, xn = oracle.input_norm(inp["ar"], inp["res"], inp["g_in"], inp["eps"])
    x8, s_x = oracle.quantize_per_token(xn)
    y = oracle.project_decode(x8, s_x, inp["w"], inp["w_scale"])
    xi = (oracle.e4m3_decode(x8) * 512).astype(np.int64)
    wi = (oracle.e4m3_decode(inp["w"]) * 512).astype(np.int64)
    acc_int = xi @ wi.T  # exact integers, < 2^49
    want = (acc_int.astype(np.float64) / 2.0**18 * s_x.astype(np.float64)[:, None]) \
        * inp["w_scale"].astype(np.float64)[None, :]
    assert np.array_equal(y, want)


def test_mxfp8_projection_close_to_exact_rational():
    from fractions import Fraction
    rng = np.random.default_rng(6)
    xq = rng.integers(0, 0x7E, size=(2, 64)).astype(np.uint8) | \
        (rng.integers(0, 2, size=(2, 64)) << 7).astype(np.uint8)
    wq = rng.integers(0, 0x7E, size=(3, 64)).astype(np.uint8)
    xs = rng.integers(100, 140, size=(2, 2)).astype(np.uint8)
    ws = rng.integers(100, 140, size=(3, 2)).astype(np.uint8)
    y = oracle.project_mxfp8(xq, xs, wq, ws)
    for m in range(2):
        for n in range(3):
            tot = Fraction(0)
            for k in range(64):
                tot += (brute.E4M3[int(xq[m, k])] * Fraction(2) ** (int(xs[m, k // 32]) - 127)
                        * brute.E4M3[int(wq[n, k])] * Fraction(2) ** (int(ws[n, k // 32]) - 127))
            assert abs(y[m, n] - float(tot)) <= 1e-14 * abs(float(tot)) + 1e-300


# ---------------------------------------------------------------- a5 head norm + RoPE
def _rope_case(seed=7, T=40):
    rng = np.random.default_rng(seed)
    yh = rng.standard_normal((T, 128)) * 3
    g = synth.inputs._bf16_bits(rng.normal(0, 0.1, 128))
    ang = rng.uniform(-np.pi, np.pi, size=(T, 32))
    return yh, g, np.cos(ang), np.sin(ang)


def test_rope_is_complex_multiplication_on_first_64_dims():
    yh, g, c, s = _rope_case()
    o, n = oracle.head_norm_rope(yh, g, c, s, 1e-6)
    z = (n[:, :32] + 1j * n[:, 32:64]) * (c + 1j * s)
    np.testing.assert_allclose(o[:, :32], z.real, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o[:, 32:64], z.imag, rtol=1e-13, atol=1e-13)
    assert np.array_equal(o[:, 64:], n[:, 64:])


def test_rope_preserves_pair_norms_and_identity_at_angle_zero():
    yh, g, c, s = _rope_case()
    o, n = oracle.head_norm_rope(yh, g, c, s, 1e-6)
    np.testing.assert_allclose(o[:, :32] ** 2 + o[:, 32:64] ** 2,
                               (n[:, :32] ** 2 + n[:, 32:64] ** 2) * (c * c + s * s),
                               rtol=1e-12)
    o0, n0 = oracle.head_norm_rope(yh, g, np.ones_like(c), np.zeros_like(s), 1e-6)
    assert np.array_equal(o0, n0)


def test_head_norm_matches_torch_rms_norm_times_one_plus_g():
    yh, g, c, s = _rope_case()
    _, n = oracle.head_norm_rope(yh, g, c, s, 1e-6)
    gamma = torch.from_numpy(1.0 + codecs.bf16_bits_to_f64(g))
    eps = float(np.float32(1e-6))
    want = torch.nn.functional.rms_norm(torch.from_numpy(yh), (128,), weight=gamma, eps=eps)
    np.testing.assert_allclose(n, want.numpy(), rtol=1e-14)


def test_rope_position_composition_with_table_angles():
    # the synthetic cos|sin table rotates position p by p * inv_freq: rotating a
    # vector by p then by q equals rotating it by p + q (float64 angles)
    i = np.arange(32)
    inv = 10000.0 ** (-2.0 * i / 64)
    rng = np.random.default_rng(8)
    v = rng.standard_normal((1, 128))
    g0 = np.zeros(128, np.uint16)
    p, q = 37, 1201
    a, _ = oracle.head_norm_rope(v, g0, np.cos(p * inv)[None], np.sin(p * inv)[None], 0.0)
    b, _ = oracle.head_norm_rope(a, g0, np.cos(q * inv)[None], np.sin(q * inv)[None], 0.0)
    c, _ = oracle.head_norm_rope(v, g0, np.cos((p + q) * inv)[None],
                                 np.sin((p + q) * inv)[None], 0.0)
    # the second call renormalizes a unit-RMS vector: a no-op up to rounding
    np.testing.assert_allclose(b, c, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------- a7-a10 caches
@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_cache_writes_one_per_slot_and_redecode(mode):
    wl = _small(mode=mode, tokens=20, skip_frac=0.25, num_pages=3)
    inp = synth.make_workload(wl)
    out = oracle.decode(inp) if mode == "decode" else oracle.prefill(inp)
    nkv = wl.nkv
    slots = inp["slot_mapping"]
    live = slots[slots >= 0]
    changed = sum(int((out[k] != inp[k]).sum()) for k in ("k_cache", "v_cache", "index_cache"))
    sc = sum(int((out[k].view(np.uint32) != inp[k].view(np.uint32)).sum())
             for k in ("k_scale", "v_scale"))
    # written bytes (codes never equal the 0x7F sentinel; scales are never NaN)
    assert changed == len(live) * (nkv * 256 + 128)
    assert sc == len(live) * nkv * 2
    for s, slot in enumerate(slots):
        if slot < 0:
            continue
        page, t = slot // 16, slot % 16
        for j in range(nkv):
            kk = out["k_cache"][page, j].reshape(8, 16, 16)[:, t, :].reshape(128)
            vv = out["v_cache"][page, j].reshape(128, 16)[:, t]
            assert np.array_equal(kk, out["k_codes"][s, j])
            assert np.array_equal(vv, out["v_codes"][s, j])
            assert out["k_scale"][page, j, t] == out["k_s"][s, j]
            assert out["v_scale"][page, j, t] == out["v_s"][s, j]
        assert np.array_equal(out["index_cache"][slot], out["ik_codes"][s])
    # K/V per-token scale: a full-scale code in every non-zero row
    assert np.all(np.any((out["k_codes"] & 0x7F) == 0x7E, axis=2))
    assert np.all(np.any((out["v_codes"] & 0x7F) == 0x7E, axis=2))


def test_all_negative_slots_write_nothing():
    wl = _small(tokens=4)
    inp = synth.make_workload(wl)
    inp["slot_mapping"][:] = -1
    out = oracle.decode(inp)
    for k in ("k_cache", "v_cache", "index_cache"):
        assert np.array_equal(out[k], inp[k])
    for k in ("k_scale", "v_scale"):
        assert np.array_equal(out[k].view(np.uint32), inp[k].view(np.uint32))


@pytest.mark.parametrize("mode", ["decode", "prefill"])
@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_slots_past_the_cache_write_nothing(mode, fmt):
    # Slots at or past num_pages * 16 are outside the caller's precondition and
    # are read like slot -1: the written bytes are exactly those of the same
    # call with those slots set to -1, the count per remaining slot is the
    # layout's, and the separately written scalar statement agrees.
    wl = _small(mode=mode, tokens=8, hidden=64 if mode == "prefill" else 128, nkv=1, num_pages=2,
                oob_frac=0.5, skip_frac=0.1)
    inp = synth.make_workload(wl, seed=31)
    if fmt == "nvfp4":
        inp = synth.with_nvfp4_caches(inp, 0.37, 1.9)
    slots = inp["slot_mapping"]
    past = slots >= 32
    assert past.sum() >= 4 and (slots >= 1 << 40).any() and (slots == 32).any()
    run = oracle.decode if mode == "decode" else oracle.prefill
    out = run(inp)
    minus = dict(inp, slot_mapping=np.where(past, -1, slots))
    ref = run(minus)
    keys = ("kv_cache", "index_cache") if fmt == "nvfp4" else ("k_cache", "v_cache", "index_cache", "k_scale", "v_scale")
    for k in keys:
        assert np.array_equal(out[k].view(np.uint8), ref[k].view(np.uint8)), k
    live = int(((slots >= 0) & ~past).sum())
    if fmt == "fp8":
        changed = sum(int((out[k] != inp[k]).sum()) for k in ("k_cache", "v_cache", "index_cache"))
        assert changed == live * (wl.nkv * 256 + 128)
        _check_against_brute(inp, out, mode)
    else:
        from tests.test_oracle_nvfp4 import _check_against_brute as check_nv
        check_nv(inp, out, mode)


def test_full_cache_written_exactly_once_by_prefill_layout():
    wl = synth.Workload("fill", "prefill", 64, 64, 1, 64, 4, "prefill", requests=2)
    inp = synth.make_workload(wl)
    assert sorted(inp["slot_mapping"].tolist()) == list(range(64))
    out = oracle.prefill(inp)
    assert not np.any(out["index_cache"] == 0x7F)
    assert not np.any(out["k_cache"] == 0x7F) and not np.any(out["v_cache"] == 0x7F)


# ---------------------------------------------------------------- whole path
def _check_against_brute(inp, out, mode):
    b = brute.run(inp, mode)
    assert np.array_equal(out["h_out"], np.array(b["h_out"], np.uint16))
    # bf16 outputs: equal, or one bf16 ulp apart where float64 sums round differently
    for key in ("q_out", "iq_out"):
        d = np.abs(out[key].astype(np.int64) - np.array(b[key], np.int64))
        assert d.max() <= 1 and (d > 0).mean() < 0.01, key
    flat = {k: out[k].reshape(-1) for k in
            ("k_cache", "v_cache", "index_cache", "k_scale", "v_scale")}
    for (name, idx), val in b["writes"].items():
        if name.endswith("scale"):
            assert flat[name][idx] == np.float32(val), (name, idx)
        else:
            assert flat[name][idx] == val, (name, idx)
    n_writes = sum(1 for _ in b["writes"])
    changed = sum(int((out[k] != inp[k]).sum()) for k in ("k_cache", "v_cache", "index_cache"))
    changed += sum(int((out[k].view(np.uint32) != inp[k].view(np.uint32)).sum())
                   for k in ("k_scale", "v_scale"))
    assert changed == n_writes


def test_decode_matches_scalar_bruteforce():
    inp = synth.make_workload(TINY_DECODE, seed=11)
    assert (inp["slot_mapping"] < 0).sum() == 1
    _check_against_brute(inp, oracle.decode(inp), "decode")


def test_prefill_matches_scalar_bruteforce():
    inp = synth.make_workload(TINY_PREFILL, seed=12)
    _check_against_brute(inp, oracle.prefill(inp), "prefill")


# ------------------------------------------------- variants of the head step
@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_variants_match_scalar_bruteforce(mode):
    # the unit K/V scale and the scaled FP8 q, against the separately written
    # scalar statement (a scale that is not a power of two, so the float32
    # reciprocal rounds)
    wl = TINY_DECODE if mode == "decode" else TINY_PREFILL
    inp = dict(synth.make_workload(wl, seed=21), static_kv_scale=True, q_fp8_scale=0.0371)
    out = oracle.decode(inp) if mode == "decode" else oracle.prefill(inp)
    _check_against_brute(inp, out, mode)
    b = brute.run(inp, mode)
    want = np.array(b["q_fp8"], np.uint8)
    got = out["q_fp8"]
    assert got.shape == want.shape
    # equal, or one code apart where float64 head sums round differently
    d = np.abs(codecs_ord(got) - codecs_ord(want))
    assert d.max() <= 1 and (d > 0).mean() < 0.01


def codecs_ord(c):
    c = c.astype(np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def test_static_scale_equals_dynamic_at_full_scale_rows():
    # a row whose max magnitude is exactly 448 has the dynamic scale 448 / 448
    # = 1, so its codes are the static ones; other rows saturate or not by the
    # static rule (|v| >= 464 -> 0x7E)
    rng = np.random.default_rng(5)
    v = rng.normal(0, 100, (6, 128))
    v[:3] *= 448.0 / np.abs(v[:3]).max(axis=1, keepdims=True)
    c_dyn, s_dyn = prologue._scaled_codes(v[:3])
    c_sta, s_sta = prologue._scaled_codes(v[:3], static=True)
    assert np.all(s_dyn == 1.0) and np.all(s_sta == 1.0)
    assert np.array_equal(c_dyn, c_sta)
    big = np.array([[500.0, -464.0, 463.9, -1e6] + [0.0] * 124])
    c, s = prologue._scaled_codes(big, static=True)
    assert s[0] == 1.0 and list(c[0, :4]) == [0x7E, 0xFE, 0x7E, 0xFE]


def test_q_fp8_codes_equal_bruteforce_near_midpoints():
    # float32 head outputs within two ulps of (E4M3 midpoint) * scale, where the
    # float32 product with the float32 reciprocal decides the rounding: the
    # codes equal the scalar statement's (exhaustive search, exact rationals)
    scale = 0.0371
    inv = brute.f32(1.0 / brute.f32(scale))
    tab = codecs.e4m3_decode_table()
    grid = np.sort(tab[:127])
    mids = (grid[:-1] + grid[1:]) / 2
    base = (mids * np.float64(np.float32(scale))).astype(np.float32)
    xs = np.concatenate([base + k * np.spacing(base) for k in (-2, -1, 0, 1, 2)]).astype(np.float32)
    xs = np.concatenate([xs, -xs])
    got = prologue.q_fp8_codes(xs.astype(np.float64), scale)
    want = np.array([brute.e4m3_round(brute.f32(float(x) * inv)) for x in xs], np.uint8)
    assert np.array_equal(got, want)


def test_q_fp8_dequant_within_half_step():
    # code * scale is within half an E4M3 step (times the scale) of the float32
    # head output, below saturation; above it the code is +-448
    rng = np.random.default_rng(6)
    o = rng.normal(0, 3, (4, 2, 128)) * np.exp(rng.normal(0, 2, (4, 2, 128)))
    scale = 0.013
    c = oracle.prologue.q_fp8_codes(o, scale)
    x = o.astype(np.float32).astype(np.float64) / np.float64(np.float32(scale))
    dq = oracle.e4m3_decode(c)
    mag = np.abs(x)
    step = np.where(mag < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3))
    inside = mag <= 448
    # the float32 rounding of the product moves x by at most 2^-24 relative
    assert np.all(np.abs(dq - x)[inside] <= 0.5 * step[inside] + mag[inside] * 2.0 ** -23)
    assert np.all(np.abs(dq[~inside]) == 448.0)


def test_head_order_roles():
    # N = (19 nkv + 1) * 128 and the role offsets of the head list
    for nkv, n in ((1, 2560), (2, 4992), (4, 9856)):
        assert synth.Workload("x", "decode", 1, 128, nkv, 16, 1).n_rows == n
    assert prologue.HEAD_DIM == 128 and prologue.ROTARY_DIM == 64
