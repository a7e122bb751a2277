"""Parity of the head-step variants (pre_attn_decode_ex / pre_attn_prefill_ex)
with the oracle, through the C ABI: unit K / V scales, and the FP8 q output
with its dequantization scale (with and without the bf16 q). Decode runs
through each launch structure (one launch; norm + GEMV then epilogue; norm then
GEMV + epilogue; three launches); prefill through both token-tile widths."""

import sys

import numpy as np
import pytest

import oracle
import synth
from tests import parity
from tests.test_parity_gpu import merge_stats, prefill_chunks

pytestmark = pytest.mark.gpu

# (static K / V scale, FP8 q scale or None, bf16 q written)
VARIANTS = [
    (True, None, True),
    (False, 0.008, True),   # q / scale reaches past 448: saturated codes
    (True, 1.0, False),     # small q values land on subnormal codes; FP8 q only
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _with_variant(inp, static, qs, q_bf16):
    inp = dict(inp)
    inp["static_kv_scale"] = static
    if qs is not None:
        inp["q_fp8_scale"] = qs
    inp["q_bf16"] = q_bf16
    return inp


def _run_gpu(inp):
    from kv_residual_add_amd.runner import Problem

    p = Problem(inp)
    p.run()
    return p, p.outputs()


def _check(inp, ref, got, rows=None):
    static, qs, q_bf16 = inp["static_kv_scale"], inp.get("q_fp8_scale"), inp["q_bf16"]
    assert ("q_out" in got) == q_bf16
    assert ("q_fp8" in got) == (qs is not None)
    stats = parity.compare(inp, ref, got, rows=rows)
    parity.check_written_sets(inp, got)
    if static:  # every written scale entry is exactly 1.0
        masks = parity.expected_written_masks(inp)
        for name in ("k_scale", "v_scale"):
            assert np.all(got[name][masks[name]] == np.float32(1.0)), name
    if qs is not None:  # both sides saturate at +-448 (codes 0x7E / 0xFE) and nothing else
        codes = got["q_fp8"]
        assert not np.any((codes & 0x7F) == 0x7F), "NaN code in the FP8 q output"
    return stats


DECODE_CASES = [
    (3, 256, 2, {"skip_frac": 0.34}),     # one launch
    (8, 6144, 1, {}),                     # norm + GEMV, then the epilogue
    (40, 2048, 2, {"outlier_frac": 0.01}),  # norm, then GEMV + epilogue
    (20, 4736, 1, {"skip_frac": 0.1}),    # 37 k slices: three launches
    (16, 1024, 4, {"skip_frac": 0.25}),   # nkv = 4: 77 heads, 8 K/V slots a page
    (24, 1024, 1, {"oob_frac": 0.25}),    # slots past the cache's end write nothing
]


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: f"static{int(v[0])}_q{v[1]}_bf16{int(v[2])}")
@pytest.mark.parametrize("S,K,nkv,kw", DECODE_CASES, ids=lambda v: str(v))
def test_decode_variants(S, K, nkv, kw, variant):
    wl = synth.Workload(name=f"decode_s{S}_k{K}_nkv{nkv}", mode="decode", tokens=S, hidden=K, nkv=nkv,
                        max_pos=4096, num_pages=max(1, -(-S // 16) + 2), layout="random", **kw)
    _say(f"decode variant {wl.name} {kw} {variant}")
    inp = _with_variant(synth.make_workload(wl, seed=S * 11 + K), *variant)
    ref = oracle.decode(inp)
    _, got = _run_gpu(inp)
    _say(f"  {_check(inp, ref, got)}")


PREFILL_CASES = [
    (5, 256, 2, {"skip_frac": 0.4}),
    (300, 1024, 4, {"skip_frac": 0.1}),   # 128-token CTAs, ragged tail
    (2560, 256, 4, {}),                   # 256-token CTAs
    (130, 512, 1, {"outlier_frac": 0.01}),  # nkv = 1, a ragged 128-token tile
    (200, 512, 2, {"oob_frac": 0.1}),     # slots past the cache's end write nothing
]


@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: f"static{int(v[0])}_q{v[1]}_bf16{int(v[2])}")
@pytest.mark.parametrize("S,K,nkv,kw", PREFILL_CASES, ids=lambda v: str(v))
def test_prefill_variants(S, K, nkv, kw, variant):
    wl = synth.Workload(name=f"prefill_s{S}_k{K}_nkv{nkv}", mode="prefill", tokens=S, hidden=K, nkv=nkv,
                        max_pos=4096, num_pages=max(1, -(-S // 16) + 2), layout="random", **kw)
    _say(f"prefill variant {wl.name} {kw} {variant}")
    inp = _with_variant(synth.make_workload(wl, seed=S * 13 + K), *variant)
    ref = oracle.prefill(inp)
    _, got = _run_gpu(inp)
    _say(f"  {_check(inp, ref, got)}")


@pytest.mark.parametrize("key", ["c3", "c4"])
def test_variants_full_workload(key):
    """Both variants at once on a full workload, every token."""
    wl = synth.named_config(key)
    _say(f"variants full {wl.name}")
    inp = _with_variant(synth.make_workload(wl, seed=0), True, 0.008, True)
    p, got = _run_gpu(inp)
    del p
    if wl.mode == "decode":
        _say(f"  {_check(inp, oracle.decode(inp), got)}")
        return
    stats = {}
    for rows, ref in prefill_chunks(inp):  # every token
        merge_stats(stats, _check(inp, ref, got, rows=rows))
    _say(f"  {stats}")


def test_plain_and_ex_calls_agree():
    """pre_attn_decode_ex with no options is pre_attn_decode, bit for bit."""
    from kv_residual_add_amd import _binding as B
    from kv_residual_add_amd.runner import Problem

    wl = synth.Workload(name="decode_s8_k1024_nkv2", mode="decode", tokens=8, hidden=1024, nkv=2,
                        max_pos=4096, num_pages=3, layout="random")
    inp = synth.make_workload(wl, seed=5)
    p = Problem(inp)
    p.run()
    a = p.outputs()
    p2 = Problem(inp)
    args = p2.args()
    B.pre_attn_decode_ex(args[0], None, *args[1:])
    b = p2.outputs()
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


# ---------------------------------------------------------------- NVFP4 caches
NV_SCALES = [(1.0, 1.0), (0.37, 1.9)]  # (K, V) global scales; non-powers of two round the reciprocals


def _nvfp4_check(inp, ref, got, rows=None):
    stats = parity.compare(inp, ref, got, rows=rows)
    parity.check_written_sets_nvfp4(inp, got)
    return stats


@pytest.mark.parametrize("scales", NV_SCALES, ids=lambda v: f"gk{v[0]}_gv{v[1]}")
@pytest.mark.parametrize("S,K,nkv,kw", DECODE_CASES, ids=lambda v: str(v))
def test_decode_nvfp4(S, K, nkv, kw, scales):
    wl = synth.Workload(name=f"decode_s{S}_k{K}_nkv{nkv}", mode="decode", tokens=S, hidden=K, nkv=nkv,
                        max_pos=4096, num_pages=max(1, -(-S // 16) + 2), layout="random", **kw)
    _say(f"decode nvfp4 {wl.name} {kw} {scales}")
    inp = synth.with_nvfp4_caches(synth.make_workload(wl, seed=S * 17 + K), *scales)
    ref = oracle.decode(inp)
    _, got = _run_gpu(inp)
    _say(f"  {_nvfp4_check(inp, ref, got)}")


@pytest.mark.parametrize("scales", NV_SCALES, ids=lambda v: f"gk{v[0]}_gv{v[1]}")
@pytest.mark.parametrize("S,K,nkv,kw", PREFILL_CASES, ids=lambda v: str(v))
def test_prefill_nvfp4(S, K, nkv, kw, scales):
    wl = synth.Workload(name=f"prefill_s{S}_k{K}_nkv{nkv}", mode="prefill", tokens=S, hidden=K, nkv=nkv,
                        max_pos=4096, num_pages=max(1, -(-S // 16) + 2), layout="random", **kw)
    _say(f"prefill nvfp4 {wl.name} {kw} {scales}")
    inp = synth.with_nvfp4_caches(synth.make_workload(wl, seed=S * 19 + K), *scales)
    ref = oracle.prefill(inp)
    _, got = _run_gpu(inp)
    _say(f"  {_nvfp4_check(inp, ref, got)}")


@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c5"])
def test_nvfp4_full_workload(key):
    """NVFP4 caches with the FP8 q output on a full workload, every token."""
    wl = synth.named_config(key)
    _say(f"nvfp4 full {wl.name}")
    inp = synth.with_nvfp4_caches(synth.make_workload(wl, seed=0), 0.37, 1.9)
    inp["q_fp8_scale"] = 0.008
    inp["q_bf16"] = True
    p, got = _run_gpu(inp)
    del p
    if wl.mode == "decode":
        _say(f"  {_nvfp4_check(inp, oracle.decode(inp), got)}")
        return
    stats = {}
    for rows, ref in prefill_chunks(inp):  # every token
        merge_stats(stats, _nvfp4_check(inp, ref, got, rows=rows))
    _say(f"  {stats}")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_nvfp4_and_fp8q_degenerate_rows(mode):
    """An all-zero row (ar = -res: every group below the scale floor, zero codes,
    signed-zero q codes), position 0 (identity RoPE), the last table row and a slot of -1,
    with NVFP4 caches and the FP8 q output only."""
    wl = synth.Workload(name=f"{mode}_degenerate", mode=mode, tokens=6, hidden=256, nkv=1, max_pos=64,
                        num_pages=3, layout="random")
    inp = synth.make_workload(wl, seed=3)
    inp["res"][0] = inp["ar"][0] ^ 0x8000  # bf16 negation: acc row 0 == 0
    inp["positions"][1] = 0
    inp["positions"][2] = 63
    inp["slot_mapping"][3] = -1
    inp = synth.with_nvfp4_caches(inp, 0.37, 1.9)
    inp["q_fp8_scale"] = 0.02
    inp["q_bf16"] = False
    ref = oracle.decode(inp) if mode == "decode" else oracle.prefill(inp)
    _, got = _run_gpu(inp)
    assert "q_out" not in got
    _say(f"  {_nvfp4_check(inp, ref, got)}")
    assert np.all((got["q_fp8"][0] & 0x7F) == 0)  # the zero row's q codes are signed zeros
    page, t = inp["slot_mapping"][0] // 16, inp["slot_mapping"][0] % 16
    for sl in range(2):  # K and V of the zero row: zero codes, floor scales (E4M3 2^-9 = 0x01)
        assert np.all(got["kv_cache"][page, sl, t * 64:(t + 1) * 64] == 0)
    assert np.all(got["kv_cache"][page, 0, 1024 + 8 * t:1024 + 8 * t + 8] == 0x01)
