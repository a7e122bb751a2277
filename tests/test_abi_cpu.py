"""Host-side checks of libpre_attn.so that need no GPU: it loads, exports every
function include/pre_attn.h declares, sizes its workspace and packed weights,
and rejects invalid arguments before anything is enqueued."""

import ctypes
import os
import re

import pytest

import kv_residual_add_amd as K
from kv_residual_add_amd import _binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "pre_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, re.M)))


def test_header_declares_the_expected_api():
    assert _declared_functions() == sorted(B.EXPORTS)


@pytest.mark.parametrize("name", _declared_functions())
def test_library_exports_declared_symbol(name):
    lib = ctypes.CDLL(B.LIB_PATH)
    assert hasattr(lib, name)


def _dims(**kw):
    base = dict(tokens=8, hidden=6144, nkv=1, num_pages=2048, max_pos=32768, eps=1e-6)
    base.update(kw)
    return K.make_dims(**base)


def test_workspace_sizes():
    dec = K.pa_workspace_bytes(_dims(), K.PA_MODE_DECODE)
    # x8 (8 x 6144) + scales + k-slice partials (8 slices x 8 x 2560 f32) + counters
    assert dec >= 8 * 6144 + 8 * 2560 * 4
    pre = K.pa_workspace_bytes(_dims(tokens=8192, nkv=4, num_pages=512, max_pos=2048),
                               K.PA_MODE_PREFILL)
    assert pre >= 8192 * 6144 + 8192 * 6144 // 32
    assert K.pa_workspace_bytes(_dims(tokens=65), K.PA_MODE_DECODE) == 0
    assert K.pa_workspace_bytes(_dims(tokens=65), K.PA_MODE_PREFILL) > 0
    assert K.pa_workspace_bytes(_dims(nkv=3), K.PA_MODE_DECODE) == 0
    assert K.pa_workspace_bytes(_dims(hidden=6100), K.PA_MODE_DECODE) == 0
    assert K.pa_workspace_bytes(_dims(), 7) == 0


def test_decode_launch_structure():
    NORM, EPI = K.PA_DECODE_NORM_FUSED, K.PA_DECODE_EPILOGUE_FUSED
    # few tokens with a small weight: norm, projection and epilogue in one
    # launch; few tokens with a larger weight whose heads do not divide over
    # the 8 XCDs: norm with the projection; more tokens, or a hidden size past
    # the fused norm's reach: the epilogue with the projection (when a head's
    # k slices are few enough to wait for each other)
    assert K.pa_decode_structure(_dims(tokens=1, hidden=1024)) == NORM | EPI
    assert K.pa_decode_structure(_dims(tokens=8)) == NORM
    assert K.pa_decode_structure(_dims(tokens=16, hidden=8192)) == NORM
    assert K.pa_decode_structure(_dims(tokens=17)) == EPI
    assert K.pa_decode_structure(_dims(tokens=64, nkv=2)) == EPI
    # 65 k slices of one chunk each (8320 = 65 x 128): too many for a head's
    # slices to wait for each other, so the epilogue is a launch of its own
    assert K.pa_decode_structure(_dims(tokens=8, hidden=8320)) == 0
    assert K.pa_decode_structure(_dims(tokens=20, hidden=4736)) == 0  # 37 slices
    assert K.pa_decode_structure(_dims(tokens=8, hidden=16384)) == EPI  # 32 slices
    assert K.pa_decode_structure(_dims(tokens=65)) < 0
    assert K.pa_decode_structure(_dims(nkv=3)) < 0
    # every valid shape has a plan, also where no grid is resident at once
    for nkv in (1, 2, 4):
        for hidden in (128, 1024, 6144, 8192, 16384):
            for tokens in (1, 16, 17, 64):
                d = _dims(tokens=tokens, hidden=hidden, nkv=nkv)
                assert K.pa_decode_structure(d) >= 0, (nkv, hidden, tokens)
                assert K.pa_workspace_bytes(d, K.PA_MODE_DECODE) > 0


def test_workspace_sync_words_fixed():
    # the synchronization words sit in the first 32 KB of every workspace, so
    # every decode and prefill workspace holds them
    for mode in (K.PA_MODE_DECODE, K.PA_MODE_PREFILL):
        for tokens in (1, 8, 64):
            assert K.pa_workspace_bytes(_dims(tokens=tokens, hidden=128), mode) > 32768


def test_packed_sizes():
    assert K.pa_packed_weight_bytes(0, 2560, 6144) == 2560 * 6144
    # FP8 codes of every row + bf16 copies of the k, v and index_k heads
    assert K.pa_packed_weight_bytes(1, 9856, 6144) == 9856 * 6144 + 9 * 128 * 6144 * 2
    assert K.pa_packed_scale_bytes(1, 9856, 6144) == 9856 * 6144 // 32
    assert K.pa_packed_weight_bytes(0, 2561, 6144) == 0
    assert K.pa_packed_weight_bytes(0, 19 * 3 * 128 + 128, 6144) == 0  # nkv = 3


def _call(fn, dims, ptrs=None, ws_bytes=1 << 30):
    lib = B.load()
    if ptrs is None:
        ptrs = [4096 * (i + 1) for i in range(21)]  # never dereferenced: rejected first
    return getattr(lib, fn)(ctypes.byref(dims) if dims is not None else None, *ptrs,
                            ws_bytes, None)


@pytest.mark.parametrize("fn", ["pre_attn_decode", "pre_attn_prefill"])
def test_invalid_arguments_rejected(fn):
    lib = B.load()
    assert _call(fn, None) == -1  # NULL dims
    assert _call(fn, _dims(nkv=3)) == -3
    assert _call(fn, _dims(hidden=100)) == -4
    assert _call(fn, _dims(hidden=20000 // 128 * 128)) == -4
    assert _call(fn, _dims(tokens=0)) == -5
    assert _call(fn, _dims(num_pages=0)) == -7
    assert _call(fn, _dims(eps=float("nan"))) == -7
    ptrs = [4096 * (i + 1) for i in range(21)]
    ptrs[3] = None
    assert _call(fn, _dims(), ptrs) == -1
    ptrs = [4096 * (i + 1) for i in range(21)]
    ptrs[0] += 8  # ar not 16-byte aligned
    assert _call(fn, _dims(), ptrs) == -2
    ptrs = [4096 * (i + 1) for i in range(21)]
    ptrs[11] += 4  # positions not 8-byte aligned
    assert _call(fn, _dims(), ptrs) == -2
    for i, off in ((6, 8), (10, 2)):  # g_q, cos_sin: read in 16-byte pieces
        ptrs = [4096 * (j + 1) for j in range(21)]
        ptrs[i] += off
        assert _call(fn, _dims(), ptrs) == -2
    assert _call(fn, _dims(), ws_bytes=16) == -6
    assert lib.pa_strerror(-6).decode().startswith("workspace")


def _call_ex(fn, opts, ptrs=None, ws_bytes=1 << 30):
    lib = B.load()
    if ptrs is None:
        ptrs = [4096 * (i + 1) for i in range(21)]  # never dereferenced: rejected first
    return getattr(lib, fn)(ctypes.byref(_dims()), None if opts is None else ctypes.byref(opts),
                            *ptrs, ws_bytes, None)


@pytest.mark.parametrize("fn", ["pre_attn_decode_ex", "pre_attn_prefill_ex"])
def test_head_options_rejected(fn):
    opts = B.pa_head_options
    qf = 1 << 20
    for bad in (0.0, -1.0, float("nan"), float("inf"), 1e-39):  # 1e-39: reciprocal overflows
        assert _call_ex(fn, opts(0, bad, qf)) == B.PA_ERR_OPTIONS, bad
    # the scale is ignored without the FP8 q output
    assert _call_ex(fn, opts(1, 0.0, None), ws_bytes=16) == -6
    assert _call_ex(fn, opts(0, 0.5, qf + 8)) == -2  # FP8 q not 16-byte aligned
    ptrs = [4096 * (i + 1) for i in range(21)]
    ptrs[18] = None  # q_out NULL: allowed only with the FP8 q output
    assert _call_ex(fn, None, ptrs) == -1
    assert _call_ex(fn, opts(1, 1.0, None), ptrs) == -1
    assert _call_ex(fn, opts(0, 0.5, qf), ptrs, ws_bytes=16) == -6
    ptrs[19] = None  # iq_out is always required
    assert _call_ex(fn, opts(0, 0.5, qf), ptrs) == -1
    assert B.load().pa_strerror(B.PA_ERR_OPTIONS).decode().startswith("bad pa_head_options")
    # NVFP4: an unknown format, static scales with NVFP4, bad global scales
    assert _call_ex(fn, opts(0, 1.0, None, 2, 1.0, 1.0)) == B.PA_ERR_OPTIONS
    assert _call_ex(fn, opts(1, 1.0, None, B.PA_KV_NVFP4, 1.0, 1.0)) == B.PA_ERR_OPTIONS
    for bad in (0.0, -2.0, float("inf"), float("nan"), 1e-39):
        assert _call_ex(fn, opts(0, 1.0, None, B.PA_KV_NVFP4, bad, 1.0)) == B.PA_ERR_OPTIONS, bad
        assert _call_ex(fn, opts(0, 1.0, None, B.PA_KV_NVFP4, 1.0, bad)) == B.PA_ERR_OPTIONS, bad
    ptrs = [4096 * (i + 1) for i in range(21)]
    ptrs[14] = ptrs[15] = ptrs[16] = None  # v_cache, k_scale, v_scale: unused with NVFP4
    assert _call_ex(fn, opts(0, 1.0, None, B.PA_KV_NVFP4, 0.5, 2.0), ptrs, ws_bytes=16) == -6
    assert _call_ex(fn, opts(0, 1.0, None, B.PA_KV_FP8, 1.0, 1.0), ptrs) == -1
    ptrs[13] = 4096 + 8  # the NVFP4 K/V cache takes 16-byte pieces
    assert _call_ex(fn, opts(0, 1.0, None, B.PA_KV_NVFP4, 0.5, 2.0), ptrs) == -2


def test_decode_token_limit():
    assert _call("pre_attn_decode", _dims(tokens=65)) == -5
    # prefill accepts 65 tokens; the tiny workspace stops it before any launch
    assert _call("pre_attn_prefill", _dims(tokens=65), ws_bytes=16) == -6


def test_pack_rejects_bad_shapes():
    lib = B.load()
    assert lib.pa_pack_weight_decode(None, 4096, 2560, 6144, None) == -1
    assert lib.pa_pack_weight_decode(4096, 8192, 2560, 6100, None) == -4
    assert lib.pa_pack_weight_decode(4096, 8192, 2600, 6144, None) == -3
    assert lib.pa_pack_weight_prefill(4096, 8192, 12288, 16384, 2560, 6144 + 8, None) == -4


def test_strerror_covers_all_codes():
    lib = B.load()
    for code in range(0, -13, -1):
        assert lib.pa_strerror(code).decode() != "unknown status"
    assert lib.pa_strerror(-99).decode() == "unknown status"


def test_binding_requires_built_library(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libpre_attn.so")
    with pytest.raises(RuntimeError, match="missing"):
        B.load()
