"""The two MFMA forms of the prefill projection, one 32x32x64 product each,
against the exact sums of their products (tests/native/mfma_numerics.hip, a
test-only library built with the package):

  - the block-scaled FP8 MFMA with the prefill kernels' operand layout: a
    lane's bytes 0..15 are k = 16 (l / 32) + [0, 16) of MX block 0 and bytes
    16..31 are k = 32 + 16 (l / 32) + [0, 16) of block 1. With unequal block
    scales only this layout gives the exact sums to within the instruction's
    own error; the layout with contiguous 32-k lane fragments does not.
  - its precision: it sums the 64 products at reduced internal precision, off
    by far more than a float32 accumulation (the reason the k, v and index_k
    heads, whose per-token scales must hold to 1e-6, do not use it);
  - the same product on bf16 MFMAs fed the exactly widened operands (code
    times block scale), as the precise heads compute it: within a few float32
    rounding steps of the exact sums.

Each product of two E4M3 values and two powers of two is exact in float64, and
math.fsum rounds their sum once, so the reference is the exact sum rounded."""

import ctypes
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "libmfma_numerics.so")


def _lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: build it with `python tests/native/build.py`")
    lib = ctypes.CDLL(LIB)
    for f in (lib.mfma_probe_fp8, lib.mfma_probe_bf16):
        f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_void_p]
        f.restype = ctypes.c_int
    return lib


def _codes(rng, n):
    c = rng.integers(0, 256, size=n, dtype=np.int64)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)  # no NaN codes


def _pack(x, contiguous=False):
    """[32, 64] codes -> the 64 lanes' 32-byte fragments."""
    out = np.zeros((64, 32), np.uint8)
    for l in range(64):
        r, h = l % 32, l // 32
        if contiguous:
            out[l] = x[r, 32 * h: 32 * h + 32]
        else:
            out[l, :16] = x[r, 16 * h: 16 * h + 16]
            out[l, 16:] = x[r, 32 + 16 * h: 48 + 16 * h]
    return out


def _run(fn, a, b, ea, eb, contiguous=False):
    dev = "cuda:0"
    A = torch.from_numpy(_pack(a, contiguous)).to(dev)
    Bt = torch.from_numpy(_pack(b, contiguous)).to(dev)
    lanes = np.arange(64)
    SA = torch.from_numpy(ea[lanes % 32, lanes // 32].astype(np.uint32).view(np.int32)).to(dev)
    SB = torch.from_numpy(eb[lanes % 32, lanes // 32].astype(np.uint32).view(np.int32)).to(dev)
    D = torch.zeros(64 * 16, dtype=torch.float32, device=dev)
    st = fn(A.data_ptr(), Bt.data_ptr(), SA.data_ptr(), SB.data_ptr(), D.data_ptr(), None)
    assert st == 0, f"launch failed: {st}"
    torch.cuda.synchronize()
    d = D.cpu().numpy().astype(np.float64)
    out = np.zeros((32, 32))
    for l in range(64):
        for r in range(16):
            out[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] = d[16 * l + r]
    return out


def _exact(a, b, ea, eb):
    """(exact sums rounded once, sums of |products|), [32, 32]."""
    av = codecs.e4m3_decode(a) * np.exp2(np.repeat(ea.astype(np.float64) - 127, 32, axis=1))
    bv = codecs.e4m3_decode(b) * np.exp2(np.repeat(eb.astype(np.float64) - 127, 32, axis=1))
    ex = np.zeros((32, 32))
    mag = np.zeros((32, 32))
    for i in range(32):
        for j in range(32):
            p = av[i] * bv[j]
            ex[i, j] = math.fsum(p)
            mag[i, j] = np.abs(p).sum()
    return ex, mag


@pytest.mark.parametrize("scales", ["unit", "blocks", "wide"])
def test_mfma_forms_against_exact_sums(scales):
    lib = _lib()
    rng = np.random.default_rng({"unit": 1, "blocks": 2, "wide": 3}[scales])
    a = _codes(rng, 32 * 64).reshape(32, 64)
    b = _codes(rng, 32 * 64).reshape(32, 64)
    if scales == "unit":
        ea = np.full((32, 2), 127)
        eb = np.full((32, 2), 127)
    elif scales == "blocks":  # the two MX blocks of a row scaled apart
        ea = np.tile([120, 127], (32, 1))
        eb = np.tile([127, 118], (32, 1))
    else:
        ea = rng.integers(100, 150, size=(32, 2))
        eb = rng.integers(100, 150, size=(32, 2))
    ex, mag = _exact(a, b, ea, eb)
    fp8 = _run(lib.mfma_probe_fp8, a, b, ea, eb)
    bf = _run(lib.mfma_probe_bf16, a, b, ea, eb)
    rel_fp8 = np.abs(fp8 - ex) / mag
    rel_bf = np.abs(bf - ex) / mag
    print(f"{scales}: FP8 MFMA max |err| / sum|p| {rel_fp8.max():.3e} (mean {rel_fp8.mean():.3e}); "
          f"bf16 MFMA on widened values {rel_bf.max():.3e}", flush=True)
    # the layout: exact to within the instruction's own error
    assert rel_fp8.max() < 1e-3
    # reduced internal precision: far past float32 accumulation (~1e-7)
    assert rel_fp8.max() > 1e-5
    # the precise heads' form: a float32 accumulation of exact products
    assert rel_bf.max() < 2.0 ** -19
    if scales == "blocks":  # contiguous 32-k fragments apply the wrong block scale to half the k
        wrong = _run(lib.mfma_probe_fp8, a, b, ea, eb, contiguous=True)
        assert (np.abs(wrong - ex) / mag).max() > 1e-2
