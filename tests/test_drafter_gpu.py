"""Parity of the drafter attention (pa_drafter_attention, through the C ABI)
with the oracle (oracle/drafter.py) on seeded synthetic requests: short
requests (one block, every key visible to every row), sliding windows past 4096
keys, partitions of 1, 2, 4 and 34 blocks, a row without a cache slot, and the
benchmark's 16-request batch.

Bars: the rows' q codes and the cache bytes the call writes are bit-exact (the
head step runs in float64 on both sides). The output's bar comes from the
arithmetic: the scores are float32 sums of exact products and P = 2^x a float32
hardware exp2, about 1e-6 relative from the exact values, so an E4M3 P code
moves (by one step, at most 1/8 of P) wherever the exact P lies that close to
a rounding midpoint: a few in a million. Such a move shifts one term of one
head's output, by up to an eighth of that key's share of it. So: every bf16
output within 2e-2 |ref| + 2e-2 rms(ref head); at most 1e-4 of them past the
prologue's q bar (2e-2 |ref| + 1e-3 rms); the MXFP8 output decodes to within
the first bar plus one E4M3 step of the reference's block scale, and at most
1 % of its codes differ."""

import sys

import numpy as np
import pytest

import synth
from oracle import drafter as D
from oracle.codecs import bf16_bits_to_f64, e4m3_decode

pytestmark = pytest.mark.gpu

Q_RTOL, Q_ATOL_RMS, CODE_FRAC = 2e-2, 1e-3, 1e-2
ATOL_RMS = 2e-2     # the floor every element meets
TIGHT_FRAC = 1e-4   # elements allowed past the prologue's q bar


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(inp, ref, got, ws):
    T = 7 * inp["requests"]
    # q codes in the workspace, past the 32 KB of synchronization words
    q8 = ws[32768: 32768 + T * 2048].reshape(T, 16, 128)
    assert np.array_equal(q8, ref["q8"]), f"{int((q8 != ref['q8']).sum())} q codes differ"
    assert np.array_equal(got["kv_cache"], ref["kv_cache"]), "cache bytes differ from the oracle's insert"
    g = bf16_bits_to_f64(got["out_bf16"])
    r = bf16_bits_to_f64(ref["out_bf16"])
    rms = np.sqrt((r * r).mean(axis=-1, keepdims=True))
    err = np.abs(g - r)
    bad = err > Q_RTOL * np.abs(r) + ATOL_RMS * rms
    past_tight = err > Q_RTOL * np.abs(r) + Q_ATOL_RMS * rms
    stats = {"out_max_err_over_rms": float((err / np.maximum(rms, 1e-30)).max()), "out_bad": int(bad.sum()),
             "out_past_q_bar": int(past_tight.sum())}
    assert not bad.any() and past_tight.mean() <= TIGHT_FRAC, stats
    Xg = np.repeat(2.0 ** (got["out_scales"].astype(np.float64) - 127), 32, axis=1)
    Xr = np.repeat(2.0 ** (ref["out_scales"].astype(np.float64) - 127), 32, axis=1)
    dg = e4m3_decode(got["out_codes"]) * Xg
    dr = e4m3_decode(ref["out_codes"]) * Xr
    rr = r.reshape(T, 2048)
    rmsr = np.repeat(rms.reshape(T, 16), 128, axis=1)
    step = 2.0 ** (np.minimum(np.floor(np.log2(np.maximum(np.abs(dr) / Xr, 2.0 ** -6))), 8.0) - 3.0) * Xr
    mx_bad = np.abs(dg - dr) > Q_RTOL * np.abs(rr) + ATOL_RMS * rmsr + step
    frac = float((got["out_codes"] != ref["out_codes"]).mean())
    stats.update(mx_bad=int(mx_bad.sum()), code_frac_diff=frac,
                 scale_frac_diff=float((got["out_scales"] != ref["out_scales"]).mean()))
    assert not mx_bad.any() and frac <= CODE_FRAC, stats
    return stats


def _run(inp):
    from kv_residual_add_amd.runner import DrafterProblem

    p = DrafterProblem(inp)
    p.run()
    got = p.outputs()
    return got, p.workspace.cpu().numpy()


CASES = [
    (1, None, [7], 4, "only the new rows: one block"),
    (2, None, [300, 130], 1, "short requests, one-block partitions"),
    (3, 9000, None, 4, "sliding windows"),
    (4, 12000, None, 34, "one partition"),
    (5, 6000, None, 2, "two-block partitions"),
]


@pytest.mark.parametrize("R,max_seq,seqs,split,what", CASES, ids=lambda v: str(v))
def test_drafter_parity(R, max_seq, seqs, split, what):
    inp = synth.make_drafter(R, max_seq or 0, seed=R * 31 + split, split=split, seq_lens=seqs)
    _say(f"drafter {what}: R={R} split={split} seq_lens={inp['seq_lens'].tolist()}")
    ref = D.attention(inp)
    got, ws = _run(inp)
    _say(f"  {_check(inp, ref, got, ws)}")


def test_drafter_row_without_slot():
    # a row whose slot is -1 writes no cache byte; the attention reads the
    # cache as it is at that key
    inp = synth.make_drafter(2, 700, seed=8, split=2)
    inp["slots"][3] = -1
    ref = D.attention(inp)
    got, ws = _run(inp)
    _check(inp, ref, got, ws)


def test_drafter_batch_16_requests():
    inp = synth.make_drafter(16, 12000, seed=0, split=2, min_seq=2048)
    _say(f"drafter batch: seq_lens {inp['seq_lens'].tolist()}")
    ref = D.attention(inp)
    got, ws = _run(inp)
    _say(f"  {_check(inp, ref, got, ws)}")
