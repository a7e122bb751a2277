"""How close the prefill q / index_q outputs come to their bar, on the two
prefill workloads (every token against the oracle): per head type, the ratio
|got - ref| / (2e-2 |ref| + 1e-3 rms(ref head)) at its maximum and its 99.9th
and 99th percentiles (the bar is ratio <= 1), |got - ref| / rms(ref head) at
its maximum, and with the FP8 q option the code-distance histogram of q.

The q and index_q heads run block-scaled FP8 MFMAs, which sum their products
at reduced internal precision; the figures printed here are the measured size
of that effect against the float64 statement. Run with -s to see them."""

import sys

import numpy as np
import pytest
import torch

import synth
from oracle import codecs
from tests import parity
from tests.test_parity_gpu import prefill_chunks

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ratios(got, ref):
    g = codecs.bf16_bits_to_f64(got)
    r = codecs.bf16_bits_to_f64(ref)
    rms = np.sqrt((r * r).mean(axis=-1, keepdims=True))
    err = np.abs(g - r)
    return (err / (parity.Q_RTOL * np.abs(r) + parity.Q_ATOL_RMS * rms)).ravel(), \
        (err / np.maximum(rms, 1e-30)).ravel()


def _summary(name, ratio, over_rms):
    p999, p99, p50 = np.percentile(ratio, [99.9, 99.0, 50.0])
    return (f"{name}: ratio max {ratio.max():.3f} p99.9 {p999:.3f} p99 {p99:.3f} p50 {p50:.4f}; "
            f"err/rms max {over_rms.max():.2e} ({ratio.size} values)")


@pytest.mark.parametrize("key,q_scale", [("c4", None), ("c5", None), ("c4", 0.008)],
                         ids=["c4", "c5", "c4_fp8q"])
def test_prefill_precision_report(key, q_scale):
    from kv_residual_add_amd.runner import Problem

    wl = synth.named_config(key)
    inp = synth.make_workload(wl, seed=0)
    if q_scale is not None:
        inp["q_fp8_scale"] = q_scale
    p = Problem(inp)
    p.run()
    got = p.outputs()
    del p
    torch.cuda.empty_cache()
    parts = {"q_out": ([], []), "iq_out": ([], [])}
    hist = np.zeros(8, np.int64)
    for rows, ref in prefill_chunks(inp):
        parity.compare(inp, ref, got, rows=rows)
        for key_out, (rs, es) in parts.items():
            ratio, over = _ratios(got[key_out][rows], ref[key_out])
            rs.append(ratio)
            es.append(over)
        if q_scale is not None:
            d = np.abs(parity.code_ord(got["q_fp8"][rows]) - parity.code_ord(ref["q_fp8"]))
            hist += np.bincount(np.minimum(d.ravel(), 7), minlength=8)
    _say(f"precision {wl.name}" + (f" with FP8 q at scale {q_scale}" if q_scale is not None else ""))
    for key_out, (rs, es) in parts.items():
        ratio, over = np.concatenate(rs), np.concatenate(es)
        _say("  " + _summary(key_out, ratio, over))
        assert ratio.max() <= 1.0
    if q_scale is not None:
        total = hist.sum()
        _say("  q_fp8 code distance histogram (0, 1, 2, ..., >=7): "
             + ", ".join(f"{int(c)}" for c in hist) + f" of {int(total)}; "
             + f"differing {1 - hist[0] / total:.2e}")
        assert 1 - hist[0] / total <= parity.Q_FP8_FRAC
