"""Parity of the HIP path (through the C ABI) with the oracle, element by
element, on seeded synthetic inputs: small shapes that span several tiles and
ragged tails, degenerate cases, and the five full workloads (the prefill ones
checked on sampled tokens plus the full written-byte sets)."""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu(inp):
    from kv_residual_add_amd.runner import Problem

    p = Problem(inp)
    p.run()
    return p, p.outputs()


def _wl(mode, S, K, nkv, **kw):
    base = dict(name=f"{mode}_s{S}_k{K}_nkv{nkv}", mode=mode, tokens=S, hidden=K, nkv=nkv,
                max_pos=kw.pop("max_pos", 4096), num_pages=kw.pop("num_pages", max(1, -(-S // 16) + 2)),
                layout="random")
    base.update(kw)
    return synth.Workload(**base)


DECODE_SMALL = [
    (1, 128, 1, {}),
    (3, 256, 2, {"skip_frac": 0.34}),
    (8, 1024, 1, {}),
    (16, 1024, 4, {"skip_frac": 0.25}),
    (17, 768, 1, {}),
    (33, 1536, 2, {"outlier_frac": 0.01}),
    (64, 2048, 1, {"skip_frac": 0.1}),
]


@pytest.mark.parametrize("S,K,nkv,kw", DECODE_SMALL, ids=lambda v: str(v))
def test_decode_parity_small(S, K, nkv, kw):
    wl = _wl("decode", S, K, nkv, **kw)
    _say(f"decode parity {wl.name} {kw}")
    inp = synth.make_workload(wl, seed=S * 7 + K)
    ref = oracle.decode(inp)
    _, got = _gpu(inp)
    stats = parity.compare(inp, ref, got)
    parity.check_written_sets(inp, got)
    _say(f"  {stats}")


PREFILL_SMALL = [
    (1, 128, 1, {}),
    (5, 256, 2, {"skip_frac": 0.4}),
    (130, 512, 1, {}),
    (300, 1024, 4, {"skip_frac": 0.1}),
    (257, 384, 2, {"outlier_frac": 0.01}),
]


@pytest.mark.parametrize("S,K,nkv,kw", PREFILL_SMALL, ids=lambda v: str(v))
def test_prefill_parity_small(S, K, nkv, kw):
    wl = _wl("prefill", S, K, nkv, **kw)
    _say(f"prefill parity {wl.name} {kw}")
    inp = synth.make_workload(wl, seed=S * 5 + K)
    ref = oracle.prefill(inp)
    _, got = _gpu(inp)
    stats = parity.compare(inp, ref, got)
    parity.check_written_sets(inp, got)
    _say(f"  {stats}")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_degenerate_rows(mode):
    # a zero row (ar = -res), position 0 (identity RoPE), the last table row,
    # and a slot of -1
    wl = _wl(mode, 6, 256, 1, max_pos=64)
    inp = synth.make_workload(wl, seed=3)
    inp["res"][0] = inp["ar"][0] ^ 0x8000  # bf16 negation: acc row 0 == 0
    inp["positions"][1] = 0
    inp["positions"][2] = 63
    inp["slot_mapping"][3] = -1
    ref = oracle.decode(inp) if mode == "decode" else oracle.prefill(inp)
    _, got = _gpu(inp)
    parity.compare(inp, ref, got)
    parity.check_written_sets(inp, got)
    page, t = inp["slot_mapping"][0] // 16, inp["slot_mapping"][0] % 16
    assert got["k_scale"][page, 0, t] == 1.0 and got["v_scale"][page, 0, t] == 1.0


@pytest.mark.parametrize("key", ["c1", "c2", "c3"])
def test_decode_parity_full_workloads(key):
    wl = synth.named_config(key)
    _say(f"decode full {wl.name}")
    inp = synth.make_workload(wl, seed=0)
    ref = oracle.decode(inp)
    _, got = _gpu(inp)
    stats = parity.compare(inp, ref, got)
    parity.check_written_sets(inp, got)
    _say(f"  {stats}")


@pytest.mark.parametrize("key", ["c4", "c5"])
def test_prefill_parity_full_workloads_sampled(key):
    wl = synth.named_config(key)
    _say(f"prefill full {wl.name} (sampled tokens)")
    inp = synth.make_workload(wl, seed=0)
    p, got = _gpu(inp)
    rng = np.random.default_rng(1)
    S = wl.tokens
    rows = np.unique(np.concatenate([[0, S - 1, 127, 128], rng.choice(S, 60, replace=False)]))
    ref = oracle.prefill(parity.subset(inp, rows))
    stats = parity.compare(inp, ref, got, rows=rows)
    parity.check_written_sets(inp, got)
    _say(f"  {stats}")
    del p
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_repeat_calls_bit_identical(mode):
    wl = _wl(mode, 24, 1024, 2)
    inp = synth.make_workload(wl, seed=9)
    p, first = _gpu(inp)
    for k in ("k_cache", "v_cache", "index_cache", "k_scale", "v_scale"):
        p.t[k].copy_(torch.from_numpy(inp[k]).to(p.device))
    p.run()
    second = p.outputs()
    for k in first:
        assert np.array_equal(first[k].view(np.uint8), second[k].view(np.uint8)), k


def test_positions_out_of_range_are_clamped():
    wl = _wl("decode", 4, 256, 1, max_pos=32)
    inp = synth.make_workload(wl, seed=4)
    clamped = dict(inp)
    clamped["positions"] = np.clip(inp["positions"], 0, 31)
    inp = dict(inp)
    inp["positions"] = inp["positions"].copy()
    inp["positions"][0] = 1 << 40
    inp["positions"][1] = -5
    clamped["positions"] = inp["positions"].clip(0, 31)
    ref = oracle.decode(clamped)
    _, got = _gpu(inp)
    parity.compare(inp, ref, got)

