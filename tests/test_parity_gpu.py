"""Parity of the HIP path (through the C ABI) with the oracle, element by
element, on seeded synthetic inputs: small shapes that span several tiles and
ragged tails, degenerate cases, slots outside the cache, wide weight block
exponents, and the five full workloads (every token of each)."""

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
    (20, 4736, 1, {}),  # 37 k slices: the epilogue in a launch of its own
    (12, 8192, 2, {}),  # the fused norm at its widest (four 8-element vectors a thread)
    (8, 16384, 1, {}),  # hidden past the fused norm's reach, 32 k slices
    (4, 16384, 2, {}),  # more CTAs than are resident at once
    # slots at or past the cache's end write nothing, in every launch structure
    (5, 1024, 1, {"oob_frac": 0.4}),               # one launch
    (8, 6144, 1, {"oob_frac": 0.25}),              # norm + GEMV, then the epilogue
    (40, 2048, 2, {"oob_frac": 0.2, "skip_frac": 0.1}),  # norm, then GEMV + epilogue
    (24, 16384, 1, {"oob_frac": 0.2}),             # the same past the fused norm's hidden
    (20, 4736, 1, {"oob_frac": 0.2}),              # three launches
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
    (300, 1024, 2, {"oob_frac": 0.1, "skip_frac": 0.05}),  # slots past the cache's end
    (2560, 256, 4, {"oob_frac": 0.05}),                   # the same with 256-token CTAs
    (40, 16384, 1, {}),                                   # hidden past 8192: the norm pass's 1024-thread form
    (65, 12288, 2, {"skip_frac": 0.1}),                   # the same with 768 threads a row
    (1000, 1024, 4, {}),                                  # more than one round of 128-token CTAs, ragged
    (1700, 2048, 2, {"skip_frac": 0.1}),                  # the same at nkv 2
]


@pytest.mark.parametrize("S,K,nkv,kw", PREFILL_SMALL, ids=lambda v: str(v))
def test_prefill_parity_small(S, K, nkv, kw):
    wl = _wl("prefill", S, K, nkv, **kw)
    _say(f"prefill parity {wl.name} {kw}")
    inp = synth.make_workload(wl, seed=S * 5 + K)
    ref = oracle.prefill(inp)
    p, got = _gpu(inp)
    stats = parity.compare(inp, ref, got)
    parity.check_written_sets(inp, got)
    parity.check_activation_codes(p.workspace.cpu().numpy(), ref, S, K)
    _say(f"  {stats}")


def _tie_rows(M, K, seed):
    """Rows whose MXFP8 quantization meets every E4M3 decision exactly.

    With g_in = 0 and eps = 0, a row whose mean square is exactly 1 has
    rstd = 1, so xn = acc exactly. Each of the first K / 32 - 4 blocks holds
    1.0 (so amax lies in [1, 2) and the block scale is 2^-8) and 31 values
    v = q 2^-8 with q from: every E4M3 grid value and every midpoint between
    neighbours (the ties, subnormal ones included), values past 448 (464 is the
    saturating tie), and values below half the smallest subnormal. The last
    four blocks hold bf16 values whose squares bring the row's sum of squares
    to exactly K; every partial sum of squares is exact in float64, so rstd is
    exactly 1 in any summation order. Returns float64 values, each exact in
    bf16, shape [M, K].
    """
    from fractions import Fraction
    grid = [oracle.e4m3_decode(np.array([c], np.uint8))[0] for c in range(127)]
    qs = list(grid) + [(grid[i] + grid[i + 1]) / 2 for i in range(126)]
    qs += [464.0, 470.0, 480.0, 500.0, 510.0, 2.0 ** -11, 2.0 ** -12, 3 * 2.0 ** -11]
    rng = np.random.default_rng(seed)
    nb = K // 32
    assert nb >= 16, "needs room for the tie set"
    out = np.zeros((M, K))
    unit = Fraction(1, 2 ** 20)  # every value here is a multiple of 2^-20
    for r in range(M):
        vals = np.array(qs)[rng.permutation(len(qs))] * 2.0 ** -8
        body = np.zeros((nb - 4) * 32)
        slots = [i for i in range(len(body)) if i % 32 != 0]
        n = min(len(slots), len(vals))
        body[slots[:n]] = vals[:n] * np.where(rng.random(n) < 0.5, -1.0, 1.0)
        body[::32] = 1.0
        ss = sum(Fraction(float(v)) ** 2 for v in body)
        rem = Fraction(K) - ss
        assert rem > 0
        fill = []
        while rem > 0:  # greedy: the largest bf16 value (multiple of 2^-20) whose square fits
            x = Fraction(int(np.sqrt(float(rem / unit ** 2))), 1) * unit
            while x * x > rem:
                x -= unit
            while (x + unit) ** 2 <= rem:
                x += unit
            n = int(x / unit)
            shift = max(0, n.bit_length() - 8)  # keep 8 significant bits
            x = Fraction((n >> shift) << shift) * unit
            fill.append(x)
            rem -= x * x
        assert len(fill) <= 128, "filler does not fit"
        row = np.concatenate([body, np.zeros(128)])
        row[len(body):len(body) + len(fill)] = [float(x) for x in fill]
        out[r] = row
    assert np.all(out.astype(np.float32).view(np.uint32) & 0xFFFF == 0), "value not exact in bf16"
    return out


def test_prefill_activation_codes_every_tie():
    # exact ties, subnormal midpoints and saturation in the MXFP8 activation
    # quantization, bit-exact against the oracle; rows span two token tiles
    M, K = 40, 1024
    wl = _wl("prefill", M, K, 1, eps=0.0)
    inp = synth.make_workload(wl, seed=11)
    vals = _tie_rows(M, K, seed=5)
    bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    inp["ar"] = bits
    inp["res"] = np.zeros_like(bits)
    inp["g_in"] = np.zeros_like(inp["g_in"])
    xn = oracle.input_norm(bits, inp["res"], inp["g_in"], inp["eps"])[2]
    assert np.array_equal(xn, vals), "construction: rstd is not exactly 1"
    ref = oracle.prefill(inp)
    p, got = _gpu(inp)
    assert np.array_equal(got["h_out"], ref["h_out"])
    parity.check_activation_codes(p.workspace.cpu().numpy(), ref, M, K)


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
    p, got = _gpu(inp)
    parity.compare(inp, ref, got)
    parity.check_written_sets(inp, got)
    if mode == "prefill":
        parity.check_activation_codes(p.workspace.cpu().numpy(), ref, 6, 256)
    page, t = inp["slot_mapping"][0] // 16, inp["slot_mapping"][0] % 16
    assert got["k_scale"][page, 0, t] == 1.0 and got["v_scale"][page, 0, t] == 1.0


def test_decode_parity_nkv4_full_hidden():
    # 77 heads x 12 k slices at hidden 6144: more GEMV CTAs than are resident
    # at once, heads spread unevenly over the XCDs
    wl = _wl("decode", 64, 6144, 4, outlier_frac=0.01)
    _say(f"decode parity {wl.name}")
    inp = synth.make_workload(wl, seed=41)
    ref = oracle.decode(inp)
    _, got = _gpu(inp)
    stats = parity.compare(inp, ref, got)
    parity.check_written_sets(inp, got)
    _say(f"  {stats}")


def test_workspace_shared_across_shapes():
    # one workspace serves decode and prefill calls of every launch structure
    # in turn; each call matches the oracle
    from kv_residual_add_amd import _binding as B
    from kv_residual_add_amd.runner import Problem

    shapes = [("decode", 64, 1024, 2), ("decode", 8, 1024, 1), ("prefill", 40, 512, 1),
              ("decode", 20, 4736, 1), ("decode", 4, 256, 1), ("decode", 16, 6144, 1)]
    probs = []
    for i, (mode, S, K, nkv) in enumerate(shapes):
        inp = synth.make_workload(_wl(mode, S, K, nkv), seed=100 + i)
        ref = oracle.decode(inp) if mode == "decode" else oracle.prefill(inp)
        probs.append((inp, ref, Problem(inp)))
    need = max(p.workspace.numel() for _, _, p in probs)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    B.pa_workspace_init(ws)
    for rnd in range(2):
        for (mode, S, K, nkv), (inp, ref, p) in zip(shapes, probs):
            _say(f"shared workspace: round {rnd} {mode} S={S} K={K} nkv={nkv}")
            for k in ("k_cache", "v_cache", "index_cache", "k_scale", "v_scale"):
                p.t[k].copy_(torch.from_numpy(inp[k]).to(p.device))
            p.run(workspace=ws)
            torch.cuda.synchronize()
            B.pa_workspace_status(ws)
            got = p.outputs()
            parity.compare(inp, ref, got)
            parity.check_written_sets(inp, got)


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


def prefill_chunks(inp, chunk=2048):
    """The oracle over every token of a prefill call, in token chunks (host
    memory): yields (rows, oracle output for those rows)."""
    S = inp["ar"].shape[0]
    for r0 in range(0, S, chunk):
        rows = np.arange(r0, min(S, r0 + chunk))
        yield rows, oracle.prefill(parity.subset(inp, rows))


def merge_stats(acc, stats):
    """Worst case over chunks of the statistics parity.compare returns."""
    for k, v in stats.items():
        if k == "failures":
            continue
        acc[k] = v + acc.get(k, 0) if k == "live_slots" else max(v, acc.get(k, v))
    return acc


@pytest.mark.parametrize("key", ["c4", "c5"])
def test_prefill_parity_full_workloads(key):
    # every token of the workload against the oracle (in token chunks), the
    # full written-byte sets and every activation code
    wl = synth.named_config(key)
    _say(f"prefill full {wl.name} (every token)")
    inp = synth.make_workload(wl, seed=0)
    p, got = _gpu(inp)
    ws = p.workspace.cpu().numpy()
    del p
    torch.cuda.empty_cache()
    S = wl.tokens
    stats, xq, xs = {}, [], []
    for rows, ref in prefill_chunks(inp):
        merge_stats(stats, parity.compare(inp, ref, got, rows=rows))
        xq.append(ref["xq"])
        xs.append(ref["xs"])
        _say(f"  tokens {rows[0]}..{rows[-1]} ok")
    assert stats["live_slots"] == S
    parity.check_written_sets(inp, got)
    parity.check_activation_codes(ws, {"xq": np.concatenate(xq), "xs": np.concatenate(xs)}, S, wl.hidden)
    _say(f"  {stats}")


def test_prefill_wide_weight_exponents():
    # Weight block exponents far from the synthetic 113..114, across the range
    # the header states for exact widening of the k, v and index_k heads
    # (E8M0 10..246; here up to 200 so the projection stays in float32's range):
    # half the rows take a band of four exponents around a per-row base in
    # [10, 196], the other half a uniform exponent per block in [10, 200].
    wl = _wl("prefill", 300, 1024, 2, skip_frac=0.05)
    _say(f"prefill wide exponents {wl.name}")
    inp = synth.make_workload(wl, seed=77)
    rng = np.random.default_rng(78)
    N, nb = inp["w_e8m0"].shape
    base = rng.integers(10, 197, size=(N, 1))
    band = base + rng.integers(0, 4, size=(N, nb))
    wide = rng.integers(10, 201, size=(N, nb))
    inp["w_e8m0"] = np.where((np.arange(N) % 2 == 0)[:, None], band, wide).astype(np.uint8)
    assert inp["w_e8m0"].min() == 10 and inp["w_e8m0"].max() >= 198
    ref = oracle.prefill(inp)
    p, got = _gpu(inp)
    stats = parity.compare(inp, ref, got)
    parity.check_written_sets(inp, got)
    _say(f"  {stats}")


# decode shapes for each launch structure: few tokens with a small weight (norm,
# GEMV and head epilogue in one launch, flags handed over in each XCD's L2), few
# tokens with a larger weight (norm + GEMV in one launch, epilogue in a second),
# more tokens (norm, then GEMV + epilogue), and 37 k slices (three launches).
# Repeated calls must reuse the in-launch flags cleanly.
REPEAT_CASES = [("decode", 4, 256, 1), ("decode", 8, 1024, 2), ("decode", 24, 1024, 2), ("decode", 20, 4736, 1),
                ("prefill", 24, 1024, 2)]


@pytest.mark.parametrize("mode,S,K,nkv", REPEAT_CASES, ids=lambda v: str(v))
def test_repeat_calls_bit_identical(mode, S, K, nkv):
    wl = _wl(mode, S, K, nkv)
    _say(f"repeat {wl.name}")
    inp = synth.make_workload(wl, seed=9)
    ref = oracle.decode(inp) if mode == "decode" else oracle.prefill(inp)
    p, first = _gpu(inp)
    parity.compare(inp, ref, first)
    for _ in range(3):
        for k in ("k_cache", "v_cache", "index_cache", "k_scale", "v_scale"):
            p.t[k].copy_(torch.from_numpy(inp[k]).to(p.device))
        p.run()
        again = p.outputs()
        for k in first:
            assert np.array_equal(first[k].view(np.uint8), again[k].view(np.uint8)), k


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



def _bf16_of(x):
    import struct
    return struct.unpack("<I", struct.pack("<f", float(x)))[0] >> 16  # exact for the values used


@pytest.mark.parametrize("S,K", [(4, 1024), (4, 6144), (20, 1024), (20, 6144)])
def test_norm_scale_with_exact_ties(S, K):
    # The decode norm takes the row's FP8 scale from the thread that holds the
    # largest |acc| (1 + g) when it is unique, and from a second block reduction
    # on an exact tie (distinct products are never within 2^-50 of each other).
    # Rows 0 and 1 tie across threads 0 and 1 (elements 0 and 8), with the same
    # and with different factors; the other rows have a unique maximum. With 4
    # tokens the norm shares the projection's launch and every XCD keeps a copy
    # of the per-token scales; with 20 it is a launch of its own that leaves the
    # scales and the activation codes in the workspace. All must equal the
    # oracle's bit for bit.
    from kv_residual_add_amd import _binding as B
    from kv_residual_add_amd.runner import Problem

    wl = _wl("decode", S, K, 1, max_pos=64)
    inp = synth.make_workload(wl, seed=9)
    g = inp["g_in"].copy()
    g[0], g[8] = _bf16_of(0.25), 0
    inp["g_in"] = g
    for r, (a0, a8) in enumerate(((40.0, 50.0), (48.0, 60.0))):  # 40 * 1.25 = 50, 48 * 1.25 = 60
        inp["ar"][r, 0], inp["ar"][r, 8] = _bf16_of(a0), _bf16_of(a8)
        inp["res"][r, 0], inp["res"][r, 8] = 0, 0
    inp["ar"][2, 16] = _bf16_of(70.0)
    inp["res"][2, 16] = 0
    ref = oracle.decode(inp)
    p = Problem(inp)
    fused = bool(B.pa_decode_structure(p.dims) & B.PA_DECODE_NORM_FUSED)
    assert fused == (S <= 16)
    p.run()
    got = p.outputs()
    parity.compare(inp, ref, got)
    parity.check_written_sets(inp, got)
    ws = p.workspace.cpu().numpy()
    base = parity.SYNC_BYTES
    off = base + -(-(S * K) // 256) * 256  # past the room for the codes [S][K]
    if fused:  # no activation codes in the workspace; 8 copies of the scales, 64 apart
        for x in range(8):
            sx = ws[off + 4 * 64 * x: off + 4 * (64 * x + S)].view(np.float32)
            assert np.array_equal(sx.view(np.uint32), ref["s_x"].view(np.uint32)), (x, sx, ref["s_x"])
    else:  # codes [S][K], then the scales from the next 256-byte boundary
        assert np.array_equal(ws[base: base + S * K].reshape(S, K), ref["x8"])
        sx = ws[off: off + 4 * S].view(np.float32)
        assert np.array_equal(sx.view(np.uint32), ref["s_x"].view(np.uint32)), (sx, ref["s_x"])


@pytest.mark.parametrize("S, K, nkv", [(4, 1024, 1), (33, 1536, 2), (20, 4736, 1)])
def test_decode_timeline_stamps(S, K, nkv):
    """Phase stamps (pa_set_timeline) leave every output bit unchanged, are in
    program order within each CTA, cover every GEMV CTA, and stay inside the
    buffer they are given."""
    from kv_residual_add_amd import _binding as B
    from kv_residual_add_amd.runner import Problem

    _say(f"timeline decode S={S} K={K} nkv={nkv}")
    wl = _wl("decode", S, K, nkv)
    ref = _gpu(synth.make_workload(wl, seed=11))[1]
    p = Problem(synth.make_workload(wl, seed=11))
    H = 19 * nkv + 1
    records = S + H * (K // 128) + S * H  # an upper bound for every structure
    sentinel = -7
    buf = torch.full((records * 8 + 64,), sentinel, dtype=torch.int64, device="cuda:0")
    buf[: records * 8].zero_()
    B.pa_set_timeline(buf[: records * 8])
    try:
        p.run()
        out = p.outputs()
    finally:
        B.pa_set_timeline(None)
    for k, v in ref.items():
        assert np.array_equal(v.view(np.uint8), out[k].view(np.uint8)), f"{k} changed with the timeline on"
    t = buf.cpu().numpy()
    assert (t[records * 8:] == sentinel).all(), "a stamp landed past the buffer"
    t = t[: records * 8].reshape(records, 8)
    flags = B.pa_decode_structure(p.dims)
    assert (t[:S, 0] > 0).all() and (t[:S, 5] >= t[:S, 0]).all()  # the norm of each token
    # then head h, k slice ks at S + ks H + h (the first H records at least:
    # k slice 0), and the epilogues after those; every stamped record is in
    # program order
    rest = t[S:]
    assert (rest[:H, 0] > 0).all()
    on = rest[:, 0] > 0
    assert (rest[on, 1] >= rest[on, 0]).all()
    if flags & B.PA_DECODE_NORM_FUSED:
        assert not rest[:, 2].any()
    else:
        # the GEMV records carry the activation-in-LDS stamp, between start and
        # end: a contiguous block of H ksplit records
        g2 = np.flatnonzero(rest[:, 2])
        ksplit = len(g2) // H
        assert len(g2) == H * ksplit and ksplit >= 1 and (K // 128) % ksplit == 0
        assert np.array_equal(g2, np.arange(H * ksplit))
        g = rest[: H * ksplit]
        assert ((g[:, 2] >= g[:, 0]) & (g[:, 2] <= g[:, 1])).all()
        if flags == B.PA_DECODE_EPILOGUE_FUSED:
            # GEMV + epilogue launch: the head's slices all stored, then the
            # slice's epilogue tokens
            assert ((g[:, 4] >= g[:, 1]) & (g[:, 5] >= g[:, 4])).all()
    # a buffer too small for the call: the stamps past it are dropped
    small = S + 3
    buf.fill_(sentinel)
    buf[: small * 8].zero_()
    B.pa_set_timeline(buf[: small * 8])
    try:
        p.run()
        out = p.outputs()
    finally:
        B.pa_set_timeline(None)
    for k, v in ref.items():
        assert np.array_equal(v.view(np.uint8), out[k].view(np.uint8)), f"{k} changed with a short timeline"
    t = buf.cpu().numpy()
    assert (t[small * 8:] == sentinel).all(), "a stamp landed past a short buffer"
    assert (t[: S * 8].reshape(S, 8)[:, 0] > 0).all()


def test_prefill_pack_checks_precise_exponents():
    # pa_pack_weight_prefill returns PA_ERR_WEIGHT_RANGE when an E8M0 code of a
    # k, v or index_k row lies outside [10, 246] (the exact bf16 widening's
    # range); codes of q and index_q rows are not restricted
    from kv_residual_add_amd import _binding as B

    nkv, K = 2, 256
    N = (19 * nkv + 1) * 128
    w = torch.zeros((N, K), dtype=torch.uint8, device="cuda:0")
    wp = torch.empty(B.pa_packed_weight_bytes(B.PA_MODE_PREFILL, N, K), dtype=torch.uint8, device="cuda:0")
    sp = torch.empty(B.pa_packed_scale_bytes(B.PA_MODE_PREFILL, N, K), dtype=torch.uint8, device="cuda:0")
    ok = torch.full((N, K // 32), 120, dtype=torch.uint8, device="cuda:0")
    B.pa_pack_weight_prefill(w, ok, wp, sp)
    edge = ok.clone()
    edge[16 * nkv * 128] = 10
    edge[19 * nkv * 128 + 127] = 246
    edge[0, 3] = 0  # a q row: any code
    edge[18 * nkv * 128, 0] = 255  # an index_q row: any code
    B.pa_pack_weight_prefill(w, edge, wp, sp)
    for row, code in ((16 * nkv * 128, 9), (17 * nkv * 128 + 5, 247), (19 * nkv * 128 + 127, 0),
                      (18 * nkv * 128 - 1, 255)):
        bad = ok.clone()
        bad[row, K // 32 - 1] = code
        with pytest.raises(B.PaError) as e:
            B.pa_pack_weight_prefill(w, bad, wp, sp)
        assert e.value.status == B.PA_ERR_WEIGHT_RANGE, (row, code)


@pytest.mark.parametrize("force", [1, 2, 3])
@pytest.mark.parametrize("S,K,nkv", [(1, 1024, 1), (8, 6144, 1), (40, 2048, 2), (64, 6144, 2)],
                         ids=lambda v: str(v))
def test_decode_forced_fallback_paths(monkeypatch, S, K, nkv, force):
    # The hand-offs' fall-back paths, forced from the host: every GEMV CTA of
    # the one-launch structures computes the token statistics itself (1), and
    # no k slice of the GEMV + epilogue launch waits for the others, so the
    # slice that arrives last runs every share of the head epilogue (2). The
    # outputs are the plain call's, bit for bit, and the oracle's.
    from kv_residual_add_amd.runner import Problem

    wl = _wl("decode", S, K, nkv, skip_frac=0.1)
    _say(f"forced paths {force} {wl.name}")
    inp = synth.make_workload(wl, seed=S + K + nkv)
    plain = Problem(inp)
    plain.run()
    want = plain.outputs()
    monkeypatch.setenv("PA_DECODE_FORCE_PATHS", str(force))
    p = Problem(inp)
    p.run()
    got = p.outputs()
    for k in want:
        assert np.array_equal(want[k].view(np.uint8), got[k].view(np.uint8)), k
    parity.compare(inp, oracle.decode(inp), got)
