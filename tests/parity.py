"""Comparison of the HIP path's outputs with the oracle's, to the tolerances the
prologue's contract states:

  h_out                         bit-exact
  q_out, iq_out (bf16)          |got - ref| <= 2e-2 |ref| + 1e-3 rms(ref head)
  which cache bytes / scales    bit-exact set (caches start as sentinels)
  FP8 cache codes               code distance <= 1, in at most 0.1% of codes
  K / V scales                  relative difference <= 1e-6
  NVFP4 caches (when requested) E2M1 element codes and E4M3 group scale codes:
                                distance <= 1, in at most 0.1% of each; the
                                written bytes exactly the slots' bytes
  FP8 q (when requested)        decoded values (times the scale) within the q bar
                                plus one E4M3 step at the oracle's value; codes
                                differ in at most 1% of elements

The FP8 q bar is the q bar in another encoding: the two sides' q values may
differ by 2e-2 |q| + 1e-3 rms(head), and rounding each to the E4M3 grid adds
at most one grid step between them. Away from zero that is a code distance of
at most 1; near zero the absolute floor spans several of the finest steps. The
q heads' f32 arithmetic (and, in prefill, the block-scaled FP8 MFMAs, whose
sums are off by up to ~3e-4 of the sum of the products' magnitudes) moves a
code only where the exact value lies that close to a rounding midpoint: on
every token of c4 with the FP8 q at scale 0.008, 1.0e-3 of the codes moved,
up to 4 steps near zero. The 1% ceiling catches a systematic rounding mistake
(truncation instead of nearest-even moves about half of all codes).

Code distance: |ord(a) - ord(b)| with ord(c) = +-(c & 0x7F) by the sign bit,
so +0 and -0 are equal.
"""

from __future__ import annotations

import numpy as np

from oracle import codecs

Q_RTOL = 2e-2
Q_ATOL_RMS = 1e-3
CODE_FRAC = 1e-3
SCALE_RTOL = 1e-6
Q_FP8_FRAC = 1e-2


def subset(inp: dict, rows) -> dict:
    """The same call restricted to token rows `rows` (fresh sentinel caches)."""
    rows = np.asarray(rows)
    out = dict(inp)
    for k in ("ar", "res", "positions", "slot_mapping"):
        out[k] = inp[k][rows]
    return out


def cache_pages(inp: dict) -> int:
    """Pages of the call's cache (FP8 or NVFP4 layout)."""
    return int((inp["kv_cache"] if inp.get("kv_format", "fp8") == "nvfp4" else inp["k_cache"]).shape[0])


def writes_cache(slot, pages: int) -> bool:
    """Whether a token with this slot writes the cache: 0 <= slot < pages * 16
    (a negative slot, or one at or past the cache's end, writes nothing)."""
    return 0 <= int(slot) < 16 * pages


def code_ord(c):
    c = np.asarray(c, np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def _bf16(a):
    return codecs.bf16_bits_to_f64(a)


def compare(inp: dict, ref: dict, got: dict, rows=None, strict: bool = True) -> dict:
    """Parity of `got` (GPU, all tokens) against `ref` (oracle on the tokens
    `rows`, all tokens if None). Collects every statistic first; with `strict`
    raises AssertionError naming each violated tolerance, else returns the
    statistics with a "failures" list."""
    S = inp["ar"].shape[0]
    rows = np.arange(S) if rows is None else np.asarray(rows)
    stats, fails = {}, []
    if not np.array_equal(got["h_out"][rows], ref["h_out"]):
        fails.append(f"h_out: {int((got['h_out'][rows] != ref['h_out']).sum())} elements differ")
    for key in ("q_out", "iq_out"):
        if key not in got:  # FP8 q only
            continue
        g = _bf16(got[key][rows])
        r = _bf16(ref[key])
        rms = np.sqrt((r * r).mean(axis=-1, keepdims=True))
        err = np.abs(g - r)
        bad = err > Q_RTOL * np.abs(r) + Q_ATOL_RMS * rms
        stats[key + "_max_err_over_rms"] = float((err / np.maximum(rms, 1e-30)).max())
        if bad.any():
            fails.append(f"{key}: {int(bad.sum())} elements out of tolerance")
    if "q_fp8" in got or "q_fp8" in ref:
        if "q_fp8" not in got or "q_fp8" not in ref:
            fails.append("q_fp8: requested on one side only")
        else:
            gc, rc = got["q_fp8"][rows], ref["q_fp8"]
            d = np.abs(code_ord(gc) - code_ord(rc))
            stats["qfp8_code_max_dist"] = int(d.max(initial=0))
            stats["qfp8_code_frac_diff"] = float((d > 0).mean())
            scale = float(inp["q_fp8_scale"])
            g = codecs.e4m3_decode(gc) * scale
            r = codecs.e4m3_decode(rc) * scale
            rms = np.sqrt((r * r).mean(axis=-1, keepdims=True))
            x = np.abs(r) / scale
            expo = np.floor(np.log2(np.maximum(x, 2.0 ** -6)))
            step = 2.0 ** (np.minimum(expo, 8.0) - 3.0) * scale  # grid spacing at the oracle's value
            bad = np.abs(g - r) > Q_RTOL * np.abs(r) + Q_ATOL_RMS * rms + step
            if bad.any():
                fails.append(f"q_fp8: {int(bad.sum())} decoded values out of tolerance")
            if (d > 0).mean() > Q_FP8_FRAC:
                fails.append(f"q_fp8: {(d > 0).mean():.2e} of codes differ (> {Q_FP8_FRAC})")

    slots = np.asarray(inp["slot_mapping"])[rows]
    pages = cache_pages(inp)
    slots = np.where((slots >= 0) & (slots < 16 * pages), slots, -1)  # the ones that write
    nkv = int(inp["nkv"])
    if inp.get("kv_format", "fp8") == "nvfp4":
        _compare_nvfp4(got, ref, slots, nkv, stats, fails)
        stats["live_slots"] = int((slots >= 0).sum())
        if strict:
            assert not fails, "; ".join(fails) + f" | {stats}"
        stats["failures"] = fails
        return stats
    for cache, idx in (("k_cache", None), ("v_cache", None), ("index_cache", None)):
        gs, rs = [], []
        for slot in slots:
            if slot < 0:
                continue
            if cache == "index_cache":
                gs.append(got[cache][slot])
                rs.append(ref[cache][slot])
            else:
                # whole pages: only positions the oracle wrote are compared
                gs.append(got[cache][slot // 16].reshape(-1))
                rs.append(ref[cache][slot // 16].reshape(-1))
        if not gs:
            continue
        g = np.concatenate(gs)
        r = np.concatenate(rs)
        wr = r != 0x7F
        if np.any(g[wr] == 0x7F):
            fails.append(f"{cache}: a byte the oracle writes was not written")
        d = np.abs(code_ord(g[wr]) - code_ord(r[wr]))
        name = cache.split("_")[0]
        stats[f"{name}_code_max_dist"] = int(d.max(initial=0))
        stats[f"{name}_code_frac_diff"] = float((d > 0).mean()) if d.size else 0.0
        if d.max(initial=0) > 1:
            fails.append(f"{cache}: FP8 code distance {d.max()} > 1")
        if d.size and (d > 0).mean() > CODE_FRAC:
            fails.append(f"{cache}: {(d > 0).mean():.2e} of codes differ (> {CODE_FRAC})")
    for name in ("k_scale", "v_scale"):
        gs, rs = [], []
        for slot in slots:
            if slot < 0:
                continue
            gs.append(got[name][slot // 16, :, slot % 16])
            rs.append(ref[name][slot // 16, :, slot % 16])
        if not gs:
            continue
        g = np.concatenate(gs).astype(np.float64)
        r = np.concatenate(rs).astype(np.float64)
        rel = np.abs(g - r) / np.abs(r)
        stats[name + "_max_rel"] = float(rel.max())
        if not rel.max() <= SCALE_RTOL:
            fails.append(f"{name}: max relative difference {rel.max():.3e} > {SCALE_RTOL}")
    stats["live_slots"] = int((slots >= 0).sum())
    if strict:
        assert not fails, "; ".join(fails) + f" | {stats}"
    stats["failures"] = fails
    return stats


def e2m1_ord(c):
    c = np.asarray(c, np.int64)
    return np.where(c & 0x8, -(c & 0x7), c & 0x7)


NV_SLOT = 1152


def _nv_rows(cache_page_slot: np.ndarray, t: int):
    """A token's 128 E2M1 codes and its slot's whole scale area."""
    data = cache_page_slot[t * 64:(t + 1) * 64]
    codes = np.stack([data & 0xF, data >> 4], axis=-1).reshape(128)
    return codes, cache_page_slot[1024:]


def _compare_nvfp4(got, ref, slots, nkv, stats, fails):
    gc, rc, gs, rs = [], [], [], []
    for slot in slots:
        if slot < 0:
            continue
        page, t = slot // 16, slot % 16
        pairs = [(got["kv_cache"][page, s], ref["kv_cache"][page, s]) for s in range(2 * nkv)]
        pairs.append((got["index_cache"][page], ref["index_cache"][page]))
        for g, r in pairs:
            a, sa = _nv_rows(g, t)
            b, sb = _nv_rows(r, t)
            gc.append(a)
            rc.append(b)
            wr = sb != SENTINEL  # the scale bytes the oracle wrote in this slot so far
            gs.append(sa[wr])
            rs.append(sb[wr])
    if not gc:
        return
    for name, g, r, ordf in (("nv_code", np.concatenate(gc), np.concatenate(rc), e2m1_ord),
                             ("nv_scale", np.concatenate(gs), np.concatenate(rs), code_ord)):
        d = np.abs(ordf(g) - ordf(r))
        stats[f"{name}_max_dist"] = int(d.max(initial=0))
        stats[f"{name}_frac_diff"] = float((d > 0).mean()) if d.size else 0.0
        if d.max(initial=0) > 1:
            fails.append(f"{name}: distance {d.max()} > 1")
        if d.size and (d > 0).mean() > CODE_FRAC:
            fails.append(f"{name}: {(d > 0).mean():.2e} differ (> {CODE_FRAC})")


SENTINEL = 0x7F


def check_written_sets_nvfp4(inp: dict, got: dict) -> None:
    """Outside the slots' data and scale bytes, the NVFP4 caches keep their
    sentinels; every scale byte of a live slot was written (E4M3 scale codes
    are never 0x7F, the sentinel)."""
    nkv = int(inp["nkv"])
    kv = np.zeros(inp["kv_cache"].shape, bool)
    ic = np.zeros(inp["index_cache"].shape, bool)
    for slot in np.asarray(inp["slot_mapping"]):
        if not writes_cache(slot, kv.shape[0]):
            continue
        page, t = slot // 16, slot % 16
        for m in (kv[page], ic[page][None, :]):
            m[:, t * 64:(t + 1) * 64] = True
        for s in range(2 * nkv):
            v = s % 2 == 1
            for g in range(8):
                off = (t // 4 * 4 + g // 2) * 8 + g % 2 * 4 + t % 4 if v else 8 * t + g
                kv[page, s, 1024 + off] = True
        ic[page, 1024 + 8 * t: 1024 + 8 * t + 8] = True
    for name, mask in (("kv_cache", kv), ("index_cache", ic)):
        assert np.array_equal(got[name][~mask], inp[name][~mask]), f"{name}: a byte outside the slots changed"
        scale_area = np.zeros(mask.shape, bool)
        scale_area[..., 1024:] = True
        written_scales = got[name][mask & scale_area]
        assert np.all(written_scales != SENTINEL), f"{name}: a live slot's scale byte was not written"


def expected_written_masks(inp: dict) -> dict:
    """Which cache bytes / scale entries a call must write, from the slots alone."""
    nkv = int(inp["nkv"])
    P = inp["k_cache"].shape[0]
    k = np.zeros((P, nkv, 2048), bool)
    v = np.zeros((P, nkv, 2048), bool)
    ks = np.zeros((P, nkv, 16), bool)
    ic = np.zeros(inp["index_cache"].shape, bool)
    d = np.arange(128)
    for slot in np.asarray(inp["slot_mapping"]):
        if not writes_cache(slot, P):
            continue
        page, t = slot // 16, slot % 16
        k[page, :, (d // 16) * 256 + t * 16 + d % 16] = True
        v[page, :, d * 16 + t] = True
        ks[page, :, t] = True
        ic[slot, :] = True
    return {"k_cache": k, "v_cache": v, "k_scale": ks, "v_scale": ks, "index_cache": ic}


def check_written_sets(inp: dict, got: dict) -> None:
    """Bytes that changed from the sentinels are exactly the slots' bytes."""
    masks = expected_written_masks(inp)
    for name in ("k_cache", "v_cache", "index_cache"):
        changed = got[name] != inp[name]
        assert np.array_equal(changed, masks[name]), f"{name}: written-byte set differs"
    for name in ("k_scale", "v_scale"):
        changed = got[name].view(np.uint32) != inp[name].view(np.uint32)
        assert np.array_equal(changed, masks[name]), f"{name}: written-entry set differs"
        assert np.all(np.isfinite(got[name][masks[name]])), f"{name}: non-finite scale"


SYNC_BYTES = 32768  # the workspace's leading synchronization words


def prefill_activation_codes(workspace: np.ndarray, M: int, K: int):
    """The MXFP8 activation codes and block scales the prefill norm pass leaves
    in the workspace, unpacked to [Mpad, K] and [Mpad, K // 32] (Mpad = M
    rounded up to 256 token rows).

    The codes start past the workspace's 32 KB of synchronization words, in
    the prefill MFMA's operand order: token tile tt = m // 32 and k step
    ks = k // 64 own the 2 KB block at (tt * nks + ks) * 2048; in it, lane
    l = m % 32 + 32 * ((k % 32) // 16) holds 16 consecutive codes at
    region * 1024 + 16 l, region = (k % 64) // 32. The scale of block
    b = k // 32 is byte (tt * nks + b // 2) * 64 + m % 32 + 32 (b % 2) of the
    region that starts at the next 256-byte boundary after the codes.
    """
    base = SYNC_BYTES
    mpad = -(-M // 256) * 256
    nks = K // 64
    m = np.arange(mpad)[:, None]
    k = np.arange(K)[None, :]
    tt, tl = m // 32, m % 32
    ks, kk = k // 64, k % 64
    off = base + (tt * nks + ks) * 2048 + (kk // 32) * 1024 + (tl + 32 * ((kk // 16) % 2)) * 16 + kk % 16
    xq = workspace[off]
    b = np.arange(K // 32)[None, :]
    xs_base = base + -(-(mpad * K) // 256) * 256
    soff = xs_base + (tt * nks + b // 2) * 64 + tl + 32 * (b % 2)
    xs = workspace[soff]
    return xq, xs


def check_activation_codes(workspace: np.ndarray, ref: dict, M: int, K: int, rows=None) -> None:
    """Bit-exact MXFP8 activation codes and scales against the oracle's (for
    token rows `rows`, default all); padding rows hold zero codes, unit scales."""
    xq, xs = prefill_activation_codes(workspace, M, K)
    sel = np.arange(M) if rows is None else np.asarray(rows)
    bad = np.argwhere(xq[sel] != ref["xq"])
    assert bad.size == 0, f"{len(bad)} activation codes differ, first (row, k) {bad[:5].tolist()}"
    assert np.array_equal(xs[sel], ref["xs"]), "activation block scales differ"
    assert np.all(xq[M:] == 0) and np.all(xs[M:] == 127), "padding rows not zero codes / unit scales"
