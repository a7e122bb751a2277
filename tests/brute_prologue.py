"""Scalar, pure-Python statement of the prologue for tiny inputs.

Written separately from ``oracle/`` (no shared code): number formats are
handled by exhaustive search over the representable values with exact rational
comparisons, sums use math.fsum or exact integers, and every cache byte is
placed by its own loop. Used only to pin the vectorized oracle.

Sources: the vLLM pages ``...amd.mono.kernels.pre_attn`` (K1 mono_pre:
``norm_quant``, the GEMV and head tasks, ``head_norm_rope``, ``page16_of``) and
``...nvidia.ops.qkv_index_fused_epilogue`` (``_rms_norm``, ``_rope64``, the head
list and the per-role epilogue branches).
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction

HEAD_DIM = 128


def f32(x: float) -> float:
    """Nearest float32 (IEEE round-to-nearest-even) of a Python float."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def bf16_round_bits(x: float) -> int:
    """bf16 bits of float32 value x: the nearer of the two neighbouring bf16
    values, ties to the one with an even last bit."""
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    lo = b >> 16
    hi = lo + 1
    vlo, vhi = Fraction(bf16_value(lo)), Fraction(bf16_value(hi))
    fx = Fraction(x)
    dlo, dhi = abs(fx - vlo), abs(vhi - fx)
    if dlo < dhi:
        return lo
    if dhi < dlo:
        return hi & 0xFFFF
    return lo if lo % 2 == 0 else hi & 0xFFFF


def _e4m3_values():
    vals = {}
    for sign in (0, 1):
        for e in range(16):
            for m in range(8):
                code = (sign << 7) | (e << 3) | m
                if e == 15 and m == 7:
                    continue  # NaN
                mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (
                    (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
                )
                vals[code] = -mag if sign else mag
    return vals


E4M3 = _e4m3_values()
_POS_CODES = sorted((c for c in E4M3 if c < 0x80), key=lambda c: E4M3[c])


def e4m3_value(code: int) -> float:
    return float(E4M3[code])


def e4m3_round(x: float) -> int:
    """Saturating round-to-nearest-even by search over all non-negative codes."""
    fx = Fraction(x)
    mag = min(abs(fx), Fraction(448))
    best, best_d = None, None
    for c in _POS_CODES:
        d = abs(E4M3[c] - mag)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    negative = x < 0 or (x == 0 and math.copysign(1.0, x) < 0)
    return best | (0x80 if negative else 0)


def _f32_neighbours(x: float):
    """x (a float32 value) and the float32 values just below and above it."""
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    out = [x]
    for step in (-1, 1):
        if x == 0.0:
            out.append(struct.unpack("<f", struct.pack("<I", 1))[0] * (1 if step > 0 else -1))
            continue
        nb = b + step if x > 0 else b - step  # toward +inf / -inf
        out.append(struct.unpack("<f", struct.pack("<I", nb & 0xFFFFFFFF))[0])
    return out


def f32_nearest(q: Fraction) -> float:
    """The float32 nearest the rational q, ties to an even last bit."""
    best, best_d = None, None
    for c in _f32_neighbours(f32(float(q))):
        d = abs(Fraction(c) - q)
        even = struct.unpack("<I", struct.pack("<f", c))[0] % 2 == 0
        if best is None or d < best_d or (d == best_d and even):
            best, best_d = c, d
    return best


def f32_toward_zero(q: Fraction) -> float:
    """The float32 of largest magnitude not above |q|, with q's sign."""
    cands = [c for c in _f32_neighbours(f32(float(q))) if abs(Fraction(c)) <= abs(q)
             and (c == 0.0 or (c > 0) == (q > 0))]
    return max(cands, key=lambda c: abs(Fraction(c)))


def _e2m1_values():
    vals = {}
    for c in range(8):
        e, m = c >> 1, c & 1
        vals[c] = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return vals


E2M1 = _e2m1_values()


def e2m1_round(x: float) -> int:
    """Saturating nearest-even E2M1 code by search; a zero magnitude is +0."""
    mag = min(abs(Fraction(x)), Fraction(6))
    best, best_d = None, None
    for c in range(8):
        d = abs(E2M1[c] - mag)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (0x8 if x < 0 and best != 0 else 0)


def nvfp4_row(vals, gs):
    """NVFP4 of 128 float32 values: 128 E2M1 codes and 8 E4M3 group scale
    codes, per the epilogue page's _nvfp4_quant32 (gs: float32 reciprocal of
    the global scale, or None)."""
    codes, scales = [], []
    sixth = f32(1.0 / 6.0)
    for g in range(8):
        grp = vals[16 * g:16 * g + 16]
        a = f32_nearest(Fraction(max(abs(v) for v in grp)) * Fraction(sixth))
        if gs is not None:
            a = f32_nearest(Fraction(a) * Fraction(gs))
        a = max(a, 2.0 ** -9)
        sf = e4m3_round(a)
        r = f32_nearest(1 / E4M3[sf])
        if gs is not None:
            r = f32_nearest(Fraction(r) * Fraction(gs))
        scales.append(sf)
        codes += [e2m1_round(f32_toward_zero(Fraction(v) * Fraction(r))) for v in grp]
    return codes, scales


def _nv_place(writes, name, base, t, codes, scales, swizzled):
    """Bytes of one token's NVFP4 row in a 1152-byte slot at `base`."""
    for b in range(64):
        writes[(name, base + t * 64 + b)] = codes[2 * b] | (codes[2 * b + 1] << 4)
    for g in range(8):
        # the epilogue page's formula for the V-swizzled scale byte h of token t
        off = (t // 4 * 4 + g // 2) * 8 + g % 2 * 4 + t % 4 if swizzled else 8 * t + g
        writes[(name, base + 1024 + off)] = scales[g]


def _norm_row(vals, gam, eps):
    """Gemma RMSNorm of a row (float64, fsum)."""
    ms = math.fsum(v * v for v in vals) / len(vals)
    r = 1.0 / math.sqrt(ms + eps)
    return [(v * r) * (1.0 + bf16_value(g)) for v, g in zip(vals, gam)]


def _scale(vals):
    amax = max(abs(v) for v in vals)
    return 1.0 if amax == 0.0 else f32(amax / 448.0)


def run(inp, mode: str):
    """The prologue on a tiny input dict (same keys as synth workloads).

    Returns a dict with h_out, q_out, iq_out (nested lists of bf16 bits) and the
    final caches as flat Python lists / dicts of written bytes. Optional inputs:
    static_kv_scale (K and V with the unit scale, the pre_attn page's
    STATIC_KV_SCALE) and q_fp8_scale (adds q_fp8: E4M3 codes of the float32
    product of q and the float32 reciprocal of the scale, the epilogue page's
    q_fp8_out)."""
    static = bool(inp.get("static_kv_scale", False))
    nvfp4 = inp.get("kv_format", "fp8") == "nvfp4"
    if nvfp4:
        gk = f32(1.0 / f32(float(inp["k_global_scale"])))
        gv = f32(1.0 / f32(float(inp["v_global_scale"])))
    qs = inp.get("q_fp8_scale")
    q_inv = None if qs is None else f32(1.0 / f32(float(qs)))
    q_fp8 = []
    S, K = inp["ar"].shape
    nkv = int(inp["nkv"])
    eps = float(inp["eps"])
    ar = inp["ar"].tolist()
    rs = inp["res"].tolist()
    gin = inp["g_in"].tolist()
    w = inp["w"].tolist()
    n_heads = 19 * nkv + 1
    N = n_heads * HEAD_DIM
    h_out, q_out, iq_out = [], [], []
    writes = {}  # (array name, flat index) -> value
    for s in range(S):
        acc = [f32(bf16_value(a) + bf16_value(b)) for a, b in zip(ar[s], rs[s])]
        h_out.append([bf16_round_bits(a) for a in acc])
        xn = _norm_row(acc, gin, eps)
        if mode == "decode":
            sx = _scale(xn)
            codes = [e4m3_round(v / sx) for v in xn]
            y = []
            for n in range(N):
                # exact: every code value is an integer multiple of 2^-9
                tot = sum(int(E4M3[c] * 512) * int(E4M3[wc] * 512)
                          for c, wc in zip(codes, w[n]))
                y.append((tot / 2.0**18 * sx) * float(inp["w_scale"][n]))
        else:
            xv = []
            for b in range(K // 32):
                blk = xn[32 * b: 32 * b + 32]
                amax = max(abs(v) for v in blk)
                if amax == 0.0:
                    e = 0
                else:
                    e = math.floor(math.log2(amax))
                    # guard log2 rounding at exact powers of two
                    while 2.0 ** e > amax:
                        e -= 1
                    while 2.0 ** (e + 1) <= amax:
                        e += 1
                    e -= 8
                for v in blk:
                    xv.append(Fraction(E4M3[e4m3_round(v / 2.0 ** e)]) * Fraction(2) ** e)
            y = []
            for n in range(N):
                tot = Fraction(0)
                for k in range(K):
                    ws = Fraction(2) ** (int(inp["w_e8m0"][n][k // 32]) - 127)
                    tot += xv[k] * E4M3[w[n][k]] * ws
                y.append(float(tot))
        pos = int(inp["positions"][s])
        cos = [bf16_value(int(inp["cos_sin"][pos][i])) for i in range(32)]
        sin = [bf16_value(int(inp["cos_sin"][pos][32 + i])) for i in range(32)]

        def head(h, gname):
            vals = y[h * HEAD_DIM:(h + 1) * HEAD_DIM]
            n_ = _norm_row(vals, inp[gname].tolist(), eps)
            o = list(n_)
            for i in range(32):
                o[i] = n_[i] * cos[i] - n_[i + 32] * sin[i]
                o[i + 32] = n_[i + 32] * cos[i] + n_[i] * sin[i]
            return o

        q_heads = [head(h, "g_q") for h in range(16 * nkv)]
        q_out.append([[bf16_round_bits(f32(v)) for v in o] for o in q_heads])
        if q_inv is not None:
            # product of two float32 values: exact in a double, then one rounding
            q_fp8.append([[e4m3_round(f32(f32(v) * q_inv)) for v in o] for o in q_heads])
        iq_out.append([[bf16_round_bits(f32(v)) for v in head(18 * nkv + j, "g_iq")]
                       for j in range(nkv)])
        slot = int(inp["slot_mapping"][s])
        pages = (inp["kv_cache"] if nvfp4 else inp["k_cache"]).shape[0]
        if slot < 0 or slot >= 16 * pages:  # outside the cache: no write, like -1
            continue
        page, t = slot // 16, slot % 16
        if nvfp4:
            for j in range(nkv):
                ok = head(16 * nkv + j, "g_k")
                yv = y[(17 * nkv + j) * HEAD_DIM:(17 * nkv + j + 1) * HEAD_DIM]
                kc, ksc = nvfp4_row([f32(v) for v in ok], gk)
                vc, vsc = nvfp4_row([f32(v) for v in yv], gv)
                _nv_place(writes, "kv_cache", (page * 2 * nkv + 2 * j) * 1152, t, kc, ksc, False)
                _nv_place(writes, "kv_cache", (page * 2 * nkv + 2 * j + 1) * 1152, t, vc, vsc, True)
            ic, isc = nvfp4_row([f32(v) for v in head(19 * nkv, "g_ik")], None)
            _nv_place(writes, "index_cache", page * 1152, t, ic, isc, False)
            continue
        for j in range(nkv):
            ok = head(16 * nkv + j, "g_k")
            yv = y[(17 * nkv + j) * HEAD_DIM:(17 * nkv + j + 1) * HEAD_DIM]
            ks = 1.0 if static else _scale(ok)
            vs = 1.0 if static else _scale(yv)
            writes[("k_scale", (page * nkv + j) * 16 + t)] = ks
            writes[("v_scale", (page * nkv + j) * 16 + t)] = vs
            base = (page * nkv + j) * 2048
            for d in range(HEAD_DIM):
                # K "shuffle": 16-dim groups of 16 rows x 16 bytes; V: dim-major
                writes[("k_cache", base + (d // 16) * 256 + t * 16 + d % 16)] = \
                    e4m3_round(ok[d] / ks)
                writes[("v_cache", base + d * 16 + t)] = e4m3_round(yv[d] / vs)
        oik = head(19 * nkv, "g_ik")
        for d in range(HEAD_DIM):
            writes[("index_cache", slot * HEAD_DIM + d)] = e4m3_round(oik[d])
    return {"h_out": h_out, "q_out": q_out, "iq_out": iq_out, "q_fp8": q_fp8, "writes": writes}
