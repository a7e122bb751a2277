"""The prologue's arithmetic, step by step, in float64 (float32 where the method
rounds in float32).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources. "pre_attn page" is the vLLM API page
``vllm.models.minimax_m3.amd.mono.kernels.pre_attn`` (K1 mono_pre); "epilogue
page" is ``vllm.models.minimax_m3.nvidia.ops.qkv_index_fused_epilogue``.

Per token (decode):
  a1  acc = f32(ar) + f32(res) in float32; the residual out is bf16(acc)
      (pre_attn page: module docstring; ``emit_pre_attn`` -> ``norm_quant``).
  a2  Gemma RMSNorm  xn = acc / sqrt(mean(acc^2) + eps) * (1 + g_in)
      (``norm_quant``; the epilogue page's ``_rms_norm`` writes the same form as
      n + n * w).
  a3  per-token FP8: s_x = amax / 448 (1 when amax == 0), x8 = E4M3(xn / s_x)
      with a true division (``norm_quant``).
  a4  y[n] = (sum_k x8[k] w8[n,k]) * s_x * s_w[n], the fused projection over the
      head list q x 16nkv | k x nkv | v x nkv | index_q x nkv | index_k x 1, each
      head 128 rows (the epilogue page's class docstring and the N-from-nkv rule
      of ``minimax_m3_qkv_index_fused_epilogue``). Nothing is rounded to bf16
      before the head step (the epilogue page's module docstring: the epilogue
      works on the float32 accumulator).
  a5  per head: Gemma RMSNorm over its 128 values, then NeoX RoPE on dims 0..63
      pairing dim i with i + 32 (``head_norm_rope``; ``_rms_norm``; ``_rope64``).
  a6  q and index_q out as bf16.
  a7  K: per-token scale max|o| / 448 (1 when 0), E4M3 codes into the page-16
      "shuffle" K layout (``emit_pre_attn`` head tasks, K branch).
  a8  V: the raw projection (no norm, no RoPE), same per-token scaling, into the
      transposed page-16 V layout (head tasks, V branch; the epilogue page's v
      branch also stores the raw accumulator).
  a9  index_k: E4M3 with unit scale into the index cache row of the slot.
  a10 slot -> (page = slot // 16, row = slot % 16); slot < 0 writes nothing
      (``page16_of`` at its default stride; slot -1 = skip in the epilogue page's
      argument list). A slot at or past the cache's end (num_pages * 16) is
      outside the caller's precondition; it is read like slot -1 and writes
      nothing, so no byte outside the caches is ever addressed.

Prefill replaces a3/a4 by MXFP8: per (row, 32-wide k block) an E8M0 scale
2^(floor(log2 amax) - 8) and E4M3 elements, and the block-scaled dot product.

Two variants of the head step, both optional inputs:
  static K/V scale  K and V take the unit scale instead of max / 448, and the
      scale entries hold 1.0 (the pre_attn page's STATIC_KV_SCALE config, in the
      K and V branches of the head tasks).
  FP8 q             besides (or instead of) bf16 q, the E4M3 code of the float32
      product q * inv, inv = float32(1 / q_fp8_scale), saturating at 448 (the
      epilogue page's q_fp8_out / q_fp8_scale, q branch: x * qfp8_inv cast to
      e4m3).

NVFP4 caches (the epilogue page's cache format; optional, inp["kv_format"] ==
"nvfp4"): K (normed + roped), V (raw) and index_k are quantized per 16-value
group instead of per token, as float32 values (``_nvfp4_quant32``):
  scale code  sf = E4M3(max(f32(f32(amax * f32(1/6)) * gs), 2^-9)), saturating
  elements    E2M1(RZ(v * f32(f32(1 / dec(sf)) * gs))), satfinite, and a code
              of magnitude zero loses its sign
with gs = f32(1 / global_scale) for K and V (k_scale / v_scale of the page's
argument list) and no gs for index_k. Layout (``_nvfp4_cache_views``): a page of
kv_cache holds 2 nkv slots (K of KV head j in slot 2j, V in 2j + 1), each of 16
tokens x 64 data bytes followed by 16 x 8 scale bytes; the index cache page holds
one such slot. Data byte b of a token holds elements 2b (low nibble) and 2b + 1
(high nibble). K and index_k scale bytes are linear (token t, group g at 8t + g
of the scale area); V scale bytes take the swizzled layout of that view.

Readings where the pages leave a point open (each also listed in the design
notes): the activation norm and the FP8 decisions that follow it are taken in
float64; eps is the float32 value the library receives; K and index_k are
quantized from the unrounded head output; MXFP8 follows the OCP MX rule; the
FP8 q code takes the float32 image of the head output times the float32
reciprocal, rounded once to E4M3.
"""

from __future__ import annotations

import numpy as np

from .codecs import (
    E4M3_MAX,
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    e8m0_decode,
    f32_mul_rz,
    f32_to_bf16_bits,
)

HEAD_DIM = 128
ROTARY_DIM = 64
PAGE = 16
MX_BLOCK = 32
NV_GROUP = 16
NV_SLOT_BYTES = PAGE * (HEAD_DIM // 2 + HEAD_DIM // NV_GROUP)  # 1152
NV_SF_OFF = PAGE * HEAD_DIM // 2  # scale area of a slot: 1024


def input_norm(ar, res, g_in, eps):
    """Steps a1-a2 for every row.

    Returns (h_out bf16 bits [S,K], acc float32 [S,K], xn float64 [S,K]).
    """
    acc = bf16_bits_to_f32(ar) + bf16_bits_to_f32(res)  # float32 add, one rounding
    h_out = f32_to_bf16_bits(acc)
    a = acc.astype(np.float64)
    K = a.shape[1]
    ms = (a * a).sum(axis=1) / K
    rstd = 1.0 / np.sqrt(ms + np.float64(np.float32(eps)))
    xn = (a * rstd[:, None]) * (1.0 + bf16_bits_to_f64(g_in))[None, :]
    return h_out, acc, xn


def quantize_per_token(xn):
    """Step a3 (decode): per-row scale amax/448 (1.0 if the row is all zero) as
    float32, and E4M3 codes of xn / scale. Returns (x8 uint8 [S,K], s_x f32 [S])."""
    amax = np.abs(xn).max(axis=1)
    s_x = np.where(amax == 0.0, np.float32(1.0), (amax / E4M3_MAX).astype(np.float32))
    s_x = s_x.astype(np.float32)
    x8 = e4m3_encode(xn / s_x.astype(np.float64)[:, None])
    return x8, s_x


def mxfp8_quantize(xn):
    """Step a3' (prefill): OCP MX quantization over 32-wide k blocks.

    Block scale X = 2^(floor(log2 amax_block) - 8) (8 = the largest E4M3
    exponent), stored as the E8M0 code; an all-zero block takes X = 1.
    Elements are E4M3(v / X), saturating. Returns (xq uint8 [M,K],
    xs uint8 [M,K/32]).
    """
    M, K = xn.shape
    blk = xn.reshape(M, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)  # amax = f * 2^ex, f in [0.5, 1): floor(log2) = ex - 1
    code = np.clip(ex.astype(np.int64) - 1 - 8 + 127, 0, 254)
    code = np.where(amax == 0.0, 127, code)
    X = e8m0_decode(code)
    xq = e4m3_encode(blk / X[:, :, None]).reshape(M, K)
    return xq, code.astype(np.uint8)


def project_decode(x8, s_x, w8, s_w):
    """Step a4 (decode): y = (x8 . w8) * s_x * s_w in float64.

    The code products are multiples of 2^-18 below 2^18 and K <= 2^13, so every
    partial sum is exact in float64 whatever the summation order."""
    acc = e4m3_decode(x8) @ e4m3_decode(w8).T
    return (acc * s_x.astype(np.float64)[:, None]) * s_w.astype(np.float64)[None, :]


def project_mxfp8(xq, xs, wq, ws):
    """Step a4 (prefill): y = sum over k of (xq_k 2^(ex_b-127)) (wq_k 2^(ew_b-127))."""
    xv = e4m3_decode(xq) * np.repeat(e8m0_decode(xs), MX_BLOCK, axis=1)
    wv = e4m3_decode(wq) * np.repeat(e8m0_decode(ws), MX_BLOCK, axis=1)
    return xv @ wv.T


def head_norm_rope(yh, g, cos, sin, eps):
    """Step a5 for rows of one head role.

    yh [T,128] float64, g [128] bf16 bits, cos/sin [T,32] float64.
    Returns (o, n): n the Gemma-normed head, o after NeoX RoPE on dims 0..63.
    """
    ms = (yh * yh).sum(axis=1) / HEAD_DIM
    r = 1.0 / np.sqrt(ms + np.float64(np.float32(eps)))
    n = (yh * r[:, None]) * (1.0 + bf16_bits_to_f64(g))[None, :]
    half = ROTARY_DIM // 2
    x1 = n[:, :half]
    x2 = n[:, half:ROTARY_DIM]
    o = n.copy()
    o[:, :half] = x1 * cos - x2 * sin
    o[:, half:ROTARY_DIM] = x2 * cos + x1 * sin
    return o, n


def _scaled_codes(v, static=False):
    """Per-row scale max|v| / 448 as float32 (1.0 for an all-zero row, and for
    every row with the static scale) and the E4M3 codes of v / scale (steps a7,
    a8)."""
    if static:
        return e4m3_encode(v), np.ones(v.shape[0], np.float32)
    amax = np.abs(v).max(axis=1)
    s = np.where(amax == 0.0, np.float32(1.0), (amax / E4M3_MAX).astype(np.float32))
    s = s.astype(np.float32)
    return e4m3_encode(v / s.astype(np.float64)[:, None]), s


def q_fp8_codes(o_q, q_fp8_scale):
    """FP8 q: E4M3 of float32(float32(o) * float32(1 / q_fp8_scale))."""
    inv = np.float32(np.float32(1.0) / np.float32(q_fp8_scale))
    x = o_q.astype(np.float32) * inv  # one float32 rounding of the product
    return e4m3_encode(x.astype(np.float64))


def nvfp4_quantize(v, gs=None):
    """NVFP4 of head rows v [T, 128] (float32 values): per 16-value group an
    E4M3 scale byte and 16 E2M1 codes, following the epilogue page's
    ``_nvfp4_quant32``. gs is float32(1 / global scale), or None (unit scale).

    Returns (data uint8 [T, 64], element 2b in the low nibble of byte b, and
    scale codes uint8 [T, 8]).
    """
    v = np.asarray(v, dtype=np.float32)
    T = v.shape[0]
    grp = v.reshape(T, HEAD_DIM // NV_GROUP, NV_GROUP)
    gmax = np.abs(grp).max(axis=2)  # exact
    a = gmax * np.float32(1.0 / 6.0)  # float32 product with the float32 constant
    if gs is not None:
        a = (a * np.float32(gs)).astype(np.float32)
    a = np.maximum(a, np.float32(2.0 ** -9))
    sf = e4m3_encode(a.astype(np.float64))  # nearest even, saturating at 448
    sfv = e4m3_decode(sf).astype(np.float32)  # exact
    r = (np.float32(1.0) / sfv).astype(np.float32)  # correctly rounded reciprocal
    if gs is not None:
        r = (r * np.float32(gs)).astype(np.float32)
    q = f32_mul_rz(grp, r[:, :, None])
    codes = e2m1_encode(q.astype(np.float64)).reshape(T, HEAD_DIM)
    codes = np.where((codes & 0x7) == 0, 0, codes).astype(np.uint8)  # no -0
    data = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return data, sf


def nvfp4_scale_offset(t, g, swizzled):
    """Byte offset, inside a slot's scale area, of token t's group-g scale.

    Linear: [8 groups, 16 tokens] with strides (1, 8). V-swizzled: the view of
    shape ((2, 4), (4, 4)) with strides ((4, 8), (1, 32)) over (group, token),
    i.e. group g = g0 + 2 g1 and token t = t0 + 4 t1 sit at
    4 g0 + 8 g1 + t0 + 32 t1 (the epilogue page's ``_nvfp4_cache_views``).
    """
    if not swizzled:
        return 8 * t + g
    g0, g1 = g % 2, g // 2
    t0, t1 = t % 4, t // 4
    return 4 * g0 + 8 * g1 + 1 * t0 + 32 * t1


def _nvfp4_insert(out, inp, o_k, y_v, o_ik):
    """Steps a7-a9 with the NVFP4 caches (kv_cache [P, 2 nkv, 1152] and
    index_cache [P, 1152])."""
    S, nkv = o_k.shape[0], o_k.shape[1]
    gk = np.float32(np.float32(1.0) / np.float32(inp.get("k_global_scale", 1.0)))
    gv = np.float32(np.float32(1.0) / np.float32(inp.get("v_global_scale", 1.0)))
    kd, ks = nvfp4_quantize(o_k.reshape(S * nkv, HEAD_DIM).astype(np.float32), gk)
    vd, vs = nvfp4_quantize(y_v.reshape(S * nkv, HEAD_DIM).astype(np.float32), gv)
    idd, ids = nvfp4_quantize(o_ik.astype(np.float32), None)
    kd, ks = kd.reshape(S, nkv, -1), ks.reshape(S, nkv, -1)
    vd, vs = vd.reshape(S, nkv, -1), vs.reshape(S, nkv, -1)
    kv = inp["kv_cache"].copy()
    ic = inp["index_cache"].copy()
    slots = np.asarray(inp["slot_mapping"], np.int64)
    P = kv.shape[0]
    for s in range(S):
        slot = int(slots[s])
        if slot < 0 or slot >= P * PAGE:
            continue
        page, t = slot // PAGE, slot % PAGE
        for j in range(nkv):
            for sl, data, sc, swz in ((2 * j, kd[s, j], ks[s, j], False), (2 * j + 1, vd[s, j], vs[s, j], True)):
                kv[page, sl, t * 64:(t + 1) * 64] = data
                for g in range(8):
                    kv[page, sl, NV_SF_OFF + nvfp4_scale_offset(t, g, swz)] = sc[g]
        ic[page, t * 64:(t + 1) * 64] = idd[s]
        for g in range(8):
            ic[page, NV_SF_OFF + nvfp4_scale_offset(t, g, False)] = ids[s, g]
    out.update(kv_cache=kv, index_cache=ic, k_nv=(kd, ks), v_nv=(vd, vs), ik_nv=(idd, ids))
    return out


def _epilogue(y, inp):
    """Steps a5-a10 on the float64 projection y [S, N]."""
    nkv = int(inp["nkv"])
    eps = inp["eps"]
    S = y.shape[0]
    heads = y.reshape(S, 19 * nkv + 1, HEAD_DIM)
    k0, v0, iq0, ik0 = 16 * nkv, 17 * nkv, 18 * nkv, 19 * nkv
    pos = np.asarray(inp["positions"], np.int64)
    cs = bf16_bits_to_f64(inp["cos_sin"][pos])
    cos, sin = cs[:, :32], cs[:, 32:64]

    def roped(h0, h1, g):
        hs = heads[:, h0:h1, :]
        T = h1 - h0
        o, _ = head_norm_rope(
            hs.reshape(S * T, HEAD_DIM), g,
            np.repeat(cos, T, axis=0), np.repeat(sin, T, axis=0), eps,
        )
        return o.reshape(S, T, HEAD_DIM)

    o_q = roped(0, k0, inp["g_q"])
    o_k = roped(k0, v0, inp["g_k"])
    o_iq = roped(iq0, ik0, inp["g_iq"])
    o_ik = roped(ik0, ik0 + 1, inp["g_ik"])[:, 0, :]
    y_v = heads[:, v0:iq0, :]

    out = {
        "q_out": f32_to_bf16_bits(o_q.astype(np.float32)),
        "iq_out": f32_to_bf16_bits(o_iq.astype(np.float32)),
    }
    if inp.get("q_fp8_scale") is not None:
        out["q_fp8"] = q_fp8_codes(o_q, inp["q_fp8_scale"])
    if inp.get("kv_format", "fp8") == "nvfp4":
        return _nvfp4_insert(out, inp, o_k, y_v, o_ik)
    static = bool(inp.get("static_kv_scale", False))
    k_codes, k_s = _scaled_codes(o_k.reshape(S * nkv, HEAD_DIM), static)
    v_codes, v_s = _scaled_codes(y_v.reshape(S * nkv, HEAD_DIM), static)
    k_codes = k_codes.reshape(S, nkv, HEAD_DIM)
    v_codes = v_codes.reshape(S, nkv, HEAD_DIM)
    k_s = k_s.reshape(S, nkv)
    v_s = v_s.reshape(S, nkv)
    ik_codes = e4m3_encode(o_ik)
    out.update(k_codes=k_codes, v_codes=v_codes, k_s=k_s, v_s=v_s, ik_codes=ik_codes)

    k_cache = inp["k_cache"].copy()
    v_cache = inp["v_cache"].copy()
    k_scale = inp["k_scale"].copy()
    v_scale = inp["v_scale"].copy()
    index_cache = inp["index_cache"].copy()
    slots = np.asarray(inp["slot_mapping"], np.int64)
    d = np.arange(HEAD_DIM)
    k_off = (d // 16) * (PAGE * 16) + d % 16  # + row * 16
    v_off = d * PAGE  # + row
    P = k_cache.shape[0]
    for s in range(S):
        slot = int(slots[s])
        if slot < 0 or slot >= P * PAGE:  # a slot outside the cache writes nothing, as slot -1
            continue
        page, row = slot // PAGE, slot % PAGE
        for j in range(nkv):
            k_cache[page, j, k_off + row * 16] = k_codes[s, j]
            v_cache[page, j, v_off + row] = v_codes[s, j]
            k_scale[page, j, row] = k_s[s, j]
            v_scale[page, j, row] = v_s[s, j]
        index_cache[slot, :] = ik_codes[s]
    out.update(
        k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale,
        index_cache=index_cache,
    )
    return out


def decode(inp):
    """The whole decode prologue (per-token FP8) on an input dict from ``synth``.

    Returns h_out, q_out [S,16nkv,128], iq_out [S,nkv,128] (bf16 bits), the
    updated caches and scale arrays, and the intermediates x8, s_x, y.
    """
    h_out, _, xn = input_norm(inp["ar"], inp["res"], inp["g_in"], inp["eps"])
    x8, s_x = quantize_per_token(xn)
    y = project_decode(x8, s_x, inp["w"], inp["w_scale"])
    out = _epilogue(y, inp)
    out.update(h_out=h_out, x8=x8, s_x=s_x, y=y)
    return out


def prefill(inp):
    """The whole prefill prologue (MXFP8 activations and weight).

    Same outputs as ``decode``, with the intermediates xq, xs, y.
    """
    h_out, _, xn = input_norm(inp["ar"], inp["res"], inp["g_in"], inp["eps"])
    xq, xs = mxfp8_quantize(xn)
    y = project_mxfp8(xq, xs, inp["w"], inp["w_e8m0"])
    out = _epilogue(y, inp)
    out.update(h_out=h_out, xq=xq, xs=xs, y=y)
    return out
