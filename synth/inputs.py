"""Seeded synthetic inputs for the prologue, one recipe per workload.

Every array is drawn from ``numpy.random.default_rng(seed)`` in a fixed order
(activations, outliers, gammas, weight codes, weight scales, request layout), so
one (workload, seed) pair always yields the same bytes. Conversions of random
draws to bf16 / E4M3 use torch's casts; nothing here computes any step of the
prologue itself.

Layouts (all row-major, raw bits in numpy):
  ar, res        uint16 (bf16 bits)  [S, K]
  g_in           uint16              [K]
  g_q/g_k/g_iq/g_ik uint16           [128]
  w              uint8  (E4M3 codes) [N, K], N = (19 nkv + 1) * 128, head order
                 q x 16nkv | k x nkv | v x nkv | index_q x nkv | index_k x 1
  w_scale        float32             [N]        (decode: per output row)
  w_e8m0         uint8               [N, K/32]  (prefill: per 32-k block)
  cos_sin        uint16              [max_pos, 64]  cos | sin
  positions      int64               [S]
  slot_mapping   int64               [S]   (-1 = no cache write)
  k_cache/v_cache uint8              [num_pages, nkv, 2048]
  k_scale/v_scale float32            [num_pages, nkv, 16]
  index_cache    uint8               [num_pages * 16, 128]
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

HEAD_DIM = 128
ROTARY_DIM = 64
PAGE = 16
PAGE_BYTES = PAGE * HEAD_DIM

# cache bytes no store ever produces: E4M3 0x7F is NaN
SENTINEL_CACHE_BYTE = 0x7F
# a quiet-NaN payload for the scale arrays
SENTINEL_SCALE_BITS = 0x7FC0DEAD


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and request layout of one synthetic prologue call."""

    name: str
    mode: str  # "decode" (per-token FP8) or "prefill" (MXFP8)
    tokens: int
    hidden: int
    nkv: int
    max_pos: int
    num_pages: int
    # "random": uniform positions, slots from a permutation of all slots
    # "decode": `requests` requests of q_len rows at the end of a random history
    # "prefill": `requests` requests of tokens/requests rows from position 0
    layout: str = "random"
    requests: int = 1
    q_len: int = 1
    outlier_frac: float = 0.0
    outlier_mult: float = 50.0
    skip_frac: float = 0.0  # fraction of tokens whose slot is -1
    # fraction of tokens whose slot lies at or past the cache's end (outside the
    # caller's precondition; such a token writes no cache byte)
    oob_frac: float = 0.0
    eps: float = 1e-6

    @property
    def n_rows(self) -> int:
        return (19 * self.nkv + 1) * HEAD_DIM

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "c1": Workload("tiny_decode_s1_k1024_nkv1", "decode", 1, 1024, 1, 4096, 8, "random"),
    "c2": Workload(
        "decode_batch_s8_k6144_nkv1", "decode", 8, 6144, 1, 32768, 2048, "decode",
        requests=8, q_len=1,
    ),
    "c3": Workload(
        "spec_decode_s64_k6144_nkv2", "decode", 64, 6144, 2, 32768, 2048, "decode",
        requests=16, q_len=4, outlier_frac=0.01,
    ),
    "c4": Workload(
        "prefill_m2048_k6144_nkv2", "prefill", 2048, 6144, 2, 2048, 128, "prefill",
        requests=1,
    ),
    "c5": Workload(
        "prefill_m8192_k6144_nkv4", "prefill", 8192, 6144, 4, 2048, 512, "prefill",
        requests=4,
    ),
}


def named_config(key: str) -> Workload:
    return CONFIGS[key]


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _e4m3_codes(x: np.ndarray) -> np.ndarray:
    # torch's cast; callers keep |x| < 448 so no NaN codes appear
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _rope_table(max_pos: int) -> np.ndarray:
    # NeoX inverse frequencies with base 10000 over the 64 rotary dims
    i = np.arange(ROTARY_DIM // 2, dtype=np.float64)
    inv_freq = 10000.0 ** (-2.0 * i / ROTARY_DIM)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return _bf16_bits(np.concatenate([np.cos(ang), np.sin(ang)], axis=1))


def _request_layout(wl: Workload, rng: np.random.Generator):
    """positions [S] and slot_mapping [S] for the workload's request layout."""
    S = wl.tokens
    n_slots = wl.num_pages * PAGE
    if wl.layout == "random":
        pos = rng.integers(0, wl.max_pos, size=S)
        if S > n_slots:
            raise ValueError("more tokens than cache slots")
        slots = rng.permutation(n_slots)[:S]
        return pos.astype(np.int64), slots.astype(np.int64)
    if wl.layout == "decode":
        R, ql = wl.requests, wl.q_len
        if R * ql != S:
            raise ValueError("requests * q_len must equal tokens")
        seq = rng.integers(ql, wl.max_pos + 1, size=R)  # history length incl. new rows
        pages = rng.permutation(wl.num_pages)
        nxt = 0
        pos = np.empty(S, np.int64)
        slots = np.empty(S, np.int64)
        for r in range(R):
            table = {}
            for j in range(ql):
                p = int(seq[r]) - ql + j
                lp = p // PAGE
                if lp not in table:  # only touched logical pages get a physical page
                    table[lp] = int(pages[nxt])
                    nxt += 1
                pos[r * ql + j] = p
                slots[r * ql + j] = table[lp] * PAGE + p % PAGE
        return pos, slots
    if wl.layout == "prefill":
        R = wl.requests
        if S % R:
            raise ValueError("tokens must split evenly over requests")
        L = S // R
        lp_per_req = -(-L // PAGE)
        if R * lp_per_req > wl.num_pages:
            raise ValueError("cache too small for the requests")
        if L > wl.max_pos:
            raise ValueError("request longer than the RoPE table")
        perm = rng.permutation(wl.num_pages)
        pos = np.tile(np.arange(L, dtype=np.int64), R)
        req = np.repeat(np.arange(R), L)
        slots = perm[req * lp_per_req + pos // PAGE] * PAGE + pos % PAGE
        return pos, slots.astype(np.int64)
    raise ValueError(f"unknown layout {wl.layout!r}")


def make_workload(wl: Workload, seed: int = 0, weights: bool = True) -> dict:
    """All inputs of one prologue call (see the module docstring for layouts).

    ``weights=False`` skips the weight draws (callers that reuse a weight set).
    """
    if wl.hidden % 32:
        raise ValueError("hidden must be a multiple of 32 (the MX block)")
    rng = np.random.default_rng(seed)
    S, K, N = wl.tokens, wl.hidden, wl.n_rows
    ar = rng.standard_normal((S, K), dtype=np.float32)
    res = rng.standard_normal((S, K), dtype=np.float32)
    if wl.outlier_frac > 0:
        # a fraction of (token, channel) positions, both inputs scaled
        n_out = max(1, int(round(wl.outlier_frac * S * K)))
        idx = rng.choice(S * K, size=n_out, replace=False)
        ar.reshape(-1)[idx] *= wl.outlier_mult
        res.reshape(-1)[idx] *= wl.outlier_mult
    out = {
        "ar": _bf16_bits(ar),
        "res": _bf16_bits(res),
        "g_in": _bf16_bits(rng.normal(0.0, 0.1, size=K)),
    }
    for g in ("g_q", "g_k", "g_iq", "g_ik"):
        out[g] = _bf16_bits(rng.normal(0.0, 0.1, size=HEAD_DIM))
    if weights:
        if wl.mode == "decode":
            out["w"] = _e4m3_codes(rng.standard_normal((N, K), dtype=np.float32))
            out["w_scale"] = (rng.uniform(0.5, 1.5, size=N) / math.sqrt(K)).astype(
                np.float32
            )
        elif wl.mode == "prefill":
            # MXFP8 weight drawn directly as codes and block exponents: element
            # magnitudes ~128 codes, block scale 2^(e-127) near 1/(128 sqrt K)
            codes = rng.standard_normal((N, K), dtype=np.float32) * 128.0
            out["w"] = _e4m3_codes(np.clip(codes, -440.0, 440.0))
            e0 = int(round(127 - 7 - 0.5 * math.log2(K)))
            out["w_e8m0"] = (e0 - rng.integers(0, 2, size=(N, K // 32))).astype(np.uint8)
        else:
            raise ValueError(wl.mode)
    pos, slots = _request_layout(wl, rng)
    if wl.skip_frac > 0:
        n_skip = int(round(wl.skip_frac * S))
        slots[rng.choice(S, size=n_skip, replace=False)] = -1
    if wl.oob_frac > 0:
        n_slots = wl.num_pages * PAGE
        live = np.flatnonzero(slots >= 0)
        n_oob = max(1, int(round(wl.oob_frac * S)))
        pick = rng.choice(live, size=min(n_oob, len(live)), replace=False)
        past = np.array([n_slots, n_slots + PAGE - 1, n_slots + 16 * PAGE + 3, 1 << 40], np.int64)
        slots[pick] = past[np.arange(len(pick)) % len(past)]
    out["positions"] = pos
    out["slot_mapping"] = slots
    out["cos_sin"] = _rope_table(wl.max_pos)
    P = wl.num_pages
    out["k_cache"] = np.full((P, wl.nkv, PAGE_BYTES), SENTINEL_CACHE_BYTE, np.uint8)
    out["v_cache"] = np.full((P, wl.nkv, PAGE_BYTES), SENTINEL_CACHE_BYTE, np.uint8)
    sent = np.full((P, wl.nkv, PAGE), SENTINEL_SCALE_BITS, np.uint32).view(np.float32)
    out["k_scale"] = sent.copy()
    out["v_scale"] = sent.copy()
    out["index_cache"] = np.full((P * PAGE, HEAD_DIM), SENTINEL_CACHE_BYTE, np.uint8)
    out["eps"] = np.float32(wl.eps)
    out["nkv"] = wl.nkv
    out["mode"] = wl.mode
    return out


NV_SLOT_BYTES = PAGE * (HEAD_DIM // 2 + HEAD_DIM // 16)  # 16 tokens x (64 data + 8 scale bytes)


def with_nvfp4_caches(inp: dict, k_global_scale: float = 1.0, v_global_scale: float = 1.0) -> dict:
    """The same call with NVFP4 caches instead of the FP8 ones: kv_cache
    [pages, 2 nkv, 1152] and index_cache [pages, 1152], sentinel-filled, plus
    the K / V global (dequantization) scales."""
    out = {k: v for k, v in inp.items() if k not in ("k_cache", "v_cache", "k_scale", "v_scale",
                                                     "index_cache")}
    P = inp["k_cache"].shape[0]
    nkv = int(inp["nkv"])
    out["kv_format"] = "nvfp4"
    out["kv_cache"] = np.full((P, 2 * nkv, NV_SLOT_BYTES), SENTINEL_CACHE_BYTE, np.uint8)
    out["index_cache"] = np.full((P, NV_SLOT_BYTES), SENTINEL_CACHE_BYTE, np.uint8)
    out["k_global_scale"] = np.float32(k_global_scale)
    out["v_global_scale"] = np.float32(v_global_scale)
    return out
