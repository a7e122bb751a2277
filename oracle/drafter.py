"""Attention of the DSpark drafter, step by step, in float64 (the method's own
rounding points kept: FP8 q / k / v / P, bf16 output, MXFP8 output).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the vLLM API page ``vllm.models.minimax_m3.amd.mono.drafter.attention``
("drafter page"): its module docstring, ``window``, ``kv_load``, ``block_math``,
``block_acc``, ``qkv_rows`` / ``qkv_pre`` and the ``merge_task`` and
``store_partial`` attributes.

What one call computes, per request r of R (each with QPR = 7 query rows):

  d1 qkv rows (``qkv_rows``): each of the 16 q heads of a row and the row's
     new k get the head RMSNorm and NeoX RoPE on the first 64 dims (the
     cos | sin table row of the row's position) and are cast to E4M3; the
     row's new v is cast to E4M3. The new k and v codes are written into the
     paged cache at the row's slot (block slot // 128, key slot % 128), K in
     bytes 0..127 of the key's 256-byte entry and V in bytes 128..255
     (``kv_load``'s K and V words).
  d2 window (``window``): p0 = the position of the request's first row;
     lo = max(p0 - 4095, 0); hi = min(seq_len - 1, (lo // 128 + MAXB) * 128 - 1);
     the request reads the blocks lo // 128 .. hi // 128 of its block table.
     Key kp is visible to row j (position qp_j) iff kp > qp_j - 4096,
     kp >= lo and kp <= hi (``block_math``'s mask): no causal mask among the
     7 rows (the module docstring: non-causal within a request's 7 rows).
  d3 split-KV partitions: the blocks are cut into partitions of `split`
     consecutive blocks each (the last may be shorter). In a partition, each
     (row, head) runs the online softmax block by block in order
     (``block_math`` for the first block, ``block_acc`` after it):
        s_k   = q8 . k8_k, the dot product of the decoded E4M3 values (raw units)
        m'    = max(m, max over visible keys of s_k)   (m starts at -inf)
        ms    = 0 if m' = -inf else m'
        alpha = 2^((m - ms) C),  C = log2(e) / sqrt(128)
        p_k   = 2^(s_k C - (ms C - 8))   (= 256 exp((s_k - m') / sqrt(128)); 0 if hidden)
        l     = l alpha + sum_k p_k              (p before its FP8 rounding)
        o     = o alpha + sum_k E4M3(p_k) v8_k   (P in e4m3, the FP8 PV)
     giving the partial (m, l, o); l and o carry the factor 256.
  d4 merge (``merge_task``): per (row, head) the partials are merged in order:
     M = max_i m_i, w_i = 2^((m_i - M) C), out = (sum_i w_i o_i) / (sum_i w_i l_i),
     rounded to bf16 and quantized to MXFP8 (E8M0 scale per 32 values of the
     row's 16 x 128 output, OCP MX rule as the prologue's prefill activations).

Readings where the page is silent (each also listed in the design notes):
  - the head norm is the Gemma form of the prologue's head_norm_rope
    (x / rms * (1 + g), one eps), and RoPE is its partial NeoX rotation of dims
    0..63 with the cos | sin table rows;
  - q, k, v and P are E4M3 with unit scales (saturating at 448): the page's
    score is q . k / sqrt(128) with no other factor, and P's only factor is 256;
  - MAXB = 34 blocks, enough for the union of the 7 rows' windows (4102 keys)
    at any alignment, so hi is seq_len - 1 whenever the window allows;
  - the partition size `split` (blocks per partition) is a parameter of the
    call: FP8 P is rounded relative to each partition's running maximum, so
    the result depends on it, and both sides take the same value;
  - a (row, head) that sees no key at all (every partial's m is -inf) outputs
    zeros (the page's msafe keeps exp2 finite; the division has no other
    reading).
"""

from __future__ import annotations

import math

import numpy as np

from .codecs import bf16_bits_to_f64, e4m3_decode, e4m3_encode, f32_to_bf16_bits
from .prologue import head_norm_rope, mxfp8_quantize

QPR = 7          # query rows per request
HEADS = 16       # q heads per row (one KV head)
HEAD_DIM = 128
BLOCK = 128      # keys per cache block
KEY_BYTES = 256  # K (128 E4M3) | V (128 E4M3)
WINDOW = 4096
MAXB = 34
ROTARY_DIM = 64
C = math.log2(math.e) / math.sqrt(HEAD_DIM)


def qkv_rows(q, k, v, qn, kn, cos_sin, positions, eps):
    """Step d1 without the cache write: (q8 [T,16,128], k8 [T,128], v8 [T,128])
    E4M3 codes from bf16 bits q [T,16,128], k [T,128], v [T,128]."""
    T = q.shape[0]
    pos = np.asarray(positions, np.int64)
    cs = bf16_bits_to_f64(cos_sin[pos])
    cos, sin = cs[:, :32], cs[:, 32:64]
    qf = bf16_bits_to_f64(q).reshape(T * HEADS, HEAD_DIM)
    qo, _ = head_norm_rope(qf, qn, np.repeat(cos, HEADS, axis=0), np.repeat(sin, HEADS, axis=0), eps)
    ko, _ = head_norm_rope(bf16_bits_to_f64(k), kn, cos, sin, eps)
    return (e4m3_encode(qo).reshape(T, HEADS, HEAD_DIM), e4m3_encode(ko),
            e4m3_encode(bf16_bits_to_f64(v)))


def insert_kv(cache, k8, v8, slots):
    """Step d1's cache write: a new copy of `cache` [num_blocks, 128, 256] with
    each row's codes at its slot (slot < 0, or past the cache: no write)."""
    out = cache.copy()
    nb = cache.shape[0]
    for t, slot in enumerate(np.asarray(slots, np.int64)):
        if slot < 0 or slot >= nb * BLOCK:
            continue
        out[slot // BLOCK, slot % BLOCK, :HEAD_DIM] = k8[t]
        out[slot // BLOCK, slot % BLOCK, HEAD_DIM:] = v8[t]
    return out


def window(p0, seq_len):
    """Step d2: (lo, hi, first block, last block) of a request."""
    lo = max(p0 - (WINDOW - 1), 0)
    hi = min(seq_len - 1, (lo // BLOCK + MAXB) * BLOCK - 1)
    return lo, hi, lo // BLOCK, hi // BLOCK


def gather_keys(cache, block_table_row, blk):
    """Logical block blk of a request: (k8 [128,128], v8 [128,128]) codes.
    The block index is clamped to the table row and the physical block to the
    cache (``kv_load`` keeps every address inside them)."""
    bt = np.asarray(block_table_row)
    col = min(max(blk, 0), len(bt) - 1)
    phys = min(max(int(bt[col]), 0), cache.shape[0] - 1)
    return cache[phys, :, :HEAD_DIM], cache[phys, :, HEAD_DIM:]


def partial(q8h, qp, lo, hi, blocks, cache, bt_row, p_fp8=True):
    """Step d3 for the heads of one row over one partition's blocks, in order.

    q8h [H, 128] codes (the row's heads), qp the row's position. Returns
    (m [H], l [H], o [H, 128]); m in raw score units, l and o scaled by 256.
    With p_fp8=False P keeps its exact value in the PV product (for the
    closed-form check only)."""
    q = e4m3_decode(q8h)
    H = q.shape[0]
    m, l, o = np.full(H, -math.inf), np.zeros(H), np.zeros((H, HEAD_DIM))
    for blk in blocks:
        k8, v8 = gather_keys(cache, bt_row, blk)
        kp = blk * BLOCK + np.arange(BLOCK)
        vis = ((kp > qp - WINDOW) & (kp >= lo) & (kp <= hi))[None, :]
        s = np.where(vis, q @ e4m3_decode(k8).T, -math.inf)  # [H, keys]
        mn = np.maximum(m, s.max(axis=1))
        ms = np.where(mn == -math.inf, 0.0, mn)
        alpha = 2.0 ** ((m - ms) * C)
        p = np.where(vis, 2.0 ** (s * C - (ms * C - 8.0)[:, None]), 0.0)
        pq = e4m3_decode(e4m3_encode(p)) if p_fp8 else p
        l = l * alpha + p.sum(axis=1)
        o = o * alpha[:, None] + pq @ e4m3_decode(v8)
        m = mn
    return m, l, o


def merge(parts):
    """Step d4 before rounding: parts [(m [H], l [H], o [H,128])] in order ->
    out [H, 128] (float64); zeros for a head no partition saw a key for."""
    M = np.max([m for m, _, _ in parts], axis=0)
    H = M.shape[0]
    L, O = np.zeros(H), np.zeros((H, HEAD_DIM))
    Ms = np.where(M == -math.inf, 0.0, M)
    for m, l, o in parts:
        w = 2.0 ** ((m - Ms) * C)
        L += w * l
        O = O + w[:, None] * o
    safe = np.where(L > 0, L, 1.0)
    return np.where((M == -math.inf)[:, None], 0.0, O / safe[:, None])


def attention(inp, p_fp8=True):
    """The whole drafter attention call on an input dict (see synth.drafter).

    Returns out_bf16 bits [T,16,128], out codes [T,2048] and scales [T,64]
    (MXFP8), the updated cache, q8/k8/v8, and out (f64, before rounding)."""
    R = int(inp["requests"])
    split = int(inp["split"])
    q8, k8, v8 = qkv_rows(inp["q"], inp["k"], inp["v"], inp["qn"], inp["kn"], inp["cos_sin"],
                          inp["positions"], inp["eps"])
    cache = insert_kv(inp["kv_cache"], k8, v8, inp["slots"])
    pos = np.asarray(inp["positions"], np.int64)
    T = R * QPR
    out = np.zeros((T, HEADS, HEAD_DIM))
    for r in range(R):
        lo, hi, b0, b1 = window(int(pos[r * QPR]), int(inp["seq_lens"][r]))
        blocks = list(range(b0, b1 + 1))
        parts_of = [blocks[i:i + split] for i in range(0, len(blocks), split)]
        bt = inp["block_table"][r]
        for j in range(QPR):
            t = r * QPR + j
            parts = [partial(q8[t], int(pos[t]), lo, hi, pb, cache, bt, p_fp8) for pb in parts_of]
            out[t] = merge(parts)
    out_bf16 = f32_to_bf16_bits(out.astype(np.float32))
    codes, scales = mxfp8_quantize(bf16_bits_to_f64(out_bf16).reshape(T, HEADS * HEAD_DIM))
    return {"out_bf16": out_bf16, "out_codes": codes, "out_scales": scales, "kv_cache": cache,
            "q8": q8, "k8": k8, "v8": v8, "out": out}
