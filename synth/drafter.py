"""Seeded synthetic inputs for the DSpark drafter's attention (one call).

Drawn from ``numpy.random.default_rng(seed)`` in a fixed order: sequence
lengths, q / k / v rows, norm weights, the cache contents, the block tables.
Conversions of random draws to bf16 / E4M3 use torch's casts; nothing here
computes any step of the attention.

Layouts (raw bits in numpy, T = 7 R query rows):
  q            uint16 (bf16 bits) [T, 16, 128]
  k, v         uint16             [T, 128]      the rows' new key and value
  qn, kn       uint16             [128]         head norm weights
  cos_sin      uint16             [max_pos, 64] cos | sin
  positions    int64              [T]           request r's rows: seq_len - 7 .. seq_len - 1
  slots        int64              [T]           cache slot of each row's new key (-1: none)
  kv_cache     uint8              [num_blocks, 128, 256]  K codes | V codes per key
  block_table  int32              [R, width]    physical block of each logical block
  seq_lens     int32              [R]
"""

from __future__ import annotations

import numpy as np

from .inputs import _bf16_bits, _e4m3_codes, _rope_table

QPR = 7
HEADS = 16
HEAD_DIM = 128
BLOCK = 128


def make_drafter(requests: int, max_seq: int, seed: int = 0, split: int = 4, min_seq: int = QPR,
                 seq_lens=None, eps: float = 1e-6) -> dict:
    """One drafter attention call: `requests` requests with seq_len ~ U[min_seq,
    max_seq] (or the given seq_lens), each owning distinct physical blocks in a
    shuffled order; every cache byte holds a finite E4M3 code."""
    rng = np.random.default_rng(seed)
    R = requests
    if seq_lens is None:
        seq_lens = rng.integers(min_seq, max_seq + 1, size=R)
    seq_lens = np.asarray(seq_lens, np.int64)
    if seq_lens.min() < QPR:
        raise ValueError("a request holds its 7 draft rows")
    T = R * QPR
    q = _bf16_bits(rng.standard_normal((T, HEADS, HEAD_DIM), dtype=np.float32))
    k = _bf16_bits(rng.standard_normal((T, HEAD_DIM), dtype=np.float32))
    v = _bf16_bits(rng.standard_normal((T, HEAD_DIM), dtype=np.float32))
    qn = _bf16_bits(rng.normal(0.0, 0.1, size=HEAD_DIM))
    kn = _bf16_bits(rng.normal(0.0, 0.1, size=HEAD_DIM))
    width = int(-(-seq_lens.max() // BLOCK))
    nblk = R * width
    # the cache: K and V codes of N(0,1) draws (history keys), never NaN
    kv = _e4m3_codes(np.clip(rng.standard_normal((nblk, BLOCK, 2 * HEAD_DIM), dtype=np.float32), -440, 440))
    perm = rng.permutation(nblk).astype(np.int32)
    block_table = perm.reshape(R, width)
    pos = np.concatenate([np.arange(s - QPR, s) for s in seq_lens]).astype(np.int64)
    req = np.repeat(np.arange(R), QPR)
    slots = (block_table[req, pos // BLOCK].astype(np.int64) * BLOCK + pos % BLOCK).astype(np.int64)
    max_pos = int(seq_lens.max())
    return {
        "requests": R, "split": int(split), "eps": np.float32(eps),
        "q": q, "k": k, "v": v, "qn": qn, "kn": kn, "cos_sin": _rope_table(max_pos),
        "positions": pos, "slots": slots, "kv_cache": kv, "block_table": block_table,
        "seq_lens": seq_lens.astype(np.int32),
    }
