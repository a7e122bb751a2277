"""Pins of the drafter attention oracle (oracle/drafter.py) against what the
drafter page and the mathematics fix: textbook softmax attention (the online
softmax, its rescaling and the partition merge are exact rewrites of it once P
keeps its exact value), the window rule restated per key, a scalar statement of
one block with P in e4m3, the e4m3 rounding bound on the whole output, the
cache insert's bytes, and planted mistakes that each of these must catch."""

import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth
from oracle import drafter as D
from oracle.codecs import bf16_bits_to_f64, e4m3_decode, e4m3_encode


def _case(R=3, max_seq=9000, seed=3, split=4, **kw):
    return synth.make_drafter(R, max_seq, seed=seed, split=split, **kw)


def _textbook(inp, q8, cache):
    """softmax(q . k / sqrt(128)) v over each row's visible keys, gathered key
    by key through the block table: the definition, with exact P."""
    R = inp["requests"]
    out = np.zeros((R * 7, 16, 128))
    pos = inp["positions"]
    for r in range(R):
        seq = int(inp["seq_lens"][r])
        p0 = int(pos[7 * r])
        first = max(p0 - 4095, 0)
        for j in range(7):
            t = 7 * r + j
            keys = [kp for kp in range(first, seq) if kp > pos[t] - 4096]
            kk, vv = [], []
            for kp in keys:
                phys = inp["block_table"][r][kp // 128]
                kk.append(cache[phys, kp % 128, :128])
                vv.append(cache[phys, kp % 128, 128:])
            K = e4m3_decode(np.array(kk))
            V = e4m3_decode(np.array(vv))
            s = e4m3_decode(q8[t]) @ K.T / math.sqrt(128)  # [16, keys]
            out[t] = softmax(s, axis=1) @ V
    return out


def test_exact_p_is_textbook_softmax_attention_for_any_split():
    # with P kept exact, the online softmax over blocks and the merge of the
    # partitions are exact rewrites of softmax attention: every split agrees
    inp = _case(R=3, max_seq=9000, seed=5)
    assert inp["seq_lens"].max() > 4200  # the sliding window bites
    ref = None
    for split in (1, 3, 34):
        got = D.attention(dict(inp, split=split), p_fp8=False)
        if ref is None:
            ref = _textbook(inp, got["q8"], got["kv_cache"])
        np.testing.assert_allclose(got["out"], ref, rtol=1e-10, atol=1e-12)


def test_short_requests_see_every_key_noncausally():
    # seq_len <= 4096: every row sees keys 0 .. seq_len - 1, its later draft
    # rows included (no causal mask among the 7 rows)
    inp = _case(R=2, max_seq=300, seed=7, seq_lens=[7, 300])
    got = D.attention(inp, p_fp8=False)
    for r, seq in enumerate(inp["seq_lens"]):
        lo, hi, b0, b1 = D.window(int(inp["positions"][7 * r]), int(seq))
        assert (lo, hi) == (0, seq - 1) and b0 == 0 and b1 == (seq - 1) // 128
    np.testing.assert_allclose(got["out"], _textbook(inp, got["q8"], got["kv_cache"]), rtol=1e-10, atol=1e-12)


def test_window_rule_per_key():
    # the docstring's semantics: a row at position qp sees the 4096 most recent
    # keys up to itself (fewer near the start) and every later key below
    # seq_len (the other draft rows): min(qp + 1, 4096) + (seq_len - 1 - qp)
    for p0, seq in ((0, 7), (100, 107), (4089, 4096), (4090, 4097), (9000, 9007), (5000, 5007)):
        lo, hi, b0, b1 = D.window(p0, seq)
        assert hi == seq - 1  # MAXB never truncates a window
        for j in range(7):
            qp = p0 + j
            n_vis = sum(1 for kp in range(b0 * 128, (b1 + 1) * 128) if kp > qp - 4096 and kp >= lo and kp <= hi)
            assert n_vis == min(qp + 1, 4096) + (seq - 1 - qp)


def _one_block_scalar(q8h, k8, v8, n_keys):
    """A scalar statement of one 128-key block with P in e4m3 (keys n_keys..
    hidden): out = sum E4M3(256 exp((s - m)/sqrt128)) v / sum 256 exp(...)."""
    s = [sum(float(e4m3_decode(np.uint8(q8h[d]))) * float(e4m3_decode(np.uint8(k8[k, d]))) for d in range(128))
         for k in range(n_keys)]
    m = max(s)
    p = [256.0 * math.exp((x - m) / math.sqrt(128)) for x in s]
    pq = [float(e4m3_decode(e4m3_encode(np.float64(x)))) for x in p]
    L = sum(p)
    return np.array([sum(pq[k] * float(e4m3_decode(np.uint8(v8[k, d]))) for k in range(n_keys)) / L
                     for d in range(128)])


def test_one_block_with_fp8_p_matches_scalar_statement():
    inp = _case(R=1, seed=9, seq_lens=[100])
    got = D.attention(inp)
    cache, q8 = got["kv_cache"], got["q8"]
    phys = inp["block_table"][0][0]
    for j in (0, 6):
        for h in (0, 15):
            want = _one_block_scalar(q8[j, h], cache[phys, :, :128], cache[phys, :, 128:], 100)
            np.testing.assert_allclose(got["out"][j, h], want, rtol=1e-11, atol=1e-13)


def test_fp8_p_stays_within_the_e4m3_rounding_bound():
    # each P value moves by at most 2^-4 of itself (e4m3 normals; P <= 256, and
    # a subnormal P is off by at most 2^-10), so the output moves from exact
    # softmax attention by at most 2^-4 max|v| + 2^-10 n max|v| / L
    inp = _case(R=2, seed=11, max_seq=6000)
    q = D.attention(inp)
    e = D.attention(inp, p_fp8=False)
    vmax = 448.0
    diff = np.abs(q["out"] - e["out"])
    assert diff.max() <= 2.0 ** -4 * vmax
    assert diff.max() > 0  # P is rounded at all


def test_cache_insert_bytes():
    inp = _case(R=2, seed=13, max_seq=2000)
    inp["slots"][3] = -1
    inp["slots"][4] = inp["kv_cache"].shape[0] * 128 + 5  # past the cache
    q8, k8, v8 = D.qkv_rows(inp["q"], inp["k"], inp["v"], inp["qn"], inp["kn"], inp["cos_sin"],
                            inp["positions"], inp["eps"])
    out = D.insert_kv(inp["kv_cache"], k8, v8, inp["slots"])
    changed = np.zeros(out.shape, bool)
    for t, slot in enumerate(inp["slots"]):
        if 0 <= slot < out.shape[0] * 128:
            np.testing.assert_array_equal(out[slot // 128, slot % 128, :128], k8[t])
            np.testing.assert_array_equal(out[slot // 128, slot % 128, 128:], v8[t])
            changed[slot // 128, slot % 128] = True
    np.testing.assert_array_equal(out[~changed], inp["kv_cache"][~changed])


def test_qkv_rows_are_the_head_norm_rope_cast_to_e4m3():
    # q and k: the prologue's pinned head step, then a saturating E4M3 cast
    inp = _case(R=1, seed=15, seq_lens=[50])
    q8, k8, v8 = D.qkv_rows(inp["q"], inp["k"], inp["v"], inp["qn"], inp["kn"], inp["cos_sin"],
                            inp["positions"], inp["eps"])
    pos = inp["positions"]
    cs = bf16_bits_to_f64(inp["cos_sin"][pos])
    o, n = oracle.head_norm_rope(bf16_bits_to_f64(inp["k"]), inp["kn"], cs[:, :32], cs[:, 32:], inp["eps"])
    np.testing.assert_array_equal(k8, e4m3_encode(o))
    np.testing.assert_array_equal(v8, e4m3_encode(bf16_bits_to_f64(inp["v"])))
    # norms of the rotated pairs are the normed head's
    qd = e4m3_decode(q8)
    assert np.all(np.abs(qd) <= 448)


def test_output_mxfp8_blocks():
    inp = _case(R=1, seed=17, seq_lens=[700])
    got = D.attention(inp)
    deq = e4m3_decode(got["out_codes"]) * np.repeat(2.0 ** (got["out_scales"].astype(np.float64) - 127), 32, axis=1)
    ref = bf16_bits_to_f64(got["out_bf16"]).reshape(7, 2048)
    X = np.repeat(2.0 ** (got["out_scales"].astype(np.float64) - 127), 32, axis=1)
    # e4m3 rounding within 2^-4 relative (2^-10 X below the normals), and the
    # OCP scale saturates a block maximum in [448, 512) X at 448 X
    sat = np.maximum(np.abs(ref) - 448.0 * X, 0.0)
    assert np.all(np.abs(deq - ref) <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * X + sat)
    assert np.all(np.abs(ref) < 512.0 * X)


# ------------------------------------------------------------- planted mistakes
def _mutant_window(monkeypatch):
    orig = D.partial

    def wrong(q8h, qp, lo, hi, blocks, cache, bt_row, p_fp8=True):
        return orig(q8h, qp + 1, lo, hi, blocks, cache, bt_row, p_fp8)  # one key too few (>= vs >)
    monkeypatch.setattr(D, "partial", wrong)


def _mutant_merge(monkeypatch):
    def wrong(parts):
        L = sum(l for _, l, _ in parts)
        return sum(o for _, _, o in parts) / L[:, None]  # no rescale to the common maximum
    monkeypatch.setattr(D, "merge", wrong)


def _mutant_scale(monkeypatch):
    monkeypatch.setattr(D, "C", math.log2(math.e) / 128.0)  # 1/128 instead of 1/sqrt(128)


@pytest.mark.parametrize("mutant", [_mutant_window, _mutant_merge, _mutant_scale])
def test_planted_mistakes_fail_the_textbook_pin(monkeypatch, mutant):
    inp = _case(R=2, max_seq=9000, seed=5)
    mutant(monkeypatch)
    got = D.attention(dict(inp, split=2), p_fp8=False)
    ref = _textbook(inp, got["q8"], got["kv_cache"])
    assert not np.allclose(got["out"], ref, rtol=1e-6, atol=1e-9)
