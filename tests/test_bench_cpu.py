"""Host-side checks of bench.py that need no GPU: the one-GPU contract and the
algorithmic work its roofline divides by (bytes for decode, flops for
prefill), pinned to the figures the tensors of each workload add up to."""

import os
import subprocess
import sys

import pytest

import bench
import synth
import kv_residual_add_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr and proc.stdout == ""


def _structure(wl):
    d = K.make_dims(tokens=wl.tokens, hidden=wl.hidden, nkv=wl.nkv, num_pages=wl.num_pages,
                    max_pos=wl.max_pos, eps=1e-6)
    return K.pa_decode_structure(d)


# (bytes of the whole call, bytes of the dominant launch) for the decode
# workloads, each the sum of what its tensors hold: c1's one launch is the whole
# call; c2's norm + GEMV launch reads the weight, ar, res and g_in and writes
# h_out (15 728 640 + 294 912 + 12 288); c3's GEMV + epilogue launch is the
# call without the norm's ar / res / h_out / g_in and with the FP8 rows
# (33 671 680 - 2 371 584 + 393 216).
DECODE_BYTES = {
    "c1": (2_645_784, 2_645_784),
    "c2": (16_086_208, 16_035_840),
    "c3": (33_671_680, 31_693_312),
}


@pytest.mark.parametrize("key", ["c1", "c2", "c3"])
def test_decode_algorithmic_bytes(key):
    wl = synth.named_config(key)
    S, Kh, nkv = wl.tokens, wl.hidden, wl.nkv
    N = (19 * nkv + 1) * 128
    # the same total from the tensors' sizes, one term per tensor
    total = (N * Kh            # FP8 weight codes
             + 4 * N           # per-row weight scales (float32)
             + 2 * S * Kh      # ar (bf16)
             + 2 * S * Kh      # res (bf16)
             + 2 * S * Kh      # h_out (bf16)
             + 2 * Kh          # g_in (bf16)
             + 4 * 2 * 128     # the four head gammas (bf16)
             + 2 * S * 16 * nkv * 128   # q_out (bf16)
             + 2 * S * nkv * 128        # iq_out (bf16)
             + S * nkv * 2 * 128        # K and V codes
             + S * nkv * 2 * 4          # K and V scales (float32)
             + S * 128                  # index_k codes
             + S * 2 * 64               # the tokens' cos / sin rows (bf16)
             + S * 8 * 2)               # positions and slots (int64)
    assert total == DECODE_BYTES[key][0]
    call_bytes, launch_bytes, flops, _ = bench.algorithmic(wl, _structure(wl))
    assert (call_bytes, launch_bytes) == DECODE_BYTES[key]
    assert flops == 2 * S * N * Kh


@pytest.mark.parametrize("key,gflop", [("c4", 125.6), ("c5", 992.1)])
def test_prefill_algorithmic_flops(key, gflop):
    wl = synth.named_config(key)
    _, _, flops, name = bench.algorithmic(wl)
    assert name == "prefill_gemm"
    N = (19 * wl.nkv + 1) * 128
    assert flops == 2 * wl.tokens * N * wl.hidden
    assert round(flops / 1e9, 1) == gflop
