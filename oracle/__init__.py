"""CPU oracle for the MiniMax-M3 pre-attention prologue and the DSpark drafter's
attention.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, NumPy (float64 unless
the method fixes float32) statement of what the prologue computes, written from
the vLLM API pages ``vllm.models.minimax_m3.amd.mono.kernels.pre_attn`` (the
"K1 mono_pre" decode kernel) and
``vllm.models.minimax_m3.nvidia.ops.qkv_index_fused_epilogue`` (the MXFP8
prefill GEMM with a fused epilogue), and, in ``drafter.py``, from
``vllm.models.minimax_m3.amd.mono.drafter.attention`` (the drafter's
split-KV attention). Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the HIP library never calls it and
shares no code, table or constant generator with it.

Every function is pinned by ``tests/test_oracle_*.py`` against something other
than itself: brute force over the format tables, torch's library casts and
``rms_norm``, complex multiplication for RoPE, exact integer dot products, and a
separately written scalar reference of the whole pipeline. No function here is
"parity unpinned".
"""

from .codecs import (  # noqa: F401
    E4M3_MAX,
    bf16_bits_to_f64,
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_decode_table,
    e4m3_encode,
    e8m0_decode,
    f32_mul_rz,
    f32_to_bf16_bits,
)
from .prologue import (  # noqa: F401
    decode,
    head_norm_rope,
    input_norm,
    mxfp8_quantize,
    nvfp4_quantize,
    nvfp4_scale_offset,
    prefill,
    project_decode,
    project_mxfp8,
    quantize_per_token,
)
from . import drafter  # noqa: F401,E402
