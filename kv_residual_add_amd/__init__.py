"""MiniMax-M3 fused pre-attention prologue for AMD Instinct MI355X (gfx950).

The compute lives in libpre_attn.so (hand-written HIP, C ABI in
include/pre_attn.h); this package is its ctypes binding plus device set-up
helpers. Importing it loads the library and fails if it has not been built.
"""

from ._binding import (  # noqa: F401
    DECODE_MAX_TOKENS,
    EXPORTS,
    LIB_PATH,
    HeadOptions,
    PA_DECODE_EPILOGUE_FUSED,
    PA_DECODE_NORM_FUSED,
    PA_ERR_OPTIONS,
    PA_ERR_SYNC,
    PA_MODE_DECODE,
    PA_MODE_PREFILL,
    PaError,
    load,
    make_dims,
    pa_dims,
    pa_head_options,
    pa_pack_weight_decode,
    pa_pack_weight_prefill,
    pa_set_kernel_events,
    pa_set_timeline,
    pa_packed_scale_bytes,
    pa_packed_weight_bytes,
    pa_workspace_bytes,
    pa_decode_structure,
    pa_workspace_init,
    pa_workspace_status,
    pre_attn_decode,
    pre_attn_prefill,
    pre_attn_decode_ex,
    pre_attn_prefill_ex,
)

load()
