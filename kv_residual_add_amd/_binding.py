"""ctypes binding of libpre_attn.so (declared in include/pre_attn.h).

The functions keep the C names and argument order. They only marshal: torch
tensors become device pointers after dtype / size / device checks (the C ABI
cannot see buffer sizes, so the checks here keep every kernel access inside
the caller's tensors), and the stream defaults to torch's current stream.
Every step of the prologue runs in the HIP kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpre_attn.so")

PA_MODE_DECODE = 0
PA_MODE_PREFILL = 1
HEAD_DIM = 128
PAGE = 16
PAGE_BYTES = 2048
DECODE_MAX_TOKENS = 64
PA_DECODE_NORM_FUSED = 1
PA_DECODE_EPILOGUE_FUSED = 2
PA_OK = 0
PA_ERR_NULL = -1
PA_ERR_ALIGN = -2
PA_ERR_NKV = -3
PA_ERR_HIDDEN = -4
PA_ERR_TOKENS = -5
PA_ERR_WORKSPACE = -6
PA_ERR_DIMS = -7
PA_ERR_HIP = -8
PA_ERR_DEVICE = -9
PA_ERR_MODE = -10
PA_ERR_SYNC = -11
PA_ERR_OPTIONS = -12
PA_ERR_WEIGHT_RANGE = -13
PA_KV_FP8 = 0
PA_KV_NVFP4 = 1
NV_SLOT_BYTES = 1152

EXPORTS = (
    "pa_workspace_bytes",
    "pa_decode_structure",
    "pa_workspace_init",
    "pa_workspace_status",
    "pa_packed_weight_bytes",
    "pa_packed_scale_bytes",
    "pa_pack_weight_decode",
    "pa_pack_weight_prefill",
    "pre_attn_decode",
    "pre_attn_prefill",
    "pre_attn_decode_ex",
    "pre_attn_prefill_ex",
    "pre_attn_decode_noalloc",
    "pa_drafter_workspace_bytes",
    "pa_drafter_attention",
    "pa_set_kernel_events",
    "pa_set_timeline",
    "pa_strerror",
    "pa_last_error_detail",
)


class pa_drafter_dims(ctypes.Structure):
    _fields_ = [
        ("requests", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("table_width", ctypes.c_int32),
        ("max_pos", ctypes.c_int32),
        ("split", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


class pa_dims(ctypes.Structure):
    _fields_ = [
        ("tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("nkv", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pos", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


class pa_head_options(ctypes.Structure):
    _fields_ = [
        ("static_kv_scale", ctypes.c_int32),
        ("q_fp8_scale", ctypes.c_float),
        ("q_fp8_out", ctypes.c_void_p),
        ("kv_cache_format", ctypes.c_int32),
        ("k_global_scale", ctypes.c_float),
        ("v_global_scale", ctypes.c_float),
    ]


class HeadOptions:
    """Head-step variants of pre_attn_decode_ex / pre_attn_prefill_ex:
    static_kv_scale (unit K / V scales), an optional FP8 q output q_fp8_out
    (uint8 [tokens, 16 nkv, 128]) with its dequantization scale, and the NVFP4
    cache format (nvfp4=True: k_cache is the K/V cache uint8
    [pages, 2 nkv, 1152], index_cache uint8 [pages, 1152]; v_cache, k_scale and
    v_scale may be None) with the K / V global scales."""

    def __init__(self, static_kv_scale: bool = False, q_fp8_out=None, q_fp8_scale: float = 1.0,
                 nvfp4: bool = False, k_global_scale: float = 1.0, v_global_scale: float = 1.0):
        self.static_kv_scale = bool(static_kv_scale)
        self.q_fp8_out = q_fp8_out
        self.q_fp8_scale = float(q_fp8_scale)
        self.nvfp4 = bool(nvfp4)
        self.k_global_scale = float(k_global_scale)
        self.v_global_scale = float(v_global_scale)


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.pa_strerror(status).decode()
        detail = lib.pa_last_error_detail().decode()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail else ""))
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python kv_residual_add_amd/build.py`"
            )
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        sz = ctypes.c_size_t
        i32 = ctypes.c_int32
        dims_p = ctypes.POINTER(pa_dims)
        lib.pa_workspace_bytes.argtypes = [dims_p, ctypes.c_int]
        lib.pa_workspace_bytes.restype = sz
        lib.pa_decode_structure.argtypes = [dims_p]
        lib.pa_decode_structure.restype = ctypes.c_int
        lib.pa_workspace_status.argtypes = [P, P]
        lib.pa_workspace_status.restype = ctypes.c_int
        lib.pa_workspace_init.argtypes = [P, sz, P]
        lib.pa_workspace_init.restype = ctypes.c_int
        lib.pa_packed_weight_bytes.argtypes = [ctypes.c_int, i32, i32]
        lib.pa_packed_weight_bytes.restype = sz
        lib.pa_packed_scale_bytes.argtypes = [ctypes.c_int, i32, i32]
        lib.pa_packed_scale_bytes.restype = sz
        lib.pa_pack_weight_decode.argtypes = [P, P, i32, i32, P]
        lib.pa_pack_weight_decode.restype = ctypes.c_int
        lib.pa_pack_weight_prefill.argtypes = [P, P, P, P, i32, i32, P]
        lib.pa_pack_weight_prefill.restype = ctypes.c_int
        lib.pre_attn_decode.argtypes = [dims_p] + [P] * 21 + [sz, P]
        lib.pre_attn_decode.restype = ctypes.c_int
        lib.pre_attn_prefill.argtypes = [dims_p] + [P] * 21 + [sz, P]
        lib.pre_attn_prefill.restype = ctypes.c_int
        opts_p = ctypes.POINTER(pa_head_options)
        lib.pre_attn_decode_ex.argtypes = [dims_p, opts_p] + [P] * 21 + [sz, P]
        lib.pre_attn_decode_ex.restype = ctypes.c_int
        lib.pre_attn_prefill_ex.argtypes = [dims_p, opts_p] + [P] * 21 + [sz, P]
        lib.pre_attn_prefill_ex.restype = ctypes.c_int
        lib.pre_attn_decode_noalloc.argtypes = [dims_p] + [P] * 20 + [P]
        lib.pre_attn_decode_noalloc.restype = ctypes.c_int
        ddims_p = ctypes.POINTER(pa_drafter_dims)
        lib.pa_drafter_workspace_bytes.argtypes = [ddims_p]
        lib.pa_drafter_workspace_bytes.restype = sz
        lib.pa_drafter_attention.argtypes = [ddims_p] + [P] * 15 + [sz, P]
        lib.pa_drafter_attention.restype = ctypes.c_int
        lib.pa_set_timeline.argtypes = [P, sz]
        lib.pa_set_timeline.restype = ctypes.c_int
        lib.pa_set_kernel_events.argtypes = [P, P]
        lib.pa_set_kernel_events.restype = ctypes.c_int
        lib.pa_strerror.argtypes = [ctypes.c_int]
        lib.pa_strerror.restype = ctypes.c_char_p
        lib.pa_last_error_detail.argtypes = []
        lib.pa_last_error_detail.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def make_dims(tokens, hidden, nkv, num_pages, max_pos, eps) -> pa_dims:
    return pa_dims(int(tokens), int(hidden), int(nkv), int(num_pages), int(max_pos), float(eps))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor, name: str, dtype, numel: int, device) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must live on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _check(status: int, where: str):
    if status != 0:
        raise PaError(status, where)


def pa_set_kernel_events(start, stop) -> None:
    """Record torch.cuda.Event pair (or None, None) around the dominant kernel of
    later calls on this thread (see include/pre_attn.h)."""
    ps = None if start is None else start.cuda_event
    pe = None if stop is None else stop.cuda_event
    if (start is not None and not ps) or (stop is not None and not pe):
        raise ValueError("record each torch.cuda.Event once before passing it (torch creates "
                         "the underlying event lazily)")
    _check(load().pa_set_kernel_events(ps, pe), "pa_set_kernel_events")


def pa_set_timeline(buffer) -> None:
    """Per-CTA phase stamps of later decode calls into a uint64 CUDA tensor (None: off)."""
    if buffer is None:
        _check(load().pa_set_timeline(None, 0), "pa_set_timeline")
        return
    if buffer.dtype != torch.int64 or not buffer.is_cuda or not buffer.is_contiguous():
        raise ValueError("timeline buffer must be a contiguous int64 CUDA tensor")
    _check(load().pa_set_timeline(buffer.data_ptr(), buffer.numel() * 8), "pa_set_timeline")


def pa_workspace_bytes(dims: pa_dims, mode: int) -> int:
    return load().pa_workspace_bytes(ctypes.byref(dims), mode)


def pa_decode_structure(dims: pa_dims) -> int:
    """PA_DECODE_* flags of a decode call with these dims (negative status on bad dims)."""
    return load().pa_decode_structure(ctypes.byref(dims))


def pa_workspace_status(workspace: torch.Tensor, stream=None) -> None:
    """Raises PaError(PA_ERR_SYNC) if a bounded in-kernel wait gave up on this
    workspace since it was initialised (synchronizes the stream)."""
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    _check(load().pa_workspace_status(workspace.data_ptr(), _stream(stream)), "pa_workspace_status")


def pa_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    _check(load().pa_workspace_init(workspace.data_ptr(), workspace.numel(), _stream(stream)),
           "pa_workspace_init")


def pa_packed_weight_bytes(mode: int, n_rows: int, hidden: int) -> int:
    return load().pa_packed_weight_bytes(mode, n_rows, hidden)


def pa_packed_scale_bytes(mode: int, n_rows: int, hidden: int) -> int:
    return load().pa_packed_scale_bytes(mode, n_rows, hidden)


def pa_pack_weight_decode(w: torch.Tensor, w_packed: torch.Tensor, stream=None) -> None:
    n, k = w.shape
    dev = w.device
    nb = pa_packed_weight_bytes(PA_MODE_DECODE, n, k)
    if nb == 0:
        raise ValueError(f"unsupported weight shape {tuple(w.shape)}")
    _check(load().pa_pack_weight_decode(
        _ptr(w, "w", torch.uint8, n * k, dev), _ptr(w_packed, "w_packed", torch.uint8, nb, dev),
        n, k, _stream(stream)), "pa_pack_weight_decode")


def pa_pack_weight_prefill(w: torch.Tensor, w_e8m0: torch.Tensor, w_packed: torch.Tensor,
                           s_packed: torch.Tensor, stream=None) -> None:
    n, k = w.shape
    dev = w.device
    nb = pa_packed_weight_bytes(PA_MODE_PREFILL, n, k)
    ns = pa_packed_scale_bytes(PA_MODE_PREFILL, n, k)
    if nb == 0:
        raise ValueError(f"unsupported weight shape {tuple(w.shape)}")
    _check(load().pa_pack_weight_prefill(
        _ptr(w, "w", torch.uint8, n * k, dev),
        _ptr(w_e8m0, "w_e8m0", torch.uint8, n * k // 32, dev),
        _ptr(w_packed, "w_packed", torch.uint8, nb, dev),
        _ptr(s_packed, "s_packed", torch.uint8, ns, dev),
        n, k, _stream(stream)), "pa_pack_weight_prefill")


def _run(fn_name: str, mode: int, dims: pa_dims, ar, res, h_out, g_in, w_packed, w_scales,
         g_q, g_k, g_iq, g_ik, cos_sin, positions, slot_mapping, k_cache, v_cache, k_scale,
         v_scale, index_cache, q_out, iq_out, workspace, stream, opts=None):
    S, K, nkv = dims.tokens, dims.hidden, dims.nkv
    P, L = dims.num_pages, dims.max_pos
    N = (19 * nkv + 1) * HEAD_DIM
    dev = ar.device
    bf, u8, f32, i64 = torch.bfloat16, torch.uint8, torch.float32, torch.int64
    lead = [ctypes.byref(dims)]
    nvfp4 = opts is not None and opts.nvfp4
    if fn_name.endswith("_ex"):
        c_opts = None
        if opts is not None:
            qf = opts.q_fp8_out
            c_opts = pa_head_options(
                int(opts.static_kv_scale), opts.q_fp8_scale,
                None if qf is None else _ptr(qf, "q_fp8_out", u8, S * 16 * nkv * HEAD_DIM, dev),
                PA_KV_NVFP4 if nvfp4 else PA_KV_FP8, opts.k_global_scale, opts.v_global_scale)
        lead.append(None if c_opts is None else ctypes.byref(c_opts))
    ws_need = pa_workspace_bytes(dims, mode)
    if ws_need == 0:
        # let the library name the invalid dimension
        _check(getattr(load(), fn_name)(*lead, *([None] * 21), 0, None), fn_name)
    if workspace.numel() < ws_need:
        raise ValueError(f"workspace: need {ws_need} bytes, got {workspace.numel()}")
    if mode == PA_MODE_DECODE:
        wp = _ptr(w_packed, "w_packed", u8, pa_packed_weight_bytes(mode, N, K), dev)
        sc = _ptr(w_scales, "w_scale", f32, N, dev)
    else:
        wp = _ptr(w_packed, "w_packed", u8, pa_packed_weight_bytes(mode, N, K), dev)
        sc = _ptr(w_scales, "s_packed", u8, pa_packed_scale_bytes(mode, N, K), dev)
    args = [
        _ptr(ar, "ar", bf, S * K, dev), _ptr(res, "res", bf, S * K, dev),
        _ptr(h_out, "h_out", bf, S * K, dev), _ptr(g_in, "g_in", bf, K, dev), wp, sc,
        _ptr(g_q, "g_q", bf, HEAD_DIM, dev), _ptr(g_k, "g_k", bf, HEAD_DIM, dev),
        _ptr(g_iq, "g_iq", bf, HEAD_DIM, dev), _ptr(g_ik, "g_ik", bf, HEAD_DIM, dev),
        _ptr(cos_sin, "cos_sin", bf, L * 64, dev),
        _ptr(positions, "positions", i64, S, dev), _ptr(slot_mapping, "slot_mapping", i64, S, dev),
        *([_ptr(k_cache, "kv_cache (NVFP4)", u8, P * 2 * nkv * NV_SLOT_BYTES, dev),
           None if v_cache is None else _ptr(v_cache, "v_cache", u8, P * nkv * PAGE_BYTES, dev),
           None if k_scale is None else _ptr(k_scale, "k_scale", f32, P * nkv * PAGE, dev),
           None if v_scale is None else _ptr(v_scale, "v_scale", f32, P * nkv * PAGE, dev),
           _ptr(index_cache, "index_cache (NVFP4)", u8, P * NV_SLOT_BYTES, dev)] if nvfp4 else
          [_ptr(k_cache, "k_cache", u8, P * nkv * PAGE_BYTES, dev),
           _ptr(v_cache, "v_cache", u8, P * nkv * PAGE_BYTES, dev),
           _ptr(k_scale, "k_scale", f32, P * nkv * PAGE, dev),
           _ptr(v_scale, "v_scale", f32, P * nkv * PAGE, dev),
           _ptr(index_cache, "index_cache", u8, P * PAGE * HEAD_DIM, dev)]),
        None if q_out is None else _ptr(q_out, "q_out", bf, S * 16 * nkv * HEAD_DIM, dev),
        _ptr(iq_out, "iq_out", bf, S * nkv * HEAD_DIM, dev),
        workspace.data_ptr(),
    ]
    if workspace.dtype != u8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    st = getattr(load(), fn_name)(*lead, *args, workspace.numel(), _stream(stream))
    _check(st, fn_name)


def pre_attn_decode(dims, ar, res, h_out, g_in, w_packed, w_scale, g_q, g_k, g_iq, g_ik,
                    cos_sin, positions, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                    index_cache, q_out, iq_out, workspace, stream=None) -> None:
    """Decode prologue; argument meaning as in include/pre_attn.h."""
    _run("pre_attn_decode", PA_MODE_DECODE, dims, ar, res, h_out, g_in, w_packed, w_scale,
         g_q, g_k, g_iq, g_ik, cos_sin, positions, slot_mapping, k_cache, v_cache, k_scale,
         v_scale, index_cache, q_out, iq_out, workspace, stream)


def pre_attn_prefill(dims, ar, res, h_out, g_in, w_packed, s_packed, g_q, g_k, g_iq, g_ik,
                     cos_sin, positions, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                     index_cache, q_out, iq_out, workspace, stream=None) -> None:
    """Prefill prologue; argument meaning as in include/pre_attn.h."""
    _run("pre_attn_prefill", PA_MODE_PREFILL, dims, ar, res, h_out, g_in, w_packed, s_packed,
         g_q, g_k, g_iq, g_ik, cos_sin, positions, slot_mapping, k_cache, v_cache, k_scale,
         v_scale, index_cache, q_out, iq_out, workspace, stream)


def pre_attn_decode_ex(dims, opts, ar, res, h_out, g_in, w_packed, w_scale, g_q, g_k, g_iq, g_ik,
                       cos_sin, positions, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                       index_cache, q_out, iq_out, workspace, stream=None) -> None:
    """Decode prologue with head-step options (a HeadOptions or None); q_out may
    be None when opts.q_fp8_out is set. As in include/pre_attn.h."""
    _run("pre_attn_decode_ex", PA_MODE_DECODE, dims, ar, res, h_out, g_in, w_packed, w_scale,
         g_q, g_k, g_iq, g_ik, cos_sin, positions, slot_mapping, k_cache, v_cache, k_scale,
         v_scale, index_cache, q_out, iq_out, workspace, stream, opts)


def pre_attn_prefill_ex(dims, opts, ar, res, h_out, g_in, w_packed, s_packed, g_q, g_k, g_iq,
                        g_ik, cos_sin, positions, slot_mapping, k_cache, v_cache, k_scale,
                        v_scale, index_cache, q_out, iq_out, workspace, stream=None) -> None:
    """Prefill prologue with head-step options, as pre_attn_decode_ex."""
    _run("pre_attn_prefill_ex", PA_MODE_PREFILL, dims, ar, res, h_out, g_in, w_packed, s_packed,
         g_q, g_k, g_iq, g_ik, cos_sin, positions, slot_mapping, k_cache, v_cache, k_scale,
         v_scale, index_cache, q_out, iq_out, workspace, stream, opts)


def pre_attn_decode_noalloc(dims, ar, res, h_out, g_in, w_packed, w_scale, g_q, g_k, g_iq, g_ik,
                            cos_sin, positions, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                            index_cache, q_out, iq_out, stream=None) -> None:
    """pre_attn_decode with the library's per-GPU scratch as its workspace (no
    allocation; calls on one GPU must not overlap). As in include/pre_attn.h."""
    S, K, nkv = dims.tokens, dims.hidden, dims.nkv
    P, L = dims.num_pages, dims.max_pos
    N = (19 * nkv + 1) * HEAD_DIM
    dev = ar.device
    bf, u8, f32, i64 = torch.bfloat16, torch.uint8, torch.float32, torch.int64
    args = [
        _ptr(ar, "ar", bf, S * K, dev), _ptr(res, "res", bf, S * K, dev),
        _ptr(h_out, "h_out", bf, S * K, dev), _ptr(g_in, "g_in", bf, K, dev),
        _ptr(w_packed, "w_packed", u8, pa_packed_weight_bytes(PA_MODE_DECODE, N, K), dev),
        _ptr(w_scale, "w_scale", f32, N, dev),
        _ptr(g_q, "g_q", bf, HEAD_DIM, dev), _ptr(g_k, "g_k", bf, HEAD_DIM, dev),
        _ptr(g_iq, "g_iq", bf, HEAD_DIM, dev), _ptr(g_ik, "g_ik", bf, HEAD_DIM, dev),
        _ptr(cos_sin, "cos_sin", bf, L * 64, dev),
        _ptr(positions, "positions", i64, S, dev), _ptr(slot_mapping, "slot_mapping", i64, S, dev),
        _ptr(k_cache, "k_cache", u8, P * nkv * PAGE_BYTES, dev),
        _ptr(v_cache, "v_cache", u8, P * nkv * PAGE_BYTES, dev),
        _ptr(k_scale, "k_scale", f32, P * nkv * PAGE, dev),
        _ptr(v_scale, "v_scale", f32, P * nkv * PAGE, dev),
        _ptr(index_cache, "index_cache", u8, P * PAGE * HEAD_DIM, dev),
        _ptr(q_out, "q_out", bf, S * 16 * nkv * HEAD_DIM, dev),
        _ptr(iq_out, "iq_out", bf, S * nkv * HEAD_DIM, dev),
    ]
    _check(load().pre_attn_decode_noalloc(ctypes.byref(dims), *args, _stream(stream)),
           "pre_attn_decode_noalloc")


def pa_drafter_workspace_bytes(dims: pa_drafter_dims) -> int:
    return load().pa_drafter_workspace_bytes(ctypes.byref(dims))


def pa_drafter_attention(dims, q, k, v, qn, kn, cos_sin, positions, slots, kv_cache, block_table,
                         seq_lens, out_codes, out_scales, out_bf16, workspace, stream=None) -> None:
    """The DSpark drafter's attention; argument meaning as in include/pre_attn.h
    (out_bf16 may be None)."""
    R, W, NB, L = dims.requests, dims.table_width, dims.num_blocks, dims.max_pos
    T = 7 * R
    dev = q.device
    bf, u8, i32, i64 = torch.bfloat16, torch.uint8, torch.int32, torch.int64
    need = pa_drafter_workspace_bytes(dims)
    if need == 0:
        _check(PA_ERR_DIMS, "pa_drafter_attention")
    if workspace.dtype != u8 or workspace.device != dev or not workspace.is_contiguous() or workspace.numel() < need:
        raise ValueError(f"workspace: need a contiguous uint8 tensor of {need} bytes on {dev}")
    args = [
        _ptr(q, "q", bf, T * 16 * HEAD_DIM, dev), _ptr(k, "k", bf, T * HEAD_DIM, dev),
        _ptr(v, "v", bf, T * HEAD_DIM, dev), _ptr(qn, "qn", bf, HEAD_DIM, dev), _ptr(kn, "kn", bf, HEAD_DIM, dev),
        _ptr(cos_sin, "cos_sin", bf, L * 64, dev), _ptr(positions, "positions", i64, T, dev),
        _ptr(slots, "slots", i64, T, dev), _ptr(kv_cache, "kv_cache", u8, NB * 128 * 256, dev),
        _ptr(block_table, "block_table", i32, R * W, dev), _ptr(seq_lens, "seq_lens", i32, R, dev),
        _ptr(out_codes, "out_codes", u8, T * 2048, dev), _ptr(out_scales, "out_scales", u8, T * 64, dev),
        None if out_bf16 is None else _ptr(out_bf16, "out_bf16", bf, T * 2048, dev),
        workspace.data_ptr(),
    ]
    _check(load().pa_drafter_attention(ctypes.byref(dims), *args, workspace.numel(), _stream(stream)),
           "pa_drafter_attention")
