"""Device-side set-up for one prologue call: uploads host arrays (raw bits in
numpy, the layouts of include/pre_attn.h), packs the weight once, allocates and
initializes the workspace, and calls pre_attn_decode / pre_attn_prefill.
"""

from __future__ import annotations

import numpy as np
import torch

from . import _binding as B

_BF16_KEYS = ("ar", "res", "g_in", "g_q", "g_k", "g_iq", "g_ik", "cos_sin")


def _to_dev(a: np.ndarray, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


class Problem:
    """All device buffers of one prologue call."""

    def __init__(self, arrays: dict, device="cuda:0"):
        self.device = torch.device(device)
        self.mode = B.PA_MODE_DECODE if arrays["mode"] == "decode" else B.PA_MODE_PREFILL
        S, K = arrays["ar"].shape
        self.nkv = int(arrays["nkv"])
        self.N = (19 * self.nkv + 1) * B.HEAD_DIM
        pages = (arrays["kv_cache"] if arrays.get("kv_format", "fp8") == "nvfp4" else arrays["k_cache"]).shape[0]
        self.dims = B.make_dims(S, K, self.nkv, pages,
                                arrays["cos_sin"].shape[0], float(arrays["eps"]))
        dev = self.device
        t = {}
        for k in _BF16_KEYS:
            t[k] = _to_dev(arrays[k].view(np.int16), dev, torch.bfloat16)
        for k in ("positions", "slot_mapping"):
            t[k] = _to_dev(arrays[k].astype(np.int64), dev)
        self.nvfp4 = arrays.get("kv_format", "fp8") == "nvfp4"
        if self.nvfp4:  # the K/V cache goes in the k_cache argument
            t["k_cache"] = _to_dev(arrays["kv_cache"], dev)
            t["index_cache"] = _to_dev(arrays["index_cache"], dev)
            t["v_cache"] = t["k_scale"] = t["v_scale"] = None
        else:
            for k in ("k_cache", "v_cache", "index_cache"):
                t[k] = _to_dev(arrays[k], dev)
            for k in ("k_scale", "v_scale"):
                t[k] = _to_dev(arrays[k], dev)
        t["h_out"] = torch.empty((S, K), dtype=torch.bfloat16, device=dev)
        t["q_out"] = torch.empty((S, 16 * self.nkv, B.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        t["iq_out"] = torch.empty((S, self.nkv, B.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        # head-step variants (the _ex entry points): inputs "static_kv_scale",
        # "q_fp8_scale" (adds the FP8 q output) and "q_bf16" (False: no bf16 q)
        self.opts = None
        qs = arrays.get("q_fp8_scale")
        if arrays.get("static_kv_scale", False) or qs is not None or self.nvfp4:
            qf = None
            if qs is not None:
                qf = torch.empty((S, 16 * self.nkv, B.HEAD_DIM), dtype=torch.uint8, device=dev)
                t["q_fp8"] = qf
            self.opts = B.HeadOptions(bool(arrays.get("static_kv_scale", False)), qf,
                                      1.0 if qs is None else float(qs), self.nvfp4,
                                      float(arrays.get("k_global_scale", 1.0)),
                                      float(arrays.get("v_global_scale", 1.0)))
        if not arrays.get("q_bf16", True):
            t["q_out"] = None
        self.t = t
        self.set_weight(arrays)
        nbytes = B.pa_workspace_bytes(self.dims, self.mode)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        B.pa_workspace_init(self.workspace)

    def set_weight(self, arrays: dict) -> None:
        dev = self.device
        K = self.dims.hidden
        w = _to_dev(arrays["w"], dev)
        nb = B.pa_packed_weight_bytes(self.mode, self.N, K)
        self.w_packed = torch.empty(nb, dtype=torch.uint8, device=dev)
        if self.mode == B.PA_MODE_DECODE:
            B.pa_pack_weight_decode(w, self.w_packed)
            self.w_scales = _to_dev(arrays["w_scale"].astype(np.float32), dev)
        else:
            we = _to_dev(arrays["w_e8m0"], dev)
            ns = B.pa_packed_scale_bytes(self.mode, self.N, K)
            self.w_scales = torch.empty(ns, dtype=torch.uint8, device=dev)
            B.pa_pack_weight_prefill(w, we, self.w_packed, self.w_scales)

    def args(self, w_packed=None, w_scales=None, workspace=None, **over):
        t = dict(self.t, **over)
        return (self.dims, t["ar"], t["res"], t["h_out"], t["g_in"],
                self.w_packed if w_packed is None else w_packed,
                self.w_scales if w_scales is None else w_scales,
                t["g_q"], t["g_k"], t["g_iq"], t["g_ik"], t["cos_sin"], t["positions"],
                t["slot_mapping"], t["k_cache"], t["v_cache"], t["k_scale"], t["v_scale"],
                t["index_cache"], t["q_out"], t["iq_out"], self.workspace if workspace is None else workspace)

    def run(self, stream=None, **over) -> None:
        if self.opts is None:
            fn = B.pre_attn_decode if self.mode == B.PA_MODE_DECODE else B.pre_attn_prefill
            fn(*self.args(**over), stream=stream)
        else:
            fn = B.pre_attn_decode_ex if self.mode == B.PA_MODE_DECODE else B.pre_attn_prefill_ex
            a = self.args(**over)
            fn(a[0], self.opts, *a[1:], stream=stream)

    def outputs(self) -> dict:
        """Outputs and caches as numpy raw bits (synchronizes). Raises if an
        in-kernel wait gave up on the workspace since it was initialised."""
        torch.cuda.synchronize(self.device)
        B.pa_workspace_status(self.workspace)
        out = {}
        for k in ("h_out", "q_out", "iq_out"):
            if self.t[k] is not None:
                out[k] = self.t[k].view(torch.int16).cpu().numpy().view(np.uint16)
        if "q_fp8" in self.t:
            out["q_fp8"] = self.t["q_fp8"].cpu().numpy()
        if self.nvfp4:
            out["kv_cache"] = self.t["k_cache"].cpu().numpy()
            out["index_cache"] = self.t["index_cache"].cpu().numpy()
            return out
        for k in ("k_cache", "v_cache", "index_cache", "k_scale", "v_scale"):
            out[k] = self.t[k].cpu().numpy()
        return out


class DrafterProblem:
    """All device buffers of one drafter attention call (inputs from
    synth.make_drafter)."""

    def __init__(self, arrays: dict, device="cuda:0"):
        self.device = torch.device(device)
        dev = self.device
        R = int(arrays["requests"])
        T = 7 * R
        bt = np.ascontiguousarray(arrays["block_table"], np.int32)
        self.dims = B.pa_drafter_dims(R, int(arrays["kv_cache"].shape[0]), int(bt.shape[1]),
                                      int(arrays["cos_sin"].shape[0]), int(arrays["split"]), float(arrays["eps"]))
        t = {}
        for key in ("q", "k", "v", "qn", "kn", "cos_sin"):
            t[key] = _to_dev(arrays[key].view(np.int16), dev, torch.bfloat16)
        t["positions"] = _to_dev(arrays["positions"].astype(np.int64), dev)
        t["slots"] = _to_dev(arrays["slots"].astype(np.int64), dev)
        t["kv_cache"] = _to_dev(arrays["kv_cache"], dev)
        t["block_table"] = _to_dev(bt, dev)
        t["seq_lens"] = _to_dev(np.asarray(arrays["seq_lens"], np.int32), dev)
        t["out_codes"] = torch.empty((T, 2048), dtype=torch.uint8, device=dev)
        t["out_scales"] = torch.empty((T, 64), dtype=torch.uint8, device=dev)
        t["out_bf16"] = torch.empty((T, 16, 128), dtype=torch.bfloat16, device=dev)
        self.t = t
        self.workspace = torch.empty(B.pa_drafter_workspace_bytes(self.dims), dtype=torch.uint8, device=dev)

    def run(self, stream=None, **over) -> None:
        t = dict(self.t, **over)
        B.pa_drafter_attention(self.dims, t["q"], t["k"], t["v"], t["qn"], t["kn"], t["cos_sin"],
                               t["positions"], t["slots"], t["kv_cache"], t["block_table"], t["seq_lens"],
                               t["out_codes"], t["out_scales"], t["out_bf16"], self.workspace, stream=stream)

    def outputs(self) -> dict:
        torch.cuda.synchronize(self.device)
        return {"out_codes": self.t["out_codes"].cpu().numpy(), "out_scales": self.t["out_scales"].cpu().numpy(),
                "out_bf16": self.t["out_bf16"].view(torch.int16).cpu().numpy().view(np.uint16),
                "kv_cache": self.t["kv_cache"].cpu().numpy()}
