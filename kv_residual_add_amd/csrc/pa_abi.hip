// extern "C" entry points of libpre_attn.so: argument validation, workspace
// carve-up and kernel launches on the caller's stream. Nothing here allocates
// device memory or synchronizes the host (except the status queries and the
// prefill weight check, which say so).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "pa_internal.hpp"
#include "pre_attn.h"

namespace {

thread_local char g_detail[256] = "";
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;
thread_local uint64_t* g_timeline = nullptr;
thread_local uint32_t g_timeline_slots = 0;

int hip_fail(hipError_t e, const char* where) {
  std::snprintf(g_detail, sizeof(g_detail), "%s: %s", where, hipGetErrorString(e));
  return PA_ERR_HIP;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_DEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? PA_OK : PA_ERR_DEVICE;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_dims(const pa_dims* d, int mode) {
  if (!d) return PA_ERR_NULL;
  if (mode != PA_MODE_DECODE && mode != PA_MODE_PREFILL) return PA_ERR_MODE;
  if (d->nkv != 1 && d->nkv != 2 && d->nkv != 4) return PA_ERR_NKV;
  if (d->hidden < 128 || d->hidden > PA_MAX_HIDDEN || d->hidden % 128) return PA_ERR_HIDDEN;
  const int max_tokens = mode == PA_MODE_DECODE ? PA_DECODE_MAX_TOKENS : (1 << 24);
  if (d->tokens < 1 || d->tokens > max_tokens) return PA_ERR_TOKENS;
  if (d->num_pages < 1 || d->max_pos < 1) return PA_ERR_DIMS;
  if (!std::isfinite(d->eps) || d->eps < 0.0f) return PA_ERR_DIMS;
  // byte offsets of the caches must fit the kernels' 64-bit index math
  if (static_cast<int64_t>(d->num_pages) * d->nkv > (int64_t(1) << 40)) return PA_ERR_DIMS;
  return PA_OK;
}

size_t workspace_for(const pa_dims* d, int mode) {
  if (mode == PA_MODE_DECODE) return pa::decode_plan(d->tokens, d->hidden, d->nkv).total;
  return pa::prefill_plan(d->tokens, d->hidden, d->nkv).total;
}

struct Ptrs {
  const uint16_t *ar, *res;
  uint16_t* h_out;
  const uint16_t* g_in;
  const uint8_t* w_packed;
  const void* w_scales;
  const uint16_t *g_q, *g_k, *g_iq, *g_ik, *cos_sin;
  const int64_t *positions, *slot_mapping;
  uint8_t *k_cache, *v_cache;
  float *k_scale, *v_scale;
  uint8_t* index_cache;
  uint16_t *q_out, *iq_out;
  void* ws;
};

// The head-step variants of the _ex entry points (defaults: per-token K / V
// scales, bf16 q only).
struct Opts {
  uint8_t* q_fp8 = nullptr;
  float q_fp8_inv = 1.0f;
  int static_kv = 0;
  int nvfp4 = 0;
  float k_gs = 1.0f, v_gs = 1.0f;
};

// float32(1 / s), correctly rounded, for a finite s > 0 whose reciprocal is finite
bool reciprocal(float s, float& out) {
  if (!std::isfinite(s) || !(s > 0.0f)) return false;
  const volatile float one = 1.0f;
  out = one / s;
  return std::isfinite(out);
}

int check_opts(const pa_head_options* o, Opts& out) {
  if (!o) return PA_OK;
  out.static_kv = o->static_kv_scale != 0;
  if (o->kv_cache_format != PA_KV_FP8 && o->kv_cache_format != PA_KV_NVFP4) return PA_ERR_OPTIONS;
  if (o->kv_cache_format == PA_KV_NVFP4) {
    if (out.static_kv) return PA_ERR_OPTIONS;  // per-group scales have no static form
    out.nvfp4 = 1;
    if (!reciprocal(o->k_global_scale, out.k_gs) || !reciprocal(o->v_global_scale, out.v_gs))
      return PA_ERR_OPTIONS;
  }
  out.q_fp8 = o->q_fp8_out;
  if (out.q_fp8) {
    if (!aligned(out.q_fp8, 16)) return PA_ERR_ALIGN;
    if (!reciprocal(o->q_fp8_scale, out.q_fp8_inv)) return PA_ERR_OPTIONS;
  }
  return PA_OK;
}

// q_out may be NULL only when the FP8 q output is requested; v_cache, k_scale
// and v_scale are not used (and may be NULL) with the NVFP4 caches.
int check_ptrs(const Ptrs& p, bool has_q_fp8, bool nvfp4) {
  const void* all[] = {p.ar, p.res, p.h_out, p.g_in, p.w_packed, p.w_scales, p.g_q, p.g_k,
                       p.g_iq, p.g_ik, p.cos_sin, p.positions, p.slot_mapping, p.k_cache,
                       p.index_cache, p.iq_out, p.ws};
  for (const void* q : all)
    if (!q) return PA_ERR_NULL;
  if (!p.q_out && !has_q_fp8) return PA_ERR_NULL;
  if (!nvfp4 && (!p.v_cache || !p.k_scale || !p.v_scale)) return PA_ERR_NULL;
  const void* a16[] = {p.ar, p.res, p.h_out, p.g_in, p.w_packed, p.q_out, p.iq_out, p.g_q, p.g_k,
                       p.g_iq, p.g_ik, p.cos_sin, p.k_cache, p.v_cache, p.index_cache, p.ws};
  for (const void* q : a16)
    if (!aligned(q, 16)) return PA_ERR_ALIGN;
  const void* a8[] = {p.positions, p.slot_mapping};
  for (const void* q : a8)
    if (!aligned(q, 8)) return PA_ERR_ALIGN;
  const void* a4[] = {p.w_scales, p.k_scale, p.v_scale};
  for (const void* q : a4)
    if (!aligned(q, 4)) return PA_ERR_ALIGN;
  return PA_OK;
}

// Test hook: PA_DECODE_FORCE_PATHS=1 makes every decode GEMV CTA compute the
// token statistics itself, =2 makes no k slice wait for the others (the slice
// that arrives last runs every share of the head epilogue), =3 both. The
// outputs are the same bits either way.
uint32_t forced_paths() {
  const char* v = std::getenv("PA_DECODE_FORCE_PATHS");
  if (!v) return 0u;
  const int f = std::atoi(v);
  return ((f & 1) ? pa::kOptLocalStats : 0u) | ((f & 2) ? pa::kOptNoSliceWait : 0u);
}

pa::Args make_args(const pa_dims* d, const Ptrs& p, void* stream) {
  pa::Args a{};
  a.S = d->tokens;
  a.K = d->hidden;
  a.nkv = d->nkv;
  a.num_pages = d->num_pages;
  a.max_pos = d->max_pos;
  a.eps = d->eps;
  a.ar = p.ar;
  a.res = p.res;
  a.g_in = p.g_in;
  a.h_out = p.h_out;
  a.w_packed = p.w_packed;
  a.g_q = p.g_q;
  a.g_k = p.g_k;
  a.g_iq = p.g_iq;
  a.g_ik = p.g_ik;
  a.cos_sin = p.cos_sin;
  a.positions = p.positions;
  a.slot_mapping = p.slot_mapping;
  a.k_cache = p.k_cache;
  a.v_cache = p.v_cache;
  a.index_cache = p.index_cache;
  a.k_scale = p.k_scale;
  a.v_scale = p.v_scale;
  a.q_out = p.q_out;
  a.iq_out = p.iq_out;
  a.ws = static_cast<uint8_t*>(p.ws);
  a.stream = static_cast<hipStream_t>(stream);
  a.ev_start = g_ev_start;
  a.ev_stop = g_ev_stop;
  a.timeline = g_timeline;
  a.timeline_slots = g_timeline_slots;
  return a;
}

int run(int mode, const pa_dims* dims, const Ptrs& p, const pa_head_options* opts, size_t ws_bytes,
        void* stream) {
  int st = check_dims(dims, mode);
  if (st) return st;
  Opts o;
  st = check_opts(opts, o);
  if (st) return st;
  st = check_ptrs(p, o.q_fp8 != nullptr, o.nvfp4 != 0);
  if (st) return st;
  if (ws_bytes < workspace_for(dims, mode)) return PA_ERR_WORKSPACE;
  st = check_device();
  if (st) return st;
  pa::Args a = make_args(dims, p, stream);
  a.q_fp8 = o.q_fp8;
  a.q_fp8_inv = o.q_fp8_inv;
  a.opts = (o.static_kv ? pa::kOptStaticKv : 0u) | (o.nvfp4 ? pa::kOptNvfp4 : 0u) | forced_paths();
  a.k_gs = o.k_gs;
  a.v_gs = o.v_gs;
  hipError_t e;
  if (mode == PA_MODE_DECODE) {
    a.w_scale = static_cast<const float*>(p.w_scales);
    e = pa::launch_decode(a, pa::decode_plan(a.S, a.K, a.nkv));
  } else {
    a.s_packed = static_cast<const uint8_t*>(p.w_scales);
    e = pa::launch_prefill(a, pa::prefill_plan(a.S, a.K, a.nkv));
  }
  if (e != hipSuccess) return hip_fail(e, mode == PA_MODE_DECODE ? "pre_attn_decode" : "pre_attn_prefill");
  return PA_OK;
}

int check_pack(int32_t n_rows, int32_t hidden) {
  if (hidden < 128 || hidden > PA_MAX_HIDDEN || hidden % 128) return PA_ERR_HIDDEN;
  const int heads = n_rows / 128;
  if (n_rows % 128 || (heads - 1) % 19 || n_rows <= 0) return PA_ERR_NKV;
  const int nkv = (heads - 1) / 19;
  if (nkv != 1 && nkv != 2 && nkv != 4) return PA_ERR_NKV;
  return PA_OK;
}

// The allocation-free decode call's workspace: one array per GPU, held until
// the process ends. Host code never passes its name to a kernel (on the host
// it is a stand-in, not a device address); it uses the address
// hipGetSymbolAddress returns for the current device, taken once per device
// with that device current.
constexpr size_t kScratchBytes = size_t(24) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, cleared on its first use (the
// synchronization words must start at zero; calls leave them zero).
int scratch_for_current_device(void*& out, void* stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if ((e = pa::probe_placement(ptr, static_cast<hipStream_t>(stream))) != hipSuccess)
      return hip_fail(e, "scratch set-up");
    if ((e = pa::launch_fill_zero(ptr, kScratchBytes, static_cast<hipStream_t>(stream))) != hipSuccess)
      return hip_fail(e, "scratch clear");
    g_scratch_ptr[dev] = ptr;
  }
  out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_workspace_bytes(const pa_dims* dims, int mode) {
  if (check_dims(dims, mode) != PA_OK) return 0;
  return workspace_for(dims, mode);
}

int pa_decode_structure(const pa_dims* d) {
  const int st = check_dims(d, PA_MODE_DECODE);
  if (st != PA_OK) return st;
  const pa::DecodePlan p = pa::decode_plan(d->tokens, d->hidden, d->nkv);
  if (p.chunks_per_cta == 0) return PA_ERR_HIDDEN;
  return (p.fused ? PA_DECODE_NORM_FUSED : 0) |
         (p.fused_epilogue || p.gemv_epilogue ? PA_DECODE_EPILOGUE_FUSED : 0);
}

int pa_workspace_status(const void* workspace, void* stream) {
  if (!workspace) return PA_ERR_NULL;
  if (!aligned(workspace, 16)) return PA_ERR_ALIGN;
  uint32_t word = 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&word, static_cast<const uint8_t*>(workspace) + pa::kSyncErr, sizeof(word),
                                hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "pa_workspace_status");
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "pa_workspace_status");
  return word ? PA_ERR_SYNC : PA_OK;
}

int pa_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace) return PA_ERR_NULL;
  if (!aligned(workspace, 16)) return PA_ERR_ALIGN;
  int st = check_device();
  if (st) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (bytes >= pa::kSyncBytes && (e = pa::probe_placement(workspace, s)) != hipSuccess)
    return hip_fail(e, "pa_workspace_init");
  e = pa::launch_fill_zero(workspace, bytes, s);
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_workspace_init");
}

size_t pa_packed_weight_bytes(int mode, int32_t n_rows, int32_t hidden) {
  if (check_pack(n_rows, hidden) != PA_OK) return 0;
  if (mode == PA_MODE_DECODE) return static_cast<size_t>(n_rows) * hidden;
  if (mode == PA_MODE_PREFILL) return pa::prefill_packed_weight_bytes(n_rows, hidden);
  return 0;
}

size_t pa_packed_scale_bytes(int mode, int32_t n_rows, int32_t hidden) {
  if (check_pack(n_rows, hidden) != PA_OK) return 0;
  if (mode == PA_MODE_PREFILL) return pa::prefill_packed_scale_bytes(n_rows, hidden);
  return 0;
}

int pa_pack_weight_decode(const uint8_t* w, uint8_t* w_packed, int32_t n_rows, int32_t hidden,
                          void* stream) {
  if (!w || !w_packed) return PA_ERR_NULL;
  if (!aligned(w, 16) || !aligned(w_packed, 16)) return PA_ERR_ALIGN;
  int st = check_pack(n_rows, hidden);
  if (st) return st;
  st = check_device();
  if (st) return st;
  hipError_t e = pa::launch_pack_decode(w, w_packed, n_rows, hidden, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_pack_weight_decode");
}

int pa_pack_weight_prefill(const uint8_t* w, const uint8_t* w_e8m0, uint8_t* w_packed,
                           uint8_t* s_packed, int32_t n_rows, int32_t hidden, void* stream) {
  if (!w || !w_e8m0 || !w_packed || !s_packed) return PA_ERR_NULL;
  if (!aligned(w, 16) || !aligned(w_packed, 16) || !aligned(s_packed, 16) || !aligned(w_e8m0, 4))
    return PA_ERR_ALIGN;
  int st = check_pack(n_rows, hidden);
  if (st) return st;
  st = check_device();
  if (st) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = pa::launch_pack_prefill(w, w_e8m0, w_packed, s_packed, n_rows, hidden, s);
  if (e != hipSuccess) return hip_fail(e, "pa_pack_weight_prefill");
  bool ok = false;
  if ((e = pa::prefill_weight_range_ok(w_e8m0, n_rows, hidden, s, ok)) != hipSuccess)
    return hip_fail(e, "pa_pack_weight_prefill");
  return ok ? PA_OK : PA_ERR_WEIGHT_RANGE;
}

int pre_attn_decode(const pa_dims* dims, const uint16_t* ar, const uint16_t* res, uint16_t* h_out,
                    const uint16_t* g_in, const uint8_t* w_packed, const float* w_scale,
                    const uint16_t* g_q, const uint16_t* g_k, const uint16_t* g_iq,
                    const uint16_t* g_ik, const uint16_t* cos_sin, const int64_t* positions,
                    const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                    float* k_scale, float* v_scale, uint8_t* index_cache, uint16_t* q_out,
                    uint16_t* iq_out, void* workspace, size_t workspace_bytes, void* stream) {
  const Ptrs p{ar, res, h_out, g_in, w_packed, w_scale, g_q, g_k, g_iq, g_ik, cos_sin,
               positions, slot_mapping, k_cache, v_cache, k_scale, v_scale, index_cache,
               q_out, iq_out, workspace};
  return run(PA_MODE_DECODE, dims, p, nullptr, workspace_bytes, stream);
}

int pre_attn_decode_noalloc(const pa_dims* dims, const uint16_t* ar, const uint16_t* res, uint16_t* h_out,
                            const uint16_t* g_in, const uint8_t* w_packed, const float* w_scale,
                            const uint16_t* g_q, const uint16_t* g_k, const uint16_t* g_iq,
                            const uint16_t* g_ik, const uint16_t* cos_sin, const int64_t* positions,
                            const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                            float* k_scale, float* v_scale, uint8_t* index_cache, uint16_t* q_out,
                            uint16_t* iq_out, void* stream) {
  int st = check_dims(dims, PA_MODE_DECODE);
  if (st) return st;
  if (workspace_for(dims, PA_MODE_DECODE) > kScratchBytes) return PA_ERR_WORKSPACE;
  st = check_device();
  if (st) return st;
  void* ws = nullptr;
  st = scratch_for_current_device(ws, stream);
  if (st) return st;
  const Ptrs p{ar, res, h_out, g_in, w_packed, w_scale, g_q, g_k, g_iq, g_ik, cos_sin,
               positions, slot_mapping, k_cache, v_cache, k_scale, v_scale, index_cache,
               q_out, iq_out, ws};
  return run(PA_MODE_DECODE, dims, p, nullptr, kScratchBytes, stream);
}

int pre_attn_decode_ex(const pa_dims* dims, const pa_head_options* opts, const uint16_t* ar,
                       const uint16_t* res, uint16_t* h_out, const uint16_t* g_in,
                       const uint8_t* w_packed, const float* w_scale, const uint16_t* g_q,
                       const uint16_t* g_k, const uint16_t* g_iq, const uint16_t* g_ik,
                       const uint16_t* cos_sin, const int64_t* positions,
                       const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                       float* k_scale, float* v_scale, uint8_t* index_cache, uint16_t* q_out,
                       uint16_t* iq_out, void* workspace, size_t workspace_bytes, void* stream) {
  const Ptrs p{ar, res, h_out, g_in, w_packed, w_scale, g_q, g_k, g_iq, g_ik, cos_sin,
               positions, slot_mapping, k_cache, v_cache, k_scale, v_scale, index_cache,
               q_out, iq_out, workspace};
  return run(PA_MODE_DECODE, dims, p, opts, workspace_bytes, stream);
}

int pre_attn_prefill(const pa_dims* dims, const uint16_t* ar, const uint16_t* res,
                     uint16_t* h_out, const uint16_t* g_in, const uint8_t* w_packed,
                     const uint8_t* s_packed, const uint16_t* g_q, const uint16_t* g_k,
                     const uint16_t* g_iq, const uint16_t* g_ik, const uint16_t* cos_sin,
                     const int64_t* positions, const int64_t* slot_mapping, uint8_t* k_cache,
                     uint8_t* v_cache, float* k_scale, float* v_scale, uint8_t* index_cache,
                     uint16_t* q_out, uint16_t* iq_out, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const Ptrs p{ar, res, h_out, g_in, w_packed, s_packed, g_q, g_k, g_iq, g_ik, cos_sin,
               positions, slot_mapping, k_cache, v_cache, k_scale, v_scale, index_cache,
               q_out, iq_out, workspace};
  return run(PA_MODE_PREFILL, dims, p, nullptr, workspace_bytes, stream);
}

int pre_attn_prefill_ex(const pa_dims* dims, const pa_head_options* opts, const uint16_t* ar,
                        const uint16_t* res, uint16_t* h_out, const uint16_t* g_in,
                        const uint8_t* w_packed, const uint8_t* s_packed, const uint16_t* g_q,
                        const uint16_t* g_k, const uint16_t* g_iq, const uint16_t* g_ik,
                        const uint16_t* cos_sin, const int64_t* positions,
                        const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                        float* k_scale, float* v_scale, uint8_t* index_cache, uint16_t* q_out,
                        uint16_t* iq_out, void* workspace, size_t workspace_bytes, void* stream) {
  const Ptrs p{ar, res, h_out, g_in, w_packed, s_packed, g_q, g_k, g_iq, g_ik, cos_sin,
               positions, slot_mapping, k_cache, v_cache, k_scale, v_scale, index_cache,
               q_out, iq_out, workspace};
  return run(PA_MODE_PREFILL, dims, p, opts, workspace_bytes, stream);
}

size_t pa_drafter_workspace_bytes(const pa_drafter_dims* d) {
  if (!d || d->requests < 1 || d->requests > (1 << 20) || d->split < 1 || d->split > PA_DRAFTER_MAX_SPLIT)
    return 0;
  return pa::drafter_plan(d->requests, d->split).total;
}

int pa_drafter_attention(const pa_drafter_dims* d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* qn, const uint16_t* kn, const uint16_t* cos_sin,
                         const int64_t* positions, const int64_t* slots, uint8_t* kv_cache,
                         const int32_t* block_table, const int32_t* seq_lens, uint8_t* out_codes,
                         uint8_t* out_scales, uint16_t* out_bf16, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!d) return PA_ERR_NULL;
  if (d->requests < 1 || d->requests > (1 << 20)) return PA_ERR_TOKENS;
  if (d->num_blocks < 1 || d->table_width < 1 || d->max_pos < 1 || d->split < 1 ||
      d->split > PA_DRAFTER_MAX_SPLIT || !std::isfinite(d->eps) || d->eps < 0.0f)
    return PA_ERR_DIMS;
  const void* req[] = {q, k, v, qn, kn, cos_sin, positions, slots, kv_cache, block_table, seq_lens,
                       out_codes, out_scales, workspace};
  for (const void* p : req)
    if (!p) return PA_ERR_NULL;
  const void* a2[] = {q, k, v, qn, kn, cos_sin};
  for (const void* p : a2)
    if (!aligned(p, 2)) return PA_ERR_ALIGN;
  if (!aligned(kv_cache, 16) || !aligned(workspace, 16) || (out_bf16 && !aligned(out_bf16, 16)) ||
      !aligned(out_codes, 8) || !aligned(positions, 8) || !aligned(slots, 8) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4))
    return PA_ERR_ALIGN;
  const pa::DrafterPlan plan = pa::drafter_plan(d->requests, d->split);
  if (workspace_bytes < plan.total) return PA_ERR_WORKSPACE;
  int st = check_device();
  if (st) return st;
  pa::DArgs a{};
  a.requests = d->requests;
  a.num_blocks = d->num_blocks;
  a.table_width = d->table_width;
  a.max_pos = d->max_pos;
  a.split = d->split;
  a.eps = d->eps;
  a.q = q, a.k = k, a.v = v, a.qn = qn, a.kn = kn, a.cos_sin = cos_sin;
  a.positions = positions, a.slots = slots, a.kv_cache = kv_cache;
  a.block_table = block_table, a.seq_lens = seq_lens;
  a.out_codes = out_codes, a.out_scales = out_scales, a.out_bf16 = out_bf16;
  a.ws = static_cast<uint8_t*>(workspace);
  a.stream = static_cast<hipStream_t>(stream);
  a.ev_start = g_ev_start;
  a.ev_stop = g_ev_stop;
  a.timeline = g_timeline;
  a.timeline_slots = g_timeline_slots;
  const hipError_t e = pa::launch_drafter(a, plan);
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_drafter_attention");
}

const char* pa_strerror(int status) {
  switch (status) {
    case PA_OK: return "success";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_ALIGN: return "a pointer is misaligned (16 B data, 8 B int64, 4 B float)";
    case PA_ERR_NKV: return "nkv must be 1, 2 or 4 (n_rows = (19 nkv + 1) * 128)";
    case PA_ERR_HIDDEN: return "hidden must be a multiple of 128 in [128, 16384]";
    case PA_ERR_TOKENS: return "tokens out of range (decode 1..64, prefill 1..2^24)";
    case PA_ERR_WORKSPACE: return "workspace smaller than pa_workspace_bytes()";
    case PA_ERR_DIMS: return "num_pages and max_pos must be >= 1 and eps finite and >= 0";
    case PA_ERR_HIP: return "HIP runtime error (see pa_last_error_detail)";
    case PA_ERR_DEVICE: return "current device is not a gfx950 GPU";
    case PA_ERR_MODE: return "unknown mode";
    case PA_ERR_SYNC: return "a kernel's bounded wait gave up: that call's outputs are not valid";
    case PA_ERR_WEIGHT_RANGE:
      return "an E8M0 code of a k, v or index_k weight row is outside [10, 246]";
    case PA_ERR_OPTIONS:
      return "bad pa_head_options: a scale not finite and > 0 (or with an infinite float32 reciprocal), "
             "an unknown kv_cache_format, or static_kv_scale with NVFP4";
    default: return "unknown status";
  }
}

const char* pa_last_error_detail(void) { return g_detail; }

int pa_set_timeline(void* buffer, size_t bytes) {
  if (buffer && !aligned(buffer, 8)) return PA_ERR_ALIGN;
  g_timeline = static_cast<uint64_t*>(buffer);
  const size_t slots = buffer ? bytes / 8 : 0;
  g_timeline_slots = static_cast<uint32_t>(slots > 0xffffffffu ? 0xffffffffu : slots);
  return PA_OK;
}

int pa_set_kernel_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return PA_ERR_NULL;
  g_ev_start = static_cast<hipEvent_t>(start);
  g_ev_stop = static_cast<hipEvent_t>(stop);
  return PA_OK;
}

}  // extern "C"
