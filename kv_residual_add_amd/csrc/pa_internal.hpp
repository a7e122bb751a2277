// Internal interfaces between the C ABI (pa_abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pre_attn.h"

namespace pa {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Everything a prologue launch reads or writes (device pointers).
struct Args {
  int S, K, nkv, num_pages, max_pos;
  float eps;
  const uint16_t *ar, *res, *g_in;
  uint16_t* h_out;
  const uint8_t* w_packed;
  const float* w_scale;    // decode
  const uint8_t* s_packed; // prefill
  const uint16_t *g_q, *g_k, *g_iq, *g_ik, *cos_sin;
  const int64_t *positions, *slot_mapping;
  uint8_t *k_cache, *v_cache, *index_cache;
  float *k_scale, *v_scale;
  uint16_t *q_out, *iq_out;
  uint8_t* ws;
  hipStream_t stream;
  hipEvent_t ev_start, ev_stop;  // optional, around the dominant kernel
  uint64_t* timeline;            // optional per-CTA phase stamps (s_memrealtime)
  uint32_t timeline_slots;       // stamps available in `timeline`
  __host__ __device__ int N() const { return (19 * nkv + 1) * 128; }
  __host__ __device__ int heads() const { return 19 * nkv + 1; }
};

// Decode: split of the GEMV's k range and the workspace carve-up.
struct DecodePlan {
  int chunks_per_cta;  // 128-wide k chunks per CTA
  int ksplit;          // CTAs along k
  bool fused;          // norm and GEMV in one launch (a per-XCD copy of the FP8 rows)
  bool fused_epilogue; // the head epilogue in that launch too
  size_t off_x8, off_sx, off_rstd, off_part, off_done, off_hdone, off_err, total;
};
DecodePlan decode_plan(int S, int K, int nkv);
hipError_t launch_decode(const Args& a, const DecodePlan& p);
hipError_t launch_pack_decode(const uint8_t* w, uint8_t* wp, int N, int K, hipStream_t s);

// Prefill.
struct PrefillPlan {
  size_t off_xq, off_xs, off_cnt, total;
};
PrefillPlan prefill_plan(int M, int K, int nkv);
hipError_t launch_prefill(const Args& a, const PrefillPlan& p);
hipError_t launch_pack_prefill(const uint8_t* w, const uint8_t* ws, uint8_t* wp, uint8_t* sp,
                               int N, int K, hipStream_t s);
size_t prefill_packed_weight_bytes(int N, int K);
size_t prefill_packed_scale_bytes(int N, int K);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

inline hipError_t mark(hipEvent_t ev, hipStream_t s) {
  return ev ? hipEventRecord(ev, s) : hipSuccess;
}

}  // namespace pa
