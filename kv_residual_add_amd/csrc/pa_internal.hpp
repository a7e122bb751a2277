// Internal interfaces between the C ABI (pa_abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pre_attn.h"

namespace pa {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Everything a prologue kernel reads or writes (device pointers), passed by
// value as the kernels' argument block: host-only state stays in Args below,
// so the block does not grow with it.
constexpr uint32_t kOptStaticKv = 1u;  // unit K / V scales
constexpr uint32_t kOptNvfp4 = 2u;     // NVFP4 caches (k_cache = K/V cache, index_cache NVFP4)
// Fall-back paths of the decode hand-offs, forced from the host for tests
// (PA_DECODE_FORCE_PATHS): every GEMV CTA computes the token statistics itself;
// no k slice waits for the others (the last arriver runs every share).
constexpr uint32_t kOptLocalStats = 4u;
constexpr uint32_t kOptNoSliceWait = 8u;

struct KArgs {
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
  uint16_t *q_out, *iq_out;      // q_out may be NULL when q_fp8 is set
  uint8_t* q_fp8;                // optional E4M3 q [S][16 nkv][128]
  float q_fp8_inv;               // float32(1 / q_fp8_scale)
  uint32_t opts;                 // kOpt* flags
  float k_gs, v_gs;              // NVFP4: float32(1 / global scale) of K and V
  uint8_t* ws;
  uint64_t* timeline;            // optional per-CTA phase stamps (s_memrealtime)
  uint32_t timeline_slots;       // stamps available in `timeline`
  __host__ __device__ int N() const { return (19 * nkv + 1) * 128; }
  __host__ __device__ int heads() const { return 19 * nkv + 1; }
  __host__ __device__ bool static_kv() const { return (opts & kOptStaticKv) != 0; }
  __host__ __device__ bool kv_nvfp4() const { return (opts & kOptNvfp4) != 0; }
};

// A call: the kernels' arguments plus the host-side launch state.
struct Args : KArgs {
  hipStream_t stream;
  hipEvent_t ev_start, ev_stop;  // optional, around the dominant kernel
};

// The words kernels synchronize through (flags, counters, published
// statistics, the failure word) sit at the start of every workspace at fixed
// offsets, whatever the call's dims and mode, and every call leaves them zero.
// Data regions start past them, so one workspace can serve calls of any shape
// in turn without a stale data byte ever reading as a flag.
constexpr size_t kSyncErr = 0;             // failure word: a call's outputs are not valid
constexpr size_t kSyncDone = 256;          // per-XCD GEMV counters, 128 bytes apart
constexpr size_t kSyncPub = 1280;          // per-XCD published rstd and scale words
constexpr size_t kSyncPubBytes = 2 * 8 * 64 * sizeof(uint64_t);
// per-head counters of the k slices (started, arrived, bailed-out mask, done),
// one 256-byte record per head
constexpr size_t kSyncHeadFlags = kSyncPub + kSyncPubBytes;
constexpr int kSyncMaxHeads = 19 * 4 + 1;  // heads at the largest nkv
constexpr int kSyncMaxSlices = 64;         // words per head record
constexpr size_t kSyncHeadCnt = kSyncHeadFlags + kSyncMaxHeads * kSyncMaxSlices * sizeof(uint32_t);
constexpr size_t kSyncBytes = 32768;
static_assert(kSyncHeadCnt + kSyncMaxHeads * sizeof(uint32_t) <= kSyncBytes, "synchronization words overflow");

// Decode: split of the GEMV's k range and the workspace carve-up.
struct DecodePlan {
  int chunks_per_cta;  // 128-wide k chunks per CTA
  int ksplit;          // CTAs along k
  bool fused;          // norm and GEMV in one launch (a per-XCD copy of the FP8 rows)
  bool fused_epilogue; // the head epilogue in that launch too
  bool gemv_epilogue;  // not fused: the head epilogue in the GEMV's launch
  size_t off_x8, off_sx, off_rstd, off_part, off_done, off_hdone, off_err, total;
};
DecodePlan decode_plan(int S, int K, int nkv);
hipError_t launch_decode(const Args& a, const DecodePlan& p);
hipError_t launch_pack_decode(const uint8_t* w, uint8_t* wp, int N, int K, hipStream_t s);

// Prefill.
struct PrefillPlan {
  size_t off_xq, off_xs, total;
};
PrefillPlan prefill_plan(int M, int K, int nkv);
hipError_t launch_prefill(const Args& a, const PrefillPlan& p);
hipError_t launch_pack_prefill(const uint8_t* w, const uint8_t* ws, uint8_t* wp, uint8_t* sp,
                               int N, int K, hipStream_t s);
// Whether every E8M0 code of the k, v and index_k rows admits the exact bf16
// widening (synchronizes s).
hipError_t prefill_weight_range_ok(const uint8_t* we, int N, int K, hipStream_t s, bool& ok);
size_t prefill_packed_weight_bytes(int N, int K);
size_t prefill_packed_scale_bytes(int N, int K);

// The DSpark drafter's attention (pa_drafter.hip).
struct DArgs {
  int requests, num_blocks, table_width, max_pos, split, nsplit;
  float eps;
  const uint16_t *q, *k, *v, *qn, *kn, *cos_sin;
  const int64_t *positions, *slots;
  uint8_t* kv_cache;
  const int32_t *block_table, *seq_lens;
  uint8_t *out_codes, *out_scales;
  uint16_t* out_bf16;  // optional
  uint8_t* ws;
  uint8_t* q8;         // workspace: the rows' q codes [7 R][16][128]
  float* part;         // workspace: partials [7 R][nsplit][16][2 + 128]
  int32_t* blocks;     // workspace: per request lo, hi, first and last block, then its physical blocks
  uint64_t* timeline;  // phase stamps (pa_set_timeline), or null
  uint32_t timeline_slots;
  hipStream_t stream;
  hipEvent_t ev_start, ev_stop;
};
struct DrafterPlan {
  int nsplit;  // partitions per request (34 blocks / split, rounded up)
  size_t off_q8, off_part, off_blocks, total;
};
DrafterPlan drafter_plan(int requests, int split);
hipError_t launch_drafter(const DArgs& a, const DrafterPlan& p);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t probe_placement(void* ws, hipStream_t s);

inline hipError_t mark(hipEvent_t ev, hipStream_t s) {
  return ev ? hipEventRecord(ev, s) : hipSuccess;
}

}  // namespace pa
