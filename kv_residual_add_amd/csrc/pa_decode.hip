// Decode prologue on gfx950: per-token FP8 activations against a per-row
// scaled FP8 weight, for up to 64 tokens.
//
// The stages (the K1 mono_pre page, vllm.models.minimax_m3.amd.mono.kernels.
// pre_attn, emit_pre_attn: norm tasks, GEMV tasks, head tasks):
//   norm      per token: residual add (f32) + bf16 residual out, Gemma RMSNorm,
//             per-token FP8 quantization (norm_quant).
//   GEMV      the fused projection as an HBM-bound GEMV: a CTA owns one 128-row
//             head x a k slice; every wave streams its 32 rows' packed weight
//             with dwordx4 loads issued before anything waits on them, the FP8
//             activation slice sits in LDS, and 32x32x16 bf16 MFMAs take up to
//             32 tokens a tile on exactly widened FP8 codes. k-slice partial
//             sums go to the workspace.
//   epilogue  per (token, head), one wave: sums the k-slice partials in a fixed
//             order, applies the activation and row scales, then the head's role
//             (head tasks; head_norm_rope; the epilogue page
//             vllm.models.minimax_m3.nvidia.ops.qkv_index_fused_epilogue,
//             per-role branches).
// Launches (decode_plan): up to 16 tokens, norm and GEMV share one launch
// (decode_fused: each XCD computes the tokens' norm statistics, and its GEMV
// CTAs take them from that XCD's L2 while their weights stream), and the
// epilogue joins it when the weight is small; otherwise decode_norm,
// decode_gemv and decode_epilogue are launches of their own. A hand-off across
// XCDs inside a launch (L2 write-back on publish, invalidate on acquire)
// measured slower than kernel boundaries under graph replay; one inside an
// XCD's L2 did not.
//
// Head-step options (pre_attn_decode_ex, runtime flags read by the epilogue):
// unit K / V scales (the K1 mono_pre page's STATIC_KV_SCALE), an FP8 q output
// (the epilogue page's q_fp8_out), and the epilogue page's NVFP4 K / V /
// index_k caches (E2M1 codes with an E4M3 scale per 16 values, 16-lane group
// maxima by shuffles).
//
// Numerics: the input norm, its FP8 decision and the head epilogue run in
// float64 with contraction off, so a code is decided from the same value the
// float64 statement of the method gives; the projection's products are exact
// and accumulate in float32 (FP8-input MFMAs sum at lower internal precision,
// which moves the per-token K / V scales by ~1e-5, so the codes are widened to
// bf16 first).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr int kLdsPad = 16;
// Where the activation slice's LDS has room for it, a GEMV CTA's partial sums
// leave through LDS, a wave's 32 tokens x 32 rows at a time (each token's 32
// floats padded to 144 bytes)
constexpr int kPartRowBytes = 144;
constexpr int kPartStageBytes = 4 * 32 * kPartRowBytes;
constexpr int kMaxLds = 64 * 1024;
// one launch for norm + GEMV: up to this many tokens and hidden <= 8192 (the
// norm at 256 threads then holds at most four 8-element vectors a thread)
constexpr int kFusedMaxS = 16;
constexpr int kFusedMaxK = 8192;
constexpr int kSxStride = 64;    // scale floats per XCD copy (and published words per XCD)
constexpr int kMaxKsplit = kSyncMaxSlices;  // slice flags per head
constexpr size_t kFusedEpiMaxWeight = 4u << 20;  // weight bytes up to which whole heads per XCD pay
// GEMV + epilogue launch: a head's slices sit on one XCD and hand their partial
// sums over in its L2; at most one slice per CU of an XCD and one bit each in
// a 32-bit mask
constexpr int kGemvEpiMaxKsplit = 32;

// Block reductions over up to 16 waves: each wave's result goes to LDS, then
// every thread combines the waves' values in the same fixed order (pairwise).
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = static_cast<int>(blockDim.x >> 6);
  if (lane == 0) red[wave] = v;
  for (int w = nw; w < 16; ++w)
    if (threadIdx.x == 0) red[w] = 0.0;
  __syncthreads();
  double t[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) t[w] = red[w] + red[w + 8];
#pragma unroll
  for (int w = 0; w < 4; ++w) t[w] += t[w + 4];
  const double r = (t[0] + t[2]) + (t[1] + t[3]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ double block_max_f64(double v, double* red) {
  v = wave_max_f64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = static_cast<int>(blockDim.x >> 6);
  if (lane == 0) red[wave] = v;
  for (int w = nw; w < 16; ++w)
    if (threadIdx.x == 0) red[w] = 0.0;
  __syncthreads();
  double t[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) t[w] = __builtin_fmax(red[w], red[w + 8]);
#pragma unroll
  for (int w = 0; w < 4; ++w) t[w] = __builtin_fmax(t[w], t[w + 4]);
  const double r = __builtin_fmax(__builtin_fmax(t[0], t[2]), __builtin_fmax(t[1], t[3]));
  __syncthreads();
  return r;
}

// One block reduction of (sum, top two of per-thread maxima) over up to 16
// waves: the sum in the same fixed order as block_sum_f64; m1 the largest
// contribution and m2 the second largest, counting each thread once (the DPP
// steps and the LDS tree combine disjoint sets of threads, as for the sum).
// Values are >= 0. red holds 48 doubles; the reduction leaves them in use.
__device__ __forceinline__ void top2_merge(double& m1, double& m2, double b1, double b2) {
  const double lo = __builtin_fmin(m1, b1);
  m1 = __builtin_fmax(m1, b1);
  m2 = __builtin_fmax(lo, __builtin_fmax(m2, b2));
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ void dpp_sum_top2(double& v, double& m1, double& m2) {
  const double bv = dpp_f64<kCtrl, kRowMask>(v, 0.0);
  const double b1 = dpp_f64<kCtrl, kRowMask>(m1, 0.0);
  const double b2 = dpp_f64<kCtrl, kRowMask>(m2, 0.0);
  v += bv;
  top2_merge(m1, m2, b1, b2);
}

__device__ __forceinline__ void block_sum_top2_f64(double& v, double& m1, double& m2, double* red) {
  dpp_sum_top2<0xB1, 0xf>(v, m1, m2);   // quad_perm [1,0,3,2]
  dpp_sum_top2<0x4E, 0xf>(v, m1, m2);   // quad_perm [2,3,0,1]
  dpp_sum_top2<0x141, 0xf>(v, m1, m2);  // row_half_mirror
  dpp_sum_top2<0x140, 0xf>(v, m1, m2);  // row_mirror
  dpp_sum_top2<0x142, 0xa>(v, m1, m2);  // row_bcast:15 into rows 1, 3
  dpp_sum_top2<0x143, 0xc>(v, m1, m2);  // row_bcast:31 into rows 2, 3
  v = lane63_f64(v);
  m1 = lane63_f64(m1);
  m2 = lane63_f64(m2);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = static_cast<int>(blockDim.x >> 6);
  if (lane == 0) red[wave] = v, red[16 + wave] = m1, red[32 + wave] = m2;
  if (threadIdx.x < 16 && threadIdx.x >= nw) red[threadIdx.x] = 0.0, red[16 + threadIdx.x] = 0.0, red[32 + threadIdx.x] = 0.0;
  __syncthreads();
  double t[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) t[w] = red[w] + red[w + 8];
#pragma unroll
  for (int w = 0; w < 4; ++w) t[w] += t[w + 4];
  v = (t[0] + t[2]) + (t[1] + t[3]);
  double a1 = red[16], a2 = red[32];
  for (int w = 1; w < 16; ++w) top2_merge(a1, a2, red[16 + w], red[32 + w]);
  m1 = a1;
  m2 = a2;
  // no trailing barrier: its one caller runs it once per CTA and gives the
  // fallback reduction a region of its own (red + 48)
}

// ---------------------------------------------------------------------------
// norm: residual add + Gemma RMSNorm + per-token FP8 for token `row`; thread
// t owns the 8-element vectors t, t + blockDim.x, ... (NV of them). The element
// loops stay rolled: each wave runs this code once, so its size, not its
// instruction count, sets the time.
// With CODES false the row's FP8 codes are left to the GEMV CTAs (codes8),
// which take the row's rstd and scale from *rstd_out and *s_out (rstd in every
// thread, the scale in the row's owner thread, see below).
// Without CODES the row's scale comes from one block reduction instead of two:
// the exact products y = |acc| (1 + g) (a float32 times a 9-bit value, exact in
// float64) order the normalized values |xn| = RN(RN(|acc| rstd) (1 + g)) except
// within 2^-50 relative of each other. When the largest per-thread y is clear
// of the second by more than that, the one thread holding it computes the
// row's max |xn| from its own values and is the row's owner (*owner_out): it
// alone holds the scale. Otherwise (near-ties, or an all-zero row) the second
// reduction runs as with CODES and thread 0 is the owner.
template <int NV, bool CODES = true>
__device__ __forceinline__ void norm_token(const KArgs& a, int row, uint8_t* __restrict__ x8,
                                           float* __restrict__ sx, double* red, int tl, bool write_h = true,
                                           double* rstd_out = nullptr, float* s_out = nullptr,
                                           bool* owner_out = nullptr) {
#pragma clang fp contract(off)
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int K = a.K;
  const int nvec = K >> 3;
  const size_t base = static_cast<size_t>(row) * K;
  uint4 av[NV], bv[NV], gv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {  // every load in flight before any use
    const int v = tid + i * nthreads;
    av[i] = bv[i] = gv[i] = make_uint4(0u, 0u, 0u, 0u);
    if (v < nvec) {
      av[i] = *reinterpret_cast<const uint4*>(a.ar + base + 8 * v);
      bv[i] = *reinterpret_cast<const uint4*>(a.res + base + 8 * v);
      gv[i] = *reinterpret_cast<const uint4*>(a.g_in + 8 * v);
    }
  }
  stamp(a.timeline, a.timeline_slots, tl, 0);
  float acc[NV][8];
  double ssp[4] = {0.0, 0.0, 0.0, 0.0};  // four chains, combined pairwise
  uint32_t hw[NV][4];  // the bf16 residual, stored with the codes at the end
  double ymine = 0.0, y1 = 0.0, y2 = 0.0;  // this thread's largest y; the row's two largest
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint32_t aw[4] = {av[i].x, av[i].y, av[i].z, av[i].w};
    const uint32_t bw[4] = {bv[i].x, bv[i].y, bv[i].z, bv[i].w};
    const uint32_t gw[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[i][2 * q] = bf16_to_f32(aw[q] & 0xffffu) + bf16_to_f32(bw[q] & 0xffffu);
      acc[i][2 * q + 1] = bf16_to_f32(aw[q] >> 16) + bf16_to_f32(bw[q] >> 16);
      hw[i][q] = pack_bf16x2(acc[i][2 * q], acc[i][2 * q + 1]);
      // a float32 square is exact in float64: the fma rounds only the sum
      ssp[q] = __builtin_fma(static_cast<double>(acc[i][2 * q]), static_cast<double>(acc[i][2 * q]), ssp[q]);
      ssp[q] = __builtin_fma(static_cast<double>(acc[i][2 * q + 1]), static_cast<double>(acc[i][2 * q + 1]), ssp[q]);
      if constexpr (!CODES) {
        ymine = __builtin_fmax(ymine, __builtin_fabs(static_cast<double>(acc[i][2 * q]) *
                                                     (1.0 + static_cast<double>(bf16_to_f32(gw[q] & 0xffffu)))));
        ymine = __builtin_fmax(ymine, __builtin_fabs(static_cast<double>(acc[i][2 * q + 1]) *
                                                     (1.0 + static_cast<double>(bf16_to_f32(gw[q] >> 16)))));
      }
    }
  }
  stamp(a.timeline, a.timeline_slots, tl, 1);
  double ss;
  if constexpr (CODES) {
    ss = block_sum_f64((ssp[0] + ssp[1]) + (ssp[2] + ssp[3]), red);
  } else {
    ss = (ssp[0] + ssp[1]) + (ssp[2] + ssp[3]);
    y1 = ymine;
    block_sum_top2_f64(ss, y1, y2, red);
  }
  stamp(a.timeline, a.timeline_slots, tl, 2);
  const double rstd = 1.0 / __builtin_sqrt(ss / static_cast<double>(K) + static_cast<double>(a.eps));
  double xn[NV][8];
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint32_t gw[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w};
    double m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t gb = (gw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      xn[i][e] = (static_cast<double>(acc[i][e]) * rstd) * (1.0 + static_cast<double>(bf16_to_f32(gb)));
      m[e] = __builtin_fabs(xn[i][e]);
    }
    const double mm = __builtin_fmax(__builtin_fmax(__builtin_fmax(m[0], m[1]), __builtin_fmax(m[2], m[3])),
                                     __builtin_fmax(__builtin_fmax(m[4], m[5]), __builtin_fmax(m[6], m[7])));
    amax = __builtin_fmax(amax, mm);
  }
  stamp(a.timeline, a.timeline_slots, tl, 3);
  bool owner = threadIdx.x == 0;
  // one clear maximum (uniform: every thread holds the same y1, y2): its thread's
  // own max |xn| is the row's; else the second reduction
  const bool clear = !CODES && y2 < y1 * (1.0 - 0x1p-50);
  if (clear)
    owner = ymine == y1;
  else
    amax = block_max_f64(amax, !CODES ? red + 48 : red);
  stamp(a.timeline, a.timeline_slots, tl, 4);
  const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
  const double sd = static_cast<double>(s);
  const double rcp = 1.0 / sd;
  const Fp8Scale unit = fp8_scale(0);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    uint32_t w[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      w[j] = e4m3x4_scaled(div_rn(xn[i][4 * j], sd, rcp), div_rn(xn[i][4 * j + 1], sd, rcp),
                           div_rn(xn[i][4 * j + 2], sd, rcp), div_rn(xn[i][4 * j + 3], sd, rcp), unit);
    const int v = tid + i * nthreads;
    if (CODES && v < nvec) *reinterpret_cast<uint2*>(x8 + base + 8 * v) = make_uint2(w[0], w[1]);
    if (v < nvec && write_h)
      *reinterpret_cast<uint4*>(a.h_out + base + 8 * v) = make_uint4(hw[i][0], hw[i][1], hw[i][2], hw[i][3]);
  }
  if (owner) sx[row] = s;
  if (rstd_out != nullptr) *rstd_out = rstd;
  if (s_out != nullptr) *s_out = s;
  if (owner_out != nullptr) *owner_out = owner;
  stamp(a.timeline, a.timeline_slots, tl, 5);
}

// The FP8 codes of eight consecutive row elements from their 16-byte pieces of
// ar, res and g_in, given the row's rstd and scale: the norm's own expressions,
// so the codes are the ones norm_token would store.
__device__ __forceinline__ uint2 codes8(const u32x4& av, const u32x4& bv, const u32x4& gv, double rstd, double sd,
                                        double rcp) {
#pragma clang fp contract(off)
  double xn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float acc = bf16_at_f32(av, e) + bf16_at_f32(bv, e);
    xn[e] = (static_cast<double>(acc) * rstd) * (1.0 + static_cast<double>(bf16_at_f32(gv, e)));
  }
  const Fp8Scale unit = fp8_scale(0);
  return make_uint2(e4m3x4_scaled(div_rn(xn[0], sd, rcp), div_rn(xn[1], sd, rcp), div_rn(xn[2], sd, rcp),
                                  div_rn(xn[3], sd, rcp), unit),
                    e4m3x4_scaled(div_rn(xn[4], sd, rcp), div_rn(xn[5], sd, rcp), div_rn(xn[6], sd, rcp),
                                  div_rn(xn[7], sd, rcp), unit));
}

// ---------------------------------------------------------------------------
// GEMV. Packed weight: head h, 128-wide k chunk c, 32-row tile m -> a 4 KB
// block at ((h * K/128 + c) * 4 + m) * 4096. Its dwordx4 piece q of lane l sits
// at q * 1024 + 16 l (each wave load is 1 KB contiguous) and holds row
// 32m + l % 32 for MFMA steps j = 2q and 2q + 1, each 8 codes at
// k = 128c + 16j + 8 (l / 32) + [0, 8). The activation B operand takes the same
// k from LDS, so the dot product needs no shuffles. Tokens past S reuse token
// S-1 and are never stored. NT = 32-token tiles (1 or 2).
// What a GEMV CTA of the single-launch decode takes from the norm CTAs of its
// XCD: each token's rstd and FP8 scale, published in the XCD's L2.
constexpr int kSpinMax = 1 << 18;  // polls before a wait gives up (well under a second)

struct Publish {
  const uint64_t* rstd;  // this XCD's per-token rstd bits (0: not yet; a real rstd is > 0)
  const uint64_t* srec;  // this XCD's per-token scale bits, tagged 1 in the upper half (0: not yet)
  float* sx;             // this XCD's per-token scales, read by the head epilogue
  uint32_t* done;        // this XCD's count of GEMV CTAs done with the values
  uint32_t* err;         // the call's failure word
  bool handoff;          // take the statistics from the XCD's norm CTAs (else compute them here)
};

// Records that this call's outputs are not valid (read by pa_workspace_status).
__device__ __forceinline__ void mark_invalid(uint32_t* err) {
  __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until the XCD's S tokens are published and returns this lane's token's
// rstd and scale (lanes t < S; the others get token 0's). Each value is one
// naturally aligned 8-byte word written once per call, and it carries its own
// readiness, so no flag and no store order is needed; a lane polls its token's
// two words with agent-scope loads (not served by the CU's L1; they read the
// XCD's L2, where the norm CTAs' plain stores land). The norm CTAs come first
// in dispatch order, so they are running or done; the wait is still bounded,
// and returns false if it gave up (the caller then computes the values itself).
__device__ __forceinline__ bool wait_stats(const Publish& pub, int S, double& rstd, float& sc) {
  const int lane = threadIdx.x & 63;
  const int t = lane < S ? lane : 0;
  uint64_t r = 0, c = 0;
  bool ok = true;
  for (int it = 0;; ++it) {
    r = __hip_atomic_load(const_cast<uint64_t*>(pub.rstd) + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    c = __hip_atomic_load(const_cast<uint64_t*>(pub.srec) + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool ready = r != 0 && (c >> 32) == 1;
    if (__builtin_amdgcn_ballot_w64(lane < S && !ready) == 0ull) break;
    if (it == kSpinMax) {
      ok = false;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  asm volatile("" ::: "memory");
  rstd = __longlong_as_double(static_cast<long long>(r));
  sc = __uint_as_float(static_cast<uint32_t>(c));
  return ok;
}


// Waits until the counter reaches n (an agent-scope load, served by the XCD's
// L2, where the counter's atomics execute). Bounded: returns false if it gave
// up, so every wave finishes.
__device__ __forceinline__ bool wait_count(const uint32_t* counter, uint32_t n) {
  bool ok = true;
  for (int it = 0;; ++it) {
    if (__hip_atomic_load(const_cast<uint32_t*>(counter), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) break;
    if (it == kSpinMax) {
      ok = false;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  asm volatile("" ::: "memory");  // the loads after the wait stay after it
  return ok;
}

// The token statistics (rstd and FP8 scale) of every row, computed by this CTA
// alone: the fall-back of a GEMV CTA whose wait for its XCD's published values
// gave up (and the path the host can force for tests). The same numbers as
// norm_token's: the sum of squares in the same per-thread chains and block
// reduction order (thread t owns the 8-element vectors t, t + 256, ...), then
// the largest |xn| over the row, which is the value norm_token's owner finds.
// Lane t of every wave gets token t's values, and thread 0 writes the XCD's
// copy of each row's scale. Few registers: the forced path runs it before the
// weight stream is issued, and the weights are in registers when a wait gives
// up only in that rare case.
template <int NV>
__device__ __forceinline__ void local_stats(const KArgs& a, float* sx, double* red, double& rstd_l, float& sc_l) {
#pragma clang fp contract(off)
  const int tid = threadIdx.x, lane = tid & 63;
  const int K = a.K, nvec = K >> 3;
  for (int t = 0; t < a.S; ++t) {
    const size_t base = static_cast<size_t>(t) * K;
    double ssp[4] = {0.0, 0.0, 0.0, 0.0};
#pragma nounroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * 256;
      if (v >= nvec) break;
      const u32x4 av = *reinterpret_cast<const u32x4*>(a.ar + base + 8 * v);
      const u32x4 bv = *reinterpret_cast<const u32x4*>(a.res + base + 8 * v);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double lo = static_cast<double>(bf16_at_f32(av, 2 * q) + bf16_at_f32(bv, 2 * q));
        const double hi = static_cast<double>(bf16_at_f32(av, 2 * q + 1) + bf16_at_f32(bv, 2 * q + 1));
        ssp[q] = __builtin_fma(lo, lo, ssp[q]);
        ssp[q] = __builtin_fma(hi, hi, ssp[q]);
      }
    }
    const double ss = block_sum_f64((ssp[0] + ssp[1]) + (ssp[2] + ssp[3]), red);
    const double rstd = 1.0 / __builtin_sqrt(ss / static_cast<double>(K) + static_cast<double>(a.eps));
    double amax = 0.0;
#pragma nounroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * 256;
      if (v >= nvec) break;
      const u32x4 av = *reinterpret_cast<const u32x4*>(a.ar + base + 8 * v);
      const u32x4 bv = *reinterpret_cast<const u32x4*>(a.res + base + 8 * v);
      const u32x4 gv = *reinterpret_cast<const u32x4*>(a.g_in + 8 * v);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float acc = bf16_at_f32(av, e) + bf16_at_f32(bv, e);
        const double xn = (static_cast<double>(acc) * rstd) * (1.0 + static_cast<double>(bf16_at_f32(gv, e)));
        amax = __builtin_fmax(amax, __builtin_fabs(xn));
      }
    }
    amax = block_max_f64(amax, red);
    const float sc = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
    if (lane == t) rstd_l = rstd, sc_l = sc;
    if (tid == 0) sx[t] = sc;
  }
}

// One GEMV CTA: head h, k chunks [ks * CPC, + CPC). With a Publish (FUSED),
// the weight stream and the CTA's slice of ar, res and g_in go out first;
// once the XCD's norm CTAs have published each token's rstd and scale, the CTA
// forms its slice's FP8 codes itself (codes8) straight into LDS.
template <int CPC, int NT, bool FUSED, int NV = 1>
__device__ __forceinline__ uint32_t gemv_tile(const KArgs& a, int h, int ks, const uint8_t* x8, float* part, int tlb,
                                              const Publish& pub, double* red = nullptr) {
  uint32_t done_before = 0;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S, K = a.K, N = a.N();
  const int nchk = K >> 7;
  constexpr int ldw = CPC * 128 + kLdsPad;
  stamp(a.timeline, a.timeline_slots, tlb, 0);

  double rstd_l = 0.0;  // FUSED: token lane's rstd and scale
  float sc_l = 0.f;
  if constexpr (FUSED) {
    if (!pub.handoff) local_stats<NV>(a, pub.sx, red, rstd_l, sc_l);  // uniform over the launch
  }
  const int per_row = CPC * 8;  // 16-byte pieces per token row
  constexpr int kMaxPieces = 64 * CPC * 8 / 256;
  i32x4 xv[kMaxPieces];
  const auto load_rows = [&]() {
    const auto xr = panel(x8, static_cast<size_t>(S) * K);
#pragma unroll
    for (int r = 0; r < kMaxPieces; ++r) {
      const int i = tid + r * 256;
      const int s = i / per_row, j = i - s * per_row;
      // past the S rows the offset is past the panel: the load reads zeros
      const uint32_t off = i < S * per_row ? static_cast<uint32_t>(s * K + ks * CPC * 128 + j * 16) : 0x7ffffff0u;
      xv[r] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
    }
  };
  // without a publisher the activation slice goes to LDS before any weight
  // load is issued: behind the grid's weight requests it would arrive only once
  // they all had, and the MFMAs below could not start on the first chunks
  // while the later ones stream
  if constexpr (!FUSED) {
    load_rows();
#pragma unroll
    for (int r = 0; r < kMaxPieces; ++r) {
      const int i = tid + r * 256;
      if (i < S * per_row) {
        const int s = i / per_row, j = i - s * per_row;
        *reinterpret_cast<i32x4*>(lds + s * ldw + j * 16) = xv[r];
      }
    }
    __syncthreads();
    stamp(a.timeline, a.timeline_slots, tlb, 2);
  }
  // with one, the raw slice: 8-element groups i = tid + 256 r, token i / (16 CPC)
  constexpr int kGroups = CPC;  // per thread: at most 16 tokens x 16 CPC groups over 256 threads
  u32x4 ga[FUSED ? kGroups : 1], gb[FUSED ? kGroups : 1], gg[FUSED ? kGroups : 1];
  if constexpr (FUSED) {
    const auto pa = panel(a.ar, static_cast<size_t>(S) * K * 2), pr = panel(a.res, static_cast<size_t>(S) * K * 2);
    const auto pg = panel(a.g_in, static_cast<size_t>(K) * 2);
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
      const int i = tid + 256 * r;
      const int s = i / (16 * CPC), j = i - s * 16 * CPC;
      const bool in = i < S * 16 * CPC;
      const uint32_t k = static_cast<uint32_t>(ks * CPC * 128 + j * 8);
      ga[r] = __builtin_amdgcn_raw_buffer_load_b128(pa, in ? 2u * (s * K + k) : 0x7ffffff0u, 0, 0);
      gb[r] = __builtin_amdgcn_raw_buffer_load_b128(pr, in ? 2u * (s * K + k) : 0x7ffffff0u, 0, 0);
      gg[r] = __builtin_amdgcn_raw_buffer_load_b128(pg, in ? 2u * k : 0x7ffffff0u, 0, 0);
    }
  }
  i32x4 wv[CPC][4];
  const uint8_t* wb = a.w_packed + ((static_cast<size_t>(h) * nchk + ks * CPC) * 4 + wave) * 4096 + lane * 16;
#pragma unroll
  for (int c = 0; c < CPC; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      wv[c][q] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wb + c * 16384 + q * 1024));
  // Every weight load is issued before the first MFMA. Left to itself the
  // scheduler sinks each load next to its MFMAs (fewer live registers), which
  // keeps two or three of a wave's loads in flight instead of all of them.
  // (With a publisher the widening below already needs them all first.)
  if constexpr (!FUSED) __builtin_amdgcn_sched_barrier(0);
  // with a publisher, the weights are widened while the norm statistics are
  // still on their way (off the critical path)
  bf16x8 aw[FUSED ? CPC : 1][FUSED ? 8 : 1];
  if constexpr (FUSED) {
#pragma unroll
    for (int c = 0; c < CPC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const i32x4& w = wv[c][j >> 1];
        aw[c][j] = fp8x8_to_bf16(w[2 * (j & 1)], w[2 * (j & 1) + 1], 1.0f);
      }
  }
  if constexpr (FUSED) {
    // lane t holds token t's values: from the XCD's norm CTAs, or computed
    // here when the wait gives up (every wave of the CTA decides alike)
    if (pub.handoff) {
      __shared__ int s_ok[4];
      const bool ok = wait_stats(pub, S, rstd_l, sc_l);
      if (lane == 0) s_ok[wave] = ok;
      __syncthreads();
      if (!(s_ok[0] && s_ok[1] && s_ok[2] && s_ok[3])) local_stats<NV>(a, pub.sx, red, rstd_l, sc_l);
    }
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
      const int i = tid + 256 * r;
      const int s = i / (16 * CPC), j = i - s * 16 * CPC;
      const int src = s < S ? s : 0;
      const double rstd = __shfl(rstd_l, src, 64);
      const double sd = static_cast<double>(__shfl(sc_l, src, 64));
      if (i < S * 16 * CPC)
        *reinterpret_cast<uint2*>(lds + s * ldw + j * 8) = codes8(ga[r], gb[r], gg[r], rstd, sd, 1.0 / sd);
    }
    __syncthreads();
    // the CTA is done with the published values: counted now, so that the
    // counter's round trip overlaps the MFMAs (its value is looked at last)
    if (threadIdx.x == 0)
      done_before = __hip_atomic_fetch_add(pub.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  const int hh = lane >> 5;
  const uint8_t* brow[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) brow[tt] = lds + min(tt * 32 + (lane & 31), S - 1) * ldw + 8 * hh;
  f32x16 acc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[tt][r] = 0.f;
#pragma unroll
  for (int c = 0; c < CPC; ++c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16x8 A;
      if constexpr (FUSED) {
        A = aw[c][j];
      } else {
        const i32x4& w = wv[c][j >> 1];
        A = fp8x8_to_bf16(w[2 * (j & 1)], w[2 * (j & 1) + 1], 1.0f);
      }
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const uint2 bv = *reinterpret_cast<const uint2*>(brow[tt] + c * 128 + 16 * j);
        const bf16x8 B = fp8x8_to_bf16(bv.x, bv.y, 1.0f);
        acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[tt], 0, 0, 0);
      }
    }
  }
  // D[i][j]: token j = lane % 32, row i = 8 (r / 4) + 4 (lane / 32) + r % 4:
  // a token's 32 rows of this wave's tile (one 128-byte line of the partial
  // sums) are spread over lanes t and t + 32. Where the activation slice's LDS
  // can hold them (at 4 chunks a CTA: 35 or more tokens) they go through LDS
  // so that each store instruction writes whole lines (8 lanes a token): for
  // the 64-token workload the step is ~1.2 us shorter than with each line
  // written in 32-byte pieces by four instructions. For few tokens, staging in
  // LDS of its own cost ~0.2 us.
  if (S * ldw >= kPartStageBytes) {  // uniform over the launch
    __syncthreads();  // every wave is past its reads of the activation slice
    uint8_t* const wl = lds + wave * 32 * kPartRowBytes;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      pin_registers(acc[tt]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(wl + (lane & 31) * kPartRowBytes + 32 * q + 16 * hh) =
            f32x4{acc[tt][4 * q], acc[tt][4 * q + 1], acc[tt][4 * q + 2], acc[tt][4 * q + 3]};
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // tokens 8u .. 8u + 7 of the tile, 16 bytes a lane
        const int tr = 8 * u + (lane >> 3), c = lane & 7;
        const f32x4 v = *reinterpret_cast<const f32x4*>(wl + tr * kPartRowBytes + 16 * c);
        const int t = tt * 32 + tr;
        if (t < S)
          *reinterpret_cast<f32x4*>(part + (static_cast<size_t>(ks) * S + t) * N + h * kHeadDim + wave * 32 + 4 * c) =
              v;
      }
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      pin_registers(acc[tt]);
      const int t = tt * 32 + (lane & 31);
      if (t < S) {
        float* dst = part + (static_cast<size_t>(ks) * S + t) * N + h * kHeadDim + wave * 32 + 4 * hh;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {acc[tt][4 * q], acc[tt][4 * q + 1], acc[tt][4 * q + 2], acc[tt][4 * q + 3]};
          *reinterpret_cast<f32x4*>(dst + 8 * q) = v;
        }
      }
    }
  }
  stamp(a.timeline, a.timeline_slots, tlb, 1);
  return done_before;
}

template <int CPC, int NT>
__global__ __launch_bounds__(256) void decode_gemv(KArgs a, size_t off_x8, size_t off_part) {
  const int tlb = a.S + blockIdx.y * gridDim.x + blockIdx.x;  // timeline slot
  gemv_tile<CPC, NT, false>(a, blockIdx.x, blockIdx.y, a.ws + off_x8, reinterpret_cast<float*>(a.ws + off_part), tlb,
                            Publish{});
}

// ---------------------------------------------------------------------------
// epilogue of head h for token tok, one wave. Lane l holds dims l and l + 64;
// the RoPE partner of dim l < 64 is dim l ^ 32, i.e. lane l ^ 32.
// A partial sum written in this launch by another CTA of the same XCD: an
// agent-scope load, which the CU's L1 does not serve.
template <bool COHERENT>
__device__ __forceinline__ float load_partial(const float* p) {
  if constexpr (COHERENT)
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
  else
    return *p;
}

// NVFP4 row of one token into a 1152-byte cache slot (the wave holds dims lane
// and lane + 64 as float32): 16-lane group maxima, then each even lane stores
// the byte of its dim pair in both halves, and lanes 0, 16, 32, 48 the scale
// bytes of their two groups. Every lane of the wave must call it.
__device__ __forceinline__ void nvfp4_row_wave(float x0, float x1, float gs, bool has_gs, uint8_t* slot, int t,
                                               bool swizzled, int lane) {
#pragma nounroll
  for (int hh = 0; hh < 2; ++hh) {  // one half at a time keeps the extra registers few
    const float x = hh ? x1 : x0;
    float m = __builtin_fabsf(x);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, 64));
    const NvScale ns = nv_scale(m, gs, has_gs);
    const uint32_t c = e2m1_code(mul_rz(x, ns.r));
    const uint32_t n = __shfl_down(c, 1, 64);
    if ((lane & 1) == 0) slot[t * 64 + 32 * hh + (lane >> 1)] = static_cast<uint8_t>(c | (n << 4));
    if ((lane & 15) == 0)
      slot[kNvScaleOff + nv_scale_offset(t, 4 * hh + (lane >> 4), swizzled)] = static_cast<uint8_t>(ns.sf);
  }
}

// OPT: the head-step options (unit K / V scales, FP8 q, NVFP4 caches) are read
// from the arguments; without it the plain path is compiled alone, since these
// short kernels fetch their code cold and every extra instruction costs.
template <bool COHERENT, bool OPT>
__device__ __forceinline__ void head_epilogue(const KArgs& a, int h, int tok, int64_t pos,
                                              const float* __restrict__ part, const float* __restrict__ sx,
                                              int ksplit, int tlb) {
#pragma clang fp contract(off)
  const int N = a.N();
  const int lane = threadIdx.x & 63;
  const int nkv = a.nkv;
  const int S = a.S;
  const int d0 = lane, d1 = lane + 64;
  const int n0 = h * kHeadDim + d0, n1 = h * kHeadDim + d1;
  stamp(a.timeline, a.timeline_slots, tlb, 0);

  // Everything the epilogue reads goes out before anything waits: the token's
  // position (pos, a load the caller issues first, since cos / sin depend on
  // it), the slice partials (sixteen slices in flight at a time, summed in
  // slice order), the scales, the slot and the gamma pair.
  double y0 = 0.0, y1 = 0.0;
  const size_t stride = static_cast<size_t>(S) * N;
  const float* p = part + static_cast<size_t>(tok) * N;
  const int k0 = 16 * nkv, v0 = 17 * nkv, iq0 = 18 * nkv, ik0 = 19 * nkv;
  const uint16_t* g = h < k0 ? a.g_q : (h < v0 ? a.g_k : (h < ik0 ? a.g_iq : a.g_ik));
  float sxf = 0.f, ws0 = 0.f, ws1 = 0.f;
  int64_t slot = 0;
  uint16_t g0 = 0, g1 = 0, cs0 = 0, cs1 = 0;
  for (int k16 = 0; k16 < ksplit; k16 += 16) {
    float v0f[16], v1f[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {  // clamped indices: every load is unconditional
      const size_t ks = static_cast<size_t>(min(k16 + u, ksplit - 1));
      v0f[u] = load_partial<COHERENT>(p + ks * stride + n0);
      v1f[u] = load_partial<COHERENT>(p + ks * stride + n1);
    }
    if (k16 == 0) {
      sxf = load_partial<COHERENT>(sx + tok);
      ws0 = a.w_scale[n0];
      ws1 = a.w_scale[n1];
      slot = a.slot_mapping[tok];
      g0 = g[d0];
      g1 = g[d1];
      pos = pos < 0 ? 0 : (pos >= a.max_pos ? a.max_pos - 1 : pos);
      cs0 = a.cos_sin[pos * kRotary + (lane & 31)];
      cs1 = a.cos_sin[pos * kRotary + 32 + (lane & 31)];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool in = k16 + u < ksplit;
      y0 += in ? static_cast<double>(v0f[u]) : 0.0;
      y1 += in ? static_cast<double>(v1f[u]) : 0.0;
    }
  }
  stamp(a.timeline, a.timeline_slots, tlb, 1);
  const double sxv = static_cast<double>(sxf);
  y0 = (y0 * sxv) * static_cast<double>(ws0);
  y1 = (y1 * sxv) * static_cast<double>(ws1);

  const bool store_cache = slot >= 0 && slot < static_cast<int64_t>(a.num_pages) * kPage;
  const int64_t page = slot_page(slot);
  const int t = slot_row(slot);

  if (OPT && h >= v0 && h < iq0 && a.kv_nvfp4()) {  // V, NVFP4: slot 2j + 1, swizzled scale bytes
    if (store_cache)
      nvfp4_row_wave(static_cast<float>(y0), static_cast<float>(y1), a.v_gs, true,
                     a.k_cache + (page * 2 * nkv + 2 * (h - v0) + 1) * kNvSlotBytes, t, true, lane);
    return;
  }
  if (h >= v0 && h < iq0) {  // V: the raw projection, per-token scale (1 when static)
    const int j = h - v0;
    const double amax = OPT && a.static_kv() ? 0.0 : wave_max_f64(fmax(__builtin_fabs(y0), __builtin_fabs(y1)));
    const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
    if (store_cache) {
      const double sd = static_cast<double>(s), rcp = 1.0 / sd;
      uint8_t* vc = a.v_cache + (page * nkv + j) * kPageBytes;
      const uint32_t c2 = e4m3x2_scaled(div_rn(y0, sd, rcp), div_rn(y1, sd, rcp), fp8_scale(0));
      vc[d0 * kPage + t] = static_cast<uint8_t>(c2);
      vc[d1 * kPage + t] = static_cast<uint8_t>(c2 >> 8);
      if (lane == 0) a.v_scale[(page * nkv + j) * kPage + t] = s;
    }
    return;
  }

  const double ss = wave_sum_f64(y0 * y0 + y1 * y1);
  const double r = 1.0 / __builtin_sqrt(ss / static_cast<double>(kHeadDim) + static_cast<double>(a.eps));
  const double nm0 = (y0 * r) * (1.0 + static_cast<double>(bf16_to_f32(g0)));
  const double nm1 = (y1 * r) * (1.0 + static_cast<double>(bf16_to_f32(g1)));
  const double c = static_cast<double>(bf16_to_f32(cs0));
  const double sn = static_cast<double>(bf16_to_f32(cs1));
  const double partner = __shfl_xor(nm0, 32, 64);
  const double o0 = lane < 32 ? nm0 * c - partner * sn : nm0 * c + partner * sn;
  const double o1 = nm1;

  if (h < k0) {
    const size_t qrow = (static_cast<size_t>(tok) * k0 + h) * kHeadDim;
    if (!OPT || a.q_out != nullptr) {
      uint16_t* q = a.q_out + qrow;
      q[d0] = static_cast<uint16_t>(f32_to_bf16(static_cast<float>(o0)));
      q[d1] = static_cast<uint16_t>(f32_to_bf16(static_cast<float>(o1)));
    }
    if (OPT && a.q_fp8 != nullptr) {  // E4M3 of the float32 product q * (1 / q_fp8_scale)
      const float p0 = static_cast<float>(o0) * a.q_fp8_inv, p1 = static_cast<float>(o1) * a.q_fp8_inv;
      const uint32_t c2 = e4m3x2_scaled(static_cast<double>(p0), static_cast<double>(p1), fp8_scale(0));
      a.q_fp8[qrow + d0] = static_cast<uint8_t>(c2);
      a.q_fp8[qrow + d1] = static_cast<uint8_t>(c2 >> 8);
    }
  } else if (OPT && h < v0 && a.kv_nvfp4()) {  // K, NVFP4: slot 2j, linear scale bytes
    if (store_cache)
      nvfp4_row_wave(static_cast<float>(o0), static_cast<float>(o1), a.k_gs, true,
                     a.k_cache + (page * 2 * nkv + 2 * (h - k0)) * kNvSlotBytes, t, false, lane);
  } else if (h < v0) {  // K: per-token scale (1 when static), shuffled page-16 layout
    const int j = h - k0;
    const double amax = OPT && a.static_kv() ? 0.0 : wave_max_f64(fmax(__builtin_fabs(o0), __builtin_fabs(o1)));
    const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
    if (store_cache) {
      const double sd = static_cast<double>(s), rcp = 1.0 / sd;
      uint8_t* kc = a.k_cache + (page * nkv + j) * kPageBytes + t * 16;
      const uint32_t c2 = e4m3x2_scaled(div_rn(o0, sd, rcp), div_rn(o1, sd, rcp), fp8_scale(0));
      kc[(d0 >> 4) * 256 + (d0 & 15)] = static_cast<uint8_t>(c2);
      kc[(d1 >> 4) * 256 + (d1 & 15)] = static_cast<uint8_t>(c2 >> 8);
      if (lane == 0) a.k_scale[(page * nkv + j) * kPage + t] = s;
    }
  } else if (h < ik0) {
    const int j = h - iq0;
    uint16_t* q = a.iq_out + (static_cast<size_t>(tok) * nkv + j) * kHeadDim;
    q[d0] = static_cast<uint16_t>(f32_to_bf16(static_cast<float>(o0)));
    q[d1] = static_cast<uint16_t>(f32_to_bf16(static_cast<float>(o1)));
  } else if (OPT && store_cache && a.kv_nvfp4()) {  // index_k, NVFP4: the page's one slot, no global scale
    nvfp4_row_wave(static_cast<float>(o0), static_cast<float>(o1), 1.0f, false,
                   a.index_cache + page * kNvSlotBytes, t, false, lane);
  } else if (store_cache) {  // index_k: unit-scale E4M3 into the slot's row
    uint8_t* ic = a.index_cache + slot * kHeadDim;
    const uint32_t c2 = e4m3x2_scaled(o0, o1, fp8_scale(0));
    ic[d0] = static_cast<uint8_t>(c2);
    ic[d1] = static_cast<uint8_t>(c2 >> 8);
  }
}

// Sums and maxima over one half-wave (32 lanes): xor butterflies, so every lane
// of the half ends with the same value.
__device__ __forceinline__ double half_sum_f64(double v) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ double half_max_f64(double v) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) v = __builtin_fmax(v, __shfl_xor(v, m, 64));
  return v;
}

// The head epilogue of two tokens of head h at once, one per half-wave (the
// plain call, without head-step options): tok[0] in lanes 0..31, tok[1] in
// lanes 32..63 (a negative token: that half computes and stores nothing). Lane
// l of a half holds dims l, l + 32, l + 64 and l + 96, so both members (l, l +
// 32) of a NeoX RoPE pair sit in one lane. The arithmetic is head_epilogue's:
// the slice partials summed in slice order in float64, the same float64 head
// norm and FP8 decisions (only the order of the head's sum of squares differs).
template <bool COHERENT>
__device__ __forceinline__ void head_epilogue_pair(const KArgs& a, int h, int tok0, int tok1,
                                                   const float* __restrict__ part, const float* __restrict__ sx,
                                                   int ksplit, int tlb) {
#pragma clang fp contract(off)
  const int N = a.N();
  const int lane = threadIdx.x & 63, li = lane & 31;
  const int tk = lane < 32 ? tok0 : tok1;
  const bool live = tk >= 0;
  const int tok = live ? tk : (tok0 >= 0 ? tok0 : 0);
  const int nkv = a.nkv, S = a.S;
  const int k0 = 16 * nkv, v0 = 17 * nkv, iq0 = 18 * nkv, ik0 = 19 * nkv;
  stamp(a.timeline, a.timeline_slots, tlb, 0);

  // every load first: the token's position (cos / sin depend on it), the
  // slice partials (four dims a lane, sixteen slices in flight at a time), the
  // scales, the slot and the gammas
  int64_t pos = a.positions[tok];
  const size_t stride = static_cast<size_t>(S) * N;
  const float* p = part + static_cast<size_t>(tok) * N + h * kHeadDim + li;
  const uint16_t* g = h < k0 ? a.g_q : (h < v0 ? a.g_k : (h < ik0 ? a.g_iq : a.g_ik));
  double y[4] = {0.0, 0.0, 0.0, 0.0};
  float sxf = 0.f, ws[4] = {0.f, 0.f, 0.f, 0.f};
  int64_t slot = 0;
  uint16_t gm[4] = {0, 0, 0, 0}, cs0 = 0, cs1 = 0;
  for (int k16 = 0; k16 < ksplit; k16 += 16) {
    float v[16][4];
#pragma unroll
    for (int u = 0; u < 16; ++u) {  // clamped indices: every load is unconditional
      const size_t ks = static_cast<size_t>(min(k16 + u, ksplit - 1));
#pragma unroll
      for (int j = 0; j < 4; ++j) v[u][j] = load_partial<COHERENT>(p + ks * stride + 32 * j);
    }
    if (k16 == 0) {
      sxf = load_partial<COHERENT>(sx + tok);
#pragma unroll
      for (int j = 0; j < 4; ++j) ws[j] = a.w_scale[h * kHeadDim + li + 32 * j], gm[j] = g[li + 32 * j];
      slot = a.slot_mapping[tok];
      pos = pos < 0 ? 0 : (pos >= a.max_pos ? a.max_pos - 1 : pos);
      cs0 = a.cos_sin[pos * kRotary + li];
      cs1 = a.cos_sin[pos * kRotary + 32 + li];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool in = k16 + u < ksplit;
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] += in ? static_cast<double>(v[u][j]) : 0.0;
    }
  }
  stamp(a.timeline, a.timeline_slots, tlb, 1);
  const double sxv = static_cast<double>(sxf);
#pragma unroll
  for (int j = 0; j < 4; ++j) y[j] = (y[j] * sxv) * static_cast<double>(ws[j]);

  const bool store_cache = live && slot >= 0 && slot < static_cast<int64_t>(a.num_pages) * kPage;
  const int64_t page = slot_page(slot);
  const int t = slot_row(slot);
  const Fp8Scale unit = fp8_scale(0);

  if (h >= v0 && h < iq0) {  // V: the raw projection, per-token scale
    const int jv = h - v0;
    const double amax = half_max_f64(__builtin_fmax(__builtin_fmax(__builtin_fabs(y[0]), __builtin_fabs(y[1])),
                                                    __builtin_fmax(__builtin_fabs(y[2]), __builtin_fabs(y[3]))));
    const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
    if (store_cache) {
      const double sd = static_cast<double>(s), rcp = 1.0 / sd;
      uint8_t* vc = a.v_cache + (page * nkv + jv) * kPageBytes + t;
      const uint32_t c01 = e4m3x2_scaled(div_rn(y[0], sd, rcp), div_rn(y[1], sd, rcp), unit);
      const uint32_t c23 = e4m3x2_scaled(div_rn(y[2], sd, rcp), div_rn(y[3], sd, rcp), unit);
      vc[(li + 0) * kPage] = static_cast<uint8_t>(c01);
      vc[(li + 32) * kPage] = static_cast<uint8_t>(c01 >> 8);
      vc[(li + 64) * kPage] = static_cast<uint8_t>(c23);
      vc[(li + 96) * kPage] = static_cast<uint8_t>(c23 >> 8);
      if (li == 0) a.v_scale[(page * nkv + jv) * kPage + t] = s;
    }
    return;
  }

  const double ss = half_sum_f64((y[0] * y[0] + y[1] * y[1]) + (y[2] * y[2] + y[3] * y[3]));
  const double r = 1.0 / __builtin_sqrt(ss / static_cast<double>(kHeadDim) + static_cast<double>(a.eps));
  double nm[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) nm[j] = (y[j] * r) * (1.0 + static_cast<double>(bf16_to_f32(gm[j])));
  const double c = static_cast<double>(bf16_to_f32(cs0));
  const double sn = static_cast<double>(bf16_to_f32(cs1));
  const double o[4] = {nm[0] * c - nm[1] * sn, nm[1] * c + nm[0] * sn, nm[2], nm[3]};

  if (h < k0 || (h >= iq0 && h < ik0)) {  // q / index_q: bf16 out
    if (!live) return;
    uint16_t* q = h < k0 ? a.q_out + (static_cast<size_t>(tok) * k0 + h) * kHeadDim
                         : a.iq_out + (static_cast<size_t>(tok) * nkv + (h - iq0)) * kHeadDim;
#pragma unroll
    for (int j = 0; j < 4; ++j) q[li + 32 * j] = static_cast<uint16_t>(f32_to_bf16(static_cast<float>(o[j])));
  } else if (h < v0) {  // K: per-token scale, shuffled page-16 layout
    const int jk = h - k0;
    const double amax = half_max_f64(__builtin_fmax(__builtin_fmax(__builtin_fabs(o[0]), __builtin_fabs(o[1])),
                                                    __builtin_fmax(__builtin_fabs(o[2]), __builtin_fabs(o[3]))));
    const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
    if (store_cache) {
      const double sd = static_cast<double>(s), rcp = 1.0 / sd;
      uint8_t* kc = a.k_cache + (page * nkv + jk) * kPageBytes + t * 16;
      const uint32_t c01 = e4m3x2_scaled(div_rn(o[0], sd, rcp), div_rn(o[1], sd, rcp), unit);
      const uint32_t c23 = e4m3x2_scaled(div_rn(o[2], sd, rcp), div_rn(o[3], sd, rcp), unit);
      const uint32_t cw[4] = {c01 & 0xffu, (c01 >> 8) & 0xffu, c23 & 0xffu, (c23 >> 8) & 0xffu};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = li + 32 * j;
        kc[(d >> 4) * 256 + (d & 15)] = static_cast<uint8_t>(cw[j]);
      }
      if (li == 0) a.k_scale[(page * nkv + jk) * kPage + t] = s;
    }
  } else if (store_cache) {  // index_k: unit-scale E4M3 into the slot's row
    uint8_t* ic = a.index_cache + slot * kHeadDim;
    const uint32_t c01 = e4m3x2_scaled(o[0], o[1], unit);
    const uint32_t c23 = e4m3x2_scaled(o[2], o[3], unit);
    ic[li] = static_cast<uint8_t>(c01);
    ic[li + 32] = static_cast<uint8_t>(c01 >> 8);
    ic[li + 64] = static_cast<uint8_t>(c23);
    ic[li + 96] = static_cast<uint8_t>(c23 >> 8);
  }
}

template <bool OPT>
__global__ __launch_bounds__(64) void decode_epilogue(KArgs a, size_t off_part, size_t off_sx, int ksplit) {
  const int H = a.heads();
  head_epilogue<false, OPT>(a, blockIdx.x % H, blockIdx.x / H, a.positions[blockIdx.x / H],
                            reinterpret_cast<const float*>(a.ws + off_part),
                       reinterpret_cast<const float*>(a.ws + off_sx), ksplit, a.S + H * ksplit + blockIdx.x);
}

// The GEMV CTAs of XCD x count themselves once done with the XCD's published
// values (gemv_tile); the one that counted last of the XCD's gx clears them
// and the counter for the next call.
__device__ __forceinline__ void xcd_clear(const KArgs& a, uint32_t done_before, int gx, uint32_t* done,
                                          uint64_t* pub_r, uint64_t* pub_s) {
  if (done_before == static_cast<uint32_t>(gx - 1)) {
    for (int t = 0; t < a.S; ++t) pub_r[t] = 0u, pub_s[t] = 0u;
    __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The decode step in one or two launches for a few tokens.
//  - Blocks b < 8 S are norm CTAs: token b / 8 for the XCD b % 8. Workgroups
//    go to the XCDs round-robin, so blocks with equal b % 8 share an XCD and
//    its L2 (with fewer XCDs the same holds for b % 4 or b % 2). Each XCD thus
//    computes every token's norm statistics (rstd and the FP8 scale) and
//    publishes them in its L2.
//  - The GEMV CTAs follow. They stream their weights and their slice of ar,
//    res and g_in at once, wait for their XCD's statistics, form the slice's
//    FP8 codes (the norm's expressions) and store partial sums.
//  - With EPI, head h runs all its k slices on XCD h % 8. Each slice stores its
//    partial sums and takes an arrival ticket on the head's counter; the slice
//    that arrives last (every partial is then in its L2) runs the head's
//    epilogue for every token. No slice waits for another. Whole heads per XCD
//    can load some XCDs with more weight than others, so without EPI the slices
//    spread evenly and the epilogue is the next launch.
// No cache write-back or invalidate is needed and nothing crosses XCDs (the
// library checks once per device, when a workspace is set up, that blocks with
// equal b % 8 share an XCD, and otherwise plans no hand-off inside a launch).
// The only wait, a GEMV CTA's for its XCD's statistics, is on norm CTAs that
// come first in dispatch order (so they are running or done), and is bounded;
// if it gives up the CTA computes the statistics itself. The GEMV CTA of an
// XCD that is the last to be done with the XCD's published values clears them,
// a head's last slice its counter, for the next call.
template <int CPC, int NV, bool EPI, bool OPT>
__global__ __launch_bounds__(256) void decode_fused(KArgs a, DecodePlan p) {
  __shared__ double red[64];
  const int b = blockIdx.x, x = b & 7, S = a.S, H = a.heads(), ksplit = p.ksplit;
  float* sx = reinterpret_cast<float*>(a.ws + p.off_sx) + x * kSxStride;
  uint64_t* pub_r = reinterpret_cast<uint64_t*>(a.ws + p.off_rstd) + x * 2 * kSxStride;
  uint64_t* pub_s = pub_r + kSxStride;
  uint32_t* err = reinterpret_cast<uint32_t*>(a.ws + p.off_err);
  const bool stats_handoff = !(a.opts & kOptLocalStats);
  if (b < 8 * S) {
    const int tok = b >> 3;
    double rstd;
    float sc;
    bool owner;
    norm_token<NV, false>(a, tok, nullptr, sx, red, x == 0 ? tok : -1, x == 0, &rstd, &sc, &owner);
    if (owner && stats_handoff) {  // the thread that holds the row's scale
      __builtin_amdgcn_s_waitcnt(0);  // sx (read by the epilogue) is in the L2 before the values are
      pub_r[tok] = static_cast<uint64_t>(__double_as_longlong(rstd));
      pub_s[tok] = (uint64_t{1} << 32) | __float_as_uint(sc);
    }
    return;
  }
  int h, ks;
  if constexpr (EPI) {
    const int j = (b - 8 * S) >> 3;  // this block's index among its XCD's GEMV blocks
    h = x + 8 * (j / ksplit);
    ks = j % ksplit;
    if (h >= H) return;  // XCDs with fewer heads have idle blocks
  } else {  // the slices spread evenly over the XCDs; the epilogue is a launch of its own
    const int g = b - 8 * S;
    h = g % H;
    ks = g / H;
  }
  float* part = reinterpret_cast<float*>(a.ws + p.off_part);
  uint32_t* done = reinterpret_cast<uint32_t*>(a.ws + p.off_done) + x * 32;
  const uint32_t done_before = gemv_tile<CPC, 1, true, NV>(a, h, ks, nullptr, part, S + ks * H + h,
                                                           Publish{pub_r, pub_s, sx, done, err, stats_handoff}, red);
  if constexpr (!EPI) {
    if (threadIdx.x == 0) xcd_clear(a, done_before, (H * ksplit - x + 7) / 8, done, pub_r, pub_s);
    return;
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have reached the L2
  __syncthreads();
  __shared__ uint32_t s_last;
  uint32_t* harrive = reinterpret_cast<uint32_t*>(a.ws + p.off_hdone) + h * kMaxKsplit + 1;
  if (threadIdx.x == 0) {
    s_last = __hip_atomic_fetch_add(harrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             static_cast<uint32_t>(ksplit - 1);
  }
  __syncthreads();
  if (s_last) {  // every other slice of the head has stored its partial sums
    if (threadIdx.x == 0) __hip_atomic_store(harrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int wave = threadIdx.x >> 6;
    for (int tok = wave; tok < S; tok += 4)
      head_epilogue<true, OPT>(a, h, tok, a.positions[tok], part, sx, ksplit, S + H * ksplit + tok * H + h);
  }
  if (threadIdx.x == 0) xcd_clear(a, done_before, (H - x + 7) / 8 * ksplit, done, pub_r, pub_s);
}

// The GEMV with the head epilogue in the same launch, after a norm launch (more
// tokens than the fused launch takes). Head h runs all its k slices on XCD
// h % 8 (blocks with equal b % 8 share an XCD), so its partial sums stay in
// that XCD's L2, and each slice runs the head's epilogue for its share of the
// tokens (ks, ks + ksplit, ...) once every slice's partial sums are stored.
// Per head, four counters in the XCD's L2: started, arrived, the slices that
// left their share to others, and done. A slice counts itself started before
// its GEMV; after storing its partials it waits for the others only if all of
// them have started (so it never waits for a CTA that has not begun, whatever
// the dispatcher does), and otherwise leaves its share to the last arriver.
// The slice that arrives last never waits: it runs its own share and every
// share left to it. A wait can only give up if a started slice never arrives;
// the call's outputs are then marked invalid. The slice that is done last
// clears the counters for the next call.
template <int CPC, int NT, bool OPT>
__global__ __launch_bounds__(256) void decode_gemv_epi(KArgs a, DecodePlan p) {
  const int b = blockIdx.x, x = b & 7, j = b >> 3, H = a.heads(), ksplit = p.ksplit;
  const int h = x + 8 * (j / ksplit), ks = j % ksplit;
  if (h >= H) return;  // XCDs with fewer heads have idle blocks
  float* part = reinterpret_cast<float*>(a.ws + p.off_part);
  const float* sx = reinterpret_cast<const float*>(a.ws + p.off_sx);
  uint32_t* err = reinterpret_cast<uint32_t*>(a.ws + p.off_err);
  uint32_t* hc = reinterpret_cast<uint32_t*>(a.ws + p.off_hdone) + h * kMaxKsplit;  // started, arrived, left, done
  if (threadIdx.x == 0) __hip_atomic_fetch_add(hc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  gemv_tile<CPC, NT, false>(a, h, ks, a.ws + p.off_x8, part, a.S + ks * H + h, Publish{});
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have reached the L2
  __syncthreads();
  __shared__ uint32_t s_role, s_mask;  // role: 0 leaves its share, 1 waits, 2 arrived last
  if (threadIdx.x == 0) {
    const uint32_t me = 1u << ks;
    const bool all_started =
        __hip_atomic_load(hc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == static_cast<uint32_t>(ksplit) &&
        !(a.opts & kOptNoSliceWait);
    if (!all_started) {
      __hip_atomic_fetch_or(hc + 2, me, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);  // in the L2 before the arrival below
    }
    const bool last = __hip_atomic_fetch_add(hc + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      static_cast<uint32_t>(ksplit - 1);
    s_role = last ? 2u : (all_started ? 1u : 0u);
    s_mask = last ? (__hip_atomic_load(hc + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) | me)
                  : (all_started ? me : 0u);
  }
  __syncthreads();
  uint32_t mask = s_mask;
  if (s_role == 1u) {
    __shared__ int s_ok;
    if (threadIdx.x == 0) {
      s_ok = wait_count(hc + 1, static_cast<uint32_t>(ksplit));
      if (!s_ok) mark_invalid(err);
    }
    __syncthreads();
    if (!s_ok) mask = 0u;
  }
  stamp(a.timeline, a.timeline_slots, a.S + ks * H + h, 4);
  // done with the counters; the slice done last clears them for the next call
  if (threadIdx.x == 192 &&
      __hip_atomic_fetch_add(hc + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == static_cast<uint32_t>(ksplit - 1)) {
    for (int f = 0; f < 4; ++f) __hip_atomic_store(hc + f, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int wave = threadIdx.x >> 6;
  if constexpr (OPT) {  // head-step options: one token a wave
    for (; mask != 0u; mask &= mask - 1u) {
      const int sl = __builtin_ctz(mask);
      for (int tok = sl + ksplit * wave; tok < a.S; tok += 4 * ksplit)
        head_epilogue<true, OPT>(a, h, tok, a.positions[tok], part, sx, ksplit, a.S + H * ksplit + tok * H + h);
    }
  } else {  // two tokens a wave, one per half; a share's token pairs dealt to the waves in turn
    int pq = 0;
    for (; mask != 0u; mask &= mask - 1u) {
      const int sl = __builtin_ctz(mask);
      const int cnt = sl < a.S ? (a.S - sl + ksplit - 1) / ksplit : 0;
      for (int q = 0; 2 * q < cnt; ++q, ++pq) {
        if ((pq & 3) != wave) continue;
        const int t0 = sl + 2 * q * ksplit;
        const int t1 = 2 * q + 1 < cnt ? t0 + ksplit : -1;
        head_epilogue_pair<true>(a, h, t0, t1, part, sx, ksplit, a.S + H * ksplit + t0 * H + h);
      }
    }
  }
  stamp(a.timeline, a.timeline_slots, a.S + ks * H + h, 5);
}

// ---------------------------------------------------------------------------
// norm kernel: blockDim.x threads (a multiple of 64, at most 1024)
template <int NV>
__global__ __launch_bounds__(1024) void decode_norm(KArgs a, size_t off_x8, size_t off_sx) {
  __shared__ double red[16];
  norm_token<NV>(a, blockIdx.x, a.ws + off_x8, reinterpret_cast<float*>(a.ws + off_sx), red,
                 blockIdx.x);
}

// Weight repack for the GEMV (one thread per 16-byte piece).
__global__ void pack_decode(const uint8_t* __restrict__ w, uint8_t* __restrict__ wp, int N, int K) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t pieces = static_cast<size_t>(N) * K / 16;
  if (idx >= pieces) return;
  const int nchk = K >> 7;
  const size_t blk = idx >> 8;  // 4 KB blocks of 256 pieces
  const int p = static_cast<int>(idx & 255);
  const int q = p >> 6, l = p & 63;
  const int m = static_cast<int>(blk & 3);
  const size_t hc = blk >> 2;
  const int h = static_cast<int>(hc / nchk), c = static_cast<int>(hc % nchk);
  const int row = h * kHeadDim + m * 32 + (l & 31);
  const uint8_t* src = w + static_cast<size_t>(row) * K + c * 128 + 8 * (l >> 5);
  // steps j = 2q (bytes 0..7) and 2q + 1 (bytes 8..15)
  const uint2 lo = *reinterpret_cast<const uint2*>(src + 16 * (2 * q));
  const uint2 hi = *reinterpret_cast<const uint2*>(src + 16 * (2 * q + 1));
  *reinterpret_cast<uint4*>(wp + blk * 4096 + q * 1024 + l * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

__global__ void fill_zero(uint32_t* p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

template <int CPC, int NT>
hipError_t launch_gemv(const Args& a, const DecodePlan& p) {
  const size_t lds = static_cast<size_t>(a.S) * (CPC * 128 + kLdsPad);
  hipLaunchKernelGGL((decode_gemv<CPC, NT>), dim3(a.heads(), p.ksplit), dim3(256), lds, a.stream, a,
                     p.off_x8, p.off_part);
  return hipGetLastError();
}

// whether a call uses any head-step option (the OPT kernel instantiations)
bool has_options(const Args& a) {
  return a.q_fp8 != nullptr || a.static_kv() || a.kv_nvfp4() || a.q_out == nullptr;
}

template <int CPC, int NT>
hipError_t launch_gemv_epi(const Args& a, const DecodePlan& p) {
  const size_t lds = static_cast<size_t>(a.S) * (CPC * 128 + kLdsPad);
  const dim3 grid(8 * ((a.heads() + 7) / 8) * p.ksplit);
  if (has_options(a))
    hipLaunchKernelGGL((decode_gemv_epi<CPC, NT, true>), grid, dim3(256), lds, a.stream, a, p);
  else
    hipLaunchKernelGGL((decode_gemv_epi<CPC, NT, false>), grid, dim3(256), lds, a.stream, a, p);
  return hipGetLastError();
}

template <int CPC>
hipError_t launch_gemv_nt(const Args& a, const DecodePlan& p) {
  if (p.gemv_epilogue) return a.S <= 32 ? launch_gemv_epi<CPC, 1>(a, p) : launch_gemv_epi<CPC, 2>(a, p);
  return a.S <= 32 ? launch_gemv<CPC, 1>(a, p) : launch_gemv<CPC, 2>(a, p);
}

template <int CPC, bool EPI, bool OPT>
hipError_t launch_fused_e(const Args& a, const DecodePlan& p) {
  const int nv = (a.K / 8 + 255) / 256;  // 8-element vectors a norm thread holds
  const int gemv = EPI ? 8 * ((a.heads() + 7) / 8) * p.ksplit : a.heads() * p.ksplit;
  const dim3 grid(8 * a.S + gemv);
  const size_t lds = static_cast<size_t>(a.S) * (CPC * 128 + kLdsPad);
  switch (nv) {
    case 1: hipLaunchKernelGGL((decode_fused<CPC, 1, EPI, OPT>), grid, dim3(256), lds, a.stream, a, p); break;
    case 2: hipLaunchKernelGGL((decode_fused<CPC, 2, EPI, OPT>), grid, dim3(256), lds, a.stream, a, p); break;
    case 3: hipLaunchKernelGGL((decode_fused<CPC, 3, EPI, OPT>), grid, dim3(256), lds, a.stream, a, p); break;
    case 4: hipLaunchKernelGGL((decode_fused<CPC, 4, EPI, OPT>), grid, dim3(256), lds, a.stream, a, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_epilogue(const Args& a, const DecodePlan& p) {
  if (has_options(a))
    hipLaunchKernelGGL(decode_epilogue<true>, dim3(a.S * a.heads()), dim3(64), 0, a.stream, a, p.off_part, p.off_sx,
                       p.ksplit);
  else
    hipLaunchKernelGGL(decode_epilogue<false>, dim3(a.S * a.heads()), dim3(64), 0, a.stream, a, p.off_part, p.off_sx,
                       p.ksplit);
  return hipGetLastError();
}

template <int CPC>
hipError_t launch_fused(const Args& a, const DecodePlan& p) {
  // without the epilogue in it the launch never reads the options
  if (!p.fused_epilogue) return launch_fused_e<CPC, false, false>(a, p);
  return has_options(a) ? launch_fused_e<CPC, true, true>(a, p) : launch_fused_e<CPC, true, false>(a, p);
}

// CTAs of one launch that fit on a CU at once, from the occupancy API (cached
// per kernel, LDS size and device), or, without a device, the counts the
// compiler reports for these kernels (registers) and the 160 KB of LDS.
int resident_per_cu(const void* fn, size_t lds, int fallback) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(dev, fn, lds);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (dev < 0 || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 256, lds) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = fallback;
    if (lds > 0) n = std::min<int>(n, static_cast<int>((160u << 10) / lds));
  }
  cache[key] = n;
  return n;
}

template <int C>
int gemv_per_cu_c(int S, int K, bool fused, bool epi, bool gemv_epi) {
  const size_t lds = static_cast<size_t>(S) * (C * 128 + kLdsPad);
  const int nv = (K / 8 + 255) / 256;
  if (fused) {
    const void* f = nullptr;
    switch (nv) {
      case 1: f = epi ? (const void*)&decode_fused<C, 1, true, false> : (const void*)&decode_fused<C, 1, false, false>; break;
      case 2: f = epi ? (const void*)&decode_fused<C, 2, true, false> : (const void*)&decode_fused<C, 2, false, false>; break;
      case 3: f = epi ? (const void*)&decode_fused<C, 3, true, false> : (const void*)&decode_fused<C, 3, false, false>; break;
      default: f = epi ? (const void*)&decode_fused<C, 4, true, false> : (const void*)&decode_fused<C, 4, false, false>; break;
    }
    return resident_per_cu(f, lds, nv == 1 ? 3 : (nv == 4 ? 1 : 2));
  }
  if (gemv_epi)
    return resident_per_cu(S <= 32 ? (const void*)&decode_gemv_epi<C, 1, false> : (const void*)&decode_gemv_epi<C, 2, false>,
                           lds, 3);
  return resident_per_cu(S <= 32 ? (const void*)&decode_gemv<C, 1> : (const void*)&decode_gemv<C, 2>, lds, 7);
}

int gemv_per_cu(int c, int S, int K, bool fused, bool epi, bool gemv_epi) {
  switch (c) {
    case 1: return gemv_per_cu_c<1>(S, K, fused, epi, gemv_epi);
    case 2: return gemv_per_cu_c<2>(S, K, fused, epi, gemv_epi);
    case 3: return gemv_per_cu_c<3>(S, K, fused, epi, gemv_epi);
    default: return gemv_per_cu_c<4>(S, K, fused, epi, gemv_epi);
  }
}

// Whether the launches of the current device may hand values between CTAs
// inside one XCD's L2: set once per device from a placement probe, true until
// then.
constexpr int kMaxDev = 64;
std::atomic<int> g_handoff[kMaxDev];  // 0 not probed, 1 blocks with equal b % 8 share an XCD, -1 not

bool handoff_ok() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return true;
  }
  return g_handoff[dev].load(std::memory_order_relaxed) >= 0;
}

// Each block records its XCD (1 + the XCC_ID hardware register).
__global__ void xcd_probe(uint32_t* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = 1u + (__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u);
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1) {
    (void)hipGetLastError();
    cus = 256;
  }
  return cus;
}

}  // namespace

DecodePlan decode_plan(int S, int K, int nkv) {
  DecodePlan p{};
  const int N = (19 * nkv + 1) * 128;
  const int nchk = K / 128;
  const int heads = N / kHeadDim;
  // The largest chunk count that still gives every CU a CTA, among those whose
  // whole grid is resident at once (a grid in two rounds streams its second
  // half only after the first has finished). The CTAs a CU holds come from the
  // occupancy API on the kernel the split would launch (its registers and LDS).
  // No correctness depends on it: no CTA waits for one that has not started.
  // When no grid is resident at once (many heads and a long k), the largest
  // chunk count, i.e. the fewest CTAs, is taken.
  // In the one-launch structure the 8 S norm CTAs also occupy CUs: counted
  // towards the CU count, they let c2 take 4 chunks a CTA (240 GEMV CTAs + 64
  // norm CTAs): 12.2 vs 12.8 us a step with 3 chunks (320 + 64).
  static const int kCands[] = {4, 3, 2, 1};
  const int cus = device_cus();
  const bool fusable = S <= kFusedMaxS && K <= kFusedMaxK;
  const bool epi_whole_heads = heads % 8 == 0 || static_cast<size_t>(N) * K <= kFusedEpiMaxWeight;
  const int norm_ctas = fusable ? 8 * S : 0;
  int pick = 0, fewest = 0;
  for (int c : kCands) {
    if (nchk % c) continue;
    if (static_cast<size_t>(S) * (c * 128 + kLdsPad) > kMaxLds) continue;
    if (fewest == 0) fewest = c;
    const int ks = nchk / c;
    const int per_cu = gemv_per_cu(c, S, K, fusable, fusable && epi_whole_heads && ks <= kMaxKsplit,
                                   !fusable && ks <= kGemvEpiMaxKsplit);
    if (heads * ks > cus * per_cu) continue;
    pick = c;  // smallest fitting candidate so far
    if (heads * ks + norm_ctas >= cus) break;
  }
  if (pick == 0) pick = fewest;  // c = 1 always fits the LDS: S * 144 bytes
  p.chunks_per_cta = pick;
  p.ksplit = pick ? nchk / pick : 0;
  const bool handoff = handoff_ok();
  p.fused = handoff && pick > 0 && S <= kFusedMaxS && K <= kFusedMaxK;
  // the head's epilogue in the same launch: heads then sit whole on XCDs, which
  // is balanced when they divide evenly, and cheap when the weight is small
  p.fused_epilogue = p.fused && p.ksplit <= kMaxKsplit && epi_whole_heads;
  // more tokens: the epilogue joins the GEMV's launch, which saves the partial
  // sums' round trip through memory (ksplit x S x N floats)
  p.gemv_epilogue = handoff && pick > 0 && !p.fused && p.ksplit <= kGemvEpiMaxKsplit;
  p.off_err = kSyncErr;
  p.off_done = kSyncDone;
  p.off_rstd = kSyncPub;  // published rstd and scale words
  p.off_hdone = kSyncHeadFlags;
  size_t off = kSyncBytes;
  p.off_x8 = off;  // the FP8 rows (not fused; sized either way, so the size never depends on the structure)
  off = align_up(off + static_cast<size_t>(S) * K, 256);
  p.off_sx = off;  // per-token scales: one copy per XCD when fused
  off = align_up(off + sizeof(float) * (p.fused ? 8 * kSxStride : S), 256);
  p.off_part = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(p.ksplit) * S * N, 256);
  p.total = off;
  return p;
}

hipError_t launch_decode(const Args& a, const DecodePlan& p) {
  hipError_t e;
  if (p.fused) {
    if ((e = mark(a.ev_start, a.stream)) != hipSuccess) return e;
    switch (p.chunks_per_cta) {
      case 1: e = launch_fused<1>(a, p); break;
      case 2: e = launch_fused<2>(a, p); break;
      case 3: e = launch_fused<3>(a, p); break;
      case 4: e = launch_fused<4>(a, p); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    if ((e = mark(a.ev_stop, a.stream)) != hipSuccess) return e;
    if (p.fused_epilogue) return hipSuccess;
    return launch_epilogue(a, p);
  }
  // norm: one thread per 8-element vector up to 1024 threads, then loop
  const int vecs = a.K / 8;
  const int threads = vecs >= 1024 ? 1024 : (vecs + 63) / 64 * 64;
  const int nv = (vecs + threads - 1) / threads;
  if (nv == 1)
    hipLaunchKernelGGL((decode_norm<1>), dim3(a.S), dim3(threads), 0, a.stream, a, p.off_x8, p.off_sx);
  else if (nv == 2)
    hipLaunchKernelGGL((decode_norm<2>), dim3(a.S), dim3(threads), 0, a.stream, a, p.off_x8, p.off_sx);
  else
    return hipErrorInvalidValue;
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = mark(a.ev_start, a.stream)) != hipSuccess) return e;
  switch (p.chunks_per_cta) {
    case 1: e = launch_gemv_nt<1>(a, p); break;
    case 2: e = launch_gemv_nt<2>(a, p); break;
    case 3: e = launch_gemv_nt<3>(a, p); break;
    case 4: e = launch_gemv_nt<4>(a, p); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if ((e = mark(a.ev_stop, a.stream)) != hipSuccess) return e;
  if (p.gemv_epilogue) return hipSuccess;
  return launch_epilogue(a, p);
}

hipError_t launch_pack_decode(const uint8_t* w, uint8_t* wp, int N, int K, hipStream_t s) {
  const size_t pieces = static_cast<size_t>(N) * K / 16;
  const unsigned blocks = static_cast<unsigned>((pieces + 255) / 256);
  hipLaunchKernelGGL(pack_decode, dim3(blocks), dim3(256), 0, s, w, wp, N, K);
  return hipGetLastError();
}

// Checks once per device, on a workspace of at least kSyncBytes, that
// workgroups with equal b % 8 run on one XCD (the dispatcher hands them to the
// XCDs round-robin; its starting XCD may move from launch to launch, which the
// hand-offs do not mind); otherwise decode plans no hand-off inside a launch.
// Synchronizes `s` the first time.
hipError_t probe_placement(void* ws, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev || g_handoff[dev].load(std::memory_order_relaxed) != 0) return hipSuccess;
  constexpr int kBlocks = 2048;
  static_assert(kBlocks * 4 <= static_cast<int>(kSyncBytes), "probe fits the synchronization words");
  uint32_t rec[kBlocks];
  hipLaunchKernelGGL(xcd_probe, dim3(kBlocks), dim3(64), 0, s, static_cast<uint32_t*>(ws));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = hipMemcpyAsync(rec, ws, sizeof(rec), hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  bool ok = true;
  for (int b = 0; b < kBlocks; ++b) ok = ok && rec[b] != 0u && rec[b] == rec[b % 8];
  g_handoff[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  return hipSuccess;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(n < 256 * 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(fill_zero, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace pa
