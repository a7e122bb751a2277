// Prefill prologue on gfx950: MXFP8 activations against an MXFP8 weight.
//
// Two kernels on the caller's stream:
//   1. prefill_prepass  one CTA per token: residual add (f32) + bf16 residual
//                       out, Gemma RMSNorm, then OCP-MX quantization (E8M0
//                       scale per 32-wide k block, E4M3 elements) into the
//                       GEMM's packed activation layout in the workspace.
//   2. prefill_gemm     C^T = W . X^T on MFMA. One CTA owns one 128-wide head
//                       x 128 tokens; each wave 32 tokens x the whole head.
//                       q and index_q heads run block-scaled FP8 MFMAs
//                       (v_mfma_scale_f32_32x32x64_f8f6f4); the k, v and
//                       index_k heads, whose per-token scales and codes must
//                       follow the exact projection closely, run bf16 MFMAs on
//                       the MXFP8 values widened exactly to bf16 (FP8-input
//                       MFMAs sum their products at reduced internal
//                       precision). Either way, after the k loop a lane holds one
//                       token's 64 dims of the head and its lane ^ 32 partner
//                       the other 64: the per-head Gemma norm is an in-register
//                       sum plus one swap, and the RoPE pair (i, i + 32) sits
//                       in the same lane and register slot of the first two
//                       32-row tiles. The epilogue (the pages' per-role
//                       branches: the qkv_index_fused_epilogue page and the
//                       K1 mono_pre head tasks) runs on the f32 accumulator;
//                       the projection is never written to memory.
//
// Numerics: as in decode, the norm / MX decision and the head epilogue run in
// float64 with contraction off.
#include <hip/hip_runtime.h>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr int kPreThreads = 256;
constexpr int kTokTile = 128;   // tokens per GEMM CTA (4 waves x 32)
constexpr int kKStep = 64;      // k per MFMA
constexpr int kTileBytes = 2048;  // one 32 x 64 FP8 operand tile

// Operand order of the 32x32x64 FP8 MFMA (measured on gfx950): lane l holds
// row / column l % 32; with h = l / 32 its bytes 0..15 are k = 16h + [0, 16)
// (MX block 0) and bytes 16..31 are k = 32 + 16h + [0, 16) (block 1); the E8M0
// scale operand of lane l is that row's scale for block l / 32.
// Packed activation: token tile tt (32 tokens), k step ks -> 2 KB block at
// (tt * nks + ks) * 2048; lane l's bytes 0..15 at 16 l, bytes 16..31 at
// 1024 + 16 l (so each dwordx4 wave load is 1 KB contiguous).
// Scales: byte (tt * nks + ks) * 64 + l.
__device__ __forceinline__ size_t xq_offset(int m, int k, int nks) {
  const int tt = m >> 5, tl = m & 31;
  const int ks = k >> 6, kk = k & 63;
  const int region = kk >> 5, h = (kk >> 4) & 1;
  return (static_cast<size_t>(tt) * nks + ks) * kTileBytes + region * 1024 + (tl + 32 * h) * 16 + (kk & 15);
}

__device__ __forceinline__ size_t xs_offset(int m, int blk, int nks) {
  const int tt = m >> 5, tl = m & 31;
  const int ks = blk >> 1, kg = blk & 1;
  return (static_cast<size_t>(tt) * nks + ks) * 64 + tl + 32 * kg;
}

template <int NV>
__global__ __launch_bounds__(kPreThreads) void prefill_prepass(
    const uint16_t* __restrict__ ar, const uint16_t* __restrict__ res,
    uint16_t* __restrict__ h_out, const uint16_t* __restrict__ g_in,
    uint8_t* __restrict__ xq, uint8_t* __restrict__ xs, int M, int K, float eps) {
#pragma clang fp contract(off)
  __shared__ double red[kPreThreads / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int nvec = K >> 3;
  const int nks = K / kKStep;
  if (row >= M) {  // padding rows of the last token tile: zero codes, unit scales
    for (int v = tid; v < nvec; v += kPreThreads)
      *reinterpret_cast<uint2*>(xq + xq_offset(row, 8 * v, nks)) = make_uint2(0u, 0u);
    for (int b = tid; b < K / 32; b += kPreThreads) xs[xs_offset(row, b, nks)] = 127;
    return;
  }
  const size_t base = static_cast<size_t>(row) * K;
  double xn[NV][8];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = tid + i * kPreThreads;
    if (v < nvec) {
      const uint4 a = *reinterpret_cast<const uint4*>(ar + base + 8 * v);
      const uint4 b = *reinterpret_cast<const uint4*>(res + base + 8 * v);
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
      uint32_t hw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = bf16_to_f32(aw[q] & 0xffffu) + bf16_to_f32(bw[q] & 0xffffu);
        const float hi = bf16_to_f32(aw[q] >> 16) + bf16_to_f32(bw[q] >> 16);
        hw[q] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
        xn[i][2 * q] = lo;
        xn[i][2 * q + 1] = hi;
        ss += static_cast<double>(lo) * lo;
        ss += static_cast<double>(hi) * hi;
      }
      *reinterpret_cast<uint4*>(h_out + base + 8 * v) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xn[i][e] = 0.0;
    }
  }
  ss = wave_sum_f64(ss);
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  double tot = red[0];
  for (int w = 1; w < kPreThreads / 64; ++w) tot += red[w];
  const double rstd = 1.0 / __builtin_sqrt(tot / static_cast<double>(K) + static_cast<double>(eps));
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = tid + i * kPreThreads;
    // 8-element vectors 4b..4b+3 form MX block b: four consecutive lanes
    double amax = 0.0;
    if (v < nvec) {
      const uint4 g = *reinterpret_cast<const uint4*>(g_in + 8 * v);
      const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t gb = (e & 1) ? (gw[e >> 1] >> 16) : (gw[e >> 1] & 0xffffu);
        xn[i][e] = (xn[i][e] * rstd) * (1.0 + static_cast<double>(bf16_to_f32(gb)));
        const double m = __builtin_fabs(xn[i][e]);
        amax = amax > m ? amax : m;
      }
    }
    {
      const double o1 = __shfl_xor(amax, 1, 64);
      amax = amax > o1 ? amax : o1;
      const double o2 = __shfl_xor(amax, 2, 64);
      amax = amax > o2 ? amax : o2;
    }
    if (v < nvec) {
      // X = 2^(floor(log2 amax) - 8); an all-zero block keeps X = 1
      int code = 127;
      if (amax != 0.0) {
        const int e = static_cast<int>((static_cast<uint64_t>(__double_as_longlong(amax)) >> 52) & 0x7ff) - 1023;
        code = e - 8 + 127;
        code = code < 0 ? 0 : (code > 254 ? 254 : code);
      }
      const double inv = __longlong_as_double(static_cast<long long>(1023 - (code - 127)) << 52);
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) w0 |= e4m3_from_f64(xn[i][e] * inv) << (8 * e);
#pragma unroll
      for (int e = 0; e < 4; ++e) w1 |= e4m3_from_f64(xn[i][4 + e] * inv) << (8 * e);
      *reinterpret_cast<uint2*>(xq + xq_offset(row, 8 * v, nks)) = make_uint2(w0, w1);
      if ((v & 3) == 0) xs[xs_offset(row, v >> 2, nks)] = static_cast<uint8_t>(code);
    }
  }
}

// Packed weight, FP8 part (every head): head h, k step ks, 32-row tile m ->
// 2 KB block at ((h * nks + ks) * 4 + m) * 2048 in the activation's lane order
// (row 32m + l % 32). Scales: dword (h * nks + ks) * 64 + l holds tiles
// m = 0..3 in bytes 0..3, each the row's E8M0 for block 2 ks + l / 32.
// bf16 part (k, v and index_k heads, index p = 0 .. 2 nkv), after the N x K FP8
// bytes: 1 KB block (((p * nks + ks) * 4 + m) * 4 + j) * 1024 for bf16 MFMA step
// j of the k step; lane l's 8 values (row 32m + l % 32) sit at 16 l and are
// k = 64 ks + 32 (j / 2) + 16 (l / 32) + 8 (j % 2) + [0, 8), times the block
// scale: exactly the FP8 bytes 8 (j % 2) .. + 8 of region j / 2 of the lane.

__device__ __forceinline__ bool precise_head(int h, int nkv) {
  return (h >= 16 * nkv && h < 18 * nkv) || h == 19 * nkv;
}

__device__ __forceinline__ int precise_index(int h, int nkv) {
  return h == 19 * nkv ? 2 * nkv : h - 16 * nkv;
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  return __uint_as_float(c ? c << 23 : 0x00400000u);
}

// q / index_q heads: block-scaled FP8 MFMA.
__device__ __forceinline__ void mainloop_fp8(const Args& a, int h, const uint8_t* xbase,
                                             const uint8_t* xsb, uint8_t* sA, f32x16 (&acc)[4]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int nks = a.K / kKStep;
  const uint8_t* wbase = a.w_packed + static_cast<size_t>(h) * nks * 4 * kTileBytes;
  const uint32_t* sbase = reinterpret_cast<const uint32_t*>(a.s_packed) + static_cast<size_t>(h) * nks * 64;
  for (int ks = 0; ks < nks; ++ks) {
    const i32x4* wsrc = reinterpret_cast<const i32x4*>(wbase + static_cast<size_t>(ks) * 4 * kTileBytes);
    const i32x4 w0 = wsrc[tid];
    const i32x4 w1 = wsrc[tid + 256];
    const uint32_t sa = sbase[static_cast<size_t>(ks) * 64 + lane];
    const i32x4* xsrc = reinterpret_cast<const i32x4*>(xbase + static_cast<size_t>(ks) * kTileBytes);
    const i32x4 b0 = xsrc[lane];
    const i32x4 b1 = xsrc[lane + 64];
    const uint32_t sb = xsb[static_cast<size_t>(ks) * 64 + lane];
    __syncthreads();
    reinterpret_cast<i32x4*>(sA)[tid] = w0;
    reinterpret_cast<i32x4*>(sA)[tid + 256] = w1;
    __syncthreads();
    const i32x8 B = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const i32x4 a0 = reinterpret_cast<const i32x4*>(sA + m * kTileBytes)[lane];
      const i32x4 a1 = reinterpret_cast<const i32x4*>(sA + m * kTileBytes + 1024)[lane];
      const i32x8 A = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      switch (m) {  // the scale byte of tile m (op_sel is an immediate)
        case 0: acc[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[0], 0, 0, 0, sa, 0, sb); break;
        case 1: acc[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[1], 0, 0, 1, sa, 0, sb); break;
        case 2: acc[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[2], 0, 0, 2, sa, 0, sb); break;
        default: acc[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[3], 0, 0, 3, sa, 0, sb); break;
      }
    }
  }
}

// k / v / index_k heads: bf16 MFMA on exactly widened MXFP8 values.
__device__ __forceinline__ void mainloop_bf16(const Args& a, int h, const uint8_t* xbase,
                                              const uint8_t* xsb, uint8_t* sA, f32x16 (&acc)[4]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int nks = a.K / kKStep;
  const int p = precise_index(h, a.nkv);
  const uint8_t* wbase = a.w_packed + static_cast<size_t>(a.N()) * a.K +
                         static_cast<size_t>(p) * nks * 16384;
  for (int ks = 0; ks < nks; ++ks) {
    const i32x4* wsrc = reinterpret_cast<const i32x4*>(wbase + static_cast<size_t>(ks) * 16384);
    const i32x4 w0 = wsrc[tid], w1 = wsrc[tid + 256], w2 = wsrc[tid + 512], w3 = wsrc[tid + 768];
    const i32x4* xsrc = reinterpret_cast<const i32x4*>(xbase + static_cast<size_t>(ks) * kTileBytes);
    const i32x4 b0 = xsrc[lane];
    const i32x4 b1 = xsrc[lane + 64];
    const float x0 = e8m0_to_f32(xsb[static_cast<size_t>(ks) * 64 + (lane & 31)]);
    const float x1 = e8m0_to_f32(xsb[static_cast<size_t>(ks) * 64 + (lane & 31) + 32]);
    __syncthreads();
    reinterpret_cast<i32x4*>(sA)[tid] = w0;
    reinterpret_cast<i32x4*>(sA)[tid + 256] = w1;
    reinterpret_cast<i32x4*>(sA)[tid + 512] = w2;
    reinterpret_cast<i32x4*>(sA)[tid + 768] = w3;
    __syncthreads();
    bf16x8 B[4];
    B[0] = fp8x8_to_bf16(b0[0], b0[1], x0);
    B[1] = fp8x8_to_bf16(b0[2], b0[3], x0);
    B[2] = fp8x8_to_bf16(b1[0], b1[1], x1);
    B[3] = fp8x8_to_bf16(b1[2], b1[3], x1);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(sA + ((m * 4 + j) * 1024) + lane * 16);
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B[j], acc[m], 0, 0, 0);
      }
  }
}

__global__ __launch_bounds__(256) void prefill_gemm(Args a, const uint8_t* __restrict__ xq,
                                                   const uint8_t* __restrict__ xs) {
  __shared__ __align__(16) uint8_t sA[16384];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x;
  const int tt = blockIdx.y * (kTokTile / 32) + wave;  // this wave's 32-token tile
  const int nks = a.K / kKStep;
  const uint8_t* xbase = xq + static_cast<size_t>(tt) * nks * kTileBytes;
  const uint8_t* xsb = xs + static_cast<size_t>(tt) * nks * 64;

  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
  if (precise_head(h, a.nkv))
    mainloop_bf16(a, h, xbase, xsb, sA, acc);
  else
    mainloop_fp8(a, h, xbase, xsb, sA, acc);
#pragma unroll
  for (int m = 0; m < 4; ++m) pin_registers(acc[m]);

  // ---------------- epilogue: lane holds token tok, dims 32m + 8(r/4) + 4(l/32) + r%4
  {
#pragma clang fp contract(off)
    const int tok = tt * 32 + (lane & 31);
    const bool live = tok < a.S;
    const int tk = live ? tok : a.S - 1;  // padded rows use clamped metadata
    const int nkv = a.nkv;
    const int k0 = 16 * nkv, v0 = 17 * nkv, iq0 = 18 * nkv, ik0 = 19 * nkv;
    const int hi = (lane >> 5) * 4;
    auto dim = [&](int m, int r) { return 32 * m + 8 * (r >> 2) + hi + (r & 3); };

    int64_t slot = a.slot_mapping[tk];
    const bool store_cache = live && slot >= 0 && slot < static_cast<int64_t>(a.num_pages) * kPage;
    const int64_t page = slot_page(slot);
    const int t = slot_row(slot);

    if (h >= v0 && h < iq0) {  // V: raw projection, per-token scale
      const int j = h - v0;
      double amax = 0.0;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) amax = fmax(amax, __builtin_fabs(static_cast<double>(acc[m][r])));
      const double o = __shfl_xor(amax, 32, 64);
      amax = amax > o ? amax : o;
      const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
      if (store_cache) {
        uint8_t* vc = a.v_cache + (page * nkv + j) * kPageBytes + t;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            vc[dim(m, r) * kPage] = static_cast<uint8_t>(
                e4m3_from_f64(static_cast<double>(acc[m][r]) / static_cast<double>(s)));
        if (lane < 32) a.v_scale[(page * nkv + j) * kPage + t] = s;
      }
      return;
    }

    const uint16_t* g = h < k0 ? a.g_q : (h < v0 ? a.g_k : (h < ik0 ? a.g_iq : a.g_ik));
    double ss = 0.0;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) ss += static_cast<double>(acc[m][r]) * static_cast<double>(acc[m][r]);
    ss += __shfl_xor(ss, 32, 64);
    const double rr = 1.0 / __builtin_sqrt(ss / static_cast<double>(kHeadDim) + static_cast<double>(a.eps));
    int64_t pos = a.positions[tk];
    pos = pos < 0 ? 0 : (pos >= a.max_pos ? a.max_pos - 1 : pos);
    const uint16_t* cs = a.cos_sin + pos * kRotary;

    double o[4][16];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        o[m][r] = (static_cast<double>(acc[m][r]) * rr) * (1.0 + static_cast<double>(bf16_to_f32(g[dim(m, r)])));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = dim(0, r);
      const double c = static_cast<double>(bf16_to_f32(cs[i]));
      const double sn = static_cast<double>(bf16_to_f32(cs[32 + i]));
      const double x1 = o[0][r], x2 = o[1][r];
      o[0][r] = x1 * c - x2 * sn;
      o[1][r] = x2 * c + x1 * sn;
    }

    if (h < k0 || (h >= iq0 && h < ik0)) {  // q / index_q: bf16 out
      uint16_t* dst = h < k0 ? a.q_out + (static_cast<size_t>(tok) * k0 + h) * kHeadDim
                             : a.iq_out + (static_cast<size_t>(tok) * nkv + (h - iq0)) * kHeadDim;
      if (live) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t p0 = f32_to_bf16(static_cast<float>(o[m][4 * q])) |
                          (f32_to_bf16(static_cast<float>(o[m][4 * q + 1])) << 16);
            uint32_t p1 = f32_to_bf16(static_cast<float>(o[m][4 * q + 2])) |
                          (f32_to_bf16(static_cast<float>(o[m][4 * q + 3])) << 16);
            *reinterpret_cast<uint2*>(dst + dim(m, 4 * q)) = make_uint2(p0, p1);
          }
      }
    } else if (h < v0) {  // K: per-token scale, shuffled page-16 layout
      const int j = h - k0;
      double amax = 0.0;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) amax = fmax(amax, __builtin_fabs(o[m][r]));
      const double ot = __shfl_xor(amax, 32, 64);
      amax = amax > ot ? amax : ot;
      const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
      if (store_cache) {
        uint8_t* kc = a.k_cache + (page * nkv + j) * kPageBytes + t * 16;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              w |= e4m3_from_f64(o[m][4 * q + e] / static_cast<double>(s)) << (8 * e);
            const int d = dim(m, 4 * q);
            *reinterpret_cast<uint32_t*>(kc + (d >> 4) * 256 + (d & 15)) = w;
          }
        if (lane < 32) a.k_scale[(page * nkv + j) * kPage + t] = s;
      }
    } else if (store_cache) {  // index_k: unit-scale E4M3 into the slot's row
      uint8_t* ic = a.index_cache + slot * kHeadDim;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t w = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) w |= e4m3_from_f64(o[m][4 * q + e]) << (8 * e);
          *reinterpret_cast<uint32_t*>(ic + dim(m, 4 * q)) = w;
        }
    }
  }
}

__global__ void pack_prefill(const uint8_t* __restrict__ w, const uint8_t* __restrict__ we,
                             uint8_t* __restrict__ wp, uint8_t* __restrict__ sp, int N, int K) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t pieces = static_cast<size_t>(N) * K / 16;
  if (idx >= pieces) return;
  const int nks = K / kKStep;
  const size_t blk = idx >> 7;  // 2 KB blocks of 128 pieces
  const int p = static_cast<int>(idx & 127);
  const int m = static_cast<int>(blk & 3);
  const size_t hk = blk >> 2;
  const int h = static_cast<int>(hk / nks), ks = static_cast<int>(hk % nks);
  const int region = p >> 6, l = p & 63;
  const int row = h * 128 + m * 32 + (l & 31);
  const int k = ks * kKStep + region * 32 + (l >> 5) * 16;
  *reinterpret_cast<i32x4*>(wp + blk * kTileBytes + region * 1024 + l * 16) =
      *reinterpret_cast<const i32x4*>(w + static_cast<size_t>(row) * K + k);
  if (region == 0)  // one scale byte per (tile, lane)
    sp[hk * 256 + l * 4 + m] = we[static_cast<size_t>(row) * (K / 32) + ks * 2 + (l >> 5)];
}

// bf16 copy of the k, v and index_k heads (one thread per 8 values).
__global__ void pack_prefill_bf16(const uint8_t* __restrict__ w, const uint8_t* __restrict__ we,
                                  uint8_t* __restrict__ wb, int nkv, int K) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int nks = K / kKStep;
  const size_t pieces = static_cast<size_t>(2 * nkv + 1) * nks * 4 * 4 * 64;
  if (idx >= pieces) return;
  const int l = static_cast<int>(idx & 63);
  const int j = static_cast<int>((idx >> 6) & 3);
  const int m = static_cast<int>((idx >> 8) & 3);
  const size_t pk = idx >> 10;
  const int p = static_cast<int>(pk / nks), ks = static_cast<int>(pk % nks);
  const int head = p < 2 * nkv ? 16 * nkv + p : 19 * nkv;
  const int row = head * 128 + m * 32 + (l & 31);
  const int k = ks * kKStep + 32 * (j >> 1) + 16 * (l >> 5) + 8 * (j & 1);
  const uint8_t* src = w + static_cast<size_t>(row) * K + k;
  const int e = we[static_cast<size_t>(row) * (K / 32) + (k >> 5)];
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t two = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t c = src[2 * i + q];
      const uint32_t sgn = c & 0x80u, ex = (c >> 3) & 0xfu, mt = c & 7u;
      // E4M3 value as float32, then times 2^(e - 127); exact in bf16
      float v = ex ? __uint_as_float(((ex + 120u) << 23) | (mt << 20)) : static_cast<float>(mt) * 0x1p-9f;
      v = __builtin_ldexpf(v, e - 127);
      uint32_t bits = (__float_as_uint(v) >> 16) | (sgn << 8);
      two |= bits << (16 * q);
    }
    out[i] = two;
  }
  *reinterpret_cast<uint4*>(wb + idx * 16) = make_uint4(out[0], out[1], out[2], out[3]);
}

template <int NV>
hipError_t launch_prepass(const Args& a, const PrefillPlan& p, int mpad) {
  hipLaunchKernelGGL(prefill_prepass<NV>, dim3(mpad), dim3(kPreThreads), 0, a.stream, a.ar, a.res,
                     a.h_out, a.g_in, a.ws + p.off_xq, a.ws + p.off_xs, a.S, a.K, a.eps);
  return hipGetLastError();
}

}  // namespace

PrefillPlan prefill_plan(int M, int K, int nkv) {
  (void)nkv;
  PrefillPlan p{};
  const size_t mpad = (static_cast<size_t>(M) + kTokTile - 1) / kTokTile * kTokTile;
  size_t off = 0;
  p.off_xq = off;
  off = align_up(off + mpad * K, 256);
  p.off_xs = off;
  off = align_up(off + mpad * K / 32, 256);
  p.off_cnt = off;
  off += 1024;
  p.total = off;
  return p;
}

size_t prefill_packed_weight_bytes(int N, int K) {
  const int nkv = (N / 128 - 1) / 19;
  return static_cast<size_t>(N) * K + static_cast<size_t>(2 * nkv + 1) * 128 * K * 2;
}
size_t prefill_packed_scale_bytes(int N, int K) { return static_cast<size_t>(N) * K / 32; }

hipError_t launch_prefill(const Args& a, const PrefillPlan& p) {
  const int mpad = (a.S + kTokTile - 1) / kTokTile * kTokTile;
  const int nv = (a.K / 8 + kPreThreads - 1) / kPreThreads;
  hipError_t e;
  switch (nv) {
    case 1: e = launch_prepass<1>(a, p, mpad); break;
    case 2: e = launch_prepass<2>(a, p, mpad); break;
    case 3: e = launch_prepass<3>(a, p, mpad); break;
    case 4: e = launch_prepass<4>(a, p, mpad); break;
    case 5: e = launch_prepass<5>(a, p, mpad); break;
    case 6: e = launch_prepass<6>(a, p, mpad); break;
    case 7: e = launch_prepass<7>(a, p, mpad); break;
    case 8: e = launch_prepass<8>(a, p, mpad); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if ((e = mark(a.ev_start, a.stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_gemm, dim3(a.heads(), mpad / kTokTile), dim3(256), 0, a.stream, a,
                     a.ws + p.off_xq, a.ws + p.off_xs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(a.ev_stop, a.stream);
}

hipError_t launch_pack_prefill(const uint8_t* w, const uint8_t* we, uint8_t* wp, uint8_t* sp,
                               int N, int K, hipStream_t s) {
  const size_t pieces = static_cast<size_t>(N) * K / 16;
  const unsigned blocks = static_cast<unsigned>((pieces + 255) / 256);
  hipLaunchKernelGGL(pack_prefill, dim3(blocks), dim3(256), 0, s, w, we, wp, sp, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkv = (N / 128 - 1) / 19;
  const size_t pieces16 = static_cast<size_t>(2 * nkv + 1) * (K / kKStep) * 1024;
  hipLaunchKernelGGL(pack_prefill_bf16, dim3(static_cast<unsigned>((pieces16 + 255) / 256)), dim3(256),
                     0, s, w, we, wp + static_cast<size_t>(N) * K, nkv, K);
  return hipGetLastError();
}

}  // namespace pa
