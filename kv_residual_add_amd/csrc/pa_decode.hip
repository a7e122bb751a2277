// Decode prologue on gfx950: per-token FP8 activations against a per-row
// scaled FP8 weight, for up to 64 tokens.
//
// Three kernels on the caller's stream:
//   1. decode_norm      one CTA per token: residual add (f32) + bf16 residual
//                       out, Gemma RMSNorm, per-token FP8 quantization into a
//                       workspace row (the K1 mono_pre page,
//                       vllm.models.minimax_m3.amd.mono.kernels.pre_attn,
//                       emit_pre_attn: norm_quant).
//   2. decode_gemv      the fused projection as an HBM-bound GEMV: each CTA
//                       owns one 128-row head x a k slice; every wave streams
//                       its 32 rows' packed weight with dwordx4 loads issued
//                       before anything waits on them, the FP8 activation slice
//                       sits in LDS, and 32x32x16 bf16 MFMAs take up to 32
//                       tokens a tile on exactly widened FP8 codes. k-slice
//                       partial sums go to the workspace.
//   3. decode_epilogue  one wave per (token, head): sums the k-slice partials,
//                       applies the activation and row scales, then the head's
//                       role (pre_attn page, head tasks; head_norm_rope; the
//                       epilogue page vllm.models.minimax_m3.nvidia.ops.
//                       qkv_index_fused_epilogue, per-role branches).
//
// Numerics: the input norm, its FP8 decision and the head epilogue run in
// float64 with contraction off, so a code is decided from the same value the
// float64 statement of the method gives; the projection's products are exact
// and accumulate in float32 (FP8-input MFMAs sum at lower internal precision,
// which moves the per-token K / V scales by ~1e-5, so the codes are widened to
// bf16 first).
#include <hip/hip_runtime.h>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr int kNormThreads = 256;
constexpr int kLdsPad = 16;
constexpr int kMaxLds = 64 * 1024;

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = red[0];
  for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) t += red[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ double block_max_f64(double v, double* red) {
  v = wave_max_f64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = red[0];
  for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) t = t > red[w] ? t : red[w];
  __syncthreads();
  return t;
}

// ---------------------------------------------------------------------------
// 1. residual add + Gemma RMSNorm + per-token FP8, one token per CTA.
//    NV = 8-element vectors per thread (hidden <= NV * 8 * 256).
template <int NV>
__global__ __launch_bounds__(kNormThreads) void decode_norm(
    const uint16_t* __restrict__ ar, const uint16_t* __restrict__ res,
    uint16_t* __restrict__ h_out, const uint16_t* __restrict__ g_in,
    uint8_t* __restrict__ x8, float* __restrict__ sx, int K, float eps) {
#pragma clang fp contract(off)
  __shared__ double red[kNormThreads / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int nvec = K >> 3;
  const size_t base = static_cast<size_t>(row) * K;
  double xn[NV][8];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = tid + i * kNormThreads;
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
  ss = block_sum_f64(ss, red);
  const double rstd = 1.0 / __builtin_sqrt(ss / static_cast<double>(K) + static_cast<double>(eps));
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = tid + i * kNormThreads;
    if (v < nvec) {
      const uint4 g = *reinterpret_cast<const uint4*>(g_in + 8 * v);
      const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t gb = (e & 1) ? (gw[e >> 1] >> 16) : (gw[e >> 1] & 0xffffu);
        const double gp = 1.0 + static_cast<double>(bf16_to_f32(gb));
        xn[i][e] = (xn[i][e] * rstd) * gp;
        const double m = __builtin_fabs(xn[i][e]);
        amax = amax > m ? amax : m;
      }
    }
  }
  amax = block_max_f64(amax, red);
  const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
  const double sd = static_cast<double>(s);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = tid + i * kNormThreads;
    if (v < nvec) {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) w0 |= e4m3_from_f64(xn[i][e] / sd) << (8 * e);
#pragma unroll
      for (int e = 0; e < 4; ++e) w1 |= e4m3_from_f64(xn[i][4 + e] / sd) << (8 * e);
      *reinterpret_cast<uint2*>(x8 + base + 8 * v) = make_uint2(w0, w1);
    }
  }
  if (tid == 0) sx[row] = s;
}

// ---------------------------------------------------------------------------
// 2. GEMV partials. Packed weight: head h, 128-wide k chunk c, 32-row tile m ->
//    a 4 KB block at ((h * K/128 + c) * 4 + m) * 4096. Its dwordx4 piece q of
//    lane l sits at q * 1024 + 16 l (each wave load is 1 KB contiguous) and holds
//    row 32m + l % 32 for MFMA steps j = 2q and 2q + 1, each 8 codes at
//    k = 128c + 16j + 8 (l / 32) + [0, 8). The activation B operand takes the
//    same k from LDS, so the dot product needs no shuffles. Tokens past S reuse
//    token S-1 and are never stored. NT = 32-token tiles (1 or 2).
template <int CPC, int NT>
__global__ __launch_bounds__(256) void decode_gemv(
    const uint8_t* __restrict__ x8, const uint8_t* __restrict__ wp, float* __restrict__ part,
    int S, int K, int N) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, ks = blockIdx.y;
  const int nchk = K >> 7;
  const int c0 = ks * CPC;
  constexpr int ldw = CPC * 128 + kLdsPad;

  // the weight stream first: nothing waits on it until the MFMAs
  i32x4 wv[CPC][4];
  const uint8_t* wb = wp + ((static_cast<size_t>(h) * nchk + c0) * 4 + wave) * 4096 + lane * 16;
#pragma unroll
  for (int c = 0; c < CPC; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      wv[c][q] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wb + c * 16384 + q * 1024));
  // the FP8 activation slice of every token into LDS
  const int per_row = CPC * 8;  // 16-byte pieces per token row
  for (int i = tid; i < S * per_row; i += 256) {
    const int s = i / per_row, j = i - s * per_row;
    const i32x4 v = *reinterpret_cast<const i32x4*>(x8 + static_cast<size_t>(s) * K + c0 * 128 + j * 16);
    *reinterpret_cast<i32x4*>(lds + s * ldw + j * 16) = v;
  }
  __syncthreads();

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
      const i32x4& w = wv[c][j >> 1];
      const bf16x8 A = fp8x8_to_bf16(w[2 * (j & 1)], w[2 * (j & 1) + 1], 1.0f);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const uint2 bv = *reinterpret_cast<const uint2*>(brow[tt] + c * 128 + 16 * j);
        const bf16x8 B = fp8x8_to_bf16(bv.x, bv.y, 1.0f);
        acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[tt], 0, 0, 0);
      }
    }
  }
  // D[i][j]: token j = lane % 32, row i = 8 (r / 4) + 4 (lane / 32) + r % 4
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

// ---------------------------------------------------------------------------
// 3. head epilogue, one wave per (token, head). Lane l holds dims l and l+64;
//    the RoPE partner of dim l < 64 is dim l ^ 32, i.e. lane l ^ 32.
__global__ __launch_bounds__(64) void decode_epilogue(Args a, const float* __restrict__ part,
                                                     const float* __restrict__ sx, int ksplit) {
#pragma clang fp contract(off)
  const int H = a.heads();
  const int N = a.N();
  const int h = blockIdx.x % H;
  const int tok = blockIdx.x / H;
  const int lane = threadIdx.x;
  const int nkv = a.nkv;
  const int S = a.S;
  const int d0 = lane, d1 = lane + 64;
  const int n0 = h * kHeadDim + d0, n1 = h * kHeadDim + d1;

  double y0 = 0.0, y1 = 0.0;
  for (int ks = 0; ks < ksplit; ++ks) {
    const float* p = part + (static_cast<size_t>(ks) * S + tok) * N;
    y0 += static_cast<double>(p[n0]);
    y1 += static_cast<double>(p[n1]);
  }
  const double sxv = static_cast<double>(sx[tok]);
  y0 = (y0 * sxv) * static_cast<double>(a.w_scale[n0]);
  y1 = (y1 * sxv) * static_cast<double>(a.w_scale[n1]);

  const int k0 = 16 * nkv, v0 = 17 * nkv, iq0 = 18 * nkv, ik0 = 19 * nkv;
  int64_t slot = a.slot_mapping[tok];
  const bool store_cache = slot >= 0 && slot < static_cast<int64_t>(a.num_pages) * kPage;
  const int64_t page = slot_page(slot);
  const int t = slot_row(slot);

  if (h >= v0 && h < iq0) {  // V: the raw projection, per-token scale
    const int j = h - v0;
    const double amax = wave_max_f64(fmax(__builtin_fabs(y0), __builtin_fabs(y1)));
    const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
    if (store_cache) {
      uint8_t* vc = a.v_cache + (page * nkv + j) * kPageBytes;
      vc[d0 * kPage + t] = static_cast<uint8_t>(e4m3_from_f64(y0 / static_cast<double>(s)));
      vc[d1 * kPage + t] = static_cast<uint8_t>(e4m3_from_f64(y1 / static_cast<double>(s)));
      if (lane == 0) a.v_scale[(page * nkv + j) * kPage + t] = s;
    }
    return;
  }

  const uint16_t* g = h < k0 ? a.g_q : (h < v0 ? a.g_k : (h < ik0 ? a.g_iq : a.g_ik));
  const double ss = wave_sum_f64(y0 * y0 + y1 * y1);
  const double r = 1.0 / __builtin_sqrt(ss / static_cast<double>(kHeadDim) + static_cast<double>(a.eps));
  const double nm0 = (y0 * r) * (1.0 + static_cast<double>(bf16_to_f32(g[d0])));
  const double nm1 = (y1 * r) * (1.0 + static_cast<double>(bf16_to_f32(g[d1])));
  int64_t pos = a.positions[tok];
  pos = pos < 0 ? 0 : (pos >= a.max_pos ? a.max_pos - 1 : pos);
  const int i = lane & 31;
  const double c = static_cast<double>(bf16_to_f32(a.cos_sin[pos * kRotary + i]));
  const double sn = static_cast<double>(bf16_to_f32(a.cos_sin[pos * kRotary + 32 + i]));
  const double partner = __shfl_xor(nm0, 32, 64);
  const double o0 = lane < 32 ? nm0 * c - partner * sn : nm0 * c + partner * sn;
  const double o1 = nm1;

  if (h < k0) {
    uint16_t* q = a.q_out + (static_cast<size_t>(tok) * k0 + h) * kHeadDim;
    q[d0] = static_cast<uint16_t>(f32_to_bf16(static_cast<float>(o0)));
    q[d1] = static_cast<uint16_t>(f32_to_bf16(static_cast<float>(o1)));
  } else if (h < v0) {  // K: per-token scale, shuffled page-16 layout
    const int j = h - k0;
    const double amax = wave_max_f64(fmax(__builtin_fabs(o0), __builtin_fabs(o1)));
    const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
    if (store_cache) {
      uint8_t* kc = a.k_cache + (page * nkv + j) * kPageBytes + t * 16;
      kc[(d0 >> 4) * 256 + (d0 & 15)] = static_cast<uint8_t>(e4m3_from_f64(o0 / static_cast<double>(s)));
      kc[(d1 >> 4) * 256 + (d1 & 15)] = static_cast<uint8_t>(e4m3_from_f64(o1 / static_cast<double>(s)));
      if (lane == 0) a.k_scale[(page * nkv + j) * kPage + t] = s;
    }
  } else if (h < ik0) {
    const int j = h - iq0;
    uint16_t* q = a.iq_out + (static_cast<size_t>(tok) * nkv + j) * kHeadDim;
    q[d0] = static_cast<uint16_t>(f32_to_bf16(static_cast<float>(o0)));
    q[d1] = static_cast<uint16_t>(f32_to_bf16(static_cast<float>(o1)));
  } else if (store_cache) {  // index_k: unit-scale E4M3 into the slot's row
    uint8_t* ic = a.index_cache + slot * kHeadDim;
    ic[d0] = static_cast<uint8_t>(e4m3_from_f64(o0));
    ic[d1] = static_cast<uint8_t>(e4m3_from_f64(o1));
  }
}

// Weight repack for decode_gemv (one thread per 16-byte piece).
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

template <int CPC>
hipError_t launch_gemv_cpc(const Args& a, const DecodePlan& p) {
  const int N = a.N();
  const size_t lds = static_cast<size_t>(a.S) * (CPC * 128 + kLdsPad);
  dim3 grid(a.heads(), p.ksplit);
  float* part = reinterpret_cast<float*>(a.ws + p.off_part);
  if (a.S <= 32)
    hipLaunchKernelGGL((decode_gemv<CPC, 1>), grid, dim3(256), lds, a.stream, a.ws + p.off_x8,
                       a.w_packed, part, a.S, a.K, N);
  else
    hipLaunchKernelGGL((decode_gemv<CPC, 2>), grid, dim3(256), lds, a.stream, a.ws + p.off_x8,
                       a.w_packed, part, a.S, a.K, N);
  return hipGetLastError();
}

template <int NV>
hipError_t launch_norm_nv(const Args& a, const DecodePlan& p) {
  hipLaunchKernelGGL(decode_norm<NV>, dim3(a.S), dim3(kNormThreads), 0, a.stream, a.ar, a.res,
                     a.h_out, a.g_in, a.ws + p.off_x8, reinterpret_cast<float*>(a.ws + p.off_sx),
                     a.K, a.eps);
  return hipGetLastError();
}

}  // namespace

DecodePlan decode_plan(int S, int K, int nkv) {
  DecodePlan p{};
  const int N = (19 * nkv + 1) * 128;
  const int nchk = K / 128;
  const int row_ctas = N / kHeadDim;
  static const int kCands[] = {4, 3, 2, 1};
  int pick = 0;
  for (int c : kCands) {
    if (nchk % c) continue;
    if (static_cast<size_t>(S) * (c * 128 + kLdsPad) > kMaxLds) continue;
    pick = c;  // smallest fitting candidate so far
    if (row_ctas * (nchk / c) >= 256) break;
  }
  p.chunks_per_cta = pick;
  p.ksplit = pick ? nchk / pick : 0;
  size_t off = 0;
  p.off_x8 = off;
  off = align_up(off + static_cast<size_t>(S) * K, 256);
  p.off_sx = off;
  off = align_up(off + sizeof(float) * S, 256);
  p.off_part = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(p.ksplit) * S * N, 256);
  p.off_cnt = off;
  off += 1024;
  p.total = off;
  return p;
}

hipError_t launch_decode(const Args& a, const DecodePlan& p) {
  hipError_t e;
  const int nv = (a.K / 8 + kNormThreads - 1) / kNormThreads;
  switch (nv) {
    case 1: e = launch_norm_nv<1>(a, p); break;
    case 2: e = launch_norm_nv<2>(a, p); break;
    case 3: e = launch_norm_nv<3>(a, p); break;
    case 4: e = launch_norm_nv<4>(a, p); break;
    case 5: e = launch_norm_nv<5>(a, p); break;
    case 6: e = launch_norm_nv<6>(a, p); break;
    case 7: e = launch_norm_nv<7>(a, p); break;
    case 8: e = launch_norm_nv<8>(a, p); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if ((e = mark(a.ev_start, a.stream)) != hipSuccess) return e;
  switch (p.chunks_per_cta) {
    case 1: e = launch_gemv_cpc<1>(a, p); break;
    case 2: e = launch_gemv_cpc<2>(a, p); break;
    case 3: e = launch_gemv_cpc<3>(a, p); break;
    case 4: e = launch_gemv_cpc<4>(a, p); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if ((e = mark(a.ev_stop, a.stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(decode_epilogue, dim3(a.S * a.heads()), dim3(64), 0, a.stream, a,
                     reinterpret_cast<const float*>(a.ws + p.off_part),
                     reinterpret_cast<const float*>(a.ws + p.off_sx), p.ksplit);
  return hipGetLastError();
}

hipError_t launch_pack_decode(const uint8_t* w, uint8_t* wp, int N, int K, hipStream_t s) {
  const size_t pieces = static_cast<size_t>(N) * K / 16;
  const unsigned blocks = static_cast<unsigned>((pieces + 255) / 256);
  hipLaunchKernelGGL(pack_decode, dim3(blocks), dim3(256), 0, s, w, wp, N, K);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(n < 256 * 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(fill_zero, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace pa
