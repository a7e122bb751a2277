// Device helpers for the prologue kernels (gfx950, wave64).
//
// Number formats: bf16 is the top half of an IEEE binary32 rounded to nearest
// even; E4M3 is OCP E4M3FN (bias 7, max 448, no infinities, S.1111.111 = NaN),
// produced here by round-to-nearest-even with saturation at +-448, the FP8
// rounding the K1 mono_pre page (vllm.models.minimax_m3.amd.mono.kernels.pre_attn)
// applies to activations and to the K / V / index_k caches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kHeadDim = 128;
constexpr int kRotary = 64;
constexpr int kPage = 16;
constexpr int kPageBytes = kPage * kHeadDim;
constexpr double kFp8Max = 448.0;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw, untyped buffer resource (gfx9 descriptor word 3) over `bytes` bytes at
// `base`. A load whose per-lane offset is at or past the size returns zeros and
// such a store is dropped (the kernels here rely on that with a zero scalar
// offset only).
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t panel(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufWord3);
}

// Eight E4M3 codes (two dwords, byte order = element order) -> eight bf16 values
// times `scale` (a power of two). Every E4M3 value, and every such product in
// bf16's normal range, is a bf16 value, so the widening is exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi, float scale) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(lo), scale, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(lo), scale, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(hi), scale, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(hi), scale, true);
  return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Keeps an MFMA result materialized in uniform control flow: without it the
// compiler may sink the last MFMA of a chain into a lane-divergent store branch,
// where the inactive lanes' operands are undefined.
template <typename T>
__device__ __forceinline__ void pin_registers(T& v) {
  asm volatile("" : "+v"(v));
}

// bf16 element e (0..7) of a 16-byte piece, widened exactly to f32 / f64
__device__ __forceinline__ float bf16_at_f32(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}
__device__ __forceinline__ double bf16_at(const u32x4& v, int e) { return static_cast<double>(bf16_at_f32(v, e)); }

// two floats to bf16 (round to nearest even, NaN quiet; the hardware conversion)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float32 -> bf16 bits, round to nearest even, NaN kept quiet (the hardware
// conversion, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// E4M3 codes of float64 values times a power of two 2^-s, made by the hardware
// float32 -> FP8 conversion (v_cvt_pk_fp8_f32: OCP E4M3FN, round to nearest
// even) from an exact stand-in. Rounding v 2^-s to float32 first and then to
// E4M3 could round twice; rounding to odd instead (truncate, then set the last
// bit if anything nonzero was dropped) keeps every value that is not already a
// float32 strictly between the same two float32 neighbours, and float32 has
// 20 more significand bits than E4M3, so the E4M3 rounding of the odd result
// (ties included: an exact tie is exact in float32) is that of v 2^-s.
// The magnitude is clamped to [2^-11, 448] 2^s first (below 2^-11 everything
// rounds to a signed zero, above 448 saturates), so the float32 exponent is
// 116..135 and can be built from the float64 one with 9-bit wrap-around
// arithmetic: alignbit takes exponent bits 8..0 and the top 23 mantissa bits,
// and adding (128 - s) << 23 turns exponent e into e - 1023 - s + 127 modulo 512.
struct Fp8Scale {
  double lo, hi;   // 2^(s - 11), 448 * 2^s
  uint32_t bias;   // (128 - s) << 23, modulo 2^32
};

__device__ __forceinline__ Fp8Scale fp8_scale(int s) {
  Fp8Scale f;
  f.lo = __hiloint2double((1023 - 11 + s) << 20, 0);
  f.hi = 448.0 * __hiloint2double((1023 + s) << 20, 0);
  f.bias = static_cast<uint32_t>(128 - s) << 23;
  return f;
}

__device__ __forceinline__ float f32_odd_scaled(double v, const Fp8Scale& f) {
  const double a = __builtin_fmin(__builtin_fmax(__builtin_fabs(v), f.lo), f.hi);
  const uint32_t h = static_cast<uint32_t>(__double2hiint(a)), l = static_cast<uint32_t>(__double2loint(a));
  uint32_t t = __builtin_amdgcn_alignbit(h, l, 29) + f.bias;  // truncated magnitude
  uint32_t sticky;  // dropped bits 28..0 nonzero -> 1 (one v_min_u32 on l << 3)
  asm("v_min_u32_e32 %0, 1, %1" : "=v"(sticky) : "v"(l << 3));
  t |= sticky | (static_cast<uint32_t>(__double2hiint(v)) & 0x80000000u);
  return __uint_as_float(t);
}

// Two E4M3 codes (bytes 0 and 1; the upper half is zero) of v0, v1 * 2^-s.
__device__ __forceinline__ uint32_t e4m3x2_scaled(double v0, double v1, const Fp8Scale& f) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_cvt_pk_fp8_f32(f32_odd_scaled(v0, f), f32_odd_scaled(v1, f), 0, false));
}

// RN64(x / s) for s > 0 without a division, given rcp = RN64(1 / s). q = x rcp
// is within two ulps of x / s; a step q + RN(r rcp) with the remainder
// r = x - q s (one fma) brings it within an ulp, where r is exact, and from
// there one more such step gives the correctly rounded quotient (Markstein's
// theorem; a quotient of two doubles is never halfway between two doubles).
// The magnitudes here are far from float64 underflow and overflow.
__device__ __forceinline__ double div_rn(double x, double s, double rcp) {
  double q = x * rcp;
  q = __builtin_fma(__builtin_fma(-q, s, x), rcp, q);
  return __builtin_fma(__builtin_fma(-q, s, x), rcp, q);
}

// Four E4M3 codes (bytes in element order) of v[0..3] * 2^-s.
__device__ __forceinline__ uint32_t e4m3x4_scaled(double v0, double v1, double v2, double v3, const Fp8Scale& f) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(f32_odd_scaled(v0, f), f32_odd_scaled(v1, f), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(f32_odd_scaled(v2, f), f32_odd_scaled(v3, f), w, true);
  return static_cast<uint32_t>(w);
}

// NVFP4 (the epilogue page's K / V / index_k cache format): per 16-value group
// an E4M3 scale byte and 16 E2M1 codes, element 2b in the low nibble of byte b.
constexpr int kNvSlotBytes = kPage * (kHeadDim / 2 + kHeadDim / 16);  // 1152
constexpr int kNvScaleOff = kPage * kHeadDim / 2;                     // 1024

// Value of a non-negative E4M3 code (exact): (1 + m/8) 2^(e-7), or m 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : static_cast<float>(m) * 0x1p-9f;
}

// A group's scale code sf and element multiplier r, from the group's largest
// magnitude (float32): sf = E4M3(max(amax * f32(1/6) [* gs], 2^-9)), saturating;
// r = RN32(1 / dec(sf)) [* gs]. The reciprocal is taken in float64 and rounded
// once more to float32: 1 / dec(sf) is m^-1 2^k with m an odd integer below 16,
// whose binary expansion repeats with a period of at most 12 bits, so the
// float64 value is never a float32 midpoint and the second rounding gives the
// correctly rounded float32 reciprocal.
struct NvScale {
  uint32_t sf;
  float r;
};

__device__ __forceinline__ NvScale nv_scale(float amax, float gs, bool has_gs) {
#pragma clang fp contract(off)
  float a = amax * (1.0f / 6.0f);
  if (has_gs) a = a * gs;
  a = __builtin_fmaxf(a, 0x1p-9f);
  NvScale s;
  s.sf = e4m3x2_scaled(static_cast<double>(a), 0.0, fp8_scale(0)) & 0xFFu;
  s.r = static_cast<float>(1.0 / static_cast<double>(e4m3_to_f32(s.sf)));
  if (has_gs) s.r = s.r * gs;
  return s;
}

// float32 product rounded toward zero: exact in float64, rounded to nearest
// float32, then one ulp back toward zero where that landed past the exact value.
__device__ __forceinline__ float mul_rz(float x, float y) {
  const double p = static_cast<double>(x) * static_cast<double>(y);
  const float f = static_cast<float>(p);
  return __builtin_fabs(static_cast<double>(f)) > __builtin_fabs(p) ? __uint_as_float(__float_as_uint(f) - 1u) : f;
}

// E2M1 code of q: nearest, ties to the even code, saturating at +-6 (the
// comparisons below are the rounding boundaries of the grid 0, .5, 1, 1.5, 2,
// 3, 4, 6, strict where the tie goes down to the even code); a zero magnitude
// keeps no sign.
__device__ __forceinline__ uint32_t e2m1_code(float q) {
  const float a = __builtin_fabsf(q);
  const uint32_t m = static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
                     static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
                     static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
                     static_cast<uint32_t>(a > 5.0f);
  return m | (q < 0.0f && m != 0u ? 8u : 0u);
}

// Offset of token t's group-g scale byte in a slot's scale area: linear
// (K, index_k) or the swizzled V view, (t/4*4 + g/2)*8 + (g%2)*4 + t%4.
__device__ __forceinline__ int nv_scale_offset(int t, int g, bool swizzled) {
  return swizzled ? ((t >> 2) * 4 + (g >> 1)) * 8 + (g & 1) * 4 + (t & 3) : 8 * t + g;
}

// Wave64 reductions of float64 with DPP row operations (no LDS traffic):
// xor-1 and xor-2 inside quads, the half-row and row mirrors, then the row
// broadcasts of lanes 15 and 31 carry the partial results up to lane 63, which
// is read back for every lane. A DPP move works on 32 bits, so each step moves
// both halves; rows outside `row_mask` receive the identity.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ double dpp_f64(double v, double identity) {
  const int lo = __builtin_amdgcn_update_dpp(__double2loint(identity), __double2loint(v), kCtrl, kRowMask, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(__double2hiint(identity), __double2hiint(v), kCtrl, kRowMask, 0xf, false);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double lane63_f64(double v) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1, 0xf>(v, 0.0);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E, 0xf>(v, 0.0);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141, 0xf>(v, 0.0);  // row_half_mirror
  v += dpp_f64<0x140, 0xf>(v, 0.0);  // row_mirror
  v += dpp_f64<0x142, 0xa>(v, 0.0);  // row_bcast:15 into rows 1, 3
  v += dpp_f64<0x143, 0xc>(v, 0.0);  // row_bcast:31 into rows 2, 3
  return lane63_f64(v);
}

// max of non-negative values (identity 0)
__device__ __forceinline__ double wave_max_f64(double v) {
  v = __builtin_fmax(v, dpp_f64<0xB1, 0xf>(v, 0.0));
  v = __builtin_fmax(v, dpp_f64<0x4E, 0xf>(v, 0.0));
  v = __builtin_fmax(v, dpp_f64<0x141, 0xf>(v, 0.0));
  v = __builtin_fmax(v, dpp_f64<0x140, 0xf>(v, 0.0));
  v = __builtin_fmax(v, dpp_f64<0x142, 0xa>(v, 0.0));
  v = __builtin_fmax(v, dpp_f64<0x143, 0xc>(v, 0.0));
  return lane63_f64(v);
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Timeline stamp k of CTA b (8 per CTA): the 100 MHz s_memrealtime counter.
__device__ __forceinline__ void stamp(uint64_t* tl, uint32_t slots, int b, int k) {
  if (tl != nullptr && threadIdx.x == 0 && static_cast<uint32_t>(b * 8 + k) < slots)
    tl[b * 8 + k] = __builtin_amdgcn_s_memrealtime();
}

// Where the stamping wave runs: XCC_ID (hardware register 20) in the upper
// word, HW_ID (register 4: wave, SIMD, CU, shader array and engine) below.
__device__ __forceinline__ void stamp_place(uint64_t* tl, uint32_t slots, int b, int k) {
  if (tl != nullptr && threadIdx.x == 0 && static_cast<uint32_t>(b * 8 + k) < slots) {
    const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
    const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);
    tl[b * 8 + k] = (static_cast<uint64_t>(xcc) << 32) | hw;
  }
}

// Page-16 addressing of a slot at the default (contiguous) page stride.
__device__ __forceinline__ int64_t slot_page(int64_t slot) { return slot >> 4; }
__device__ __forceinline__ int slot_row(int64_t slot) { return static_cast<int>(slot & 15); }

}  // namespace pa
