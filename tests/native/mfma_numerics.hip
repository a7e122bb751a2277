// Test-only probes of the two MFMA forms the prefill projection uses, one wave
// and one 32x32x64 product each, for tests/test_mfma_numerics_gpu.py:
//  - the block-scaled FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) with the
//    operand layout the prefill kernels pack: lane l holds row (A) or column
//    (B) l % 32; its bytes 0..15 are k = 16 (l / 32) + [0, 16) (MX block 0) and
//    bytes 16..31 are k = 32 + 16 (l / 32) + [0, 16) (block 1); its scale byte
//    is the E8M0 code of block l / 32 of its row or column;
//  - four 32x32x16 bf16 MFMAs on the same operands widened exactly (code times
//    its block scale), step j taking bytes 8 j .. 8 j + 7 of each fragment, as
//    the precise heads do.
// D[i][j] (A row i, B column j) comes back as d[16 l + r] with j = l % 32 and
// i = 8 (r / 4) + 4 (l / 32) + r % 4.
#include <hip/hip_runtime.h>

#include <cstdint>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

namespace {

__device__ bf16x8 widen8(uint32_t lo, uint32_t hi, float scale) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
  return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ float e8m0(uint32_t c) { return __uint_as_float(c ? c << 23 : 0x00400000u); }

__global__ __launch_bounds__(64) void k_fp8(const uint32_t* a, const uint32_t* b, const uint32_t* sa,
                                            const uint32_t* sb, float* d) {
  const int l = threadIdx.x;
  i32x8 av, bv;
  for (int i = 0; i < 8; ++i) av[i] = static_cast<int>(a[8 * l + i]), bv[i] = static_cast<int>(b[8 * l + i]);
  f32x16 acc;
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, sa[l], 0, sb[l]);
  for (int r = 0; r < 16; ++r) d[16 * l + r] = acc[r];
}

__global__ __launch_bounds__(64) void k_bf16(const uint32_t* a, const uint32_t* b, const uint32_t* sa,
                                             const uint32_t* sb, float* d) {
  const int l = threadIdx.x;
  const bool low = l < 32;
  const uint32_t sa_own = sa[l], sa_x = sa[l ^ 32], sb_own = sb[l], sb_x = sb[l ^ 32];
  f32x16 acc;
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int j = 0; j < 4; ++j) {
    const bool own = (j < 2) == low;  // bytes 0..15 are block 0, 16..31 block 1
    const bf16x8 A = widen8(a[8 * l + 2 * j], a[8 * l + 2 * j + 1], e8m0(own ? sa_own : sa_x));
    const bf16x8 B = widen8(b[8 * l + 2 * j], b[8 * l + 2 * j + 1], e8m0(own ? sb_own : sb_x));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc, 0, 0, 0);
  }
  for (int r = 0; r < 16; ++r) d[16 * l + r] = acc[r];
}

}  // namespace

// a, b: 64 lanes x 32 bytes; sa, sb: 64 words (E8M0 code in the low byte);
// d: 64 x 16 floats. All device pointers; one wave on `stream`. Returns the
// HIP error code of the launch (0 on success).
extern "C" int mfma_probe_fp8(const void* a, const void* b, const void* sa, const void* sb, float* d, void* stream) {
  hipLaunchKernelGGL(k_fp8, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), static_cast<const uint32_t*>(a),
                     static_cast<const uint32_t*>(b), static_cast<const uint32_t*>(sa),
                     static_cast<const uint32_t*>(sb), d);
  return static_cast<int>(hipGetLastError());
}

extern "C" int mfma_probe_bf16(const void* a, const void* b, const void* sa, const void* sb, float* d, void* stream) {
  hipLaunchKernelGGL(k_bf16, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), static_cast<const uint32_t*>(a),
                     static_cast<const uint32_t*>(b), static_cast<const uint32_t*>(sa),
                     static_cast<const uint32_t*>(sb), d);
  return static_cast<int>(hipGetLastError());
}
