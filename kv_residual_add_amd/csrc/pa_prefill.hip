// Prefill prologue on gfx950: MXFP8 activations against an MXFP8 weight.
//
// Two kernels on the caller's stream:
//   1. prefill_prepass  token rows walked by one CTA per resident slot:
//                       residual add (f32) + bf16 residual out, Gemma RMSNorm,
//                       then OCP-MX quantization (E8M0 scale per 32-wide k
//                       block, E4M3 elements) into the GEMM's packed activation
//                       layout in the workspace.
//   2. prefill_gemm     C^T = W . X^T on MFMA. One CTA owns one 128-wide head
//                       x 128 NTW tokens; each wave 32 NTW tokens x the whole
//                       head.
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
// Head-step options (pre_attn_prefill_ex) as in decode: unit K / V scales,
// an FP8 q output, NVFP4 K / V / index_k caches (lane-local 16-value groups;
// K and index_k stage their float32 values in the lane's own LDS row half).
//
// Numerics: as in decode, the norm / MX decision and the head epilogue run in
// float64 with contraction off.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr int kTokAlign = 256;  // token rows of the packed activation (largest CTA tile)
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

// Norm pass. A CTA walks the token rows blockIdx.x, + gridDim.x, ...; a thread
// owns one 16-element chunk of every row (blockDim = hidden / 16 rounded up to
// a wave; at most 1024 since hidden <= 16384). The chunk's 16 codes are 16
// contiguous bytes of the packed layout, written with one store; an MX block is
// the chunk pair of lanes 2j, 2j + 1. Up to hidden 8192 (WIDE false) a thread
// keeps its chunk's 1 + g factors in float64 registers for all its rows and
// issues the next row's loads before working on the current one; above that
// the register budget of 1024 threads allows neither.
//
// Every global access goes through a buffer resource sized to what it may
// touch: rows past the last token get size 0 (their loads read zeros and their
// stores vanish), threads past the row and the odd lanes of the scale byte
// store fall outside by offset. No access is predicated by a branch, so the
// compiler's wait counts stay exact across the row loop.
template <bool WIDE>
__global__ __launch_bounds__(WIDE ? 1024 : 512) void prefill_prepass(
    const uint16_t* __restrict__ ar, const uint16_t* __restrict__ res,
    uint16_t* __restrict__ h_out, const uint16_t* __restrict__ g_in,
    uint8_t* __restrict__ xq, uint8_t* __restrict__ xs, int M, int mpad, int K, float eps) {
#pragma clang fp contract(off)
  __shared__ double red[2][16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = static_cast<int>(blockDim.x >> 6);
  const int nks = K / kKStep;
  const uint32_t row_bytes = 2u * static_cast<uint32_t>(K);
  const uint32_t voff = 32u * tid;  // at or past row_bytes for threads past the row
  const auto row_rsrc = [&](const uint16_t* base, int r) {
    const bool live = r < M;
    return panel(base + static_cast<size_t>(live ? r : 0) * K, live ? row_bytes : 0u);
  };
  const auto gr = panel(g_in, row_bytes);
  u32x4 gv[2] = {__builtin_amdgcn_raw_buffer_load_b128(gr, voff, 0, 0),
                 __builtin_amdgcn_raw_buffer_load_b128(gr, voff + 16, 0, 0)};
  double g1[16];
  if constexpr (!WIDE) {
#pragma unroll
    for (int e = 0; e < 16; ++e) g1[e] = 1.0 + bf16_at(gv[e >> 3], e & 7);
  }
  // chunk offsets in the packed activation of a token tile (past the tile for
  // threads past the row; the odd lane of a block pair stores no scale)
  const int k = 16 * tid;
  const uint32_t xq_off = static_cast<uint32_t>(xq_offset(0, k, nks));
  const uint32_t xs_off = (tid & 1) ? 0x7ffffff0u : static_cast<uint32_t>(xs_offset(0, tid >> 1, nks));
  const uint32_t tile_q = static_cast<uint32_t>(nks) * kTileBytes, tile_s = static_cast<uint32_t>(nks) * 64;

  // Rows 8i .. 8i + 7 of a token tile fill the packed activation's 128-byte
  // lines together (16 bytes each), so they go to the 8 blocks of one XCD
  // (equal index mod 8) in the same pass, and each line is assembled in one
  // L2 rather than written back in pieces by all eight. The grid is a multiple
  // of 64 and the mapping a bijection onto [0, grid) whatever the placement.
  const int G = static_cast<int>(gridDim.x);
  const int bx = static_cast<int>(blockIdx.x) & 7, bj = static_cast<int>(blockIdx.x) >> 3;
  int row = 8 * (bx * (G >> 6) + (bj >> 3)) + (bj & 7);
  u32x4 av[2], bv[2];
  const auto load_row = [&](int r, u32x4* x, u32x4* y) {
    const auto ra = row_rsrc(ar, r), rb = row_rsrc(res, r);
    x[0] = __builtin_amdgcn_raw_buffer_load_b128(ra, voff, 0, 0);
    x[1] = __builtin_amdgcn_raw_buffer_load_b128(ra, voff + 16, 0, 0);
    y[0] = __builtin_amdgcn_raw_buffer_load_b128(rb, voff, 0, 0);
    y[1] = __builtin_amdgcn_raw_buffer_load_b128(rb, voff + 16, 0, 0);
  };
  if constexpr (!WIDE) load_row(row, av, bv);
  // A row's codes and scale are stored one row later, right after the next
  // row's data has arrived. Loads and stores share the vector-memory counter
  // and may complete out of order, so a wave with stores in flight can only
  // wait for all of them: stored at the end of its row, they made every next
  // row wait out their acknowledgements; stored early, they are done by then.
  u32x4 pw = {0u, 0u, 0u, 0u};
  uint32_t pcode = 0;
  int prow = -1;  // uniform: no row pending
  const auto store_codes = [&]() {
    const size_t tt = static_cast<size_t>(prow >> 5);
    const uint32_t tl = static_cast<uint32_t>(prow & 31);
    __builtin_amdgcn_raw_buffer_store_b128(pw, panel(xq + tt * tile_q, tile_q), xq_off + 16u * tl, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(pcode), panel(xs + tt * tile_s, tile_s), xs_off + tl, 0,
                                         0);
  };
  for (int it = 0; row < mpad; ++it) {
    const int next = row + static_cast<int>(gridDim.x);
    u32x4 an[2], bn[2];
    if constexpr (WIDE) {
      load_row(row, av, bv);
      asm volatile("" : "+v"(gv[0]), "+v"(gv[1]));  // rebuilt every row, not hoisted
#pragma unroll
      for (int e = 0; e < 16; ++e) g1[e] = 1.0 + bf16_at(gv[e >> 3], e & 7);
    } else {
      load_row(next, an, bn);
    }
    // residual add in float32, bf16 residual out, sum of squares in float64
    // (a float32 square is exact in float64, so the fma rounds only the sum)
    double acc[16];  // the float32 sums, widened once
    double ssp[4] = {0.0, 0.0, 0.0, 0.0};
    u32x4 hv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = bf16_at_f32(av[i], 2 * q) + bf16_at_f32(bv[i], 2 * q);
        const float hi = bf16_at_f32(av[i], 2 * q + 1) + bf16_at_f32(bv[i], 2 * q + 1);
        hv[i][q] = pack_bf16x2(lo, hi);
        const double dl = static_cast<double>(lo), dh = static_cast<double>(hi);
        acc[8 * i + 2 * q] = dl;
        acc[8 * i + 2 * q + 1] = dh;
        ssp[q] = __builtin_fma(dl, dl, ssp[q]);
        ssp[q] = __builtin_fma(dh, dh, ssp[q]);
      }
    }
    const auto hr = row_rsrc(h_out, row);
    __builtin_amdgcn_raw_buffer_store_b128(hv[0], hr, voff, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(hv[1], hr, voff + 16, 0, 0);
    if (prow >= 0) store_codes();
    // row sum: DPP wave sums, then the waves' values in a fixed order; the two
    // halves of `red` alternate between rows, so one barrier per row suffices
    const double ss = wave_sum_f64((ssp[0] + ssp[1]) + (ssp[2] + ssp[3]));
    double* part = red[it & 1];
    if (lane == 0) part[wave] = ss;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    double tot = part[0];
    for (int w = 1; w < nw; ++w) tot += part[w];
    double rstd = 1.0 / __builtin_sqrt(tot / static_cast<double>(K) + static_cast<double>(eps));
    const bool live = row < M;
    rstd = live ? rstd : 0.0;
    double xn[16];
    double amax = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      xn[e] = (acc[e] * rstd) * g1[e];
      amax = __builtin_fmax(amax, __builtin_fabs(xn[e]));
    }
    amax = __builtin_fmax(amax, dpp_f64<0xB1, 0xf>(amax, 0.0));  // the block's other chunk: lane ^ 1
    // X = 2^(floor(log2 amax) - 8) as an E8M0 code; an all-zero block keeps X = 1
    int code = static_cast<int>((static_cast<uint32_t>(__double2hiint(amax)) >> 20) & 0x7ffu) - 1023 - 8 + 127;
    code = code < 0 ? 0 : (code > 254 ? 254 : code);
    code = amax != 0.0 ? code : 127;
    const Fp8Scale f = fp8_scale(code - 127);
    const uint32_t keep = live ? ~0u : 0u;  // a padding row stores zero codes (a mask, not a branch)
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = e4m3x4_scaled(xn[4 * j], xn[4 * j + 1], xn[4 * j + 2], xn[4 * j + 3], f) & keep;
    pw = w;
    pcode = static_cast<uint32_t>(code);
    prow = row;
    if constexpr (!WIDE) {
      av[0] = an[0], av[1] = an[1], bv[0] = bn[0], bv[1] = bn[1];
    }
    row = next;
  }
  if (prow >= 0) store_codes();  // the last row's
}

// Packed weight: head h, k step ks, 32-row tile m -> 2 KB block at
// ((h * nks + ks) * 4 + m) * 2048 in the activation's lane order (row
// 32m + l % 32). Scales: dword (h * nks + ks) * 64 + l holds tiles m = 0..3 in
// bytes 0..3, each the row's E8M0 for block 2 ks + l / 32.
// After the FP8 blocks of every head, the precise heads (k heads, v heads,
// then index_k: precise index p) carry a bf16 copy of their weight, each value
// code * 2^(e - 127) exactly (E8M0 codes in [10, 246]), in the bf16 MFMA's
// operand order: a 16 KB block per k step; in it row tile m and MFMA step j
// (16 k) hold 1 KB at m * 4096 + j * 1024, lane l's 8 values at 16 l: row
// 32 m + l % 32, k = 64 ks + 32 (j / 2) + 16 (l / 32) + 8 (j % 2) + [0, 8)
// (the k order the activation operand takes from its FP8 fragment).
constexpr int kBf16StepBytes = 16384;

__device__ __forceinline__ bool precise_head(int h, int nkv) {
  return (h >= 16 * nkv && h < 18 * nkv) || h == 19 * nkv;
}

__host__ __device__ __forceinline__ int precise_index(int h, int nkv) { return h < 18 * nkv ? h - 16 * nkv : 2 * nkv; }

__host__ __device__ __forceinline__ size_t precise_panel_offset(int N, int K, int p) {
  return static_cast<size_t>(N) * K + static_cast<size_t>(p) * kHeadDim * K * 2;
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  return __uint_as_float(c ? c << 23 : 0x00400000u);
}

// ---------------------------------------------------------------------------
// Main loop. A wave owns the whole 128-row head x NTW 32-token tiles. The CTA's
// four waves share the head's weight tile of each 64-wide k step, which the
// buffer unit writes straight into a four-slot LDS ring (no registers on the
// way), while each wave keeps its own activation tiles and the scales in one of
// four register sets. A stage (SUB k steps: two in one-tile CTAs, whose
// registers allow it, one otherwise) is issued kPrefetch stages ahead of its
// MFMAs, so L2 and Infinity Cache latency (up to about a microsecond when a
// load misses) overlaps that many stages of MFMA work; the barrier and the
// wait come once a stage.
//
// Per step: weight 8 KB (4 row tiles x 2 KB) + one scale dword per lane;
// activations per token tile 2 KB + one scale byte per lane. FP8 heads feed
// them to the block-scaled FP8 MFMA; precise heads widen both operands exactly
// to bf16 (the code times its block scale) for the bf16 MFMA.

// k steps that a step's loads are issued ahead of its MFMAs; ring slots and
// register sets: kPrefetch + 1
constexpr int kPrefetch = 3;
constexpr int kSlots = kPrefetch + 1;
constexpr int kSlotBytes = 16384;  // a weight step uses 8 KB; a slot also holds one wave's 32 x 128 f32 output tile
constexpr int kSubSingle = 2;      // k steps per stage in one-tile CTAs

// A stage is SUB consecutive k steps: their weight tiles share one ring slot
// (8 KB each) and their register loads one set.
//
// The precise heads keep the activation scale as a byte: a register set can be
// consumed after the loop's back edge, and a byte widened to 32 bits where it
// is loaded would make the compiler wait for that load (and so for every load
// issued before it) right there, draining the lookahead once a loop iteration.
// Widened where it is used, after the stage's own wait, it costs nothing.
template <bool PRECISE, int NTW, int SUB>
struct Stage {
  using ScaleByte = std::conditional_t<PRECISE, uint8_t, uint32_t>;
  uint32_t sa[SUB];        // weight scale dword (row tiles in bytes 0..3) for block lane / 32
  i32x4 b[SUB][NTW][2];    // activation bytes 0..15 and 16..31 of the lane
  ScaleByte sb[SUB][NTW];  // the lane's activation scale (its token, block lane / 32)
};

// Loads of one k step go through buffer resources, one per operand panel (the
// head's weight rows, the wave's token tiles): the per-lane offset stays in one
// vector register for the whole loop and the step's offset is a scalar. A
// resource also bounds its panel: a read past its size returns zeros.

struct Panels {
  __amdgpu_buffer_rsrc_t a, sa, b, sb;
};

template <bool PRECISE, int NTW>
__device__ __forceinline__ Panels make_panels(const KArgs& a, int h, int tt0, const uint8_t* xq, const uint8_t* xs) {
  const size_t nks = a.K / kKStep;
  Panels p;
  if (PRECISE)  // the head's bf16 panel
    p.a = panel(a.w_packed + precise_panel_offset(a.N(), a.K, precise_index(h, a.nkv)), nks * kBf16StepBytes);
  else
    p.a = panel(a.w_packed + static_cast<size_t>(h) * nks * 4 * kTileBytes, nks * 4 * kTileBytes);
  p.sa = panel(a.s_packed + static_cast<size_t>(h) * nks * 256, nks * 256);
  p.b = panel(xq + static_cast<size_t>(tt0) * nks * kTileBytes, NTW * nks * kTileBytes);
  p.sb = panel(xs + static_cast<size_t>(tt0) * nks * 64, NTW * nks * 64);
  return p;
}

// Vector-memory instructions one stage issues per wave (the waits count them):
// per k step the weight tile's LDS copies (FP8: 2, bf16: 4) and, FP8 only, the
// weight scale dword, then two activation loads and a scale byte per token tile.
template <bool PRECISE, int NTW, int SUB>
constexpr int step_vm_ops() {
  return SUB * ((PRECISE ? 4 : 3) + 2 * NTW + NTW);
}

// s_waitcnt immediate that waits until at most n vector-memory instructions of
// this wave are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; the
// export and LDS/scalar counters left at their no-wait maxima)
constexpr int vmcnt_at_most(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Issues stage st (k steps SUB st ..): the register loads first, then the
// weight tiles' LDS writes.
template <bool PRECISE, int NTW, int SUB>
__device__ __forceinline__ void stage_issue(Stage<PRECISE, NTW, SUB>& st, const Panels& p, int nks, int stage,
                                            uint8_t* slot, int wave) {
  const int tid = threadIdx.x, lane = tid & 63;
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    const int ks = stage * SUB + u;
    if constexpr (!PRECISE) st.sa[u] = __builtin_amdgcn_raw_buffer_load_b32(p.sa, lane * 4, ks * 256, 0);
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
      const int blk = n * nks + ks;
      st.b[u][n][0] = __builtin_amdgcn_raw_buffer_load_b128(p.b, lane * 16, blk * kTileBytes, 0);
      st.b[u][n][1] = __builtin_amdgcn_raw_buffer_load_b128(p.b, lane * 16, blk * kTileBytes + 1024, 0);
      st.sb[u][n] = __builtin_amdgcn_raw_buffer_load_b8(p.sb, lane, blk * 64, 0);
    }
  }
  // weight tiles: instruction q of wave w moves bytes (256 q + 64 w + lane) * 16
  // of step u's tile, which land at the same offset of the slot's part u
  // (FP8: two 8 KB steps a slot; bf16: one 16 KB step a slot, SUB = 1)
  if constexpr (PRECISE) {
    static_assert(SUB == 1, "a bf16 weight step fills a ring slot");
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(p.a, (__attribute__((address_space(3))) void*)(slot + q * 4096 + wave * 1024),
                                               16, tid * 16, stage * kBf16StepBytes + q * 4096, 0, 0);
  } else {
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            p.a, (__attribute__((address_space(3))) void*)(slot + u * 8192 + q * 4096 + wave * 1024), 16, tid * 16,
            (stage * SUB + u) * 4 * kTileBytes + q * 4096, 0, 0);
  }
}

// The MFMAs of one k step: weight scale dword sa0, activation fragments b0 and
// scales sb0, the weight tile at `slot`.
template <bool PRECISE, int NTW, typename ScaleByte>
__device__ __forceinline__ void step_mfma(uint32_t sa0, const i32x4 (&b0)[NTW][2], const ScaleByte (&sb0)[NTW],
                                          const uint8_t* slot, f32x16 (&acc)[NTW][4]) {
  const int lane = threadIdx.x & 63;
  if (PRECISE) {
    // bf16 MFMA step j takes bytes 8j .. 8j + 7 of each lane's 32-byte
    // activation fragment (k = 32 (j / 2) + 16 (lane / 32) + 8 (j % 2) + [0, 8)),
    // widened exactly with the block scale (bytes 0..15 are MX block 0 and
    // 16..31 block 1; the lane ^ 32 partner holds the scale of the other
    // block); the weight operand is the same k of the slot's bf16 tile.
    (void)sa0;
    uint32_t sb_x[NTW];
#pragma unroll
    for (int n = 0; n < NTW; ++n) sb_x[n] = __shfl_xor(sb0[n], 32, 64);
    const bool low = lane < 32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool own = (j < 2) == low;  // this lane's own block
      bf16x8 B[NTW];
#pragma unroll
      for (int n = 0; n < NTW; ++n) {
        const i32x4& src = b0[n][j >> 1];
        B[n] = fp8x8_to_bf16(src[2 * (j & 1)], src[2 * (j & 1) + 1], e8m0_to_f32((own ? sb0[n] : sb_x[n]) & 0xffu));
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(slot + m * 4096 + j * 1024 + lane * 16);
#pragma unroll
        for (int n = 0; n < NTW; ++n) acc[n][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B[n], acc[n][m], 0, 0, 0);
      }
    }
  } else {
    i32x8 Am[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const i32x4 a0 = reinterpret_cast<const i32x4*>(slot + m * kTileBytes)[lane];
      const i32x4 a1 = reinterpret_cast<const i32x4*>(slot + m * kTileBytes + 1024)[lane];
      Am[m] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const i32x8 A = Am[m];
#pragma unroll
      for (int n = 0; n < NTW; ++n) {
        const i32x8 B = {b0[n][0][0], b0[n][0][1], b0[n][0][2], b0[n][0][3],
                         b0[n][1][0], b0[n][1][1], b0[n][1][2], b0[n][1][3]};
        switch (m) {  // the scale byte of row tile m (op_sel is an immediate)
          case 0: acc[n][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[n][0], 0, 0, 0, sa0, 0, sb0[n]); break;
          case 1: acc[n][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[n][1], 0, 0, 1, sa0, 0, sb0[n]); break;
          case 2: acc[n][2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[n][2], 0, 0, 2, sa0, 0, sb0[n]); break;
          default: acc[n][3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[n][3], 0, 0, 3, sa0, 0, sb0[n]); break;
        }
      }
    }
  }
}

// The precise heads' weight-operand LDS reads are issued ahead of the MFMAs
// that take them (scheduling groups, in order). Left to itself the compiler
// reads each operand just before its MFMA and waits for it there, so each of
// a step's 16 reads paid the LDS latency against one 32-cycle bf16 MFMA (two
// in two-tile CTAs); they now run 8 reads ahead in one-tile CTAs and 4 in
// two-tile CTAs, whose registers are full. The two-tile FP8 step is grouped
// as each row tile's reads, then its two MFMAs: the compiler's own order for
// the reads (a row tile read ahead measured no better), but the groups also
// keep the stage's loads out of the MFMA run, ~0.5 % faster on the 8192-token
// workload than without them. The one-tile FP8 step keeps the compiler's order.
template <bool PRECISE, int NTW, int SUB>
__device__ __forceinline__ void stage_mfma(const Stage<PRECISE, NTW, SUB>& st, const uint8_t* slot,
                                           f32x16 (&acc)[NTW][4]) {
#pragma unroll
  for (int u = 0; u < SUB; ++u) step_mfma<PRECISE, NTW>(st.sa[u], st.b[u], st.sb[u], slot + u * 8192, acc);
  constexpr int kDs = 0x080, kDsRead = 0x100, kMfma = 0x008;  // sched_group_barrier masks
  if constexpr (PRECISE) {
    static_assert(SUB == 1, "one bf16 step a stage");
    constexpr int ahead = NTW == 1 ? 8 : 4;
    __builtin_amdgcn_sched_group_barrier(kDs, ahead + NTW, 0);  // + the scale shuffles
#pragma unroll
    for (int i = 0; i < 16 - ahead; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, NTW, 0);
      __builtin_amdgcn_sched_group_barrier(kDs, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfma, ahead * NTW, 0);
  } else if constexpr (NTW == 2) {
    __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfma, 2, 0);
  }
}

// One stage of the pipeline: wait until this wave's loads of stage s have
// landed (the two later stages' loads may still fly), barrier so every wave's
// part of the weight tiles is in LDS and every wave is done with stage s - 1,
// then issue stage s + kPrefetch into the slot and register set stage s - 1
// used, and run stage s. The scheduling barriers keep each stage's loads in
// issue order, which the wait count relies on.
template <bool PRECISE, int NTW, int SUB, int I>
__device__ __forceinline__ void pipeline_step(Stage<PRECISE, NTW, SUB> (&st)[kSlots], uint8_t* const (&ring)[kSlots],
                                              const Panels& p, int nks, int s, int wave, f32x16 (&acc)[NTW][4]) {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_at_most((kPrefetch - 1) * step_vm_ops<PRECISE, NTW, SUB>()));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  const int last = nks / SUB - 1;
  const int ahead = s + kPrefetch < last ? s + kPrefetch : last;  // clamped; extra steps are never used
  stage_issue(st[(I + kPrefetch) % kSlots], p, nks, ahead, ring[(I + kPrefetch) % kSlots], wave);
  __builtin_amdgcn_sched_barrier(0);
  stage_mfma(st[I], ring[I], acc);
}

template <bool PRECISE, int NTW, int SUB>
__device__ __forceinline__ void mainloop(const KArgs& a, int h, int tt0, const uint8_t* __restrict__ xq,
                                         const uint8_t* __restrict__ xs, uint8_t* const (&ring)[kSlots], int wave,
                                         f32x16 (&acc)[NTW][4]) {
  const int nks = a.K / kKStep;
  const int nst = nks / SUB;  // stages (hidden is a multiple of 128: nks is even)
  const int last = nst - 1;
  const Panels p = make_panels<PRECISE, NTW>(a, h, tt0, xq, xs);
  Stage<PRECISE, NTW, SUB> st[kSlots];
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) {
    stage_issue(st[i], p, nks, i < last ? i : last, ring[i], wave);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Whole groups of kSlots steps keep ring slot and register set indices
  // static; the tail covers nks % kSlots steps.
  int s0 = 0;
  for (; s0 + kSlots <= nst; s0 += kSlots) {
    pipeline_step<PRECISE, NTW, SUB, 0>(st, ring, p, nks, s0 + 0, wave, acc);
    pipeline_step<PRECISE, NTW, SUB, 1>(st, ring, p, nks, s0 + 1, wave, acc);
    pipeline_step<PRECISE, NTW, SUB, 2>(st, ring, p, nks, s0 + 2, wave, acc);
    pipeline_step<PRECISE, NTW, SUB, 3>(st, ring, p, nks, s0 + 3, wave, acc);
  }
  if (s0 + 0 < nst) pipeline_step<PRECISE, NTW, SUB, 0>(st, ring, p, nks, s0 + 0, wave, acc);
  if (s0 + 1 < nst) pipeline_step<PRECISE, NTW, SUB, 1>(st, ring, p, nks, s0 + 1, wave, acc);
  if (s0 + 2 < nst) pipeline_step<PRECISE, NTW, SUB, 2>(st, ring, p, nks, s0 + 2, wave, acc);
  static_assert(kSlots == 4, "the group above is written out for four slots");
  // every load (including the clamped extra steps) has landed and every wave
  // is past its last LDS read before the ring is reused
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// Epilogue of one 32-token tile, read back from LDS where each wave has left its
// 32 x 128 f32 tile in one ring slot: token row r holds 32 16-byte chunks (4
// dims each), chunk c stored at position c ^ r so that the 32 rows written or
// read together fall on different banks. Lane l takes token tt * 32 + l % 32
// and dims [64 (l / 32), 64 (l / 32) + 64): the lower half holds both members
// (d, d + 32) of every rotated pair, the upper half none, and runs the same
// code with cos = 1 and sin = 0, an exact identity. The values are read from
// LDS as they are needed, so the 64 of them never live in registers as f64.
struct TileRow {
  const float* row;  // the token's row
  int r;             // row index 0..31 (the swizzle key)
  __device__ __forceinline__ float4 chunk(int c) const {  // dims 4c .. 4c + 3
    return *reinterpret_cast<const float4*>(row + 4 * (c ^ r));
  }
  __device__ __forceinline__ float at(int d) const { return row[4 * ((d >> 2) ^ r) + (d & 3)]; }
};

// The epilogue's per-token inputs, requested before the accumulators go to LDS
// so that their latency overlaps that hand-off: for the lower half of the lanes
// the 32 cos and 32 sin values of the token. (The head's gamma row is staged
// in LDS when the CTA starts.)
struct EpiIn {
  u32x4 c[4];   // cos of rotary index 8j .. + 7
  u32x4 sn[4];  // sin of rotary index 8j .. + 7
};

__device__ __forceinline__ EpiIn epilogue_loads(const KArgs& a, int64_t pos) {
  const int half = (threadIdx.x & 63) >> 5;
  EpiIn in;
  if (half == 0) {
    const u32x4* cp = reinterpret_cast<const u32x4*>(a.cos_sin + pos * kRotary);
#pragma unroll
    for (int j = 0; j < 4; ++j) in.c[j] = cp[j], in.sn[j] = cp[4 + j];
  } else {  // no rotation: cos = 1.0 (bf16 0x3f80), sin = 0
#pragma unroll
    for (int j = 0; j < 4; ++j) in.c[j] = u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u},
                                in.sn[j] = u32x4{0u, 0u, 0u, 0u};
  }
  return in;
}

// the gamma row of head h's role
__device__ __forceinline__ const uint16_t* head_gamma(const KArgs& a, int h) {
  const int nkv = a.nkv;
  return h < 16 * nkv ? a.g_q : (h < 17 * nkv ? a.g_k : (h < 19 * nkv ? a.g_iq : a.g_ik));
}


// A lane's half row of NVFP4 (64 dims = 4 groups, dims dbase + 16 gl ..): the
// 32 data bytes as 8 words and the 4 scale bytes, stored into a 1152-byte
// cache slot at token row t.
__device__ __forceinline__ void nv_store_half(uint8_t* slot, int t, int half, const uint32_t (&w)[8],
                                              const uint32_t (&sf)[4], bool swizzled) {
  uint8_t* d = slot + t * 64 + 32 * half;
  *reinterpret_cast<u32x4*>(d) = u32x4{w[0], w[1], w[2], w[3]};
  *reinterpret_cast<u32x4*>(d + 16) = u32x4{w[4], w[5], w[6], w[7]};
  if (!swizzled) {
    *reinterpret_cast<uint32_t*>(slot + kNvScaleOff + 8 * t + 4 * half) =
        sf[0] | (sf[1] << 8) | (sf[2] << 16) | (sf[3] << 24);
  } else {
#pragma unroll
    for (int gl = 0; gl < 4; ++gl) slot[kNvScaleOff + nv_scale_offset(t, 4 * half + gl, true)] = static_cast<uint8_t>(sf[gl]);
  }
}

// K / index_k values of the lane's half row in float64: Gemma norm with rr and
// the gamma row, NeoX rotation with the token's cos / sin (identity for the
// upper half), for the dim pair (i + e, i + 32 + e), rounded to float32 (the
// values the NVFP4 quantizer takes).
__device__ __forceinline__ void k_pair_f32(const TileRow& x, const uint16_t* gam, const u32x4 (&c)[4],
                                           const u32x4 (&sn)[4], double rr, int c0, int dbase, int i, float (&f1)[4],
                                           float (&f2)[4]) {
#pragma clang fp contract(off)
  const float4 a1 = x.chunk(c0 + (i >> 2));
  const float4 a2 = x.chunk(c0 + (i >> 2) + 8);
  const float x1s[4] = {a1.x, a1.y, a1.z, a1.w}, x2s[4] = {a2.x, a2.y, a2.z, a2.w};
  const u32x4 ga = *reinterpret_cast<const u32x4*>(gam + dbase + (i & ~7));
  const u32x4 gb = *reinterpret_cast<const u32x4*>(gam + dbase + 32 + (i & ~7));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int d = i + e;
    const double x1 = (static_cast<double>(x1s[e]) * rr) * (1.0 + bf16_at(ga, d & 7));
    const double x2 = (static_cast<double>(x2s[e]) * rr) * (1.0 + bf16_at(gb, d & 7));
    const double cd = bf16_at(c[d >> 3], d & 7), sd2 = bf16_at(sn[d >> 3], d & 7);
    f1[e] = static_cast<float>(x1 * cd - x2 * sd2);
    f2[e] = static_cast<float>(x2 * cd + x1 * sd2);
  }
}

// NVFP4 of the lane's half row: 64 float32 values read from the wave's LDS
// tile row (dims dbase + 16 gl .. for groups gl = 0..3, chunks c0 + 4 gl ..),
// into a 1152-byte cache slot at token row t.
__device__ __forceinline__ void nv_half_from_tile(const TileRow& x, int c0, float gs, bool has_gs, uint8_t* slot,
                                                  int t, int half, bool swizzled) {
  uint32_t w[8], sf[4];
#pragma unroll
  for (int gl = 0; gl < 4; ++gl) {
    float am = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 v = x.chunk(c0 + 4 * gl + c);
      am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)),
                                               __builtin_fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w))));
    }
    const NvScale ns = nv_scale(am, gs, has_gs);
    sf[gl] = ns.sf;
#pragma unroll
    for (int c = 0; c < 4; c += 2) {
      const float4 p = x.chunk(c0 + 4 * gl + c), q = x.chunk(c0 + 4 * gl + c + 1);
      const float f[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) word |= e2m1_code(mul_rz(f[e], ns.r)) << (4 * e);
      w[2 * gl + (c >> 1)] = word;
    }
  }
  nv_store_half(slot, t, half, w, sf, swizzled);
}

// NVFP4 of the lane's half row of K (global scale gs) or index_k (none). The
// float32 images of the normed and roped values replace the lane's own 64
// accumulators in its LDS tile row (a rotation pair (i, i + 32) lies inside
// one lane's half, and no other lane reads them), and the quantizer reads
// them back: the 64 values are never live in registers at once.
__device__ __forceinline__ void nv_k_half(const TileRow& x, const uint16_t* gam, const EpiIn& in, double rr, int c0,
                                          int dbase, bool has_gs, float gs, uint8_t* slot, int t, int half) {
  float* rowp = const_cast<float*>(x.row);
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    float f1[4], f2[4];
    k_pair_f32(x, gam, in.c, in.sn, rr, c0, dbase, i, f1, f2);
    *reinterpret_cast<float4*>(rowp + 4 * ((c0 + (i >> 2)) ^ x.r)) = float4{f1[0], f1[1], f1[2], f1[3]};
    *reinterpret_cast<float4*>(rowp + 4 * ((c0 + (i >> 2) + 8) ^ x.r)) = float4{f2[0], f2[1], f2[2], f2[3]};
  }
  nv_half_from_tile(x, c0, gs, has_gs, slot, t, half, false);
}

// The q / index_q head step straight from the accumulators, with no LDS hand-off.
// In the 32x32 MFMA output, lane l holds token l % 32 and, in acc[m][r], dim
// 32 m + 8 (r / 4) + 4 (l / 32) + r % 4: the lane's 64 dims of the token, the
// other 64 in lane l ^ 32. A NeoX RoPE pair (i, i + 32), i < 32, is then
// acc[0][r] and acc[1][r] of one lane. RopeRegs holds the cos / sin values of
// the lane's rotary indices 8 g + 4 (l / 32) + [0, 4), g = 0..3, as bf16 pairs.
struct RopeRegs {
  uint32_t c[8], s[8];
};

__device__ __forceinline__ RopeRegs rope_loads(const KArgs& a, int64_t pos) {
  const int hb = (threadIdx.x & 63) >> 5;
  const uint16_t* row = a.cos_sin + pos * kRotary;
  RopeRegs r;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint2 cv = *reinterpret_cast<const uint2*>(row + 8 * g + 4 * hb);
    const uint2 sv = *reinterpret_cast<const uint2*>(row + 32 + 8 * g + 4 * hb);
    r.c[2 * g] = cv.x, r.c[2 * g + 1] = cv.y;
    r.s[2 * g] = sv.x, r.s[2 * g + 1] = sv.y;
  }
  return r;
}

// bf16 element e of a pair array: word e / 2, half e % 2
__device__ __forceinline__ float bf16_pair_at(const uint32_t* w, int e) {
  return bf16_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
}

// The q / index_q head step of the lane's token, with the pages' float32
// precision (contraction off): the head's sum of squares in float32 (again in
// float64 if it overflows), x / rms * (1 + gamma), the NeoX rotation of dims
// 0..63, bf16 out, and for q heads the FP8 q codes when requested.
// The bf16 rows go out through `stage` (this wave's 8.5 KB of LDS, free after
// the main loop): written there at the accumulator layout (row stride 272
// bytes), read back 16 bytes a lane with 16 lanes a row, so that each global
// store instruction writes four whole 256-byte rows; stored straight from the
// accumulators, a row took sixteen 16-byte pieces.
constexpr int kQStageRow = 272;
__device__ __forceinline__ void q_tile_regs(const KArgs& a, const f32x16 (&acc)[4], const uint16_t* gam, int h,
                                            int tok, const RopeRegs& cs, uint8_t* stage) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, hb = lane >> 5;
  float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) s4[r & 3] = __builtin_fmaf(acc[m][r], acc[m][r], s4[r & 3]);
  float ssf = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  ssf += __shfl_xor(ssf, 32, 64);
  float rf;
  if (__builtin_expect(!(ssf <= 3.4028234663852886e38f), 0)) {
    // the float32 sum of squares overflowed: again in float64 (both lanes of
    // the token take this branch together)
    double sd = 0.0;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) sd += static_cast<double>(acc[m][r]) * acc[m][r];
    sd += __shfl_xor(sd, 32, 64);
    rf = static_cast<float>(1.0 / __builtin_sqrt(sd / static_cast<double>(kHeadDim) + static_cast<double>(a.eps)));
  } else {
    rf = 1.0f / __builtin_sqrtf(ssf / static_cast<float>(kHeadDim) + a.eps);
  }
  const int nkv = a.nkv, k0 = 16 * nkv, iq0 = 18 * nkv;
  const bool live = tok < a.S;
  const bool bf16_rows = h >= k0 || a.q_out != nullptr;  // uniform
  const bool fp8_row = live && h < k0 && a.q_fp8 != nullptr;
  uint8_t* const srow = stage + (lane & 31) * kQStageRow;
  uint8_t* qf = fp8_row ? a.q_fp8 + (static_cast<size_t>(tok) * k0 + h) * kHeadDim : nullptr;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t gw[4][2];  // gamma of dims 32 m + 8 g + 4 hb + [0, 4)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint2 gv = *reinterpret_cast<const uint2*>(gam + 32 * m + 8 * g + 4 * hb);
      gw[m][0] = gv.x, gw[m][1] = gv.y;
    }
    float o[4][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * g + e;
      const float x1 = (acc[0][r] * rf) * (1.0f + bf16_pair_at(gw[0], e));
      const float x2 = (acc[1][r] * rf) * (1.0f + bf16_pair_at(gw[1], e));
      const float c = bf16_pair_at(cs.c + 2 * g, e), sn = bf16_pair_at(cs.s + 2 * g, e);
      o[0][e] = x1 * c - x2 * sn;
      o[1][e] = x2 * c + x1 * sn;
      o[2][e] = (acc[2][r] * rf) * (1.0f + bf16_pair_at(gw[2], e));
      o[3][e] = (acc[3][r] * rf) * (1.0f + bf16_pair_at(gw[3], e));
    }
    if (bf16_rows) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        *reinterpret_cast<uint2*>(srow + 2 * (32 * m + 8 * g + 4 * hb)) =
            make_uint2(pack_bf16x2(o[m][0], o[m][1]), pack_bf16x2(o[m][2], o[m][3]));
    }
    if (fp8_row) {  // E4M3 of the float32 products q * (1 / q_fp8_scale)
      const float inv = a.q_fp8_inv;
      const Fp8Scale unit = fp8_scale(0);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        *reinterpret_cast<uint32_t*>(qf + 32 * m + 8 * g + 4 * hb) =
            e4m3x4_scaled(o[m][0] * inv, o[m][1] * inv, o[m][2] * inv, o[m][3] * inv, unit);
    }
  }
  if (bf16_rows) {  // LDS keeps one wave's accesses in order: no barrier
    const int tok0 = tok - (lane & 31);  // the tile's first token
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = 4 * u + (lane >> 4), c = lane & 15;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * kQStageRow + 16 * c);
      const int t = tok0 + r;
      if (t < a.S) {
        uint16_t* dst = h < k0 ? a.q_out + (static_cast<size_t>(t) * k0 + h) * kHeadDim
                               : a.iq_out + (static_cast<size_t>(t) * nkv + (h - iq0)) * kHeadDim;
        *reinterpret_cast<u32x4*>(dst + 8 * c) = v;
      }
    }
  }
}

// The k, v and index_k head step of the lane's token from the wave's output
// tile in LDS (a lane holds 64 contiguous dims of its token).
__device__ __forceinline__ void tile_epilogue(const KArgs& a, const TileRow& x, const uint16_t* gam, int h, int tok,
                                              int64_t slot, const EpiIn& in) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const bool live = tok < a.S;
  const int nkv = a.nkv;
  const int k0 = 16 * nkv, v0 = 17 * nkv, iq0 = 18 * nkv;
  const int dbase = 64 * half;
  const int c0 = 16 * half;  // the lane's first chunk: dims dbase + 4 (c - c0) ..

  const bool store_cache = live && slot >= 0 && slot < static_cast<int64_t>(a.num_pages) * kPage;
  const int64_t page = slot_page(slot);
  const int t = slot_row(slot);

  if (h >= v0 && h < iq0 && a.kv_nvfp4()) {  // V, NVFP4: slot 2j + 1, swizzled scale bytes
    if (store_cache)
      nv_half_from_tile(x, c0, a.v_gs, true, a.k_cache + (page * 2 * nkv + 2 * (h - v0) + 1) * kNvSlotBytes, t, half,
                        true);
    return;
  }

  if (h >= v0 && h < iq0) {  // V: raw projection, per-token scale (1 when static)
    const int j = h - v0;
    float am = 0.f;
    if (!a.static_kv()) {
#pragma unroll 4
      for (int i = 0; i < 64; i += 4) {
        const float4 v = x.chunk(c0 + (i >> 2));
        am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)),
                                                 __builtin_fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w))));
      }
    }
    double amax = static_cast<double>(am);  // a maximum of magnitudes is exact in f32
    amax = __builtin_fmax(amax, __shfl_xor(amax, 32, 64));
    const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
    if (store_cache) {
      const double sd = static_cast<double>(s), rcp = 1.0 / sd;
      uint8_t* vc = a.v_cache + (page * nkv + j) * kPageBytes + t + dbase * kPage;
      const Fp8Scale unit = fp8_scale(0);
#pragma nounroll
      for (int i = 0; i < 64; i += 4) {
        const float4 v = x.chunk(c0 + (i >> 2));
        const uint32_t w = e4m3x4_scaled(div_rn(v.x, sd, rcp), div_rn(v.y, sd, rcp), div_rn(v.z, sd, rcp),
                                         div_rn(v.w, sd, rcp), unit);
#pragma unroll
        for (int e = 0; e < 4; ++e) vc[(i + e) * kPage] = static_cast<uint8_t>(w >> (8 * e));
      }
      if (lane < 32) a.v_scale[(page * nkv + j) * kPage + t] = s;
    }
    return;
  }

  // K and index_k: the head norm in f64, so the FP8 decisions match the exact
  // statement of the method
  double ssm[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
  for (int i = 0; i < 64; i += 4) {
    const float4 v = x.chunk(c0 + (i >> 2));
    ssm[0] += static_cast<double>(v.x) * static_cast<double>(v.x);
    ssm[1] += static_cast<double>(v.y) * static_cast<double>(v.y);
    ssm[2] += static_cast<double>(v.z) * static_cast<double>(v.z);
    ssm[3] += static_cast<double>(v.w) * static_cast<double>(v.w);
  }
  double ss = (ssm[0] + ssm[1]) + (ssm[2] + ssm[3]);
  ss += __shfl_xor(ss, 32, 64);
  double rr = 1.0 / __builtin_sqrt(ss / static_cast<double>(kHeadDim) + static_cast<double>(a.eps));

  // K and index_k share one copy of the f64 group code: pass kAmax finds the K
  // row's scale, pass kCodes writes E4M3 codes (K with its scale into the
  // shuffled page layout, index_k with unit scale into its row).
  if (a.kv_nvfp4()) {  // K into slot 2j, index_k into the page's slot, linear scale bytes
    if (!store_cache) return;
    uint8_t* slot_base =
        h < v0 ? a.k_cache + (page * 2 * nkv + 2 * (h - k0)) * kNvSlotBytes : a.index_cache + page * kNvSlotBytes;
    nv_k_half(x, gam, in, rr, c0, dbase, h < v0, a.k_gs, slot_base, t, half);
    return;
  }

  enum { kAmax, kCodes };
  int mode;
  uint8_t* cbase = nullptr;
  int cstride = 0;  // bytes between 16-dim groups of the code row
  double sd = 1.0, rcp = 1.0;
  if (h < v0 && a.static_kv()) {  // K with the unit scale: codes of the values themselves
    if (!store_cache) return;
    if (lane < 32) a.k_scale[(page * nkv + (h - k0)) * kPage + t] = 1.0f;
    mode = kCodes;
    cbase = a.k_cache + (page * nkv + (h - k0)) * kPageBytes + t * 16 + (dbase >> 4) * 256;
    cstride = 256;
  } else if (h < v0) {
    mode = kAmax;
    cbase = a.k_cache + (page * nkv + (h - k0)) * kPageBytes + t * 16 + (dbase >> 4) * 256;
    cstride = 256;
  } else {
    if (!store_cache) return;
    mode = kCodes;
    cbase = a.index_cache + slot * kHeadDim + dbase;
    cstride = 16;
  }
  auto consume = [&](int i, const double (&v)[4], double& amax) {  // dims dbase + i .. + 3
    if (mode == kAmax) {
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = __builtin_fmax(amax, __builtin_fabs(v[e]));
    } else {
      // index_k and K with the unit scale keep sd = rcp = 1, where div_rn returns v unchanged
      const uint32_t w = e4m3x4_scaled(div_rn(v[0], sd, rcp), div_rn(v[1], sd, rcp), div_rn(v[2], sd, rcp),
                                       div_rn(v[3], sd, rcp), fp8_scale(0));
      *reinterpret_cast<uint32_t*>(cbase + (i >> 4) * cstride + (i & 15)) = w;
    }
  };
  u32x4 c[4], sn[4];  // private copies the passes can mark as changed
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = in.c[j], sn[j] = in.sn[j];
  double amax = 0.0;
#pragma nounroll
  for (;;) {
    // each pass recomputes the values: hoisted out of the loop, all 64 of them
    // would be live in f64 at once
    asm volatile("" : "+v"(rr)::"memory");
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(c[j]), "+v"(sn[j]));
#pragma unroll
    for (int i = 0; i < 32; i += 4) {  // the pair (i, i + 32) of the lane's dims
      const float4 a1 = x.chunk(c0 + (i >> 2));
      const float4 a2 = x.chunk(c0 + (i >> 2) + 8);
      const float f1[4] = {a1.x, a1.y, a1.z, a1.w}, f2[4] = {a2.x, a2.y, a2.z, a2.w};
      const u32x4 ga = *reinterpret_cast<const u32x4*>(gam + dbase + (i & ~7));
      const u32x4 gb = *reinterpret_cast<const u32x4*>(gam + dbase + 32 + (i & ~7));
      double v1[4], v2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = i + e;  // 0..31
        const double x1 = (static_cast<double>(f1[e]) * rr) * (1.0 + bf16_at(ga, d & 7));
        const double x2 = (static_cast<double>(f2[e]) * rr) * (1.0 + bf16_at(gb, d & 7));
        const double cd = bf16_at(c[d >> 3], d & 7), sd2 = bf16_at(sn[d >> 3], d & 7);
        v1[e] = x1 * cd - x2 * sd2;
        v2[e] = x2 * cd + x1 * sd2;
      }
      consume(i, v1, amax);
      consume(i + 32, v2, amax);
    }
    if (mode != kAmax) break;
    amax = __builtin_fmax(amax, __shfl_xor(amax, 32, 64));
    const float s = amax == 0.0 ? 1.0f : static_cast<float>(amax / kFp8Max);
    if (!store_cache) break;
    if (lane < 32) a.k_scale[(page * nkv + (h - k0)) * kPage + t] = s;
    sd = static_cast<double>(s);
    rcp = 1.0 / sd;
    mode = kCodes;
  }
}

// Heads per XCD for the GEMM grid. Blocks b with the same b % 8 run on one XCD
// (workgroups are dispatched round-robin over the eight XCDs), and each XCD
// takes a list of heads across every token tile, so the CTAs running together
// re-read those heads' weight panels and the token tiles' activation panels
// from that XCD's L2. A precise head (bf16 MFMA) costs 1.7 FP8 heads in the
// lists (the span was shortest at that weight among 1.4, 1.7 and 2.2, on c4 and
// c5 alike); the lists balance that cost (longest first, each to the least
// loaded XCD) and put the precise heads first, so the longest CTAs of an XCD
// start earliest.
constexpr int kMaxHeads = 19 * 4 + 1;  // 128-row heads at nkv = 4, the largest nkv accepted

struct HeadMap {
  uint8_t head[kMaxHeads];  // the XCDs' lists, one after another
  uint8_t start[9];         // XCD x owns head[start[x] .. start[x + 1])
  uint8_t nprecise[8];      // its first nprecise[x] heads are precise heads
};

// One CTA = one head x (4 * NTW) 32-token tiles. An XCD first runs every tile
// of its precise heads (the longest CTAs start first, so they do not form the
// kernel's tail), then those of its FP8 heads; within each part the heads vary
// fastest, so CTAs dispatched together share token tiles. The mapping is a
// bijection onto the tiles whatever the hardware's placement.
template <int NTW>
__global__ __launch_bounds__(256, 2) void prefill_gemm(KArgs a, const uint8_t* __restrict__ xq,
                                                      const uint8_t* __restrict__ xs, int mtiles, HeadMap map) {
  // the weight ring; afterwards slot w holds wave w's output tile
  __shared__ __align__(16) uint8_t ring0[kSlotBytes];
  __shared__ __align__(16) uint8_t ring1[kSlotBytes];
  __shared__ __align__(16) uint8_t ring2[kSlotBytes];
  __shared__ __align__(16) uint8_t ring3[kSlotBytes];
  __shared__ __align__(16) uint16_t gam_lds[kHeadDim];  // the head's gamma row
  uint8_t* const ring[kSlots] = {ring0, ring1, ring2, ring3};
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: bases stay scalar
  const int b = blockIdx.x;
  const int xcd = b & 7, idx = b >> 3;
  const int hx0 = map.start[xcd];
  const int hxn = map.start[xcd + 1] - hx0;
  if (idx >= hxn * mtiles) return;  // blocks beyond this XCD's share
  const int np = map.nprecise[xcd];
  int h, mt;
  if (idx < np * mtiles) {
    h = map.head[hx0 + idx % np];
    mt = idx / np;
  } else {
    const int j = idx - np * mtiles, nf = hxn - np;
    h = map.head[hx0 + np + j % nf];
    mt = j / nf;
  }
  const int tt0 = (mt * 4 + wave) * NTW;  // this wave's first 32-token tile
  stamp(a.timeline, a.timeline_slots, b, 0);
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < kHeadDim / 8)  // read before the epilogue: the main loop's barriers order it
    reinterpret_cast<u32x4*>(gam_lds)[threadIdx.x] = reinterpret_cast<const u32x4*>(head_gamma(a, h))[threadIdx.x];
  // the tokens' slots and clamped positions, fetched now for the epilogue
  int64_t slot_n[NTW], pos_n[NTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n) {
    const int tok = (tt0 + n) * 32 + (lane & 31);
    const int tk = tok < a.S ? tok : a.S - 1;  // padded rows use clamped metadata
    slot_n[n] = a.slot_mapping[tk];
    const int64_t pos = a.positions[tk];
    pos_n[n] = pos < 0 ? 0 : (pos >= a.max_pos ? a.max_pos - 1 : pos);
  }

  f32x16 acc[NTW][4];
#pragma unroll
  for (int n = 0; n < NTW; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[n][m][r] = 0.f;
  // one-tile FP8 CTAs have the registers for two k steps a stage: twice the
  // lookahead (a bf16 weight step fills a ring slot by itself)
  constexpr int SUB = NTW == 1 ? kSubSingle : 1;
  // The main loop ends with every load landed and every wave past its last LDS
  // read. Lane l holds token l % 32 and dims 32m + 8(r/4) + 4(l/32) + r%4 in
  // acc[n][m][r]: chunk 8m + 2(r/4) + l/32 of row l % 32.
  float* tile = reinterpret_cast<float*>(wave == 0 ? ring0 : wave == 1 ? ring1 : wave == 2 ? ring2 : ring3);
  const int row = lane & 31;
  const TileRow tr{tile + row * kHeadDim, row};
  // one token tile at a time (written out per tile: a loop over n would index
  // the accumulators at run time)
  auto epilogue = [&](const f32x16 (&accn)[4], int n, int64_t slot, int64_t pos) __attribute__((always_inline)) {
    const EpiIn in = epilogue_loads(a, pos);
    // Each wave hands its tile over through its own ring slot (every wave is
    // past its last read of the ring), reading it back in the same instruction
    // stream: LDS keeps one wave's accesses in order, so no CTA barrier (which
    // would also wait for the previous tile's global stores).
    asm volatile("" ::: "memory");
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 8 * m + 2 * q + (lane >> 5);
        *reinterpret_cast<f32x4*>(tile + row * kHeadDim + 4 * (c ^ row)) =
            f32x4{accn[m][4 * q], accn[m][4 * q + 1], accn[m][4 * q + 2], accn[m][4 * q + 3]};
      }
    asm volatile("" ::: "memory");
    if (n == 0) stamp(a.timeline, a.timeline_slots, b, 3);
    tile_epilogue(a, tr, gam_lds, h, (tt0 + n) * 32 + row, slot, in);
  };
  auto epilogue_lds = [&]() __attribute__((always_inline)) {
    epilogue(acc[0], 0, slot_n[0], pos_n[0]);
    stamp(a.timeline, a.timeline_slots, b, 4);
    if constexpr (NTW > 1) epilogue(acc[1], 1, slot_n[1], pos_n[1]);
  };
  static_assert(NTW <= 2, "the epilogue calls cover two token tiles");
  auto pin_stamp = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < NTW; ++n)
#pragma unroll
      for (int m = 0; m < 4; ++m) pin_registers(acc[n][m]);
    stamp(a.timeline, a.timeline_slots, b, 1);
  };
  if (precise_head(h, a.nkv)) {  // k, v and index_k
    mainloop<true, NTW, 1>(a, h, tt0, xq, xs, ring, wave, acc);
    pin_stamp();
    epilogue_lds();
  } else {  // q and index_q
    mainloop<false, NTW, SUB>(a, h, tt0, xq, xs, ring, wave, acc);
    pin_stamp();
    // straight from the accumulators; every tile's cos / sin requested first,
    // so the second tile's wait overlaps the first tile's work
    RopeRegs cs[NTW];
#pragma unroll
    for (int n = 0; n < NTW; ++n) cs[n] = rope_loads(a, pos_n[n]);
    stamp(a.timeline, a.timeline_slots, b, 3);
    uint8_t* const stage = wave == 0 ? ring0 : wave == 1 ? ring1 : wave == 2 ? ring2 : ring3;  // free now
    q_tile_regs(a, acc[0], gam_lds, h, tt0 * 32 + row, cs[0], stage);
    stamp(a.timeline, a.timeline_slots, b, 4);
    if constexpr (NTW > 1) q_tile_regs(a, acc[1], gam_lds, h, (tt0 + 1) * 32 + row, cs[1], stage);
  }
  stamp(a.timeline, a.timeline_slots, b, 2);
  stamp_place(a.timeline, a.timeline_slots, b, 7);
}

// The precise heads' bf16 panels (one thread per 16-byte piece: 8 values).
__global__ void pack_prefill_bf16(const uint8_t* __restrict__ w, const uint8_t* __restrict__ we,
                                  uint8_t* __restrict__ wp, int N, int K) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int nkv = (N / kHeadDim - 1) / 19;
  const size_t per_head = static_cast<size_t>(kHeadDim) * K * 2 / 16;  // pieces of one panel
  if (idx >= per_head * (2 * nkv + 1)) return;
  const int pidx = static_cast<int>(idx / per_head);
  const size_t r = idx % per_head;
  const int ks = static_cast<int>(r / 1024), q = static_cast<int>(r % 1024);
  const int m = q >> 8, j = (q >> 6) & 3, l = q & 63;
  const int h = pidx < 2 * nkv ? 16 * nkv + pidx : 19 * nkv;
  const int row = h * kHeadDim + 32 * m + (l & 31);
  const int k = ks * kKStep + 32 * (j >> 1) + 16 * (l >> 5) + 8 * (j & 1);
  const uint2 codes = *reinterpret_cast<const uint2*>(w + static_cast<size_t>(row) * K + k);
  const uint32_t e = we[static_cast<size_t>(row) * (K / 32) + k / 32];
  *reinterpret_cast<bf16x8*>(wp + precise_panel_offset(N, K, pidx) + static_cast<size_t>(ks) * kBf16StepBytes +
                             m * 4096 + j * 1024 + l * 16) = fp8x8_to_bf16(codes.x, codes.y, e8m0_to_f32(e));
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

// The precondition of the exact widening on the k, v and index_k heads: every
// weight value code * 2^(e - 127) is a normal bf16 number, i.e. the block's
// E8M0 code e lies in [kPreciseMinE8m0, kPreciseMaxE8m0] (the smallest nonzero
// code is 2^-9, the largest 448 < 2^9). One word per device records a code
// outside that range for the check at pack time.
constexpr int kPreciseMinE8m0 = 10;
constexpr int kPreciseMaxE8m0 = 246;
__device__ uint32_t g_precise_range_bad;

__global__ void clear_range_flag() { g_precise_range_bad = 0u; }

// One thread per dword of the precise rows' E8M0 codes (rows of the k and v
// heads, then the index_k head's).
__global__ void check_precise_e8m0(const uint8_t* __restrict__ we, int N, int K, int nkv) {
  const size_t per_row = static_cast<size_t>(K) / 32;  // codes per row, a multiple of 4
  const size_t kv_rows = static_cast<size_t>(2 * nkv) * kHeadDim;
  const size_t words = (kv_rows + kHeadDim) * per_row / 4;
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= words) return;
  const size_t r = i * 4 / per_row;  // among the precise rows
  const size_t row = r < kv_rows ? static_cast<size_t>(16 * nkv) * kHeadDim + r
                                 : static_cast<size_t>(19 * nkv) * kHeadDim + (r - kv_rows);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(we + row * per_row + (i * 4 - r * per_row));
  bool bad = false;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int c = static_cast<int>((w >> (8 * b)) & 0xffu);
    bad |= c < kPreciseMinE8m0 || c > kPreciseMaxE8m0;
  }
  if (bad) atomicOr(&g_precise_range_bad, 1u);
  (void)N;
}

// Norm pass launch: one CTA per resident slot (the CTAs per CU that the
// kernel's registers allow, times the CUs), each walking the rows at the grid
// stride, so the next row's loads overlap the current row's work.
template <bool WIDE>
hipError_t launch_prepass_t(const Args& a, const PrefillPlan& p, int mpad, int cus) {
  const int threads = ((a.K / 16 + 63) / 64) * 64;  // one 16-element chunk a thread
  static std::atomic<int> per_cu_cache[17];         // by waves per CTA
  int per_cu = per_cu_cache[threads >> 6].load(std::memory_order_relaxed);
  if (per_cu == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prefill_prepass<WIDE>, threads, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    per_cu_cache[threads >> 6].store(per_cu, std::memory_order_relaxed);
  }
  const int grid = std::max(64, std::min(mpad, per_cu * cus) / 64 * 64);  // mpad is a multiple of 256
  hipLaunchKernelGGL(prefill_prepass<WIDE>, dim3(grid), dim3(threads), 0, a.stream, a.ar, a.res, a.h_out, a.g_in,
                     a.ws + p.off_xq, a.ws + p.off_xs, a.S, mpad, a.K, a.eps);
  return hipGetLastError();
}

hipError_t launch_prepass(const Args& a, const PrefillPlan& p, int mpad, int cus) {
  return a.K > 8192 ? launch_prepass_t<true>(a, p, mpad, cus) : launch_prepass_t<false>(a, p, mpad, cus);
}

}  // namespace

PrefillPlan prefill_plan(int M, int K, int nkv) {
  (void)nkv;
  PrefillPlan p{};
  const size_t mpad = (static_cast<size_t>(M) + kTokAlign - 1) / kTokAlign * kTokAlign;
  size_t off = kSyncBytes;  // the synchronization words stay untouched
  p.off_xq = off;
  off = align_up(off + mpad * K, 256);
  p.off_xs = off;
  off = align_up(off + mpad * K / 32, 256);
  p.total = off;
  return p;
}

size_t prefill_packed_weight_bytes(int N, int K) {
  const int nkv = (N / kHeadDim - 1) / 19;
  return precise_panel_offset(N, K, 2 * nkv + 1);
}
size_t prefill_packed_scale_bytes(int N, int K) { return static_cast<size_t>(N) * K / 32; }

// Token tiles of 32 per wave: 1 (128-token CTAs) or 2 (256-token CTAs, half
// the LDS and a quarter less L2 traffic per MFMA). A CU finishes about one CTA
// per CTA-time however many it holds at once, so a launch of n CTAs takes
// ceil(n / CUs) CTA-times; the larger tile is taken unless that quantization
// costs it more than its per-flop gain (about 1.3x).
int prefill_token_tiles_per_wave(int M, int heads, int cus) {
  auto eff = [&](int tok) {
    const double n = static_cast<double>(heads) * ((M + tok - 1) / tok) / cus;
    return n / std::ceil(n);
  };
  return eff(256) * 1.3 >= eff(128) ? 2 : 1;
}

HeadMap make_head_map(int nkv) {
  const int H = 19 * nkv + 1;
  auto precise = [&](int h) { return (h >= 16 * nkv && h < 18 * nkv) || h == 19 * nkv; };
  int load[8] = {0}, count[8] = {0};  // in tenths of an FP8 head
  int owner[kMaxHeads];
  for (int pass = 0; pass < 2; ++pass)  // precise heads (cost 17) first, then FP8 heads (cost 10)
    for (int h = 0; h < H; ++h) {
      if (precise(h) != (pass == 0)) continue;
      int best = 0;
      for (int x = 1; x < 8; ++x)
        if (load[x] < load[best] || (load[x] == load[best] && count[x] < count[best])) best = x;
      owner[h] = best;
      load[best] += precise(h) ? 17 : 10;
      ++count[best];
    }
  HeadMap m{};
  int k = 0;
  for (int x = 0; x < 8; ++x) {
    m.start[x] = static_cast<uint8_t>(k);
    for (int pass = 0; pass < 2; ++pass)
      for (int h = 0; h < H; ++h)
        if (owner[h] == x && precise(h) == (pass == 0)) {
          m.head[k++] = static_cast<uint8_t>(h);
          if (pass == 0) ++m.nprecise[x];
        }
  }
  m.start[8] = static_cast<uint8_t>(k);
  return m;
}

hipError_t launch_prefill(const Args& a, const PrefillPlan& p) {
  const int mpad = (a.S + kTokAlign - 1) / kTokAlign * kTokAlign;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  hipError_t e = launch_prepass(a, p, mpad, cus);
  if (e != hipSuccess) return e;
  const int ntw = prefill_token_tiles_per_wave(a.S, a.heads(), cus);
  const int mtiles = (a.S + 128 * ntw - 1) / (128 * ntw);
  const HeadMap map = make_head_map(a.nkv);
  int most = 0;  // heads of the largest XCD list
  for (int x = 0; x < 8; ++x) most = map.start[x + 1] - map.start[x] > most ? map.start[x + 1] - map.start[x] : most;
  const int per_xcd = most * mtiles;
  if ((e = mark(a.ev_start, a.stream)) != hipSuccess) return e;
  if (ntw == 2)
    hipLaunchKernelGGL(prefill_gemm<2>, dim3(8 * per_xcd), dim3(256), 0, a.stream, a, a.ws + p.off_xq,
                       a.ws + p.off_xs, mtiles, map);
  else
    hipLaunchKernelGGL(prefill_gemm<1>, dim3(8 * per_xcd), dim3(256), 0, a.stream, a, a.ws + p.off_xq,
                       a.ws + p.off_xs, mtiles, map);
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
  const int nkv = (N / kHeadDim - 1) / 19;
  const size_t bf_pieces = static_cast<size_t>(2 * nkv + 1) * kHeadDim * K * 2 / 16;
  hipLaunchKernelGGL(pack_prefill_bf16, dim3(static_cast<unsigned>((bf_pieces + 255) / 256)), dim3(256), 0, s, w, we,
                     wp, N, K);
  return hipGetLastError();
}

hipError_t prefill_weight_range_ok(const uint8_t* we, int N, int K, hipStream_t s, bool& ok) {
  static std::mutex mu;  // one device word per device, shared by the calling threads
  std::lock_guard<std::mutex> lock(mu);
  const int nkv = (N / kHeadDim - 1) / 19;
  const size_t words = static_cast<size_t>(2 * nkv + 1) * kHeadDim * (K / 32) / 4;
  hipLaunchKernelGGL(clear_range_flag, dim3(1), dim3(1), 0, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(check_precise_e8m0, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0, s, we, N,
                     K, nkv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  uint32_t bad = 0;
  if ((e = hipMemcpyFromSymbolAsync(&bad, HIP_SYMBOL(g_precise_range_bad), sizeof(bad), 0, hipMemcpyDeviceToHost,
                                    s)) != hipSuccess)
    return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  ok = bad == 0u;
  return hipSuccess;
}

}  // namespace pa
