// Attention of the DSpark drafter on gfx950: the split-KV partitions with the q
// and k head norms and RoPE in front of them, and the merge that writes MXFP8
// for o_proj (the vLLM API page vllm.models.minimax_m3.amd.mono.drafter.
// attention: module docstring, window, kv_load, block_math, block_acc,
// qkv_rows, merge_task, store_partial).
//
// Three launches on the caller's stream:
//   1. drafter_rows   one CTA per query row: its 16 q heads and its new k get
//                     the head RMSNorm (Gemma form) and NeoX RoPE on dims 0..63
//                     in float64 and are cast to E4M3 (unit scale, saturating);
//                     the new v is cast to E4M3. q codes go to the workspace,
//                     the new k and v codes into the paged cache at the row's
//                     slot.
//   2. drafter_split  one CTA per (request, partition of `split` blocks): the
//                     128-key blocks of the request's window, each staged in
//                     LDS as bf16 (K row-major, V transposed with its keys in
//                     the PV operand's order), then one wave per query row runs
//                     the online softmax for its 16 heads: S^T = K Q^T on
//                     16x16x32 bf16 MFMAs leaves keys 16 i + 4 g .. + 3 of a
//                     head in one lane, which is exactly the PV operand's k
//                     slice, so P never leaves the registers: P = 256
//                     exp((s - m) / sqrt(128)) is rounded to E4M3 and O^T =
//                     V^T P^T accumulates on the same MFMAs. The partial
//                     (m, l, o) goes to the workspace.
//   3. drafter_merge  one CTA per query row: the partitions merged in order,
//                     o / l rounded to bf16 and quantized to MXFP8 (E8M0 per 32
//                     values, OCP MX rule).
//
// The page computes q . k and P V on FP8 MFMAs; those sum their products at a
// reduced internal precision, so here every FP8 operand is widened exactly to
// bf16 and the products are summed in float32 (the same exact products).
#include <hip/hip_runtime.h>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr int kQpr = 7;          // query rows per request
constexpr int kHeads = 16;       // q heads per row
constexpr int kBlock = 128;      // keys per cache block
constexpr int kKeyBytes = 256;   // K codes | V codes
constexpr int kWindow = 4096;
constexpr int kMaxB = 34;        // blocks a request's window may span
constexpr float kQkC = 0.127517430824598679f;  // log2(e) / sqrt(128)
constexpr int kRecInts = 4 + kMaxB;  // a request's window record: lo, hi, b0, b1, physical blocks b0 .. b1

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int64_t clamp_pos(int64_t p, int max_pos) {
  return p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
}

// The request's window (step d2): first / last visible key and block.
struct Window {
  int lo, hi, b0, b1;
};

__device__ __forceinline__ Window request_window(const DArgs& a, int r) {
  const int p0 = static_cast<int>(clamp_pos(a.positions[r * kQpr], 1 << 30));
  const int seq = a.seq_lens[r];
  Window w;
  w.lo = p0 - (kWindow - 1) > 0 ? p0 - (kWindow - 1) : 0;
  const int cap = (w.lo / kBlock + kMaxB) * kBlock - 1;
  w.hi = seq - 1 < cap ? seq - 1 : cap;
  w.b0 = w.lo / kBlock;
  w.b1 = w.hi >= w.lo ? w.hi / kBlock : w.b0 - 1;  // no block when the window is empty
  return w;
}

// Step d1 for one query row: its 18 tasks (16 q heads, k, v) one wave each,
// four to a CTA (blockIdx.y picks the four). Lane l holds dims l and l + 64;
// the RoPE partner of dim l < 64 is dim l ^ 32, i.e. lane l ^ 32.
__global__ __launch_bounds__(256) void drafter_rows(DArgs a) {
#pragma clang fp contract(off)
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int task = static_cast<int>(blockIdx.y) * 4 + wave;
  if (task == kHeads + 2) {
    // the request's window (step d2) and its physical blocks, once per request,
    // for the split-KV launch (one round trip there instead of three dependent
    // ones); blocks and table columns clamped as kv_load does
    if (t % kQpr != 0) return;
    const int r = t / kQpr;
    const Window w = request_window(a, r);
    int32_t* rec = a.blocks + static_cast<size_t>(r) * kRecInts;
    if (lane == 0) rec[0] = w.lo, rec[1] = w.hi, rec[2] = w.b0, rec[3] = w.b1;
    if (lane < kMaxB) {
      const int blk = w.b0 + lane;
      const int col = blk < a.table_width ? blk : a.table_width - 1;
      const int phys = a.block_table[static_cast<size_t>(r) * a.table_width + (col < 0 ? 0 : col)];
      rec[4 + lane] = phys < 0 ? 0 : (phys >= a.num_blocks ? a.num_blocks - 1 : phys);
    }
    return;
  }
  if (task > kHeads + 2) return;
  const int64_t pos = clamp_pos(a.positions[t], a.max_pos);
  const double c = static_cast<double>(bf16_to_f32(a.cos_sin[pos * kRotary + (lane & 31)]));
  const double sn = static_cast<double>(bf16_to_f32(a.cos_sin[pos * kRotary + 32 + (lane & 31)]));
  const int64_t slot = a.slots[t];
  const bool store = slot >= 0 && slot < static_cast<int64_t>(a.num_blocks) * kBlock;
  uint8_t* key = a.kv_cache + (store ? slot : 0) * kKeyBytes;
  {
    if (task == kHeads + 1) {  // v: its E4M3 codes (bf16 values, exact in float64)
      const uint16_t* v = a.v + static_cast<size_t>(t) * kHeadDim;
      const uint32_t c2 = e4m3x2_scaled(bf16_to_f32(v[lane]), bf16_to_f32(v[lane + 64]), fp8_scale(0));
      if (store) {
        key[kHeadDim + lane] = static_cast<uint8_t>(c2);
        key[kHeadDim + lane + 64] = static_cast<uint8_t>(c2 >> 8);
      }
      return;
    }
    const uint16_t* x = task < kHeads ? a.q + (static_cast<size_t>(t) * kHeads + task) * kHeadDim
                                      : a.k + static_cast<size_t>(t) * kHeadDim;
    const uint16_t* g = task < kHeads ? a.qn : a.kn;
    const double y0 = bf16_to_f32(x[lane]), y1 = bf16_to_f32(x[lane + 64]);
    const double ss = wave_sum_f64(y0 * y0 + y1 * y1);
    const double r = 1.0 / __builtin_sqrt(ss / static_cast<double>(kHeadDim) + static_cast<double>(a.eps));
    const double n0 = (y0 * r) * (1.0 + static_cast<double>(bf16_to_f32(g[lane])));
    const double n1 = (y1 * r) * (1.0 + static_cast<double>(bf16_to_f32(g[lane + 64])));
    const double partner = __shfl_xor(n0, 32, 64);
    const double o0 = lane < 32 ? n0 * c - partner * sn : n0 * c + partner * sn;
    const uint32_t c2 = e4m3x2_scaled(o0, n1, fp8_scale(0));
    if (task < kHeads) {
      uint8_t* q8 = a.q8 + (static_cast<size_t>(t) * kHeads + task) * kHeadDim;
      q8[lane] = static_cast<uint8_t>(c2);
      q8[lane + 64] = static_cast<uint8_t>(c2 >> 8);
    } else if (store) {
      key[lane] = static_cast<uint8_t>(c2);
      key[lane + 64] = static_cast<uint8_t>(c2 >> 8);
    }
  }
}

// Key slot o (0..31) of a 32-key group in the V^T tile: the PV operand's lane
// group g takes keys 4g .. 4g + 3 of the group's two 16-key S tiles, so key
// 16 a + 4 g + e sits at 8 g + 4 a + e.
__device__ __forceinline__ int vt_slot(int o) { return ((o >> 2) & 3) * 8 + (o >> 4) * 4 + (o & 3); }

// Step d3 for one partition of one request: 8 waves; wave j < 7 holds query
// row j (its 16 heads: lane l has head l % 16). LDS: K of the block as bf16
// [key][dim] and V^T as bf16 [dim][key slot], 32 KB each, rows of 256 bytes
// whose 16-byte chunks are XOR-swizzled: K by row % 16 (the 16 rows an MFMA
// operand read takes, and the 16 a staging write covers, fall on 16 chunk
// positions); V^T by (d % 16) ^ (d / 16 % 16), which does the same for the
// 16 dims of an operand read (d = 16 n + l) and of a staging write (d = 8 q + e).
__device__ __forceinline__ int swz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }
__device__ __forceinline__ int vt_off(int d, int ks) {  // element offset of V^T row d, key slot ks
  return d * 128 + ((((ks >> 3) ^ ((d & 15) ^ ((d >> 4) & 15))) << 3) | (ks & 7));
}

__global__ __launch_bounds__(512, 4) void drafter_split(DArgs a) {
  __shared__ __align__(16) bf16x8_t k_lds[kBlock * 16];     // 128 rows x 16 chunks of 8 bf16
  __shared__ __align__(16) __bf16 vt_lds[kHeadDim * kBlock];  // 128 rows x 128 bf16
  const int part = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int32_t* rec = a.blocks + static_cast<size_t>(r) * kRecInts;
  const Window w{rec[0], rec[1], rec[2], rec[3]};
  const int bs = w.b0 + part * a.split;
  const int be = bs + a.split - 1 < w.b1 ? bs + a.split - 1 : w.b1;
  const int row = r * kQpr + wave;  // this wave's query row (waves < 7)
  const int tlb = r * a.nsplit + part;  // timeline record
  stamp(a.timeline, a.timeline_slots, tlb, 0);
  const int qp = wave < kQpr ? static_cast<int>(clamp_pos(a.positions[row], 1 << 30)) : 0;

  // Q^T operand: head l16, dims 32 kk + 8 g4 .. + 7, kept as codes and widened
  // exactly for each block (half the registers)
  uint2 qc[4] = {};
  if (wave < kQpr) {
    const uint8_t* q8 = a.q8 + (static_cast<size_t>(row) * kHeads + l16) * kHeadDim + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qc[kk] = *reinterpret_cast<const uint2*>(q8 + 32 * kk);
  }
  float m = -__builtin_inff(), l = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One block's codes in this thread's registers: K bytes 32 (tid % 4) .. + 31
  // of key tid / 4, and V bytes 8 (tid % 16) .. + 7 of keys 4 (tid / 16) .. + 3
  // (the 8 dims the thread transposes; 16 lanes read each key's V line).
  // Clamped metadata keeps every address inside the table row and the cache
  // (kv_load); keys outside [lo, hi] stage as zeros.
  struct Codes {
    u32x4 k0, k1;
    uint2 v[4];
  };
  const int km = tid >> 2, kq = tid & 3, vkg = tid >> 4, vdg = tid & 15;
  // the partition's physical blocks (already clamped), into LDS
  __shared__ int s_phys[kMaxB];
  if (tid < a.split && part * a.split + tid < kMaxB) s_phys[tid] = rec[4 + part * a.split + tid];
  __syncthreads();
  auto load_block = [&](int blk, Codes& c) {
    int ko = km * kKeyBytes + 32 * kq, vo = 4 * vkg * kKeyBytes + kHeadDim + 8 * vdg;
    asm volatile("" : "+v"(ko), "+v"(vo));  // formed here, not held across the loop (registers)
    const uint8_t* base = a.kv_cache + static_cast<size_t>(s_phys[blk - bs]) * kBlock * kKeyBytes;
    c.k0 = *reinterpret_cast<const u32x4*>(base + ko);
    c.k1 = *reinterpret_cast<const u32x4*>(base + ko + 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) c.v[j] = *reinterpret_cast<const uint2*>(base + vo + j * kKeyBytes);
  };
  auto stage_block = [&](int blk, const Codes& c) {
    int sk = km, sv = vdg;  // addresses formed here, not hoisted out of the loop (registers)
    asm volatile("" : "+v"(sk), "+v"(sv));
    const int kp = blk * kBlock + sk;
    const uint32_t z = kp >= w.lo && kp <= w.hi ? ~0u : 0u;
    k_lds[swz(sk, 4 * kq + 0)] = fp8x8_to_bf16(c.k0[0] & z, c.k0[1] & z, 1.0f);
    k_lds[swz(sk, 4 * kq + 1)] = fp8x8_to_bf16(c.k0[2] & z, c.k0[3] & z, 1.0f);
    k_lds[swz(sk, 4 * kq + 2)] = fp8x8_to_bf16(c.k1[0] & z, c.k1[1] & z, 1.0f);
    k_lds[swz(sk, 4 * kq + 3)] = fp8x8_to_bf16(c.k1[2] & z, c.k1[3] & z, 1.0f);
    bf16x8_t vb[4];  // key 4 vkg + j, dims 8 vdg .. + 7
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vp = blk * kBlock + 4 * vkg + j;
      const uint32_t vz = vp >= w.lo && vp <= w.hi ? ~0u : 0u;
      vb[j] = fp8x8_to_bf16(c.v[j].x & vz, c.v[j].y & vz, 1.0f);
    }
    // the four keys take four consecutive key slots of each dim's row
    const int ks = (4 * vkg & ~31) + vt_slot(4 * vkg & 31);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * sv + e;
      const bf16x2 lo2 = {vb[0][e], vb[1][e]}, hi2 = {vb[2][e], vb[3][e]};
      *reinterpret_cast<uint2*>(vt_lds + vt_off(d, ks)) =
          make_uint2(__builtin_bit_cast(uint32_t, lo2), __builtin_bit_cast(uint32_t, hi2));
    }
  };

  Codes cur;
  if (bs <= be) load_block(bs, cur);
  for (int blk = bs; blk <= be; ++blk) {
    __syncthreads();  // the previous block's tiles are no longer read
    stage_block(blk, cur);
    if (blk < be) load_block(blk + 1, cur);  // in flight during this block's math
    __syncthreads();
    if (blk - bs < 3) stamp(a.timeline, a.timeline_slots, tlb, 1 + 2 * (blk - bs));
    if (wave >= kQpr) continue;
    // The operand addresses are formed in the loop from this copy of the lane's
    // head index: hoisted out of it they would hold 64 registers for the whole
    // loop, and two CTAs a CU need the kernel within 128.
    int lh = l16;
    asm volatile("" : "+v"(lh));

    // S^T = K Q^T: s[4 i + e] is key 16 i + 4 g4 + e of the block for head l16;
    // a block whose every key this row sees needs no mask (wave-uniform)
    const int k0 = blk * kBlock;
    const bool full = k0 > qp - kWindow && k0 >= w.lo && k0 + kBlock - 1 <= w.hi;
    float s[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_lds[swz(16 * i + lh, 4 * kk + g4)],
                                                      fp8x8_to_bf16(qc[kk].x, qc[kk].y, 1.0f), acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * i + e] = acc[e];
    }
    if (!full) {  // keys outside [max(lo, qp - 4095), hi] get -inf (selects, no branches)
      int qw = qp - kWindow + 1;
      asm volatile("" : "+v"(qw));
      const int vlo = w.lo > qw ? w.lo : qw;
#pragma unroll
      for (int x = 0; x < 32; ++x) {
        const int kp = k0 + 16 * (x >> 2) + 4 * g4 + (x & 3);
        s[x] = kp >= vlo && kp <= w.hi ? s[x] : -__builtin_inff();
      }
    }
    float mb = s[0];
#pragma unroll
    for (int x = 1; x < 32; ++x) mb = fmaxf(mb, s[x]);
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float mn = fmaxf(m, mb);
    const float ms = mn == -__builtin_inff() ? 0.f : mn;
    const float alpha = __builtin_amdgcn_exp2f((m - ms) * kQkC);
    const float off = ms * kQkC - 8.0f;
    // p = 256 exp((s - m) / sqrt(128)), eight keys at a time: summed (before
    // rounding) and rounded to e4m3 (p <= 256: no saturation) as they come, so
    // no more than eight of them are live. The PV operand of key step t is
    // keys 32 t + 4 g4 + [0, 4) and 32 t + 16 + 4 g4 + [0, 4), i.e. p[8 t .. 8 t + 7].
    float ps = 0.f;
    uint32_t pc[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float p8[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        p8[x] = __builtin_amdgcn_exp2f(s[8 * t + x] * kQkC - off);
        ps += p8[x];
      }
      int lo8 = __builtin_amdgcn_cvt_pk_fp8_f32(p8[0], p8[1], 0, false);
      lo8 = __builtin_amdgcn_cvt_pk_fp8_f32(p8[2], p8[3], lo8, true);
      int hi8 = __builtin_amdgcn_cvt_pk_fp8_f32(p8[4], p8[5], 0, false);
      hi8 = __builtin_amdgcn_cvt_pk_fp8_f32(p8[6], p8[7], hi8, true);
      pc[2 * t] = static_cast<uint32_t>(lo8);
      pc[2 * t + 1] = static_cast<uint32_t>(hi8);
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l = l * alpha + ps;
    m = mn;
    bf16x8_t pb[4];  // widened back exactly
#pragma unroll
    for (int t = 0; t < 4; ++t) pb[t] = fp8x8_to_bf16(pc[2 * t], pc[2 * t + 1], 1.0f);
    // O^T += V^T P^T: o[n][e] is dim 16 n + 4 g4 + e of head l16
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      f32x4 acc = o[n] * alpha;
      const int d = 16 * n + lh;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int ks = 32 * t + 8 * g4;  // 8 key slots
        const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(vt_lds + vt_off(d, ks));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[t], acc, 0, 0, 0);
      }
      o[n] = acc;
    }
    if (blk - bs < 3) stamp(a.timeline, a.timeline_slots, tlb, 2 + 2 * (blk - bs));
  }
  if (wave >= kQpr) return;
  // the partial of (row, partition): m and l per head, o [16][128]
  float* pm = a.part + (static_cast<size_t>(row) * a.nsplit + part) * kHeads * (2 + kHeadDim);
  if (g4 == 0) {
    pm[l16] = m;
    pm[kHeads + l16] = l;
  }
  float* po = pm + 2 * kHeads + l16 * kHeadDim;
#pragma unroll
  for (int n = 0; n < 8; ++n) *reinterpret_cast<f32x4*>(po + 16 * n + 4 * g4) = o[n];
  stamp(a.timeline, a.timeline_slots, tlb, 7);
}

// Step d4: thread (head tid / 16, dims 8 (tid % 16) .. + 7) merges the
// partitions in order; four threads make one 32-value MX block. The partials
// were written by the previous launch, so every load is a trip to the memory
// side: m, l and the o slice of up to 17 partitions are all issued in one
// straight run with clamped indices (no branch between them), and a second run
// takes partitions 17 .. 33 when there are more.
constexpr int kBatch = 17;

__global__ __launch_bounds__(256) void drafter_merge(DArgs a) {
#pragma clang fp contract(off)
  const int row = blockIdx.x, tid = threadIdx.x;
  const int h = tid >> 4, d0 = 8 * (tid & 15);
  const int np = a.nsplit;
  const size_t stride = static_cast<size_t>(kHeads) * (2 + kHeadDim);
  const float* pr = a.part + static_cast<size_t>(row) * np * stride;
  float M = -__builtin_inff(), L = 0.f, O[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < np; g += kBatch) {
    float mv[kBatch], lv[kBatch];
    float4 ov[kBatch][2];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = g + u < np ? g + u : np - 1;
      const float* p = pr + i * stride;
      mv[u] = p[h];
      lv[u] = p[kHeads + h];
      ov[u][0] = *reinterpret_cast<const float4*>(p + 2 * kHeads + h * kHeadDim + d0);
      ov[u][1] = *reinterpret_cast<const float4*>(p + 2 * kHeads + h * kHeadDim + d0 + 4);
    }
    // the running maximum over the partitions so far; the sums carried so far
    // are rescaled to it
    float Mn = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) Mn = fmaxf(Mn, mv[u]);
    const float Ms = Mn == -__builtin_inff() ? 0.f : Mn;
    const float carry = __builtin_amdgcn_exp2f((M - Ms) * kQkC);
    L = L * carry;
#pragma unroll
    for (int e = 0; e < 8; ++e) O[e] = O[e] * carry;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {  // in order
      const float wgt = g + u < np ? __builtin_amdgcn_exp2f((mv[u] - Ms) * kQkC) : 0.f;
      L = L + wgt * lv[u];
      const float o8[8] = {ov[u][0].x, ov[u][0].y, ov[u][0].z, ov[u][0].w,
                           ov[u][1].x, ov[u][1].y, ov[u][1].z, ov[u][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) O[e] = O[e] + wgt * o8[e];
    }
    M = Mn;
  }
  const bool none = M == -__builtin_inff();
  float ob[8];  // the bf16 outputs as float32
  u32x4 hb;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const float x0 = none ? 0.f : O[e] / L, x1 = none ? 0.f : O[e + 1] / L;
    hb[e >> 1] = pack_bf16x2(x0, x1);
    ob[e] = bf16_to_f32(hb[e >> 1] & 0xffffu);
    ob[e + 1] = bf16_to_f32(hb[e >> 1] >> 16);
  }
  const size_t oi = static_cast<size_t>(row) * kHeads * kHeadDim + h * kHeadDim + d0;
  if (a.out_bf16) *reinterpret_cast<u32x4*>(a.out_bf16 + oi) = hb;
  // MX block of dims 32 b .. + 31: threads tid & ~3 .. + 3
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = fmaxf(am, __builtin_fabsf(ob[e]));
  am = fmaxf(am, __shfl_xor(am, 1, 64));
  am = fmaxf(am, __shfl_xor(am, 2, 64));
  int code = static_cast<int>((__float_as_uint(am) >> 23) & 0xffu) - 8;  // floor(log2 amax) - 8 + 127
  code = code < 0 ? 0 : (code > 254 ? 254 : code);
  code = am != 0.f ? code : 127;
  const Fp8Scale f = fp8_scale(code - 127);
  const uint32_t w0 = e4m3x4_scaled(ob[0], ob[1], ob[2], ob[3], f);
  const uint32_t w1 = e4m3x4_scaled(ob[4], ob[5], ob[6], ob[7], f);
  *reinterpret_cast<uint2*>(a.out_codes + oi) = make_uint2(w0, w1);
  if ((tid & 3) == 0) a.out_scales[oi / 32] = static_cast<uint8_t>(code);
}

}  // namespace

DrafterPlan drafter_plan(int requests, int split) {
  DrafterPlan p{};
  p.nsplit = (kMaxB + split - 1) / split;
  const size_t rows = static_cast<size_t>(requests) * kQpr;
  size_t off = kSyncBytes;
  p.off_q8 = off;
  off = align_up(off + rows * kHeads * kHeadDim, 256);
  p.off_part = off;
  off = align_up(off + rows * p.nsplit * kHeads * (2 + kHeadDim) * sizeof(float), 256);
  p.off_blocks = off;
  off = align_up(off + static_cast<size_t>(requests) * kRecInts * sizeof(int32_t), 256);
  p.total = off;
  return p;
}

hipError_t launch_drafter(const DArgs& a0, const DrafterPlan& p) {
  DArgs a = a0;
  a.q8 = a.ws + p.off_q8;
  a.part = reinterpret_cast<float*>(a.ws + p.off_part);
  a.blocks = reinterpret_cast<int32_t*>(a.ws + p.off_blocks);
  a.nsplit = p.nsplit;
  const int rows = a.requests * kQpr;
  hipLaunchKernelGGL(drafter_rows, dim3(rows, (kHeads + 2 + 3) / 4), dim3(256), 0, a.stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = mark(a.ev_start, a.stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(drafter_split, dim3(p.nsplit, a.requests), dim3(512), 0, a.stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(a.ev_stop, a.stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(drafter_merge, dim3(rows), dim3(256), 0, a.stream, a);
  return hipGetLastError();
}

}  // namespace pa
