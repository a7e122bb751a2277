/*
 * pre_attn.h — C ABI of the MiniMax-M3 fused pre-attention prologue for one
 * layer on one GPU (AMD Instinct MI355X, gfx950).
 *
 * What one call computes, per token (row) of the batch. Sources are the vLLM
 * API pages "vllm.models.minimax_m3.amd.mono.kernels.pre_attn" (K1 mono_pre:
 * module docstring, emit_pre_attn with norm_quant, the GEMV tasks and the head
 * tasks, head_norm_rope, page16_of) and
 * "vllm.models.minimax_m3.nvidia.ops.qkv_index_fused_epilogue" (module and class
 * docstrings, _rms_norm, _rope64, the per-role epilogue branches and the
 * argument rules of minimax_m3_qkv_index_fused_epilogue):
 *
 *   acc   = f32(ar) + f32(res)                      h_out = bf16(acc)
 *   xn    = acc / sqrt(mean(acc^2) + eps) * (1 + g_in)          (Gemma RMSNorm)
 *   decode : per-token FP8   s_x = max|xn| / 448 (1 if 0), x8 = E4M3(xn / s_x)
 *            y[n] = (x8 . w8[n]) * s_x * w_scale[n]
 *   prefill: MXFP8           per 32-wide k block, scale 2^(floor(log2 amax) - 8)
 *            y[n] = sum_k xq_k 2^(ex-127) * wq_k 2^(ew-127)
 *   y is split into 128-wide heads  q x 16nkv | k x nkv | v x nkv | iq x nkv | ik
 *   (N = (19 nkv + 1) * 128 rows); it is never written to memory.
 *   q, k, iq, ik heads: Gemma RMSNorm over the head with g_q / g_k / g_iq / g_ik,
 *            then NeoX RoPE on dims 0..63 (dim i pairs with i + 32),
 *            cos = cos_sin[pos][0..31], sin = cos_sin[pos][32..63].
 *   q_out, iq_out = bf16 of the result.
 *   K  (normed + roped) and V (raw y) per KV head j: scale s = max|.| / 448
 *            (1 if 0), codes E4M3(. / s), into the page-16 caches at the
 *            token's slot; index_k (normed + roped) as E4M3 with unit scale.
 *   E4M3 is OCP E4M3FN, round to nearest even, saturating at +-448.
 *
 * Memory layouts (all device memory, row-major, owned by the caller):
 *   ar, res, h_out   bf16 [tokens][hidden]
 *   g_in             bf16 [hidden];   g_q, g_k, g_iq, g_ik  bf16 [128]
 *   cos_sin          bf16 [max_pos][64]   (cos | sin)
 *   positions        int64 [tokens], each in [0, max_pos)
 *   slot_mapping     int64 [tokens]; slot < 0: the token writes no cache byte;
 *                    otherwise page = slot / 16, row t = slot % 16 and
 *                    slot < num_pages * 16; slots of one call are distinct
 *   k_cache, v_cache uint8 [num_pages][nkv][2048]
 *       K byte of dim d: (d / 16) * 256 + t * 16 + d % 16   ("shuffle" layout)
 *       V byte of dim d: d * 16 + t                          (dim-major)
 *   k_scale, v_scale float [num_pages][nkv][16], entry t
 *   index_cache      uint8 [num_pages * 16][128], row = slot
 *   q_out            bf16 [tokens][16 nkv][128]
 *   iq_out           bf16 [tokens][nkv][128]
 *
 * Conventions for every entry point:
 *   - All data pointers are device pointers. ar, res, h_out, the five norm
 *     weights, cos_sin, the packed weights, q_out, iq_out, the caches and the
 *     workspace must be 16-byte aligned; positions and slot_mapping 8-byte
 *     aligned; the float scale arrays 4-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *     work on it: they never synchronize the host and never allocate memory.
 *   - The library never frees or keeps caller memory. Outputs h_out, q_out
 *     and iq_out are written in full; cache bytes and scales only at the
 *     slots of tokens with slot >= 0; nothing else is written.
 *   - Return 0 (PA_OK) on success, a negative pa_status otherwise. Argument
 *     errors are detected before anything is enqueued. Device preconditions
 *     (positions in range, slots in range and distinct) are the caller's; an
 *     out-of-range position or slot is clamped or skipped, never dereferenced
 *     out of bounds.
 *   - Calls on different streams with distinct workspaces are independent.
 *     Two calls that share a workspace must be ordered (same stream).
 */
#ifndef PRE_ATTN_H
#define PRE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_HEAD_DIM 128
#define PA_ROTARY_DIM 64
#define PA_PAGE 16
#define PA_PAGE_BYTES 2048
#define PA_MAX_HIDDEN 16384
#define PA_DECODE_MAX_TOKENS 64

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,      /* a required pointer is NULL */
  PA_ERR_ALIGN = -2,     /* a pointer is not aligned as stated above */
  PA_ERR_NKV = -3,       /* nkv is not 1, 2 or 4 */
  PA_ERR_HIDDEN = -4,    /* hidden is not a multiple of 128 in [128, 16384] */
  PA_ERR_TOKENS = -5,    /* tokens < 1, or > 64 for decode, or > 2^24 */
  PA_ERR_WORKSPACE = -6, /* workspace smaller than pa_workspace_bytes() */
  PA_ERR_DIMS = -7,      /* num_pages < 1, max_pos < 1 or eps not finite >= 0 */
  PA_ERR_HIP = -8,       /* a HIP runtime call or launch failed */
  PA_ERR_DEVICE = -9,    /* the current device is not a gfx950 GPU */
  PA_ERR_MODE = -10,     /* unknown mode argument */
  PA_ERR_SYNC = -11,     /* a kernel's bounded wait for another CTA gave up */
  PA_ERR_OPTIONS = -12,  /* pa_head_options: a scale not finite and > 0 (or its float32
                            reciprocal not finite), an unknown kv_cache_format, or
                            static_kv_scale together with NVFP4 */
  PA_ERR_WEIGHT_RANGE = -13 /* pa_pack_weight_prefill: an E8M0 code of a k, v or index_k
                               row outside [10, 246] */
} pa_status;

/* Problem size of one call. */
typedef struct pa_dims {
  int32_t tokens;    /* rows of ar / res (decode: 1..64, prefill: 1..2^24) */
  int32_t hidden;    /* K, a multiple of 128, at most 16384 */
  int32_t nkv;       /* KV heads on this GPU: 1, 2 or 4 */
  int32_t num_pages; /* pages of k_cache / v_cache (16 slots each) */
  int32_t max_pos;   /* rows of cos_sin */
  float eps;         /* RMSNorm epsilon, used by the input norm and every head norm */
} pa_dims;

#define PA_MODE_DECODE 0
#define PA_MODE_PREFILL 1

/* Bytes of device workspace a call with these dims needs (0 on bad dims or
 * mode). The workspace is caller-owned scratch; it may be reused by any later
 * call, of either mode and any dims, whose requirement it meets, once
 * pa_workspace_init has run on it: the words the kernels synchronize through
 * sit at the same offsets for every call, and each call leaves them cleared. */
size_t pa_workspace_bytes(const pa_dims* dims, int mode);

/* How pre_attn_decode runs a call with these dims on the device, for
 * reporting and tests (the outputs do not depend on it): a set of flags.
 * The projection always has a launch of its own; PA_DECODE_NORM_FUSED puts the
 * input norm into it and PA_DECODE_EPILOGUE_FUSED the head epilogue (per-head
 * norm, RoPE, outputs and cache inserts). Launches per call: 3 minus the
 * flags set. Negative pa_status on bad dims. */
#define PA_DECODE_NORM_FUSED 1
#define PA_DECODE_EPILOGUE_FUSED 2
int pa_decode_structure(const pa_dims* dims);

/* Prepares a freshly allocated workspace of `bytes` bytes for use (clears the
 * library's counters with a fill kernel on `stream`). Needed once per
 * allocation; calls leave it ready for the next call. The first time on each
 * device it also checks where the dispatcher places workgroups (blocks with
 * equal index mod 8 must share an XCD for the decode launches' hand-offs; if
 * they do not, decode runs its stages in separate launches on that device),
 * and for that synchronizes `stream` once. */
int pa_workspace_init(void* workspace, size_t bytes, void* stream);

/* Whether every call on this workspace since pa_workspace_init produced valid
 * outputs: they are valid exactly when this returns PA_OK, so a caller that
 * must be certain checks it after its calls. Decode launches hand values
 * between the CTAs of one XCD through its L2 (workgroups go to the XCDs
 * round-robin, so blocks with equal index mod 8 share one; pa_workspace_init
 * checks that once per device). No CTA waits for one that has not started,
 * every wait is bounded, and a GEMV CTA whose wait for the token statistics
 * gives up computes them itself. A call marks the workspace when a wait for
 * the k slices' partial sums gave up (a started CTA never arrived); that
 * call's outputs are not valid. Returns PA_OK, or PA_ERR_SYNC once marked
 * (until the next pa_workspace_init). Unlike the other entry points this one
 * synchronizes: it waits for `stream` to finish, then reads one word of the
 * workspace. */
int pa_workspace_status(const void* workspace, void* stream);

/* Bytes of the packed weight (and packed block scales) for N rows x hidden. */
size_t pa_packed_weight_bytes(int mode, int32_t n_rows, int32_t hidden);
size_t pa_packed_scale_bytes(int mode, int32_t n_rows, int32_t hidden);

/* Decode weight: the fused projection's per-output-channel FP8 weight (the
 * pre_attn page's "preshuffled ptpc-FP8 weight", prepared once at load time).
 *   w         E4M3 codes [n_rows][hidden], row-major, head order as above
 *   w_packed  output, pa_packed_weight_bytes(PA_MODE_DECODE, ...) bytes
 * n_rows must be (19 nkv + 1) * 128 for nkv in {1, 2, 4}. */
int pa_pack_weight_decode(const uint8_t* w, uint8_t* w_packed, int32_t n_rows,
                          int32_t hidden, void* stream);

/* Prefill weight: MXFP8 codes plus one E8M0 scale per 32-wide k block (the
 * epilogue page's K-major MXFP8 weight and its scales), repacked for the
 * library's MFMA tiles.
 *   w         E4M3 codes [n_rows][hidden]
 *   w_e8m0    E8M0 codes [n_rows][hidden / 32]
 *   w_packed  output, pa_packed_weight_bytes(PA_MODE_PREFILL, ...) bytes
 *   s_packed  output, pa_packed_scale_bytes(PA_MODE_PREFILL, ...) bytes
 * The k, v and index_k heads (whose per-token FP8 scales and codes must follow
 * the exact projection to 1e-6) are computed on bf16 MFMAs from the MXFP8
 * values widened exactly to bf16 (the packed weight carries a bf16 copy of
 * those 2 nkv + 1 heads' rows), which holds while every weight value
 * code * 2^(e - 127) is a normal bf16 number: each E8M0 code e of those rows
 * must lie in [10, 246]. This call checks that and returns PA_ERR_WEIGHT_RANGE
 * otherwise (the packed buffers are written either way). Unlike the other
 * packing and prologue calls it synchronizes `stream` (a load-time call).
 * Precision notes for pre_attn_prefill: the projection accumulates in
 * float32, so its partial sums must stay below 2^127 in magnitude; an
 * activation 32-block whose largest normalized magnitude is below 2^-109
 * (but not zero) widens to bf16 subnormals, where the k, v and index_k
 * products are no longer exact. */
int pa_pack_weight_prefill(const uint8_t* w, const uint8_t* w_e8m0, uint8_t* w_packed,
                           uint8_t* s_packed, int32_t n_rows, int32_t hidden,
                           void* stream);

/* Decode prologue (per-token FP8 activations, per-row FP8 weight scales).
 *   w_packed  from pa_pack_weight_decode;  w_scale  float [N] per output row.
 * tokens <= PA_DECODE_MAX_TOKENS. */
int pre_attn_decode(const pa_dims* dims, const uint16_t* ar, const uint16_t* res,
                    uint16_t* h_out, const uint16_t* g_in, const uint8_t* w_packed,
                    const float* w_scale, const uint16_t* g_q, const uint16_t* g_k,
                    const uint16_t* g_iq, const uint16_t* g_ik, const uint16_t* cos_sin,
                    const int64_t* positions, const int64_t* slot_mapping,
                    uint8_t* k_cache, uint8_t* v_cache, float* k_scale, float* v_scale,
                    uint8_t* index_cache, uint16_t* q_out, uint16_t* iq_out,
                    void* workspace, size_t workspace_bytes, void* stream);

/* pre_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Its workspace is a library-owned array of
 * 24 MiB per GPU (PA_NOALLOC_SCRATCH_BYTES), held until the process ends and
 * cleared by a fill kernel on `stream` at the first call on each GPU; the call
 * itself allocates nothing. A call whose pa_workspace_bytes(dims,
 * PA_MODE_DECODE) exceeds that size returns PA_ERR_WORKSPACE (hidden 6144 at
 * nkv <= 2 fits up to 64 tokens; at nkv = 4 up to 48). Every call on one GPU
 * shares the array, and each call leaves its synchronization words cleared
 * for the next: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller. Other arguments and
 * results as pre_attn_decode. */
#define PA_NOALLOC_SCRATCH_BYTES (24u << 20)
int pre_attn_decode_noalloc(const pa_dims* dims, const uint16_t* ar, const uint16_t* res,
                            uint16_t* h_out, const uint16_t* g_in, const uint8_t* w_packed,
                            const float* w_scale, const uint16_t* g_q, const uint16_t* g_k,
                            const uint16_t* g_iq, const uint16_t* g_ik, const uint16_t* cos_sin,
                            const int64_t* positions, const int64_t* slot_mapping,
                            uint8_t* k_cache, uint8_t* v_cache, float* k_scale, float* v_scale,
                            uint8_t* index_cache, uint16_t* q_out, uint16_t* iq_out, void* stream);

/* Prefill prologue (MXFP8 activations and weight).
 *   w_packed, s_packed  from pa_pack_weight_prefill. */
int pre_attn_prefill(const pa_dims* dims, const uint16_t* ar, const uint16_t* res,
                     uint16_t* h_out, const uint16_t* g_in, const uint8_t* w_packed,
                     const uint8_t* s_packed, const uint16_t* g_q, const uint16_t* g_k,
                     const uint16_t* g_iq, const uint16_t* g_ik, const uint16_t* cos_sin,
                     const int64_t* positions, const int64_t* slot_mapping,
                     uint8_t* k_cache, uint8_t* v_cache, float* k_scale, float* v_scale,
                     uint8_t* index_cache, uint16_t* q_out, uint16_t* iq_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Variants of the head step, for pre_attn_decode_ex / pre_attn_prefill_ex.
 * A NULL options pointer, or all fields zero, gives the plain calls' results.
 *
 * static_kv_scale  nonzero: K and V take the unit scale instead of the
 *     per-token max / 448: their codes are E4M3 (saturating) of the values
 *     themselves, and every k_scale / v_scale entry the call writes is 1.0.
 *     Source: the pre_attn page's STATIC_KV_SCALE config, read in the K and V
 *     branches of the head tasks of emit_pre_attn.
 * q_fp8_out        NULL, or an extra q output: uint8 E4M3 codes
 *     [tokens][16 nkv][128] (16-byte aligned, caller-owned, written in full):
 *     code = E4M3(float32(q) * float32(1 / q_fp8_scale)), one float32
 *     rounding of the product, saturating at +-448, where q is the normed and
 *     roped head before its bf16 rounding. Source: the epilogue page's
 *     q_fp8_out / q_fp8_scale (the q branch of the per-role epilogue and the
 *     argument list of minimax_m3_qkv_index_fused_epilogue).
 * q_fp8_scale      the dequantization scale of q_fp8_out; with q_fp8_out set it
 *     must be finite and > 0 with a finite float32 reciprocal (else
 *     PA_ERR_OPTIONS). Ignored when q_fp8_out is NULL. */
/* kv_cache_format  PA_KV_FP8 (0): the caches of the plain calls.
 *     PA_KV_NVFP4 (1): the epilogue page's NVFP4 caches (its _nvfp4_quant32
 *     quantizer and _nvfp4_cache_views layout, the k / v / index_k branches of
 *     the per-role epilogue). Per 16-value group of a row (as float32):
 *       sf = E4M3(max(amax * f32(1/6) * gs, 2^-9)), saturating;
 *       element codes E2M1(RZ(v * f32(f32(1 / sf) * gs))), nearest even,
 *       saturating at +-6; a zero magnitude is stored as +0;
 *     gs = f32(1 / k_global_scale) for K (normed + roped), f32(1 / v_global_scale)
 *     for V (raw), none for index_k (normed + roped).
 *     Layouts (uint8, 16-byte aligned, caller-owned):
 *       k_cache      the K/V cache [num_pages][2 nkv][1152]: slot 2j holds
 *                    K of KV head j, slot 2j + 1 its V;
 *       index_cache  [num_pages][1152], one slot per page;
 *     a 1152-byte slot holds the 16 tokens' data, 64 bytes each (byte b of
 *     token t at 64 t + b: element 2b in the low nibble, 2b + 1 in the high),
 *     then their scale bytes from offset 1024: K and index_k linear (token t,
 *     group g at 1024 + 8 t + g); V swizzled, at 1024 + (t / 4 * 4 + g / 2) * 8
 *     + (g % 2) * 4 + t % 4. v_cache, k_scale and v_scale are unused (NULL is
 *     allowed). static_kv_scale must be 0.
 * k_global_scale, v_global_scale  NVFP4 only: the dequantization (global)
 *     scales of the K and V entries, finite and > 0 with finite float32
 *     reciprocals. */
#define PA_KV_FP8 0
#define PA_KV_NVFP4 1
typedef struct pa_head_options {
  int32_t static_kv_scale;
  float q_fp8_scale;
  uint8_t* q_fp8_out;
  int32_t kv_cache_format;
  float k_global_scale;
  float v_global_scale;
} pa_head_options;

/* pre_attn_decode with head-step options. Same arguments and results, except:
 * with opts->q_fp8_out set, q_out may be NULL (then only the FP8 q is
 * written; the epilogue page requires at least one of the two q outputs),
 * and K / V follow opts->static_kv_scale. */
int pre_attn_decode_ex(const pa_dims* dims, const pa_head_options* opts, const uint16_t* ar,
                       const uint16_t* res, uint16_t* h_out, const uint16_t* g_in,
                       const uint8_t* w_packed, const float* w_scale, const uint16_t* g_q,
                       const uint16_t* g_k, const uint16_t* g_iq, const uint16_t* g_ik,
                       const uint16_t* cos_sin, const int64_t* positions,
                       const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                       float* k_scale, float* v_scale, uint8_t* index_cache, uint16_t* q_out,
                       uint16_t* iq_out, void* workspace, size_t workspace_bytes, void* stream);

/* pre_attn_prefill with head-step options, as pre_attn_decode_ex. */
int pre_attn_prefill_ex(const pa_dims* dims, const pa_head_options* opts, const uint16_t* ar,
                        const uint16_t* res, uint16_t* h_out, const uint16_t* g_in,
                        const uint8_t* w_packed, const uint8_t* s_packed, const uint16_t* g_q,
                        const uint16_t* g_k, const uint16_t* g_iq, const uint16_t* g_ik,
                        const uint16_t* cos_sin, const int64_t* positions,
                        const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                        float* k_scale, float* v_scale, uint8_t* index_cache, uint16_t* q_out,
                        uint16_t* iq_out, void* workspace, size_t workspace_bytes, void* stream);

/* ---- The DSpark drafter's attention ------------------------------------------
 * Source: the vLLM API page "vllm.models.minimax_m3.amd.mono.drafter.attention"
 * (module docstring; window; kv_load; block_math; block_acc; qkv_rows;
 * merge_task; store_partial). Per request r (query rows 7 r .. 7 r + 6, one KV
 * head shared by 16 q heads of 128 dims):
 *   - each q head of a row and the row's new k: Gemma RMSNorm over the head
 *     (qn / kn, eps), NeoX RoPE on dims 0..63 (cos_sin row of the row's
 *     position), E4M3 with unit scale (nearest even, saturating); the new v:
 *     E4M3. The new k and v codes are written to the cache at the row's slot.
 *   - the window: p0 = the first row's position, lo = max(p0 - 4095, 0),
 *     hi = min(seq_len - 1, (lo / 128 + 34) * 128 - 1); key kp is visible to a
 *     row at position qp iff kp > qp - 4096 and lo <= kp <= hi (no causal mask
 *     among the 7 rows).
 *   - the blocks lo / 128 .. hi / 128 are cut into partitions of `split`
 *     blocks; per partition and (row, head) an online softmax block by block:
 *     s = q8 . k8 (decoded codes), m' = max(m, block max), alpha =
 *     2^((m - m') C), p = 2^(s C - (m' C - 8)) with C = log2(e) / sqrt(128),
 *     l = l alpha + sum p, o = o alpha + sum E4M3(p) v8 (P in e4m3).
 *   - the partitions are merged in order (weights 2^((m_i - M) C)); o / l is
 *     rounded to bf16 and quantized to MXFP8 (OCP MX: E8M0 scale
 *     2^(floor(log2 amax) - 8) per 32 values, E4M3 codes, saturating). A head
 *     that sees no key outputs zeros.
 * The result depends on `split` (P is rounded relative to each partition's
 * running maximum). The FP8 products are summed exactly widened to bf16 on
 * bf16 MFMAs with float32 accumulation.
 * Layouts (device memory, caller-owned):
 *   q            bf16 [7 R][16][128];  k, v  bf16 [7 R][128]   (new rows)
 *   qn, kn       bf16 [128];  cos_sin  bf16 [max_pos][64] (cos | sin)
 *   positions    int64 [7 R];  slots  int64 [7 R] (cache slot of the row's new
 *                key: block slot / 128, key slot % 128; < 0 or past the cache:
 *                not written)
 *   kv_cache     uint8 [num_blocks][128][256]: key entry = 128 K codes then
 *                128 V codes
 *   block_table  int32 [R][table_width] (physical block of each logical block;
 *                out-of-range entries are clamped, never dereferenced)
 *   seq_lens     int32 [R] (keys 0 .. seq_len - 1 exist, the new rows included)
 *   out_codes    uint8 [7 R][16 * 128] E4M3;  out_scales uint8 [7 R][64] E8M0
 *   out_bf16     bf16 [7 R][16][128], optional (NULL: not written)
 * Alignment: kv_cache, out_bf16 and the workspace 16 bytes; out_codes 8;
 * positions and slots 8; block_table and seq_lens 4; the bf16 inputs 2.
 * Three launches on `stream`; no allocation, no synchronization. Errors as the
 * prologue's (PA_ERR_DIMS for a bad field of the dims). */
#define PA_DRAFTER_ROWS 7
#define PA_DRAFTER_HEADS 16
#define PA_DRAFTER_BLOCK 128
#define PA_DRAFTER_MAX_SPLIT 34
typedef struct pa_drafter_dims {
  int32_t requests;     /* R, 1 .. 2^20 */
  int32_t num_blocks;   /* blocks of kv_cache, >= 1 */
  int32_t table_width;  /* columns of block_table, >= 1 */
  int32_t max_pos;      /* rows of cos_sin, >= 1 */
  int32_t split;        /* blocks per split-KV partition, 1 .. 34 */
  float eps;            /* the head norms' epsilon */
} pa_drafter_dims;

/* Workspace bytes of a drafter call (0 on bad dims). */
size_t pa_drafter_workspace_bytes(const pa_drafter_dims* dims);

int pa_drafter_attention(const pa_drafter_dims* dims, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const uint16_t* qn, const uint16_t* kn,
                         const uint16_t* cos_sin, const int64_t* positions, const int64_t* slots,
                         uint8_t* kv_cache, const int32_t* block_table, const int32_t* seq_lens,
                         uint8_t* out_codes, uint8_t* out_scales, uint16_t* out_bf16,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Instrumentation: from now on, calls on this host thread record `start` and
 * `stop` (hipEvent_t, created by the caller) on their stream immediately
 * before and after their dominant kernel (decode: the projection GEMV;
 * prefill: the MFMA GEMM with the fused epilogue), so that
 * hipEventElapsedTime gives that kernel's duration (the drafter: its split-KV
 * attention launch). Both NULL turns it off.
 * The events stay owned by the caller. */
int pa_set_kernel_events(void* start, void* stop);

/* Instrumentation: from now on, calls on this host thread have thread 0 of
 * each CTA store the 100 MHz s_memrealtime counter at its phase boundaries
 * into `buffer` (device memory, a record of 8 uint64 slots each). Decode records: token t's input norm at record t (slots 0 = loads
 * issued ... 5 = done; in the one-launch structure, one XCD's copy); the
 * GEMV CTA of head h and k slice ks at S + ks * heads + h (0 = start,
 * 1 = partial sums stored; without the norm in its launch 2 = activation
 * slice in LDS; in the GEMV + epilogue launch 4 = the head's slices all
 * stored, 5 = its epilogue tokens done); the epilogue of token t and head h
 * at S + heads * ksplit + t * heads + h (0 = start, 1 = inputs loaded; only
 * the tokens a CTA's first wave runs).
 * Prefill: the GEMM CTAs' own phases. Drafter: the split-KV CTA of request r
 * and partition p at r * partitions + p (0 = start, then for its first three
 * blocks 1 + 2 i = block i staged in LDS and 2 + 2 i = its math done; 7 =
 * partial stored). Stamps beyond `bytes` are dropped and the outputs do not
 * depend on the stamps. NULL turns it off. */
int pa_set_timeline(void* buffer, size_t bytes);

/* Static text for a pa_status value. */
const char* pa_strerror(int status);

/* Detail of the last PA_ERR_HIP on the calling thread ("" if none). */
const char* pa_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* PRE_ATTN_H */
