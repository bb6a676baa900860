/*
 * mla_kv.h -- C ABI of the MI355X (gfx950) MLA latent-KV library.
 *
 * The library computes the data-parallel path around the MLA latent KV cache
 * of a multi-layer draft model:
 *   projection  mla_ctx_kv_proj        Y = X . W  (one KV-only GEMM for all layers)
 *               mla_transpose_bf16     [K, N] weight -> the [N, K] storage the projection reads
 *   epilogue    mla_ctx_kv_epilogue    RMSNorm(kv_c) | RoPE(k_pe) -> fp8/bf16 -> paged caches
 *   insert      mla_kv_insert_grouped  [kv_c | k_pe] -> fp8/bf16 -> paged caches, all layers
 *   gather      mla_ctx_latent_gather  paged cache rows -> contiguous bf16 (or raw fp8) workspace
 *   pack        mla_ctx_kv_pack        [k_nope | k_pe] full key (+ fp8 V), contiguous
 *               mla_ctx_kv_pack_gather the pack of one chunk and the gather of the next, one launch
 *   merge       mla_ctx_merge_chunk    chunk attention partials -> accumulator (log-sum-exp)
 *   new tokens  mla_new_token_epilogue RoPE(q_pe, k_pe) -> query row, full key (+ fp8 V),
 *                                      and the cache insert of [kv_c | RoPE(k_pe)]
 *
 * Pages cited (title and section heading):
 *   [P1] "PR #51772 完整报告" -- [Attention][MLA] Fuse Kimi-K3 chunked-context K/V packing
 *   [P2] "PR #50585 完整报告" -- [K3 Perf] Optimize k3 dspark fused kv
 *   [P3] "PR #55356 完整报告" -- [Kimi Perf] Group fp8 mla cache insertion
 *
 * Conventions for every entry point
 *   - Pointers marked "device" are HIP device pointers the caller owns; the
 *     library never allocates, frees or retains them.  Host pointers are
 *     marked "host".  Buffers must stay alive until the stream work is done.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and is asynchronous; nothing synchronises inside the library.
 *     Kernels run on the calling thread's current HIP device: `stream` and
 *     every device pointer must belong to it (the library reads the
 *     device's compute-unit count, and sets the projection's LDS attribute,
 *     on that device).
 *   - Strides are in ELEMENTS of the array they describe.
 *   - bf16 arrays hold IEEE bfloat16, fp16 arrays IEEE binary16; fp8 arrays
 *     hold OCP e4m3fn codes (bias 7, no infinity, NaN = 0x7F/0xFF, max 448)
 *     -- the torch.float8_e4m3fn format.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error nothing is launched, the status is returned and
 *     mla_last_error() describes it.  Values that live in device memory
 *     (slot numbers, cache base pointers, positions) cannot be checked from
 *     the host: they are preconditions, stated per entry point.
 *   - A call with zero tokens (or zero layers) succeeds without launching.
 *   - fp8 quantisation divides by a dequantisation scale s read from device
 *     memory (kv_scales, k_scale, ...).  The codes equal those of the IEEE
 *     fp32 quotient x / s for every scale with 2^-85 <= |s| < 2^126 (checked
 *     exhaustively on the host by tests/quotient_exactness.c); scales outside
 *     that range, zero and non-finite scales are a precondition violation
 *     (codes may then differ from the quotient's).
 */
#ifndef MLA_KV_H
#define MLA_KV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* mla_stream_t; /* hipStream_t */

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1, /* bad size, null pointer, wrong dtype/scale combination */
  MLA_ERR_UNSUPPORTED = 2,      /* a valid request the library does not implement */
  MLA_ERR_MISALIGNED = 3,       /* a pointer or stride breaks 16-byte row alignment */
  MLA_ERR_DEVICE = 4            /* the HIP runtime reported an error at launch */
} mla_status_t;

/* KV cache element type.  [P3] 实现拆解 item 3 and 关键源码片段
 * (cache_kernels.cu host checks): "auto" and "bfloat16" store raw bf16,
 * "fp8" and "fp8_e4m3" store e4m3fn scaled per layer, "fp8_e5m2" stores OCP
 * e5m2 scaled per layer (the page's ROCm build refuses it; gfx950 converts
 * e5m2 natively, so it is implemented here). */
typedef enum {
  MLA_KV_AUTO = 0,
  MLA_KV_BF16 = 1,
  MLA_KV_FP8_E4M3 = 2,
  MLA_KV_FP8_E5M2 = 3,
  MLA_KV_FP16 = 4   /* IEEE fp16: a source format of the pack, never a cache */
} mla_kv_dtype_t;

/* Output layout of the chunked-context pack ([P1] 关键源码片段,
 * fused_mla_kv_concat and fused_mla_kv_concat_quant_fp8). */
typedef enum {
  MLA_PACK_KEY_BF16 = 0,          /* 16-bit full key only, in the source format */
  MLA_PACK_KEY_V_FP8 = 1,         /* fp8 full key and fp8 V */
  MLA_PACK_KEY_V_FP8_KPE_RAW = 2  /* as KEY_V_FP8, k_pe given as fp8 codes, copied as is */
} mla_pack_mode_t;

/* How a chunk's attention partial enters the accumulator ([P1] 实现拆解
 * item 3, accumulate_mla_context_chunk and its output_written flag). */
typedef enum {
  MLA_MERGE_INIT_COPY = 0,     /* first chunk: the accumulator takes the partial */
  MLA_MERGE_INIT_WRITTEN = 1,  /* first chunk already written into the accumulator:
                                  only its lse is taken */
  MLA_MERGE_ACCUMULATE = 2     /* continuation chunk: log-sum-exp merge */
} mla_merge_mode_t;

/* Description of the last error on the calling thread ("" if none). */
const char* mla_last_error(void);

/* Library version string, e.g. "mla_kv 0.1.0 gfx950". */
const char* mla_version(void);

/* Diagnostics: the next kernel this thread enqueues through the library
 * records start_event as it begins executing and stop_event as it ends
 * (hipEvent_t handles created by the caller; hipExtLaunchKernel semantics),
 * so the pair brackets that kernel alone, without the dispatch gap that
 * events recorded on the stream around the call would include.  The setting
 * is consumed by that one launch; pass NULL, NULL to clear it.  Both or
 * neither must be NULL (MLA_ERR_INVALID_ARGUMENT otherwise). */
int32_t mla_set_launch_events(void* start_event, void* stop_event);

/* Parse a KV-cache dtype string into *out.  Accepts "auto", "bfloat16",
 * "fp8", "fp8_e4m3", "fp8_e5m2" (MLA_OK); anything else
 * MLA_ERR_INVALID_ARGUMENT.  Same whitelist as [P3] 关键源码片段
 * (_GROUPED_KV_CACHE_DTYPES and the host checks of cache_kernels.cu). */
int32_t mla_parse_kv_cache_dtype(const char* s, int32_t* out);

/* ------------------------------------------------------------------------
 * mla_kv_insert_grouped -- grouped concat-and-cache over all layers in one
 * launch ([P3] 功能与动机, 实现拆解 items 2-3, 关键源码片段 cache_kernels.cu).
 *
 * For every layer l < num_layers and token t < num_tokens:
 *   s = slot_mapping[l * slot_layer_stride + t]      (device int64)
 *   if s < 0 the token is skipped for that layer;
 *   else block = s / block_size, offset = s % block_size and the entry at
 *     kv_cache_ptrs[l] + block * block_stride + offset * entry_stride
 *   receives conv(kv_c[l, t, 0:kv_lora_rank]) at element 0 and
 *   conv(k_pe[l, t, 0:pe_dim]) at element kv_lora_rank.
 * conv is a raw 16-bit copy for AUTO/BF16 and, for FP8_E4M3,
 *   e4m3fn(fl32(x) / kv_scales[l]) rounded to nearest-even, saturating at
 *   +-448 (the quotient is the IEEE fp32 quotient); for FP8_E5M2 the same
 *   with the e5m2 format, saturating at +-57344.  NaN gives code 0x7F | sign
 *   in both formats.
 * Result: bit-identical to num_layers independent single-layer inserts
 * ([P3] 关键源码片段 test_cache.py).
 *
 * kv_c   device bf16; element [l, t, i] at l*kv_c_layer_stride + t*kv_c_token_stride + i
 * k_pe   device bf16; element [l, t, j] at l*k_pe_layer_stride + t*k_pe_token_stride + j
 *        (token-major [T, L, D] and layer-major [L, T, D] storage are both
 *        expressed through the two strides)
 * kv_cache_ptrs  device int64 [num_layers]: base address of each layer's cache
 *        (bf16 elements for AUTO/BF16, bytes for FP8); all layers share
 *        block_size / block_stride / entry_stride, in cache elements.
 * kv_scales      device fp32 [num_layers] for FP8 (read when the kernel runs,
 *        never cached by the library); must be NULL for AUTO/BF16.
 * slot_mapping   device int64; slot_layer_stride 0 = one mapping for all layers.
 * kv_cache_dtype an mla_kv_dtype_t.
 *
 * Alignment (MLA_ERR_MISALIGNED otherwise): kv_c and k_pe base addresses and
 * their strides (in bytes) multiples of 16 (k_pe is not read, nor checked,
 * when pe_dim is 0); block_stride and entry_stride in bytes multiples of 16.
 * kv_lora_rank and pe_dim must be multiples of 16 (MLA_ERR_UNSUPPORTED
 * otherwise); entry_stride >= kv_lora_rank + pe_dim.
 * Preconditions (not checked): each cache base is 16-byte aligned and holds
 * every slot used; the valid slots of one layer are distinct; layers' caches
 * do not overlap each other or the inputs.
 * ------------------------------------------------------------------------ */
int32_t mla_kv_insert_grouped(
    const void* kv_c, int64_t kv_c_layer_stride, int64_t kv_c_token_stride,
    const void* k_pe, int64_t k_pe_layer_stride, int64_t k_pe_token_stride,
    const int64_t* kv_cache_ptrs, const float* kv_scales,
    const int64_t* slot_mapping, int64_t slot_layer_stride,
    int64_t num_layers, int64_t num_tokens, int64_t kv_lora_rank, int64_t pe_dim,
    int64_t block_size, int64_t block_stride, int64_t entry_stride,
    int32_t kv_cache_dtype, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_rope_cos_sin_cache -- fill the rotary table used by the epilogues.
 * out (device fp32 [max_pos, 2 * rope_dim]) row p holds, for the angles
 * theta_i = p * base^(-2i/d), i < d/2, evaluated in float64 on the device:
 *   [0, d/2)      cos_hi = RN32(cos theta_i)     [d/2, d)   sin_hi = RN32(sin theta_i)
 *   [d, 3d/2)     cos_lo = RN32(cos - cos_hi)    [3d/2, 2d) sin_lo = RN32(sin - sin_hi)
 * (hi + lo carries about 48 significant bits of each value).  The epilogues
 * rotate with the hi values in fp32 and, where that result could round to
 * a different bf16 value than the exact rotation (the two products nearly
 * cancelling, or the fp32 value next to a rounding boundary), recompute it
 * in float64 from hi + lo and rounds once.  Every rotated value is thus one
 * rounding of the rotation by the table's values, carried out with an error
 * of about 2^-52 relative to the magnitudes of the pair: the correctly
 * rounded bf16 of that rotation unless it lies that close to a rounding
 * boundary (then at most one ulp away).
 * ([P2] 关键源码片段: RoPE of k_pe at each context position, the positions
 * being the same for every layer; the formula itself is not printed, the
 * non-interleaved form with the given base is the reading taken.)
 * rope_dim must be even and > 0; max_pos >= 0.
 * ------------------------------------------------------------------------ */
int32_t mla_rope_cos_sin_cache(float* out, int64_t max_pos, int64_t rope_dim,
                               double base, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_ctx_kv_epilogue -- fused context-KV epilogue for all layers in one
 * launch: per-layer RMSNorm of kv_c, RoPE of k_pe, bf16 rounding, then the
 * grouped insert ([P2] 关键源码片段 _precompute_fused_context_kv; [P3]
 * 关键源码片段 dspark_mla.py grouped path).
 *
 * all_kv  device bf16, the projection output viewed as [T, L, kv_lora_rank + pe_dim]:
 *         element [t, l, i] at t*kv_token_stride + l*kv_layer_stride + i
 *         (for a [T, L*576] GEMM output: kv_token_stride = L*576, kv_layer_stride = 576).
 * gamma   device bf16 [num_layers, kv_lora_rank] (row l = layer l's norm weight).
 * eps     RMSNorm epsilon.
 * positions device int64 [num_tokens], each in [0, max_pos).
 * cos_sin device fp32 [max_pos, 2 * pe_dim] from mla_rope_cos_sin_cache.
 * For each (l, t):
 *   row[0:R]   = bf16(x_i * (mean(x^2) + eps)^(-1/2) * gamma[l, i])  (fp32 math)
 *   row[R:R+P] = bf16(rotation of k_pe by theta(positions[t]))   (pairs (i, i+P/2);
 *                rounded once, see mla_rope_cos_sin_cache)
 *   then row is inserted exactly as mla_kv_insert_grouped inserts [kv_c | k_pe].
 * dbg_rows  optional device bf16 [L, T, R+P] contiguous: receives every row
 *   (also those whose slot is negative); NULL to skip.
 * Cache, scale, slot and alignment arguments as mla_kv_insert_grouped; in
 * addition all_kv and its strides must be 16-byte aligned, kv_lora_rank must
 * be 512 and pe_dim 64 (MLA_ERR_UNSUPPORTED otherwise).
 * ------------------------------------------------------------------------ */
int32_t mla_ctx_kv_epilogue(
    const void* all_kv, int64_t kv_layer_stride, int64_t kv_token_stride,
    const void* gamma, float eps, const int64_t* positions, const float* cos_sin,
    int64_t max_pos,
    const int64_t* kv_cache_ptrs, const float* kv_scales,
    const int64_t* slot_mapping, int64_t slot_layer_stride,
    int64_t num_layers, int64_t num_tokens, int64_t kv_lora_rank, int64_t pe_dim,
    int64_t block_size, int64_t block_stride, int64_t entry_stride,
    int32_t kv_cache_dtype, void* dbg_rows, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_ctx_kv_proj -- the fused KV-only context projection: one GEMM producing
 * the latent KV of every draft layer at once ([P2] 功能与动机, 实现拆解 item 2:
 * hidden -> L * 576 instead of L projections hidden -> 2112).
 *   Y[t, n] = bf16( sum_k X[t, k] * W[n, k] )   fp32 accumulation (MFMA)
 * X device bf16 [T, K] row-major (row stride x_row_stride, elements).
 * W device bf16 [N, K] row-major and dense (row stride K): the linear
 *   layer's [out, in] weight storage, i.e. the transpose of the [K, N]
 *   matrix X is multiplied by.  A caller holding the [K, N] matrix converts
 *   it once with mla_transpose_bf16 (rows K, cols N).
 * Y device bf16 [T, N] row-major (row stride y_row_stride).
 * K must be a multiple of 64 and N a multiple of 16; pointers and row
 * strides 16-byte aligned.  T may be any value >= 0.  The kernel addresses
 * a 256-row tile of X by 32-bit byte offsets: 255 * x_row_stride + K must
 * stay below 2^30 elements (else MLA_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------ */
int32_t mla_ctx_kv_proj(const void* X, int64_t x_row_stride, int64_t T,
                        int64_t K, const void* W, int64_t N, void* Y,
                        int64_t y_row_stride, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_transpose_bf16 -- weight preparation for mla_ctx_kv_proj: dst[c, r] =
 * src[r, c] for r < rows, c < cols, bit for bit ([P2] 实现拆解 item 2: the
 * merged linear layer holds its weight as [out, in]; a weight held as the
 * [in, out] = [K, N] matrix that X is multiplied by is converted once with
 * this call into the [N, K] storage mla_ctx_kv_proj reads).  A weight does
 * not change between calls, so the conversion is not part of the
 * per-call path.
 * src device bf16 [rows, cols] (row stride src_row_stride >= cols);
 * dst device bf16 [cols, rows] (row stride dst_row_stride >= rows).
 * rows and cols multiples of 8; addresses and row strides 16-byte aligned
 * (MLA_ERR_UNSUPPORTED / MLA_ERR_MISALIGNED otherwise); src and dst must not
 * overlap (MLA_ERR_INVALID_ARGUMENT).
 * ------------------------------------------------------------------------ */
int32_t mla_transpose_bf16(const void* src, int64_t rows, int64_t cols, int64_t src_row_stride,
                           void* dst, int64_t dst_row_stride, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_ctx_latent_gather -- read one sequence's context rows out of a paged
 * latent cache into a contiguous workspace ([P1] 实现拆解 item 2:
 * _gather_context_latent before kv_b_proj, dispatched on the cache dtype;
 * 关键源码片段: with a plain fp8 cache the gather does not dequantise, and
 * 实现拆解 item 5: a bf16 kv_b_proj must then still receive bf16).
 *   s = src_slots[j]; row = cache + (s / block_size) * block_stride
 *                               + (s % block_size) * entry_stride
 *   out_dtype BF16, fp8 cache:  out[j, i] = bf16(fl32(decode(row[i])) * cache_scale[0])
 *                               (decode: e4m3fn or e5m2 per cache_dtype; NaN
 *                               codes give the quiet NaN with their sign)
 *   out_dtype BF16, bf16 cache: out[j, i] = row[i]  bit for bit
 *   out_dtype = cache_dtype (FP8_E4M3 or FP8_E5M2): out[j, i] = row[i] code
 *                               for code, no dequantisation (cache_scale NULL)
 * cache       device, element type from cache_dtype (AUTO/BF16, FP8_E4M3 or
 *             FP8_E5M2).
 * cache_scale device fp32 [1] for the dequantising fp8 gather (read at kernel
 *             time), NULL otherwise.
 * src_slots   device int64 [num_tokens]; every entry >= 0 and inside the cache
 *             (precondition).
 * out         device [num_tokens, width] contiguous, bf16 or fp8 codes per
 *             out_dtype; width must be a multiple of 16 and <= entry_stride.
 * max_blocks  grid cap (0 = library default); the kernel loops grid-stride.
 * ------------------------------------------------------------------------ */
int32_t mla_ctx_latent_gather(const void* cache, int32_t cache_dtype,
                              const float* cache_scale, int64_t block_size,
                              int64_t block_stride, int64_t entry_stride,
                              const int64_t* src_slots, int64_t num_tokens,
                              int64_t width, int32_t out_dtype, void* out,
                              int64_t max_blocks, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_ctx_kv_pack -- build the contiguous full key [k_nope | k_pe] (and, in
 * fp8 modes, the contiguous fp8 V) of one context chunk in one launch,
 * reading k_nope / v straight from the strided kv_b_proj output and k_pe
 * straight from the gather workspace ([P1] 实现拆解 item 1, 关键源码片段
 * fused_mla_key_concat_kv_cache.py, 评论区精华 on the tested input types).
 *   key[t, h, 0:nope]         = k_nope[t, h, :]
 *   key[t, h, nope:nope+rope] = k_pe[t, :]           (same for every head)
 *   v_out[t, h, :]            = v[t, h, :]            (fp8 modes only)
 * src_dtype: MLA_KV_BF16 or MLA_KV_FP16, the format of k_nope, v and (unless
 *   KPE_RAW) k_pe.
 * KEY_BF16:   key_out [T, H, nope+rope] in the source format (a 16-bit copy);
 *   v, v_out and the scales must be NULL.
 * KEY_V_FP8:  key_out and v_out fp8 [T, H, nope+rope] / [T, H, vdim]; each
 *   element x becomes e4m3fn(fl32(x) / scale), RNE, saturating at +-448;
 *   k_scale / v_scale are device fp32 [1] or NULL for 1.0 (a plain cast,
 *   bit-identical to torch's float8_e4m3fn cast -- the page's op has no scale).
 * KEY_V_FP8_KPE_RAW: as KEY_V_FP8, except that k_pe holds e4m3fn codes (one
 *   byte each; kpe_tok_stride in bytes), which are copied into the key
 *   unchanged -- the page's KPE_FP8 branch for a plain fp8 cache.  The codes
 *   keep the cache's scale, so this matches KEY_V_FP8 only when that scale
 *   equals k_scale (the caller's choice; not checked).
 * k_nope  device: [t, h, i] at t*kn_tok_stride + h*kn_head_stride + i
 * k_pe    device: [t, j]    at t*kpe_tok_stride + j
 * v       device: [t, h, i] at t*v_tok_stride + h*v_head_stride + i
 * nope, rope, vdim must be multiples of 16; pointers and strides (in bytes)
 * 16-byte aligned.  max_blocks caps the grid (0 = default); the kernel loops
 * grid-stride over T * H rows, so any T fits.
 * ------------------------------------------------------------------------ */
int32_t mla_ctx_kv_pack(const void* k_nope, int64_t kn_tok_stride,
                        int64_t kn_head_stride, const void* k_pe,
                        int64_t kpe_tok_stride, const void* v,
                        int64_t v_tok_stride, int64_t v_head_stride,
                        int64_t num_tokens, int64_t num_heads, int64_t nope,
                        int64_t rope, int64_t vdim, int32_t mode, int32_t src_dtype,
                        const float* k_scale, const float* v_scale,
                        void* key_out, void* v_out, int64_t max_blocks,
                        mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_ctx_kv_pack_gather -- one launch doing the pack of context chunk c and
 * the latent gather of chunk c + 1 ([P1] 实现拆解 item 2: every chunk first
 * gathers its latent rows from the cache, then runs kv_b_proj, then packs;
 * the pack of chunk c needs nothing from chunk c + 1 and the gather of
 * chunk c + 1 needs nothing from chunk c, so in a chunk loop
 *   gather(0); kv_b_proj(0); pack(0) + gather(1); kv_b_proj(1); pack(1) + gather(2); ...
 * is the same computation with one launch fewer per chunk).
 * The first 19 arguments are those of mla_ctx_kv_pack, the next 11 those of
 * mla_ctx_latent_gather; max_blocks caps the pack's part of the grid (0 =
 * one thread per output chunk; the pack then loops grid-stride), the
 * gather's part has one thread per chunk.  Result: identical to
 *   mla_ctx_kv_pack(pack arguments, max_blocks, stream);
 *   mla_ctx_latent_gather(gather arguments, 0, stream);
 * Each part is validated as its own entry point validates it, before
 * anything is launched.  In addition gather_out must not overlap k_nope,
 * k_pe, v, key_out or v_out (MLA_ERR_INVALID_ARGUMENT; checked on the
 * address ranges the views span): the two parts run concurrently.  When both
 * parts have work, the pack's sources must be bf16 with a 16-bit k_pe (modes
 * KEY_BF16 and KEY_V_FP8; MLA_ERR_UNSUPPORTED otherwise -- call the two entry
 * points); when one part is empty the other runs as its own entry point.
 * ------------------------------------------------------------------------ */
int32_t mla_ctx_kv_pack_gather(
    const void* k_nope, int64_t kn_tok_stride, int64_t kn_head_stride, const void* k_pe,
    int64_t kpe_tok_stride, const void* v, int64_t v_tok_stride, int64_t v_head_stride,
    int64_t num_tokens, int64_t num_heads, int64_t nope, int64_t rope, int64_t vdim,
    int32_t mode, int32_t src_dtype, const float* k_scale, const float* v_scale, void* key_out,
    void* v_out, const void* cache, int32_t cache_dtype, const float* cache_scale,
    int64_t block_size, int64_t block_stride, int64_t entry_stride, const int64_t* src_slots,
    int64_t gather_tokens, int64_t width, int32_t out_dtype, void* gather_out,
    int64_t max_blocks, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_ctx_merge_chunk -- fold one context chunk's attention partial into the
 * accumulator of the chunked-context loop ([P1] 实现拆解 item 3: the
 * accumulator is allocated before any chunk; a non-continuation chunk may
 * write its output straight into it, after which only its log-sum-exp is
 * folded in; continuation chunks are merged).  For every token t and head h:
 *   INIT_COPY:    out[t, h, :] = part[t, h, :];  lse[h, t] = part_lse[h, t]
 *   INIT_WRITTEN: lse[h, t] = part_lse[h, t]   (out already holds the
 *                 chunk's output; part is not read and may be NULL)
 *   ACCUMULATE:   m = max(lse, part_lse), w_x = exp(lse_x - m),
 *                 out = bf16((w_a out + w_b part) / (w_a + w_b)),
 *                 lse = m + log(w_a + w_b)  (natural log; fp32 arithmetic)
 *                 A partial whose lse is -inf covers no key and contributes
 *                 nothing (its output is not used); if both are -inf the
 *                 result is the neutral partial (0, -inf).
 * out, part  device bf16 [t, h, i] at t*tok_stride + h*head_stride + i; rows
 *            16-byte aligned; head_dim a multiple of 8.  out is updated in
 *            place; ACCUMULATE refuses part == out (a continuation chunk's
 *            output cannot already sit in the accumulator -- the page's
 *            assertion on output_written).
 * lse, part_lse  device fp32 [h, t] at h*head_stride + t*tok_stride.
 * ------------------------------------------------------------------------ */
int32_t mla_ctx_merge_chunk(void* out, int64_t out_tok_stride, int64_t out_head_stride,
                            float* lse, int64_t lse_head_stride, int64_t lse_tok_stride,
                            const void* part, int64_t part_tok_stride,
                            int64_t part_head_stride, const float* part_lse,
                            int64_t part_lse_head_stride, int64_t part_lse_tok_stride,
                            int64_t num_tokens, int64_t num_heads, int64_t head_dim,
                            int32_t mode, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_ctx_neutralize_partials -- set the neutral partial (out = 0,
 * lse = -inf) for every token t with no_context[t] != 0: prefill tokens
 * whose request has no context start the merge from it ([P1] 实现拆解
 * item 3, neutralize_empty_context_partials).  Layouts as for
 * mla_ctx_merge_chunk; no_context is a device uint8 [num_tokens].
 * ------------------------------------------------------------------------ */
int32_t mla_ctx_neutralize_partials(void* out, int64_t out_tok_stride, int64_t out_head_stride,
                                    float* lse, int64_t lse_head_stride, int64_t lse_tok_stride,
                                    const uint8_t* no_context, int64_t num_tokens,
                                    int64_t num_heads, int64_t head_dim, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_new_token_epilogue -- the new-token counterpart of the chunked-context
 * pack, for one layer's prefill tokens ([P1] 功能与动机: the new-token epilogue
 * already quantises the query; 关键源码片段, fused_mla_key_concat_kv_cache.py:
 * the chunked-context pack is fused_mla_key_concat_kv_cache_insert without
 * the query, without the cache insert and without RoPE).  The pages name the
 * op only; this entry point is that reading, with every step done as
 * elsewhere in this library:
 *   pe_q = RoPE(q_pe[t, h, :], pos[t]),  pe_k = RoPE(k_pe[t, :], pos[t])
 *            (half-split rotation, angles from cos_sin as in
 *            mla_ctx_kv_epilogue; each result rounded once to bf16)
 *   q_out[t, h, :]   = [q_nope[t, h, :] | pe_q]
 *   key_out[t, h, :] = [k_nope[t, h, :] | pe_k]     (same pe_k for every head)
 *   v_out[t, h, :]   = v[t, h, :]                    (KEY_V_FP8 only)
 *   cache entry slot_mapping[t] = [kv_c[t, :] | pe_k] (as mla_kv_insert_grouped
 *            with one layer; slot < 0 skips the token; cache NULL skips the insert)
 * mode KEY_BF16:  q_out / key_out bf16 [T, H, nope+rope] contiguous; v, v_out
 *   and q/k/v scales must be NULL.
 * mode KEY_V_FP8: q_out / key_out / v_out e4m3fn codes, each bf16 value x
 *   (for the rope parts, the rounded rotation) becomes e4m3fn(fl32(x) / scale),
 *   RNE, saturating at +-448; q_scale / k_scale / v_scale are device fp32 [1],
 *   or NULL for 1.0.
 * Inputs are bf16 device views: [t, h, i] at t*tok_stride + h*head_stride + i
 *   (q_nope, q_pe, k_nope, v), [t, i] at t*tok_stride + i (kv_c, k_pe).
 * positions   device int64 [T], each in [0, max_pos) (precondition; values
 *             outside are clamped to that range).
 * cos_sin     device fp32 [max_pos, 2 * rope] (mla_rope_cos_sin_cache fills it).
 * cache       device; element type from cache_dtype (AUTO/BF16, FP8_E4M3,
 *             FP8_E5M2); cache_scale device fp32 [1] for an fp8 cache, NULL
 *             for bf16; slot_mapping device int64 [T] with distinct
 *             non-negative slots inside the cache, or -1 (precondition).
 * rope must be 64; nope, vdim and kv_lora_rank multiples
 * of 16; addresses and strides (in bytes) 16-byte aligned.  num_heads may be
 * 0 (cache insert only).  max_blocks caps the grid (0 = the library's
 * default: the full grid -- one (token, head) task per 16-lane row, or, for
 * fp8 outputs with nope = vdim = 128 and heads a multiple of 16, one task of
 * 16 heads per wavefront -- except fp8 outputs of other shapes, which run 4
 * workgroups per CU); the kernel loops grid-stride.  Host-side validation
 * happens before any launch, so a rejected call writes nothing.
 * ------------------------------------------------------------------------ */
int32_t mla_new_token_epilogue(
    const void* q_nope, int64_t qn_tok_stride, int64_t qn_head_stride, const void* q_pe,
    int64_t qp_tok_stride, int64_t qp_head_stride, const void* k_nope, int64_t kn_tok_stride,
    int64_t kn_head_stride, const void* v, int64_t v_tok_stride, int64_t v_head_stride,
    const void* kv_c, int64_t kv_c_tok_stride, const void* k_pe, int64_t k_pe_tok_stride,
    const int64_t* positions, const float* cos_sin, int64_t max_pos, int64_t num_tokens,
    int64_t num_heads, int64_t nope, int64_t rope, int64_t vdim, int64_t kv_lora_rank,
    int32_t mode, const float* q_scale, const float* k_scale, const float* v_scale,
    void* q_out, void* key_out, void* v_out, void* cache, int32_t cache_dtype,
    const float* cache_scale, const int64_t* slot_mapping, int64_t block_size,
    int64_t block_stride, int64_t entry_stride, int64_t max_blocks, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_stream_copy -- measurement aid, not a step of the path: copy `bytes`
 * bytes from src to dst (device, 16-byte aligned, size a multiple of 16, no
 * overlap) with the launch shape of the library's streaming kernels (one
 * 16-byte chunk per thread over the full grid, cache-bypassing loads,
 * streaming stores).  Its rate at a given size is the ceiling the
 * bandwidth-bound kernels are compared with (the roofline's "measured
 * device-to-device copy bandwidth").
 * ------------------------------------------------------------------------ */
int32_t mla_stream_copy(void* dst, const void* src, int64_t bytes, mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_stream_mix -- measurement aid, not a step of the path: the launch
 * shape of mla_stream_copy with reads_per_write (1 to 4) 16-byte loads per
 * 16-byte store: output chunk i is the XOR of input chunks
 * reads_per_write * i ... reads_per_write * i + reads_per_write - 1.  dst
 * holds dst_bytes, src reads_per_write * dst_bytes (device, 16-byte aligned,
 * sizes multiples of 16, no overlap).  With reads_per_write = 2 it has the
 * fp8 pack's read:write mix, and its rate at the pack's size is the ceiling
 * the pack is compared with.  reads_per_write = 1 is mla_stream_copy.
 * ------------------------------------------------------------------------ */
int32_t mla_stream_mix(void* dst, const void* src, int64_t dst_bytes, int32_t reads_per_write,
                       mla_stream_t stream);

/* ------------------------------------------------------------------------
 * mla_mfma_rate -- measurement aid, not a step of the path: one workgroup of
 * 4 wavefronts on every compute unit, each wavefront issuing iters x 12
 * v_mfma_f32_32x32x16_bf16 (16384 multiply-adds each) on a 4 x 3 tile of
 * accumulators, with pseudo-random operands in +-[1, 2) that alternate
 * between two sets every step, between two reads of the shader clock and of
 * the 100 MHz real-time counter.
 * Wavefront w of workgroup g writes clocks[(4 g + w) * 4 + 0..3] = shader
 * clock at start, at end, real-time counter at start, at end (device memory,
 * at least 16 words per compute unit: clock_words >= 16 x CU count).  From
 * them: cycles per MFMA issue per SIMD and the clock held under full MFMA
 * load, hence the bf16 matrix peak the projection is compared with
 * (MLA_ERR_INVALID_ARGUMENT for an odd iters or one outside [2, 2^20], a
 * NULL or short clocks array).
 * ------------------------------------------------------------------------ */
int32_t mla_mfma_rate(int64_t iters, uint64_t* clocks, int64_t clock_words, mla_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_KV_H */
