/*
 * mla_oracle.c -- plain, slow, serial CPU oracle for the MLA latent-KV
 * insert / epilogue / gather / pack path.
 *
 * TEST INFRASTRUCTURE ONLY: only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load this.  It shares no code, header, table
 * or helper with the HIP library, and it never calls into it.
 *
 * Built with gcc -O2 -fno-fast-math -ffp-contract=off, so every float
 * operation below is one IEEE-754 operation in the precision written.
 *
 * Pages (cited by title and section heading):
 *   [P1] "PR #51772 完整报告" ([Attention][MLA] Fuse Kimi-K3 chunked-context
 *        K/V packing)
 *   [P2] "PR #50585 完整报告" ([K3 Perf] Optimize k3 dspark fused kv)
 *   [P3] "PR #55356 完整报告" ([Kimi Perf] Group fp8 mla cache insertion)
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function.  Pins: every function here is checked by the CPU tests against
 * closed forms, library routines (torch CPU fp8/bf16 casts, float64 matmul),
 * brute force on tiny inputs, or invariants; none is "parity unpinned".
 */
#include "mla_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================== */
/* Number formats                                                            */
/* ======================================================================== */

/* bf16 -> f32: a bf16 value is the top half of an IEEE binary32 pattern. */
float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/*
 * Round a double to the nearest bfloat16 (8 significant bits, exponent range
 * of binary32, IEEE subnormals), ties to even.  NaN becomes the quiet NaN
 * 0x7FC0 with the sign kept; overflow becomes +-Inf, as round-to-nearest
 * requires.
 *
 * Method: write |x| = r * 2^q where 2^q is the bf16 spacing in the binade of
 * |x| (or the subnormal spacing 2^-133 below the normal range) and round the
 * real r to an integer with nearbyint() in the default ties-to-even mode.
 */
uint16_t orc_f64_to_bf16(double x) {
  const uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
  double a = fabs(x);
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  if (a == 0.0) return sign;
  int e;
  (void)frexp(a, &e);            /* a = m * 2^e, 0.5 <= m < 1 */
  int q = e - 8;                 /* 8 significant bits in this binade */
  if (q < -133) q = -133;        /* subnormal spacing of bf16 */
  double r = nearbyint(ldexp(a, -q));
  double v = ldexp(r, q);
  if (v >= 0x1p128) return (uint16_t)(sign | 0x7F80u);
  float f = (float)v;            /* exact: v has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/*
 * OCP FP8 e4m3fn decode: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; there is
 * no infinity, so the largest finite magnitude is code 0x7E = 448.  This is
 * the format behind torch.float8_e4m3fn, which [P1] 实现拆解 item 1 and the
 * 关键源码片段 docstring of fused_mla_kv_concat_quant_fp8 name as the cast the
 * fp8 path must match bit for bit.
 */
double orc_e4m3_decode(uint8_t code) {
  const int s = code >> 7;
  const int e = (code >> 3) & 0xF;
  const int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return s ? -NAN : NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

/*
 * e4m3fn encode, round to nearest with ties to even, saturating:
 *   NaN -> 0x7F | sign;  |x| >= 448 (Inf included) -> 0x7E | sign;
 *   otherwise the finite code whose value is nearest |x|; on a tie between two
 *   neighbouring codes the one with an even code (mantissa LSB 0) wins; the
 *   sign bit is then attached, so -0 and tiny negatives give 0x80.
 * Reading: the pages fix bit-identity with torch's e4m3fn cast ([P1] 风险与影响
 * item 3) but not the overflow rule; the saturating rule is taken (it agrees
 * with torch for every |x| <= 464, which covers all workloads here).
 * Implementation: a plain nearest-value search over the 127 finite codes.
 */
static double g_e4m3_values[0x7F];
static int g_e4m3_values_ready = 0;

/* The 127 finite non-negative code values, decoded once (codes 0x00..0x7E). */
static const double* e4m3_values(void) {
  if (!g_e4m3_values_ready) {
    for (int c = 0; c <= 0x7E; ++c) g_e4m3_values[c] = orc_e4m3_decode((uint8_t)c);
    g_e4m3_values_ready = 1;
  }
  return g_e4m3_values;
}

uint8_t orc_e4m3_encode(double x) {
  const uint8_t sign = signbit(x) ? 0x80u : 0u;
  if (isnan(x)) return (uint8_t)(sign | 0x7Fu);
  const double a = fabs(x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
  const double* val = e4m3_values();
  int best = 0;
  double best_d = fabs(a - val[0]);
  for (int c = 1; c <= 0x7E; ++c) {
    const double d = fabs(a - val[c]);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(sign | (uint8_t)best);
}

/*
 * Quantise one bf16 value into the fp8 cache with a per-layer scale.
 * [P3] 实现拆解 item 2 and 关键源码片段 (cache_kernels.cu): the fp8 branch
 * converts each bf16 element with the layer's kv_scales entry.  Reading: the
 * scale is a dequantisation scale, so the stored code is
 * encode(fl32(x) / scale) with one IEEE fp32 division (never a reciprocal
 * multiply).
 */
uint8_t orc_quantize(uint16_t x_bf16, float scale) {
  return orc_quantize_f32(orc_bf16_to_f32(x_bf16), scale);
}

/* The same quantisation for a value already in fp32 (an fp16 source value,
 * which converts to fp32 exactly). */
uint8_t orc_quantize_f32(float x, float scale) {
  const float q = x / scale;
  return orc_e4m3_encode((double)q);
}

/*
 * IEEE binary16 -> fp32, from the format's definition: sign bit, 5 exponent
 * bits with bias 15, 10 fraction bits; exponent 0 is subnormal (m * 2^-24),
 * exponent 31 is infinity (m = 0) or NaN.  Every value is exact in fp32.
 * Used for the fp16 inputs of the fp8 pack ([P1] 评论区精华: the pack's
 * bit-level tests cover bf16 and fp16 inputs).
 */
float orc_f16_to_f32(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24);
  } else if (e == 31) {
    if (m != 0) {
      const float nan = sign ? -NAN : NAN;
      return nan;
    }
    v = INFINITY;
  } else {
    v = ldexp((double)(1024 + m), e - 25);
  }
  return (float)(sign ? -v : v);
}

void orc_f16_to_f32_n(const uint16_t* h, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f32(h[i]);
}

/* Dequantise: bf16(fl32(decode(code) * scale)), one fp32 multiply, then one
 * rounding to bf16.  Reading of the gather's "dequant" step ([P1] 实现拆解
 * item 2: the plain-fp8 gather path feeding kv_b_proj in bf16). */
uint16_t orc_dequantize(uint8_t code, float scale) {
  const float d = (float)orc_e4m3_decode(code); /* exact */
  const float p = d * scale;
  return orc_f64_to_bf16((double)p);
}

/*
 * OCP FP8 e5m2 decode: 1 sign bit, 5 exponent bits with bias 15, 2 mantissa
 * bits; exponent field 0 is subnormal (m * 2^-16); exponent field 31 is
 * infinity (m = 0) or NaN (m != 0); the largest finite magnitude is code
 * 0x7B = 57344.  The format behind torch.float8_e5m2 and the "fp8_e5m2"
 * cache dtype of [P3] 实现拆解 item 3 (the kFp8E5M2 template instance).
 */
double orc_e5m2_decode(uint8_t code) {
  const int s = code >> 7;
  const int e = (code >> 2) & 0x1F;
  const int m = code & 0x3;
  double v;
  if (e == 0x1F) {
    if (m != 0) return s ? -NAN : NAN;
    v = INFINITY;
  } else if (e == 0) {
    v = ldexp((double)m, -16);
  } else {
    v = ldexp((double)(4 + m), e - 17);
  }
  return s ? -v : v;
}

/*
 * e5m2 encode, round to nearest with ties to even, saturating:
 *   NaN -> 0x7F | sign;  |x| >= 57344 (Inf included) -> 0x7B | sign;
 *   otherwise the finite code nearest |x|, ties to the even code.
 * Reading: the pages only name scaled_convert for this dtype; the same
 * saturating rule as for e4m3fn is taken (torch's own e5m2 cast rounds to
 * infinity from 61440 up and agrees everywhere below).
 */
static double g_e5m2_values[0x7C];
static int g_e5m2_values_ready = 0;

uint8_t orc_e5m2_encode(double x) {
  const uint8_t sign = signbit(x) ? 0x80u : 0u;
  if (isnan(x)) return (uint8_t)(sign | 0x7Fu);
  const double a = fabs(x);
  if (a >= 57344.0) return (uint8_t)(sign | 0x7Bu);
  if (!g_e5m2_values_ready) {
    for (int c = 0; c <= 0x7B; ++c) g_e5m2_values[c] = orc_e5m2_decode((uint8_t)c);
    g_e5m2_values_ready = 1;
  }
  int best = 0;
  double best_d = fabs(a - g_e5m2_values[0]);
  for (int c = 1; c <= 0x7B; ++c) {
    const double d = fabs(a - g_e5m2_values[c]);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(sign | (uint8_t)best);
}

/* The e5m2 cache's quantisation and dequantisation: the same steps as the
 * e4m3fn ones, with the e5m2 codec. */
uint8_t orc_quantize_e5m2(uint16_t x_bf16, float scale) {
  const float q = orc_bf16_to_f32(x_bf16) / scale;
  return orc_e5m2_encode((double)q);
}

uint16_t orc_dequantize_e5m2(uint8_t code, float scale) {
  const float d = (float)orc_e5m2_decode(code); /* exact */
  const float p = d * scale;
  return orc_f64_to_bf16((double)p);
}

void orc_e5m2_encode_f32_n(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_encode((double)x[i]);
}
void orc_e5m2_decode_n(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_decode(c[i]);
}
void orc_quantize_e5m2_n(const uint16_t* x, int64_t n, float scale, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_quantize_e5m2(x[i], scale);
}
void orc_dequantize_e5m2_n(const uint8_t* c, int64_t n, float scale, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_dequantize_e5m2(c[i], scale);
}

/* Quantise / dequantise for an fp8 cache dtype. */
static uint8_t quantize_as(uint16_t x_bf16, float scale, int cache_dtype) {
  return cache_dtype == ORC_CACHE_FP8_E5M2 ? orc_quantize_e5m2(x_bf16, scale)
                                           : orc_quantize(x_bf16, scale);
}
static uint16_t dequantize_as(uint8_t code, float scale, int cache_dtype) {
  return cache_dtype == ORC_CACHE_FP8_E5M2 ? orc_dequantize_e5m2(code, scale)
                                           : orc_dequantize(code, scale);
}
static int is_fp8_cache(int cache_dtype) {
  return cache_dtype == ORC_CACHE_FP8_E4M3 || cache_dtype == ORC_CACHE_FP8_E5M2;
}

void orc_f64_to_bf16_n(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(x[i]);
}
void orc_e4m3_encode_f32_n(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode((double)x[i]);
}
void orc_e4m3_decode_n(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}
void orc_quantize_n(const uint16_t* x, int64_t n, float scale, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_quantize(x[i], scale);
}
void orc_dequantize_n(const uint8_t* c, int64_t n, float scale, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_dequantize(c[i], scale);
}

/* ======================================================================== */
/* Insert                                                                    */
/* ======================================================================== */

static int cmp_i64(const void* a, const void* b) {
  const int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x > y) - (x < y);
}

/* Two valid tokens of one layer must not name the same slot: the pages give
 * no order between such writes, so the oracle refuses that input. */
static int has_duplicate_slots(const int64_t* slots, int64_t n) {
  int64_t* tmp = (int64_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
  int64_t m = 0;
  int dup = 0;
  if (!tmp) return 1;
  for (int64_t i = 0; i < n; ++i)
    if (slots[i] >= 0) tmp[m++] = slots[i];
  qsort(tmp, (size_t)m, sizeof(int64_t), cmp_i64);
  for (int64_t i = 1; i < m; ++i)
    if (tmp[i] == tmp[i - 1]) dup = 1;
  free(tmp);
  return dup;
}

/*
 * Single-layer concat-and-cache, the per-layer operation that the grouped
 * insert must reproduce exactly ([P3] 关键源码片段, test_cache.py: the
 * reference is built from one concat_and_cache_mla call per layer).
 * Per token t ([P3] 关键源码片段, cache_kernels.cu):
 *   s = slots[t]; a negative slot means the token is skipped;
 *   block = s / block_size, offset = s % block_size;
 *   entry = block * block_stride + offset * entry_stride;
 *   cache[entry + i]                = conv(kv_c[t, i])  for i < kv_lora_rank
 *   cache[entry + kv_lora_rank + j] = conv(k_pe[t, j])  for j < pe_dim
 * conv is a raw 16-bit copy for the bf16/auto cache, orc_quantize for the
 * e4m3fn cache and orc_quantize_e5m2 for the e5m2 cache.
 * No other cache element is touched.
 */
int orc_insert_single(const uint16_t* kv_c, int64_t kv_c_tok_stride,
                      const uint16_t* k_pe, int64_t k_pe_tok_stride,
                      const int64_t* slots, int64_t num_tokens,
                      int64_t kv_lora_rank, int64_t pe_dim,
                      void* cache, int64_t block_size, int64_t block_stride,
                      int64_t entry_stride, int cache_dtype, float scale) {
  if (num_tokens < 0 || kv_lora_rank < 0 || pe_dim < 0 || block_size <= 0)
    return ORC_EINVAL;
  if (cache_dtype != ORC_CACHE_BF16 && !is_fp8_cache(cache_dtype)) return ORC_EINVAL;
  if (has_duplicate_slots(slots, num_tokens)) return ORC_EDUPSLOT;
  for (int64_t t = 0; t < num_tokens; ++t) {
    const int64_t s = slots[t];
    if (s < 0) continue;
    const int64_t block = s / block_size;
    const int64_t offset = s % block_size;
    const int64_t entry = block * block_stride + offset * entry_stride;
    const uint16_t* src_c = kv_c + t * kv_c_tok_stride;
    const uint16_t* src_p = k_pe + t * k_pe_tok_stride;
    if (cache_dtype == ORC_CACHE_BF16) {
      uint16_t* dst = (uint16_t*)cache + entry;
      for (int64_t i = 0; i < kv_lora_rank; ++i) dst[i] = src_c[i];
      for (int64_t j = 0; j < pe_dim; ++j) dst[kv_lora_rank + j] = src_p[j];
    } else {
      uint8_t* dst = (uint8_t*)cache + entry;
      for (int64_t i = 0; i < kv_lora_rank; ++i)
        dst[i] = quantize_as(src_c[i], scale, cache_dtype);
      for (int64_t j = 0; j < pe_dim; ++j)
        dst[kv_lora_rank + j] = quantize_as(src_p[j], scale, cache_dtype);
    }
  }
  return ORC_OK;
}

/*
 * Grouped insert over num_layers layers in one call ([P3] 功能与动机 and
 * 实现拆解 items 2-3): layer l uses its own cache base caches[l], its own
 * scale scales[l] (fp8 only) and the slot row slot_mapping + l *
 * slot_layer_stride (stride 0 = one mapping shared by all layers, as the
 * shared_slot_mapping case of [P3] 关键源码片段 test_cache.py does with
 * expand).  By definition this is num_layers independent single-layer
 * inserts, which is exactly the equality [P3]'s test asserts.
 */
int orc_insert_grouped(const uint16_t* kv_c, int64_t kv_c_layer_stride,
                       int64_t kv_c_tok_stride,
                       const uint16_t* k_pe, int64_t k_pe_layer_stride,
                       int64_t k_pe_tok_stride,
                       void* const* caches, const float* scales,
                       const int64_t* slot_mapping, int64_t slot_layer_stride,
                       int64_t num_layers, int64_t num_tokens,
                       int64_t kv_lora_rank, int64_t pe_dim,
                       int64_t block_size, int64_t block_stride,
                       int64_t entry_stride, int cache_dtype) {
  if (num_layers < 0) return ORC_EINVAL;
  if (is_fp8_cache(cache_dtype) && num_layers > 0 && !scales) return ORC_EINVAL;
  for (int64_t l = 0; l < num_layers; ++l) {
    const float sc = is_fp8_cache(cache_dtype) ? scales[l] : 1.0f;
    const int rc = orc_insert_single(
        kv_c + l * kv_c_layer_stride, kv_c_tok_stride,
        k_pe + l * k_pe_layer_stride, k_pe_tok_stride,
        slot_mapping + l * slot_layer_stride, num_tokens, kv_lora_rank, pe_dim,
        caches[l], block_size, block_stride, entry_stride, cache_dtype, sc);
    if (rc != ORC_OK) return rc;
  }
  return ORC_OK;
}

/* ======================================================================== */
/* Projection, RMSNorm, RoPE, epilogue                                       */
/* ======================================================================== */

/*
 * KV-only context projection Y = X . W for selected rows ([P2] 功能与动机 and
 * 实现拆解 item 2: one projection hidden -> L * 576 replaces L full Q+KV
 * projections).  Reading: bf16 operands, exact products accumulated in
 * float64 in k order, one rounding to bf16.  W is addressed as the
 * mathematical [K, N] matrix through (w_k_stride, w_n_stride).
 * out is [num_rows, N].
 */
int orc_gemm_rows(const uint16_t* x, int64_t x_row_stride,
                  const uint16_t* w, int64_t w_k_stride, int64_t w_n_stride,
                  int64_t K, int64_t N, const int64_t* rows, int64_t num_rows,
                  uint16_t* out) {
  if (K < 0 || N < 0 || num_rows < 0) return ORC_EINVAL;
  double* acc = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
  if (!acc) return ORC_EINVAL;
  for (int64_t r = 0; r < num_rows; ++r) {
    const uint16_t* xr = x + rows[r] * x_row_stride;
    for (int64_t n = 0; n < N; ++n) acc[n] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double xv = (double)orc_bf16_to_f32(xr[k]);
      const uint16_t* wk = w + k * w_k_stride;
      for (int64_t n = 0; n < N; ++n)
        acc[n] += xv * (double)orc_bf16_to_f32(wk[n * w_n_stride]);
    }
    for (int64_t n = 0; n < N; ++n) out[r * N + n] = orc_f64_to_bf16(acc[n]);
  }
  free(acc);
  return ORC_OK;
}

/*
 * RMSNorm of one kv_c row with the row of the 2-D weight that belongs to its
 * layer ([P2] 关键源码片段, _precompute_fused_context_kv: ops.rms_norm with a
 * [L, kv_lora_rank] weight, one row per draft layer).
 * Reading (the kernel is not printed): y_i = x_i * (mean(x^2) + eps)^(-1/2) *
 * gamma_i, evaluated in float64 and rounded once to bf16; eps is the binary32
 * value the caller passes.
 */
int orc_rmsnorm_row(const uint16_t* x, int64_t n, const uint16_t* gamma,
                    float eps, uint16_t* out) {
  if (n <= 0) return ORC_EINVAL;
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double v = (double)orc_bf16_to_f32(x[i]);
    ss += v * v;
  }
  const double r = 1.0 / sqrt(ss / (double)n + (double)eps);
  for (int64_t i = 0; i < n; ++i) {
    const double v = (double)orc_bf16_to_f32(x[i]);
    const double g = (double)orc_bf16_to_f32(gamma[i]);
    out[i] = orc_f64_to_bf16(v * r * g);
  }
  return ORC_OK;
}

/*
 * Rotary embedding of one k_pe row ([P2] 关键源码片段: RoPE is applied to k_pe
 * with the context position of each token, the same positions for every
 * layer).  Reading (the formula is elided on the page): the non-interleaved
 * ("half split") form with base `base`: for i < d/2,
 *   theta_i = pos * base^(-2i/d),
 *   y_i       = x_i * cos(theta_i) - x_{i+d/2} * sin(theta_i)
 *   y_{i+d/2} = x_{i+d/2} * cos(theta_i) + x_i * sin(theta_i),
 * in float64, each output rounded once to bf16.
 */
int orc_rope_row(const uint16_t* x, int64_t rope_dim, int64_t pos, double base,
                 uint16_t* out) {
  if (rope_dim <= 0 || (rope_dim & 1)) return ORC_EINVAL;
  const int64_t half = rope_dim / 2;
  for (int64_t i = 0; i < half; ++i) {
    const double theta =
        (double)pos * pow(base, -2.0 * (double)i / (double)rope_dim);
    const double c = cos(theta), s = sin(theta);
    const double x1 = (double)orc_bf16_to_f32(x[i]);
    const double x2 = (double)orc_bf16_to_f32(x[i + half]);
    out[i] = orc_f64_to_bf16(x1 * c - x2 * s);
    out[i + half] = orc_f64_to_bf16(x2 * c + x1 * s);
  }
  return ORC_OK;
}

/*
 * The context-KV epilogue ([P2] 关键源码片段 _precompute_fused_context_kv, then
 * [P3] 关键源码片段 dspark_mla.py): the projection output all_kv is viewed as
 * [T, L, kv_lora_rank + pe_dim]; each (layer, token) row is split into kv_c
 * and k_pe; kv_c goes through the layer's RMSNorm, k_pe through RoPE at the
 * token's position; both are materialised as bf16 (the pages hold bf16
 * all_kv_c_normed and rotated k_pe before the insert) into
 * rows_out[L, T, kv_lora_rank + pe_dim]; then the grouped insert writes them.
 */
int orc_ctx_kv_epilogue(const uint16_t* all_kv, int64_t kv_layer_stride,
                        int64_t kv_token_stride, const uint16_t* gamma,
                        float eps, const int64_t* positions, double rope_base,
                        int64_t num_layers, int64_t num_tokens,
                        int64_t kv_lora_rank, int64_t pe_dim,
                        void* const* caches, const float* scales,
                        const int64_t* slot_mapping, int64_t slot_layer_stride,
                        int64_t block_size, int64_t block_stride,
                        int64_t entry_stride, int cache_dtype,
                        uint16_t* rows_out) {
  if (num_layers < 0 || num_tokens < 0) return ORC_EINVAL;
  const int64_t width = kv_lora_rank + pe_dim;
  for (int64_t l = 0; l < num_layers; ++l) {
    for (int64_t t = 0; t < num_tokens; ++t) {
      const uint16_t* src = all_kv + t * kv_token_stride + l * kv_layer_stride;
      uint16_t* dst = rows_out + (l * num_tokens + t) * width;
      int rc = orc_rmsnorm_row(src, kv_lora_rank, gamma + l * kv_lora_rank,
                               eps, dst);
      if (rc != ORC_OK) return rc;
      rc = orc_rope_row(src + kv_lora_rank, pe_dim, positions[t], rope_base,
                        dst + kv_lora_rank);
      if (rc != ORC_OK) return rc;
    }
  }
  if (!caches) return ORC_OK; /* rows only */
  return orc_insert_grouped(rows_out, num_tokens * width, width,
                            rows_out + kv_lora_rank, num_tokens * width, width,
                            caches, scales, slot_mapping, slot_layer_stride,
                            num_layers, num_tokens, kv_lora_rank, pe_dim,
                            block_size, block_stride, entry_stride,
                            cache_dtype);
}

/* ======================================================================== */
/* Chunked-context gather and pack                                           */
/* ======================================================================== */

/*
 * Gather latent rows of one sequence's context from a paged cache into a
 * contiguous [T, width] bf16 workspace ([P1] 实现拆解 item 2:
 * _gather_context_latent reads the context from the cache before kv_b_proj;
 * the plain-fp8 case feeds a bf16 kv_b_proj, see the second commit's fix).
 * Readings: the token -> slot map is a flat int64 array src_slots[T] (every
 * entry >= 0); fp8 codes are dequantised with the cache's scale
 * (orc_dequantize); bf16 caches are copied bit for bit.
 */
int orc_gather(const void* cache, int cache_dtype, float cache_scale,
               int64_t block_size, int64_t block_stride, int64_t entry_stride,
               const int64_t* src_slots, int64_t num_tokens, int64_t width,
               int out_kind, void* out) {
  if (num_tokens < 0 || width < 0 || block_size <= 0) return ORC_EINVAL;
  if (!is_fp8_cache(cache_dtype) && cache_dtype != ORC_CACHE_BF16) return ORC_EINVAL;
  if (out_kind != ORC_GATHER_BF16 && out_kind != ORC_GATHER_FP8_RAW) return ORC_EINVAL;
  /* the raw output exists only for an fp8 cache: its codes, not dequantised */
  if (out_kind == ORC_GATHER_FP8_RAW && !is_fp8_cache(cache_dtype)) return ORC_EINVAL;
  for (int64_t j = 0; j < num_tokens; ++j) {
    const int64_t s = src_slots[j];
    if (s < 0) return ORC_EINVAL;
    const int64_t entry = (s / block_size) * block_stride + (s % block_size) * entry_stride;
    for (int64_t i = 0; i < width; ++i) {
      if (out_kind == ORC_GATHER_FP8_RAW)
        ((uint8_t*)out)[j * width + i] = ((const uint8_t*)cache)[entry + i];
      else if (is_fp8_cache(cache_dtype))
        ((uint16_t*)out)[j * width + i] =
            dequantize_as(((const uint8_t*)cache)[entry + i], cache_scale, cache_dtype);
      else
        ((uint16_t*)out)[j * width + i] = ((const uint16_t*)cache)[entry + i];
    }
  }
  return ORC_OK;
}

/*
 * Full-key (and fp8 V) pack ([P1] 关键源码片段,
 * fused_mla_key_concat_kv_cache.py: fused_mla_kv_concat and
 * fused_mla_kv_concat_quant_fp8):
 *   key[t, h, 0:nope]            = k_nope[t, h, :]
 *   key[t, h, nope:nope+rope]    = k_pe[t, :]      (same for every head h)
 *   v_out[t, h, :]               = v[t, h, :]      (fp8 mode only)
 * Outputs are contiguous [T, H, nope+rope] and [T, H, v_dim].
 * mode KEY_BF16: key is a 16-bit copy in the source format, v is not used.
 * mode KEY_V_FP8: every element x of key and of v becomes
 *   encode(fl32(x) / scale) with k_scale for the key and v_scale for V.
 * mode KEY_V_FP8_KPE_RAW: as KEY_V_FP8, but k_pe holds e4m3fn codes
 *   (uint8, kpe_tok_stride in bytes) that are copied into the key unchanged.
 * src_format: the 16-bit format of k_nope, v (and k_pe unless raw): bf16 or
 *   IEEE fp16 ([P1] 评论区精华: bf16 and fp16 inputs are both tested).
 * Reading: the page's op takes no scale (a plain cast, bit-identical to
 * torch's e4m3fn cast), which is scale = 1.0.
 */
/* One 16-bit source value as fp32 (bf16 or fp16 bits; both exact). */
static float src_to_f32(uint16_t x, int src_format) {
  return src_format == ORC_SRC_FP16 ? orc_f16_to_f32(x) : orc_bf16_to_f32(x);
}

int orc_pack(const uint16_t* k_nope, int64_t kn_tok_stride, int64_t kn_head_stride,
             const void* k_pe, int64_t kpe_tok_stride,
             const uint16_t* v, int64_t v_tok_stride, int64_t v_head_stride,
             int64_t num_tokens, int64_t num_heads, int64_t nope_dim,
             int64_t rope_dim, int64_t v_dim, int mode, int src_format,
             float k_scale, float v_scale, void* key_out, uint8_t* v_out) {
  if (num_tokens < 0 || num_heads < 0 || nope_dim < 0 || rope_dim < 0 || v_dim < 0)
    return ORC_EINVAL;
  if (mode != ORC_PACK_KEY_BF16 && mode != ORC_PACK_KEY_V_FP8 &&
      mode != ORC_PACK_KEY_V_FP8_KPE_RAW)
    return ORC_EINVAL;
  if (src_format != ORC_SRC_BF16 && src_format != ORC_SRC_FP16) return ORC_EINVAL;
  const int64_t kw = nope_dim + rope_dim;
  for (int64_t t = 0; t < num_tokens; ++t) {
    for (int64_t h = 0; h < num_heads; ++h) {
      const int64_t ko = (t * num_heads + h) * kw;
      const uint16_t* kn = k_nope + t * kn_tok_stride + h * kn_head_stride;
      if (mode == ORC_PACK_KEY_BF16) {
        /* a 16-bit copy: the key keeps the source format */
        const uint16_t* kp = (const uint16_t*)k_pe + t * kpe_tok_stride;
        uint16_t* key = (uint16_t*)key_out + ko;
        for (int64_t i = 0; i < nope_dim; ++i) key[i] = kn[i];
        for (int64_t j = 0; j < rope_dim; ++j) key[nope_dim + j] = kp[j];
        continue;
      }
      uint8_t* key = (uint8_t*)key_out + ko;
      for (int64_t i = 0; i < nope_dim; ++i)
        key[i] = orc_quantize_f32(src_to_f32(kn[i], src_format), k_scale);
      if (mode == ORC_PACK_KEY_V_FP8_KPE_RAW) {
        /* [P1] 关键源码片段 (fused_mla_kv_concat_quant_fp8): a k_pe that is
         * already fp8 (the plain-fp8 gather does not dequantise) is copied
         * into the key byte for byte. */
        const uint8_t* kp = (const uint8_t*)k_pe + t * kpe_tok_stride;
        for (int64_t j = 0; j < rope_dim; ++j) key[nope_dim + j] = kp[j];
      } else {
        const uint16_t* kp = (const uint16_t*)k_pe + t * kpe_tok_stride;
        for (int64_t j = 0; j < rope_dim; ++j)
          key[nope_dim + j] = orc_quantize_f32(src_to_f32(kp[j], src_format), k_scale);
      }
      const uint16_t* vs = v + t * v_tok_stride + h * v_head_stride;
      uint8_t* vo = v_out + (t * num_heads + h) * v_dim;
      for (int64_t i = 0; i < v_dim; ++i)
        vo[i] = orc_quantize_f32(src_to_f32(vs[i], src_format), v_scale);
    }
  }
  return ORC_OK;
}

/*
 * New-token epilogue ([P1] 功能与动机: the new-token epilogue already
 * quantises the query; [P1] 关键源码片段, fused_mla_key_concat_kv_cache.py:
 * the chunked-context pack is the new-token op without the query, without
 * the cache insert and without RoPE, because gathered context k_pe is already
 * rotated).  The pages name the op (fused_mla_key_concat_kv_cache_insert) and
 * nothing more; the reading is that op = the chunked-context pack plus the
 * three parts it lacks, each done as elsewhere on the path:
 *   1. RoPE at the token's position, of k_pe[t, :] once and of q_pe[t, h, :]
 *      for every head (orc_rope_row; bf16 results);
 *   2. query:  q_out[t, h, :] = [q_nope[t, h, :] | rope(q_pe[t, h, :])],
 *      a bf16 copy in mode KEY_BF16, e4m3fn codes of fl32(x) / q_scale in
 *      mode KEY_V_FP8;
 *   3. key (and V in fp8 mode): the chunked-context pack (orc_pack) of
 *      k_nope and v with the rotated k_pe;
 *   4. cache insert of [kv_c[t, :] | rope(k_pe[t, :])] at slots[t]
 *      (orc_insert_single; a negative slot skips the token); cache may be
 *      NULL to skip the insert.
 * Outputs q_out and key_out are contiguous [T, H, nope + rope] (uint16 bf16
 * bits or uint8 codes), v_out contiguous [T, H, v_dim] codes (fp8 mode).
 */
int orc_new_token_epilogue(
    const uint16_t* q_nope, int64_t qn_tok_stride, int64_t qn_head_stride,
    const uint16_t* q_pe, int64_t qp_tok_stride, int64_t qp_head_stride,
    const uint16_t* k_nope, int64_t kn_tok_stride, int64_t kn_head_stride,
    const uint16_t* v, int64_t v_tok_stride, int64_t v_head_stride,
    const uint16_t* kv_c, int64_t kv_c_tok_stride,
    const uint16_t* k_pe, int64_t k_pe_tok_stride,
    const int64_t* positions, double rope_base,
    int64_t num_tokens, int64_t num_heads, int64_t nope_dim, int64_t rope_dim,
    int64_t v_dim, int64_t kv_lora_rank, int mode,
    float q_scale, float k_scale, float v_scale,
    void* q_out, void* key_out, uint8_t* v_out,
    void* cache, const int64_t* slots, int64_t block_size, int64_t block_stride,
    int64_t entry_stride, int cache_dtype, float cache_scale) {
  if (num_tokens < 0 || num_heads < 0 || nope_dim < 0 || rope_dim <= 0 || (rope_dim & 1) ||
      v_dim < 0 || kv_lora_rank < 0)
    return ORC_EINVAL;
  if (mode != ORC_PACK_KEY_BF16 && mode != ORC_PACK_KEY_V_FP8) return ORC_EINVAL;
  for (int64_t t = 0; t < num_tokens; ++t)
    if (positions[t] < 0) return ORC_EINVAL;
  const int64_t qw = nope_dim + rope_dim;
  uint16_t* kpe_rot = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(num_tokens * rope_dim + 1));
  uint16_t* qpe_rot = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)rope_dim);
  if (!kpe_rot || !qpe_rot) {
    free(kpe_rot);
    free(qpe_rot);
    return ORC_EINVAL;
  }
  int rc = ORC_OK;
  /* 1. RoPE of k_pe, once per token */
  for (int64_t t = 0; t < num_tokens && rc == ORC_OK; ++t)
    rc = orc_rope_row(k_pe + t * k_pe_tok_stride, rope_dim, positions[t], rope_base,
                      kpe_rot + t * rope_dim);
  /* 1 + 2. RoPE of q_pe per head, and the query row */
  for (int64_t t = 0; t < num_tokens && rc == ORC_OK; ++t) {
    for (int64_t h = 0; h < num_heads && rc == ORC_OK; ++h) {
      const uint16_t* qn = q_nope + t * qn_tok_stride + h * qn_head_stride;
      rc = orc_rope_row(q_pe + t * qp_tok_stride + h * qp_head_stride, rope_dim, positions[t],
                        rope_base, qpe_rot);
      const int64_t o = (t * num_heads + h) * qw;
      if (mode == ORC_PACK_KEY_BF16) {
        uint16_t* q = (uint16_t*)q_out + o;
        for (int64_t i = 0; i < nope_dim; ++i) q[i] = qn[i];
        for (int64_t j = 0; j < rope_dim; ++j) q[nope_dim + j] = qpe_rot[j];
      } else {
        uint8_t* q = (uint8_t*)q_out + o;
        for (int64_t i = 0; i < nope_dim; ++i)
          q[i] = orc_quantize_f32(orc_bf16_to_f32(qn[i]), q_scale);
        for (int64_t j = 0; j < rope_dim; ++j)
          q[nope_dim + j] = orc_quantize_f32(orc_bf16_to_f32(qpe_rot[j]), q_scale);
      }
    }
  }
  /* 3. key (and V): the chunked-context pack with the rotated k_pe */
  if (rc == ORC_OK)
    rc = orc_pack(k_nope, kn_tok_stride, kn_head_stride, kpe_rot, rope_dim, v, v_tok_stride,
                  v_head_stride, num_tokens, num_heads, nope_dim, rope_dim, v_dim, mode,
                  ORC_SRC_BF16, k_scale, v_scale, key_out, v_out);
  /* 4. the cache row [kv_c | rotated k_pe] */
  if (rc == ORC_OK && cache)
    rc = orc_insert_single(kv_c, kv_c_tok_stride, kpe_rot, rope_dim, slots, num_tokens,
                           kv_lora_rank, rope_dim, cache, block_size, block_stride,
                           entry_stride, cache_dtype, cache_scale);
  free(kpe_rot);
  free(qpe_rot);
  return rc;
}

/* ======================================================================== */
/* Chunk-partial merge                                                       */
/* ======================================================================== */

/*
 * Merge of chunked-context attention partials ([P1] 实现拆解 item 3:
 * accumulate_mla_context_chunk with output_written, and
 * neutralize_empty_context_partials; the pages give the behaviour, not the
 * arithmetic).  Reading: a partial over one chunk of keys is the normalised
 * output O_c[t, h, :] (bf16, the backend's output) and the natural-log
 * log-sum-exp lse_c[h, t] (fp32) of that chunk's scores; two partials over
 * disjoint key sets combine into the partial over their union by
 *   m = max(lse_a, lse_b), w_x = exp(lse_x - m),
 *   O = (w_a O_a + w_b O_b) / (w_a + w_b),  lse = m + log(w_a + w_b),
 * computed here in float64 and rounded once (O to bf16, lse to fp32).  A
 * partial whose lse is -inf covers no keys: it contributes nothing, whatever
 * its O holds, and two such partials give (0, -inf), the neutral partial.
 * Modes: INIT_COPY (the first chunk: the accumulator takes the partial),
 * INIT_WRITTEN (the first chunk's output is already in the accumulator, so
 * only its lse is taken -- the page's output_written), ACCUMULATE (a
 * continuation chunk, merged as above).
 */
int orc_merge_chunk(uint16_t* out, int64_t out_tok_stride, int64_t out_head_stride,
                    float* lse, int64_t lse_head_stride, int64_t lse_tok_stride,
                    const uint16_t* part, int64_t part_tok_stride, int64_t part_head_stride,
                    const float* part_lse, int64_t plse_head_stride, int64_t plse_tok_stride,
                    int64_t num_tokens, int64_t num_heads, int64_t head_dim, int mode) {
  if (num_tokens < 0 || num_heads < 0 || head_dim < 0) return ORC_EINVAL;
  if (mode != ORC_MERGE_INIT_COPY && mode != ORC_MERGE_INIT_WRITTEN &&
      mode != ORC_MERGE_ACCUMULATE)
    return ORC_EINVAL;
  for (int64_t t = 0; t < num_tokens; ++t) {
    for (int64_t h = 0; h < num_heads; ++h) {
      uint16_t* o = out + t * out_tok_stride + h * out_head_stride;
      const uint16_t* p = part + t * part_tok_stride + h * part_head_stride;
      float* l = lse + h * lse_head_stride + t * lse_tok_stride;
      const float lp = part_lse[h * plse_head_stride + t * plse_tok_stride];
      if (mode == ORC_MERGE_INIT_COPY) {
        for (int64_t i = 0; i < head_dim; ++i) o[i] = p[i];
        *l = lp;
        continue;
      }
      if (mode == ORC_MERGE_INIT_WRITTEN) {
        *l = lp;
        continue;
      }
      const double la = (double)*l, lb = (double)lp;
      const double m = la > lb ? la : lb;
      if (m == -INFINITY) {                 /* neither partial covers a key */
        for (int64_t i = 0; i < head_dim; ++i) o[i] = 0;
        *l = -INFINITY;
        continue;
      }
      const double wa = exp(la - m), wb = exp(lb - m);
      const double sum = wa + wb;
      for (int64_t i = 0; i < head_dim; ++i) {
        double acc = 0.0;
        if (wa != 0.0) acc += wa * (double)orc_bf16_to_f32(o[i]);
        if (wb != 0.0) acc += wb * (double)orc_bf16_to_f32(p[i]);
        o[i] = orc_f64_to_bf16(acc / sum);
      }
      *l = (float)(m + log(sum));
    }
  }
  return ORC_OK;
}

/* The neutral partial (O = 0, lse = -inf) for every token whose flag is set:
 * a prefill token with no context ([P1] 实现拆解 item 3,
 * neutralize_empty_context_partials). */
int orc_neutralize_partials(uint16_t* out, int64_t out_tok_stride, int64_t out_head_stride,
                            float* lse, int64_t lse_head_stride, int64_t lse_tok_stride,
                            const uint8_t* no_context, int64_t num_tokens,
                            int64_t num_heads, int64_t head_dim) {
  if (num_tokens < 0 || num_heads < 0 || head_dim < 0) return ORC_EINVAL;
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (!no_context[t]) continue;
    for (int64_t h = 0; h < num_heads; ++h) {
      uint16_t* o = out + t * out_tok_stride + h * out_head_stride;
      for (int64_t i = 0; i < head_dim; ++i) o[i] = 0;
      lse[h * lse_head_stride + t * lse_tok_stride] = -INFINITY;
    }
  }
  return ORC_OK;
}

/*
 * Weight preparation for the fused KV projection ([P2] 实现拆解 item 2: the
 * merged linear layer holds its weight as [out, in]; the fused context-KV
 * workload states the weight as the [in, out] matrix).  The definition of
 * a transpose: dst[c][r] = src[r][c], bit for bit.
 */
int orc_transpose_u16(const uint16_t* src, int64_t rows, int64_t cols, int64_t src_row_stride,
                      uint16_t* dst, int64_t dst_row_stride) {
  if (rows < 0 || cols < 0) return ORC_EINVAL;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) dst[c * dst_row_stride + r] = src[r * src_row_stride + c];
  return ORC_OK;
}
