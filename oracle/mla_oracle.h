/*
 * mla_oracle.h -- plain, slow CPU oracle for the MLA latent-KV insert/pack path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include, link
 * or call this code; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source with the HIP implementation.
 *
 * Pages cited (by title and section):
 *   [P1] "PR #51772 完整报告" -- [Attention][MLA] Fuse Kimi-K3 chunked-context K/V packing
 *   [P2] "PR #50585 完整报告" -- [K3 Perf] Optimize k3 dspark fused kv
 *   [P3] "PR #55356 完整报告" -- [Kimi Perf] Group fp8 mla cache insertion
 * Section names are the pages' headings: 功能与动机 (motivation), 实现拆解
 * (implementation breakdown), 关键源码片段 (key source snippets), 风险与影响
 * (risks and impact).
 *
 * Conventions: bf16 values travel as their uint16 bit patterns, fp8 e4m3fn as
 * uint8 codes.  All strides are in elements.  Every function returns 0 on
 * success or a negative code on a rejected input.
 */
#ifndef MLA_ORACLE_H
#define MLA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_EDUPSLOT = -2 };
enum { ORC_CACHE_BF16 = 0, ORC_CACHE_FP8_E4M3 = 1, ORC_CACHE_FP8_E5M2 = 2 };
enum { ORC_PACK_KEY_BF16 = 0, ORC_PACK_KEY_V_FP8 = 1, ORC_PACK_KEY_V_FP8_KPE_RAW = 2 };
enum { ORC_SRC_BF16 = 0, ORC_SRC_FP16 = 1 };          /* 16-bit source format of the pack */
enum { ORC_GATHER_BF16 = 0, ORC_GATHER_FP8_RAW = 1 };  /* gather output */
enum { ORC_MERGE_INIT_COPY = 0, ORC_MERGE_INIT_WRITTEN = 1, ORC_MERGE_ACCUMULATE = 2 };

/* ---- number formats --------------------------------------------------- */
float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_f64_to_bf16(double x);
double   orc_e4m3_decode(uint8_t code);
uint8_t  orc_e4m3_encode(double x);
uint8_t  orc_quantize(uint16_t x_bf16, float scale);
float    orc_f16_to_f32(uint16_t h);
uint8_t  orc_quantize_f32(float x, float scale);
uint16_t orc_dequantize(uint8_t code, float scale);
double   orc_e5m2_decode(uint8_t code);
uint8_t  orc_e5m2_encode(double x);
uint8_t  orc_quantize_e5m2(uint16_t x_bf16, float scale);
uint16_t orc_dequantize_e5m2(uint8_t code, float scale);

void orc_f64_to_bf16_n(const double* x, int64_t n, uint16_t* out);
void orc_e4m3_encode_f32_n(const float* x, int64_t n, uint8_t* out);
void orc_e4m3_decode_n(const uint8_t* c, int64_t n, double* out);
void orc_quantize_n(const uint16_t* x, int64_t n, float scale, uint8_t* out);
void orc_dequantize_n(const uint8_t* c, int64_t n, float scale, uint16_t* out);
void orc_f16_to_f32_n(const uint16_t* h, int64_t n, float* out);
void orc_e5m2_encode_f32_n(const float* x, int64_t n, uint8_t* out);
void orc_e5m2_decode_n(const uint8_t* c, int64_t n, double* out);
void orc_quantize_e5m2_n(const uint16_t* x, int64_t n, float scale, uint8_t* out);
void orc_dequantize_e5m2_n(const uint8_t* c, int64_t n, float scale, uint16_t* out);

/* ---- insert ------------------------------------------------------------ */
int orc_insert_single(const uint16_t* kv_c, int64_t kv_c_tok_stride,
                      const uint16_t* k_pe, int64_t k_pe_tok_stride,
                      const int64_t* slots, int64_t num_tokens,
                      int64_t kv_lora_rank, int64_t pe_dim,
                      void* cache, int64_t block_size, int64_t block_stride,
                      int64_t entry_stride, int cache_dtype, float scale);

int orc_insert_grouped(const uint16_t* kv_c, int64_t kv_c_layer_stride,
                       int64_t kv_c_tok_stride,
                       const uint16_t* k_pe, int64_t k_pe_layer_stride,
                       int64_t k_pe_tok_stride,
                       void* const* caches, const float* scales,
                       const int64_t* slot_mapping, int64_t slot_layer_stride,
                       int64_t num_layers, int64_t num_tokens,
                       int64_t kv_lora_rank, int64_t pe_dim,
                       int64_t block_size, int64_t block_stride,
                       int64_t entry_stride, int cache_dtype);

/* ---- projection, norm, rotary, epilogue --------------------------------- */
int orc_gemm_rows(const uint16_t* x, int64_t x_row_stride,
                  const uint16_t* w, int64_t w_k_stride, int64_t w_n_stride,
                  int64_t K, int64_t N, const int64_t* rows, int64_t num_rows,
                  uint16_t* out);

int orc_rmsnorm_row(const uint16_t* x, int64_t n, const uint16_t* gamma,
                    float eps, uint16_t* out);

int orc_rope_row(const uint16_t* x, int64_t rope_dim, int64_t pos, double base,
                 uint16_t* out);

int orc_ctx_kv_epilogue(const uint16_t* all_kv, int64_t kv_layer_stride,
                        int64_t kv_token_stride, const uint16_t* gamma,
                        float eps, const int64_t* positions, double rope_base,
                        int64_t num_layers, int64_t num_tokens,
                        int64_t kv_lora_rank, int64_t pe_dim,
                        void* const* caches, const float* scales,
                        const int64_t* slot_mapping, int64_t slot_layer_stride,
                        int64_t block_size, int64_t block_stride,
                        int64_t entry_stride, int cache_dtype,
                        uint16_t* rows_out);

/* ---- chunked-context gather and pack ------------------------------------ */
int orc_gather(const void* cache, int cache_dtype, float cache_scale,
               int64_t block_size, int64_t block_stride, int64_t entry_stride,
               const int64_t* src_slots, int64_t num_tokens, int64_t width,
               int out_kind, void* out);

int orc_pack(const uint16_t* k_nope, int64_t kn_tok_stride, int64_t kn_head_stride,
             const void* k_pe, int64_t kpe_tok_stride,
             const uint16_t* v, int64_t v_tok_stride, int64_t v_head_stride,
             int64_t num_tokens, int64_t num_heads, int64_t nope_dim,
             int64_t rope_dim, int64_t v_dim, int mode, int src_format,
             float k_scale, float v_scale, void* key_out, uint8_t* v_out);

/* ---- new-token epilogue ------------------------------------------------- */
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
    int64_t entry_stride, int cache_dtype, float cache_scale);

/* ---- chunk-partial merge ------------------------------------------------ */
int orc_merge_chunk(uint16_t* out, int64_t out_tok_stride, int64_t out_head_stride,
                    float* lse, int64_t lse_head_stride, int64_t lse_tok_stride,
                    const uint16_t* part, int64_t part_tok_stride, int64_t part_head_stride,
                    const float* part_lse, int64_t plse_head_stride, int64_t plse_tok_stride,
                    int64_t num_tokens, int64_t num_heads, int64_t head_dim, int mode);

int orc_neutralize_partials(uint16_t* out, int64_t out_tok_stride, int64_t out_head_stride,
                            float* lse, int64_t lse_head_stride, int64_t lse_tok_stride,
                            const uint8_t* no_context, int64_t num_tokens,
                            int64_t num_heads, int64_t head_dim);

/* dst[c][r] = src[r][c] (16-bit elements, bit for bit). */
int orc_transpose_u16(const uint16_t* src, int64_t rows, int64_t cols, int64_t src_row_stride,
                      uint16_t* dst, int64_t dst_row_stride);

#ifdef __cplusplus
}
#endif
#endif /* MLA_ORACLE_H */
