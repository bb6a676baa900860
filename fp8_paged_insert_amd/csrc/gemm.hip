// gemm.hip -- fused KV-only context projection (MFMA bf16 GEMM).
#include "mla_common.hpp"

using namespace mla;

extern "C" int32_t mla_ctx_kv_proj(const void* X, int64_t x_row_stride, int64_t T, int64_t K,
                                   const void* W, int64_t N, void* Y, int64_t y_row_stride,
                                   mla_stream_t stream) {
  clear_error();
  (void)X; (void)x_row_stride; (void)T; (void)K; (void)W; (void)N; (void)Y;
  (void)y_row_stride; (void)stream;
  return fail(MLA_ERR_UNSUPPORTED, "mla_ctx_kv_proj: not built yet");
}
