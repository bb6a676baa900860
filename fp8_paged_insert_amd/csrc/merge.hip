// merge.hip -- merging chunked-context attention partials into the
// accumulator, and the neutral partial for prefills without context.
//
// Page: "PR #51772 完整报告" ([Attention][MLA] Fuse Kimi-K3 chunked-context
// K/V packing), 实现拆解 item 3: the accumulator is allocated before any
// chunk runs; prefills without context start from the neutral partial
// (neutralize_empty_context_partials); a non-continuation chunk's output may
// be written straight into the accumulator, after which only its
// log-sum-exp is folded in (accumulate_mla_context_chunk with
// output_written); continuation chunks are merged.  The pages give no
// arithmetic; the merge of two partials over disjoint key sets is the
// log-sum-exp combination
//   m = max(lse_a, lse_b), w = exp(lse - m),
//   O = (w_a O_a + w_b O_b) / (w_a + w_b),  lse = m + log(w_a + w_b),
// where a partial with lse = -inf covers no key and contributes nothing.
//
// gfx950 design: a (token, head) row of head_dim bf16 values belongs to 16
// lanes (4 rows per wavefront); lane j moves the row's 16-byte chunks j,
// j + 16, ... with 16-byte loads and stores.  Every lane of a row reads the
// row's old lse before the row's lane 0 writes the new one, and a row never
// spans two wavefronts, so the in-place update needs no synchronisation.
// The weights are computed once per row in fp32 (expf / logf), the output
// rounded once to bf16.
#include <cmath>

#include "mla_common.hpp"

namespace mla {
namespace {

constexpr int kRowLanes = 16;
constexpr int kRowsPerBlock = 256 / kRowLanes;

struct MergeArgs {
  uint16_t* out;
  int64_t o_ts, o_hs;
  float* lse;
  int64_t l_hs, l_ts;
  const uint16_t* part;
  int64_t p_ts, p_hs;
  const float* plse;
  int64_t pl_hs, pl_ts;
  const uint8_t* no_context;
  FastDiv heads;
  uint32_t rows;    // num_tokens * num_heads
  uint32_t chunks;  // 16-byte chunks per row (head_dim / 8)
};

// 16-byte load that does not keep its line in the caches: a chunk's partial
// is read once (126 -> 124.5 us at 16384 x 64 x 128); the accumulator, read
// and written back, keeps ordinary loads.
__device__ __forceinline__ uint4 ld16_once(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// bf16 pair -> weighted fp32 sum -> bf16 pair, skipping a term whose weight
// is exactly zero (that partial covers no key; its values may be anything).
__device__ __forceinline__ uint32_t merge2(uint32_t a, uint32_t b, float ca, float cb,
                                           bool use_a, bool use_b) {
  float lo = 0.0f, hi = 0.0f;
  if (use_a) {
    lo = ca * bf16_lo(a);
    hi = ca * bf16_hi(a);
  }
  if (use_b) {
    lo = __builtin_fmaf(cb, bf16_lo(b), lo);
    hi = __builtin_fmaf(cb, bf16_hi(b), hi);
  }
  return cvt_bf16x2(lo, hi);
}

template <int kMode>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
  const int j = threadIdx.x % kRowLanes;
  for (uint32_t row = blockIdx.x * kRowsPerBlock + threadIdx.x / kRowLanes; row < a.rows;
       row += gridDim.x * kRowsPerBlock) {
    const uint32_t t = fdiv(row, a.heads);
    const uint32_t h = row - t * a.heads.d;
    const float lp = a.plse[int64_t(h) * a.pl_hs + int64_t(t) * a.pl_ts];
    float* lse = a.lse + int64_t(h) * a.l_hs + int64_t(t) * a.l_ts;
    uint16_t* o = a.out + int64_t(t) * a.o_ts + int64_t(h) * a.o_hs;
    if constexpr (kMode == MLA_MERGE_INIT_WRITTEN) {
      if (j == 0) *lse = lp;
      continue;
    }
    const uint16_t* p = a.part + int64_t(t) * a.p_ts + int64_t(h) * a.p_hs;
    if constexpr (kMode == MLA_MERGE_INIT_COPY) {
      for (uint32_t c = j; c < a.chunks; c += kRowLanes) st16(o + 8 * c, ld16(p + 8 * c));
      if (j == 0) *lse = lp;
      continue;
    }
    // MLA_MERGE_ACCUMULATE
    const float la = *lse;
    const float m = fmaxf(la, lp);
    const bool empty = m == -INFINITY;       // neither partial covers a key
    const float wa = empty ? 0.0f : expf(la - m);
    const float wb = empty ? 0.0f : expf(lp - m);
    const float sum = wa + wb;
    const float ca = empty ? 0.0f : wa / sum;
    const float cb = empty ? 0.0f : wb / sum;
    const bool use_a = wa != 0.0f, use_b = wb != 0.0f;
    for (uint32_t c = j; c < a.chunks; c += kRowLanes) {
      const uint4 x = ld16(o + 8 * c);
      const uint4 y = ld16_once(p + 8 * c);
      st16(o + 8 * c, make_uint4(merge2(x.x, y.x, ca, cb, use_a, use_b),
                                 merge2(x.y, y.y, ca, cb, use_a, use_b),
                                 merge2(x.z, y.z, ca, cb, use_a, use_b),
                                 merge2(x.w, y.w, ca, cb, use_a, use_b)));
    }
    if (j == 0) *lse = empty ? -INFINITY : m + logf(sum);
  }
}

__global__ __launch_bounds__(256) void neutralize_kernel(const MergeArgs a) {
  const int j = threadIdx.x % kRowLanes;
  for (uint32_t row = blockIdx.x * kRowsPerBlock + threadIdx.x / kRowLanes; row < a.rows;
       row += gridDim.x * kRowsPerBlock) {
    const uint32_t t = fdiv(row, a.heads);
    if (!a.no_context[t]) continue;
    const uint32_t h = row - t * a.heads.d;
    uint16_t* o = a.out + int64_t(t) * a.o_ts + int64_t(h) * a.o_hs;
    for (uint32_t c = j; c < a.chunks; c += kRowLanes) st16(o + 8 * c, make_uint4(0, 0, 0, 0));
    if (j == 0) a.lse[int64_t(h) * a.l_hs + int64_t(t) * a.l_ts] = -INFINITY;
  }
}

// Shared checks of the accumulator's shape, alignment and sizes.
int32_t check_acc(const char* fn, const void* out, int64_t o_ts, int64_t o_hs, const float* lse,
                  int64_t T, int64_t H, int64_t D) {
  if (T < 0 || H < 0 || D < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
  if (T == 0 || H == 0 || D == 0) return MLA_OK;
  if (!out || !lse) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL out or lse", fn);
  if (D % 8 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "%s: head_dim must be a multiple of 8", fn);
  if (!aligned16(out) || !bytes16(o_ts, 2) || !bytes16(o_hs, 2) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(MLA_ERR_MISALIGNED, "%s: output rows must be 16-byte aligned, lse 4-byte", fn);
  if (T * H >= (int64_t(1) << 31) - kRowsPerBlock || H > 0x7FFFFFFF)
    return fail(MLA_ERR_UNSUPPORTED, "%s: too many rows for one launch", fn);
  return MLA_OK;
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int32_t mla_ctx_merge_chunk(void* out, int64_t out_tok_stride, int64_t out_head_stride,
                                       float* lse, int64_t lse_head_stride, int64_t lse_tok_stride,
                                       const void* part, int64_t part_tok_stride,
                                       int64_t part_head_stride, const float* part_lse,
                                       int64_t part_lse_head_stride, int64_t part_lse_tok_stride,
                                       int64_t num_tokens, int64_t num_heads, int64_t head_dim,
                                       int32_t mode, mla_stream_t stream) {
  static const char* fn = "mla_ctx_merge_chunk";
  clear_error();
  if (mode != MLA_MERGE_INIT_COPY && mode != MLA_MERGE_INIT_WRITTEN &&
      mode != MLA_MERGE_ACCUMULATE)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: unknown mode %d", fn, mode);
  int32_t st = check_acc(fn, out, out_tok_stride, out_head_stride, lse, num_tokens, num_heads,
                         head_dim);
  if (st != MLA_OK) return st;
  if (num_tokens == 0 || num_heads == 0 || head_dim == 0) return MLA_OK;
  if (!part_lse) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL part_lse", fn);
  if (mode != MLA_MERGE_INIT_WRITTEN) {
    if (!part) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL part", fn);
    if (!aligned16(part) || !bytes16(part_tok_stride, 2) || !bytes16(part_head_stride, 2))
      return fail(MLA_ERR_MISALIGNED, "%s: partial rows must be 16-byte aligned", fn);
  }
  if (mode == MLA_MERGE_ACCUMULATE && part == out)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "%s: a continuation chunk is merged from its own buffer; its output cannot "
                "already sit in the accumulator", fn);
  if (reinterpret_cast<uintptr_t>(part_lse) & 3u)
    return fail(MLA_ERR_MISALIGNED, "%s: part_lse must be 4-byte aligned", fn);
  MergeArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.o_ts = out_tok_stride;
  a.o_hs = out_head_stride;
  a.lse = lse;
  a.l_hs = lse_head_stride;
  a.l_ts = lse_tok_stride;
  a.part = static_cast<const uint16_t*>(part);
  a.p_ts = part_tok_stride;
  a.p_hs = part_head_stride;
  a.plse = part_lse;
  a.pl_hs = part_lse_head_stride;
  a.pl_ts = part_lse_tok_stride;
  a.no_context = nullptr;
  a.heads = make_fastdiv(static_cast<uint32_t>(num_heads));
  a.rows = static_cast<uint32_t>(num_tokens * num_heads);
  a.chunks = static_cast<uint32_t>(head_dim / 8);
  const int64_t blocks = ceil_div(num_tokens * num_heads, kRowsPerBlock);
  auto s = static_cast<hipStream_t>(stream);
  if (mode == MLA_MERGE_ACCUMULATE)
    launch(merge_kernel<MLA_MERGE_ACCUMULATE>, dim3(blocks), dim3(256), 0, s, a);
  else if (mode == MLA_MERGE_INIT_COPY)
    launch(merge_kernel<MLA_MERGE_INIT_COPY>, dim3(blocks), dim3(256), 0, s, a);
  else
    launch(merge_kernel<MLA_MERGE_INIT_WRITTEN>, dim3(blocks), dim3(256), 0, s, a);
  return launch_status(fn);
}

extern "C" int32_t mla_ctx_neutralize_partials(void* out, int64_t out_tok_stride,
                                               int64_t out_head_stride, float* lse,
                                               int64_t lse_head_stride, int64_t lse_tok_stride,
                                               const uint8_t* no_context, int64_t num_tokens,
                                               int64_t num_heads, int64_t head_dim,
                                               mla_stream_t stream) {
  static const char* fn = "mla_ctx_neutralize_partials";
  clear_error();
  int32_t st = check_acc(fn, out, out_tok_stride, out_head_stride, lse, num_tokens, num_heads,
                         head_dim);
  if (st != MLA_OK) return st;
  if (num_tokens == 0 || num_heads == 0 || head_dim == 0) return MLA_OK;
  if (!no_context) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL no_context", fn);
  MergeArgs a{};
  a.out = static_cast<uint16_t*>(out);
  a.o_ts = out_tok_stride;
  a.o_hs = out_head_stride;
  a.lse = lse;
  a.l_hs = lse_head_stride;
  a.l_ts = lse_tok_stride;
  a.no_context = no_context;
  a.heads = make_fastdiv(static_cast<uint32_t>(num_heads));
  a.rows = static_cast<uint32_t>(num_tokens * num_heads);
  a.chunks = static_cast<uint32_t>(head_dim / 8);
  const int64_t blocks = ceil_div(num_tokens * num_heads, kRowsPerBlock);
  launch(neutralize_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return launch_status(fn);
}
