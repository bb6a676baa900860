// transpose.hip -- bf16 matrix transpose for weight preparation.
//
// Page: "PR #50585 完整报告", 实现拆解 item 2: the fused KV projection is a
// MergedColumnParallelLinear whose weight is held as [out, in]; a caller that
// holds the same weight as the [in, out] matrix the projection multiplies
// by (the fused context-KV workload states it that way) converts it once with
// this entry point -- a weight is constant across calls, so the conversion is
// a preparation step, not a step of every projection.
//
// gfx950 design: 64 x 64 tiles through LDS; 16-byte global loads along the
// source rows and 16-byte global stores along the destination rows (every
// global access is a full contiguous chunk); the tile's LDS rows are padded
// by 16 bytes so the column reads of the transposed store phase spread over
// the banks.
#include "mla_common.hpp"

namespace mla {
namespace {

constexpr int kTile = 64;
constexpr int kPadRow = kTile + 8;  // bf16 elements per LDS row (144 bytes)

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* src, int64_t lds_,
                                                             uint16_t* dst, int64_t ldd,
                                                             int32_t rows, int32_t cols) {
  __shared__ __align__(16) uint16_t tile[kTile * kPadRow];
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  // load: 64 rows x 8 chunks of 8 values, both of a thread's loads issued
  // before either LDS write
  const int lrow = threadIdx.x >> 3, lch = threadIdx.x & 7;
  const bool cin = c0 + lch * 8 < cols;
  uint4 lv[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (cin && r0 + lrow + 32 * k < rows)
      lv[k] = ld16(src + int64_t(r0 + lrow + 32 * k) * lds_ + c0 + lch * 8);
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (cin && r0 + lrow + 32 * k < rows)
      *reinterpret_cast<uint4*>(&tile[(lrow + 32 * k) * kPadRow + lch * 8]) = lv[k];
  __syncthreads();
  // store: destination row = source column, 8 chunks of 8 source rows each
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = threadIdx.x + 256 * k;
    const int col = c >> 3, ch = c & 7;
    if (c0 + col < cols && r0 + ch * 8 < rows) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = uint32_t(tile[(ch * 8 + 2 * i) * kPadRow + col]) |
               (uint32_t(tile[(ch * 8 + 2 * i + 1) * kPadRow + col]) << 16);
      st16(dst + int64_t(c0 + col) * ldd + r0 + ch * 8, make_uint4(w[0], w[1], w[2], w[3]));
    }
  }
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int32_t mla_transpose_bf16(const void* src, int64_t rows, int64_t cols,
                                      int64_t src_row_stride, void* dst, int64_t dst_row_stride,
                                      mla_stream_t stream) {
  static const char* fn = "mla_transpose_bf16";
  clear_error();
  if (rows < 0 || cols < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
  if (rows == 0 || cols == 0) return MLA_OK;
  if (!src || !dst) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL src or dst", fn);
  if (src_row_stride < cols || dst_row_stride < rows)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: row strides smaller than the rows", fn);
  if (rows % 8 || cols % 8)
    return fail(MLA_ERR_UNSUPPORTED, "%s: rows and cols must be multiples of 8", fn);
  if (!aligned16(src) || !aligned16(dst) || !bytes16(src_row_stride, 2) ||
      !bytes16(dst_row_stride, 2))
    return fail(MLA_ERR_MISALIGNED, "%s: addresses and row strides must be 16-byte aligned", fn);
  if (rows > 0x7FFFFFFF - kTile || cols > 0x7FFFFFFF - kTile)
    return fail(MLA_ERR_UNSUPPORTED, "%s: sizes beyond 2^31", fn);
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  const int64_t sbytes = ((rows - 1) * src_row_stride + cols) * 2;
  const int64_t dbytes = ((cols - 1) * dst_row_stride + rows) * 2;
  if (d < s + sbytes && s < d + dbytes)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: src and dst overlap", fn);
  const dim3 grid(static_cast<uint32_t>(ceil_div(cols, kTile)),
                  static_cast<uint32_t>(ceil_div(rows, kTile)));
  if (grid.y > 65535)
    return fail(MLA_ERR_UNSUPPORTED, "%s: more than 65535 tile rows", fn);
  launch(transpose_bf16_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
         static_cast<const uint16_t*>(src), src_row_stride, static_cast<uint16_t*>(dst),
         dst_row_stride, static_cast<int32_t>(rows), static_cast<int32_t>(cols));
  return launch_status(fn);
}
