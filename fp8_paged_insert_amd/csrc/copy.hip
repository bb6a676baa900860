// copy.hip -- a plain device-to-device copy with the launch shape of the
// library's streaming kernels (one 16-byte chunk per thread over the full
// grid, loads that bypass the last-level cache, streaming stores).  It is a
// measurement aid: the rate it reaches on a given size is what a
// bandwidth-bound kernel of this library can expect at that size, the
// ceiling its other kernels are compared with.
#include "mla_common.hpp"

namespace mla {
namespace {

__global__ __launch_bounds__(256) void stream_copy_kernel(uint4* dst, const uint4* src,
                                                          int64_t chunks) {
  const int64_t i = blockIdx.x * int64_t(256) + threadIdx.x;
  if (i < chunks) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i));
    st16<true>(dst + i, make_uint4(v.x, v.y, v.z, v.w));
  }
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int32_t mla_stream_copy(void* dst, const void* src, int64_t bytes,
                                   mla_stream_t stream) {
  static const char* fn = "mla_stream_copy";
  clear_error();
  if (bytes < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
  if (bytes == 0) return MLA_OK;
  if (!dst || !src) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL dst or src", fn);
  if (!aligned16(dst) || !aligned16(src) || (bytes & 15))
    return fail(MLA_ERR_MISALIGNED, "%s: addresses and size must be multiples of 16 bytes", fn);
  const int64_t chunks = bytes / 16;
  const int64_t blocks = ceil_div(chunks, 256);
  if (blocks > 0x7FFFFFFF) return fail(MLA_ERR_UNSUPPORTED, "%s: too large for one launch", fn);
  const char* d = static_cast<const char*>(dst);
  const char* s = static_cast<const char*>(src);
  if (d < s + bytes && s < d + bytes)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: dst and src overlap", fn);
  launch(stream_copy_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
         static_cast<hipStream_t>(stream), static_cast<uint4*>(dst),
         static_cast<const uint4*>(src), chunks);
  return launch_status(fn);
}
