// copy.hip -- measurement aids, not steps of the path.
//  * mla_stream_copy: a plain device-to-device copy with the launch shape of
//    the library's streaming kernels (one 16-byte chunk per thread over the
//    full grid, loads that bypass the last-level cache, streaming stores):
//    the rate it reaches on a given size is what a bandwidth-bound kernel of
//    this library can expect at that size, the ceiling its other kernels are
//    compared with.
//  * mla_stream_mix: the same launch shape with 2 to 4 loads per store (each
//    16-byte output chunk the XOR of that many input chunks): the ceiling
//    for a kernel with that read:write mix (the fp8 pack reads twice the
//    bytes it writes).
//  * mla_mfma_rate: one workgroup of 4 wavefronts per compute unit, each
//    wavefront issuing a long run of v_mfma_f32_32x32x16_bf16 on a 4 x 3
//    tile of accumulators (the projection's) with operands that change every
//    step, between two reads of the shader clock and of the 100 MHz
//    real-time counter: the matrix cores' issue rate in cycles and the clock
//    they hold under full MFMA load, the ceiling the projection is compared
//    with.
#include "mla_common.hpp"

namespace mla {
namespace {

// dst chunk i = XOR of src chunks kReads i .. kReads i + kReads - 1 (a plain
// copy for kReads = 1): kReads x 16 bytes read per 16 bytes written.
template <int kReads>
__global__ __launch_bounds__(256) void stream_copy_kernel(uint4* dst, const uint4* src,
                                                          int64_t chunks) {
  const int64_t i = blockIdx.x * int64_t(256) + threadIdx.x;
  if (i < chunks) {
    const u32x4* s = reinterpret_cast<const u32x4*>(src) + i * kReads;
    u32x4 v = __builtin_nontemporal_load(s);
#pragma unroll
    for (int r = 1; r < kReads; ++r) v ^= __builtin_nontemporal_load(s + r);
    st16<true>(dst + i, make_uint4(v.x, v.y, v.z, v.w));
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Operands like the projection's: a wavefront's 4 x 3 tile of accumulators,
// each step multiplying 4 A fragments by 3 B fragments, with two fragment
// sets used on alternate steps; values in +-[1, 2) with pseudo-random
// significands, so the matrix cores switch like they do on real data (the
// clock they hold under load depends on it).
__device__ __forceinline__ bf16x8_t rate_operand(uint32_t seed) {
  bf16x8_t v;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    seed = seed * 1664525u + 1013904223u;
    const uint32_t bits = 0x3F80u | ((seed >> 9) & 0x7Fu) | ((seed >> 16) & 0x8000u);
    v[i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(bits));
  }
  return v;
}

__global__ __launch_bounds__(256) void mfma_rate_kernel(uint64_t* clocks, int32_t iters) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t seed = 0x9E3779B9u * static_cast<uint32_t>(threadIdx.x + 1) + blockIdx.x;
  bf16x8_t fa[2][4], fb[2][3];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[s][i] = rate_operand(seed + 101u * (s * 7 + i));
#pragma unroll
    for (int j = 0; j < 3; ++j) fb[s][j] = rate_operand(seed + 101u * (s * 7 + 4 + j));
  }
  f32x16_t acc[4][3];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  __syncthreads();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int32_t it = 0; it < iters; it += 2) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    uint64_t* p = clocks + (blockIdx.x * 4 + wave) * 4;
    p[0] = c0;
    p[1] = c1;
    p[2] = r0;
    p[3] = r1;
  }
  if (!(sum == sum)) clocks[0] = 0;  // never true (the sums are finite); keeps the MFMAs
}

int32_t stream_launch(const char* fn, void* dst, const void* src, int64_t dst_bytes,
                      int32_t reads, mla_stream_t stream) {
  if (dst_bytes < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
  if (reads < 1 || reads > 4)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: reads_per_write must be 1 to 4", fn);
  if (dst_bytes == 0) return MLA_OK;
  if (!dst || !src) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL dst or src", fn);
  if (!aligned16(dst) || !aligned16(src) || (dst_bytes & 15))
    return fail(MLA_ERR_MISALIGNED, "%s: addresses and size must be multiples of 16 bytes", fn);
  const int64_t chunks = dst_bytes / 16;
  const int64_t blocks = ceil_div(chunks, 256);
  if (blocks > 0x7FFFFFFF) return fail(MLA_ERR_UNSUPPORTED, "%s: too large for one launch", fn);
  const char* d = static_cast<const char*>(dst);
  const char* s = static_cast<const char*>(src);
  if (d < s + dst_bytes * reads && s < d + dst_bytes)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: dst and src overlap", fn);
  const dim3 g(static_cast<uint32_t>(blocks)), b(256);
  auto st = static_cast<hipStream_t>(stream);
  auto* o = static_cast<uint4*>(dst);
  auto* i = static_cast<const uint4*>(src);
  switch (reads) {
    case 1: launch(stream_copy_kernel<1>, g, b, 0, st, o, i, chunks); break;
    case 2: launch(stream_copy_kernel<2>, g, b, 0, st, o, i, chunks); break;
    case 3: launch(stream_copy_kernel<3>, g, b, 0, st, o, i, chunks); break;
    default: launch(stream_copy_kernel<4>, g, b, 0, st, o, i, chunks); break;
  }
  return launch_status(fn);
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int32_t mla_stream_copy(void* dst, const void* src, int64_t bytes,
                                   mla_stream_t stream) {
  clear_error();
  return stream_launch("mla_stream_copy", dst, src, bytes, 1, stream);
}

extern "C" int32_t mla_stream_mix(void* dst, const void* src, int64_t dst_bytes,
                                  int32_t reads_per_write, mla_stream_t stream) {
  clear_error();
  return stream_launch("mla_stream_mix", dst, src, dst_bytes, reads_per_write, stream);
}

extern "C" int32_t mla_mfma_rate(int64_t iters, uint64_t* clocks, int64_t clock_words,
                                 mla_stream_t stream) {
  static const char* fn = "mla_mfma_rate";
  clear_error();
  if (iters <= 0 || iters > (int64_t(1) << 20) || (iters & 1))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: iters must be even, in [2, 2^20]", fn);
  if (!clocks) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: clocks is NULL", fn);
  const int64_t cus = cu_count();
  if (clock_words < 16 * cus)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: clocks holds %lld words, %lld needed", fn,
                (long long)clock_words, (long long)(16 * cus));
  launch(mfma_rate_kernel, dim3(static_cast<uint32_t>(cus)), dim3(256), 0,
         static_cast<hipStream_t>(stream), clocks, static_cast<int32_t>(iters));
  return launch_status(fn);
}
