// mla_common.hpp -- shared device helpers and host plumbing of the gfx950
// MLA latent-KV library (number formats, vector access, error state, launch
// geometry).  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "../../include/mla_kv.h"

namespace mla {

// ===========================================================================
// Host side
// ===========================================================================

// Records a formatted message for mla_last_error() and returns `status`.
int32_t fail(int32_t status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Compute units of the current device, queried once per device.
int cu_count();

// Status after a launch: MLA_ERR_DEVICE if the runtime reports an error.
int32_t launch_status(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool bytes16(int64_t elems, int64_t elem_bytes) { return ((elems * elem_bytes) & 15) == 0; }

// Default grid cap for grid-stride kernels: enough workgroups to keep every
// compute unit busy with several resident workgroups.
inline int64_t default_grid_cap() { return int64_t(cu_count()) * 16; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool is_fp8(int32_t dt) { return dt == MLA_KV_FP8_E4M3; }

// Checks the cache-dtype / scale pairing shared by the insert and epilogue
// ([P3] "PR #55356 完整报告", 关键源码片段, cache_kernels.cu host checks).
int32_t check_cache_dtype(const char* fn, int32_t dt, const float* scales);

// ===========================================================================
// Device side
// ===========================================================================

// bf16 halves of a 32-bit word, widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN 0x7FC0 with sign.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? (((u >> 16) & 0x8000u) | 0x7FC0u) : r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Correctly rounded fp32 quotient x / s from r = RN(1/s): q0 = RN(x*r) is
// within one ulp, the remainder x - q0*s is exact under FMA, and one
// correction step rounds correctly (Markstein).  Checked exhaustively on the
// CPU for every bf16 significand against every fp32 significand of s.  For
// zeros, infinities, NaN and fp32 subnormals q0 is kept: those quotients all
// encode to a signed zero, a saturated +-448 or NaN in e4m3fn, and q0 carries
// the right sign (the correction would turn -0 into +0 and Inf into NaN).
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  const float q1 = __builtin_fmaf(e, r, q0);
  // v_cmp_class mask: snan|qnan|-inf|-denorm|-zero|+zero|+denorm|+inf
  return __builtin_amdgcn_classf(q0, 0x2F7) ? q0 : q1;
}

// Saturate finite values (and +-Inf) to the e4m3fn range; NaN passes through.
__device__ __forceinline__ float sat448(float q) {
  const float c = __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
  return (q != q) ? q : c;
}

// Byte k of w := the e4m3fn NaN code carrying the sign of x.
__device__ __forceinline__ uint32_t put_nan(uint32_t w, float x, int k) {
  const uint32_t code = 0x7Fu | ((__float_as_uint(x) >> 24) & 0x80u);
  return (w & ~(0xFFu << (8 * k))) | (code << (8 * k));
}

// Four fp32 values -> four e4m3fn codes (byte k = value k), RNE, saturating
// at +-448.  On gfx950 the packed converter produces the OCP e4m3fn
// encoding; its NaN output does not keep the input's sign, so NaN bytes are
// rewritten (a branch that no lane takes unless an input is NaN).
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
  uint32_t r = static_cast<uint32_t>(w);
  if (__builtin_expect((a != a) | (b != b) | (c != c) | (d != d), 0)) {
    if (a != a) r = put_nan(r, a, 0);
    if (b != b) r = put_nan(r, b, 1);
    if (c != c) r = put_nan(r, c, 2);
    if (d != d) r = put_nan(r, d, 3);
  }
  return r;
}

// 8 bf16 (one uint4) -> 8 e4m3fn codes (uint2), dividing by s (r = RN(1/s)).
template <bool kScaled>
__device__ __forceinline__ uint2 quant8(uint4 v, float s, float r) {
  float f[8];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
  if constexpr (kScaled) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = div_by_scale(f[i], s, r);
  }
  return make_uint2(cvt4_e4m3(f[0], f[1], f[2], f[3]), cvt4_e4m3(f[4], f[5], f[6], f[7]));
}

// 16 bf16 (two uint4) -> 16 e4m3fn codes (uint4).
template <bool kScaled>
__device__ __forceinline__ uint4 quant16(uint4 a, uint4 b, float s, float r) {
  const uint2 lo = quant8<kScaled>(a, s, r);
  const uint2 hi = quant8<kScaled>(b, s, r);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Four e4m3fn codes (one word) -> four fp32 values (exact).
__device__ __forceinline__ void dec4_e4m3(uint32_t w, float* out) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// Division of n < 2^31 by a fixed divisor d >= 1 with one high multiply:
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l.
// Checked on the CPU against the hardware divide.
struct FastDiv {
  uint32_t d, m, l;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((((uint64_t(1) << l) - d) << 32) / d) + 1;
  return FastDiv{d, static_cast<uint32_t>(m), l};
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  return (__umulhi(n, f.m) + n) >> f.l;
}

// Vector loads / stores of 16 bytes.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }

}  // namespace mla
