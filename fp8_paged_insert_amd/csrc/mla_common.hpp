// mla_common.hpp -- shared device helpers and host plumbing of the gfx950
// MLA latent-KV library (number formats, vector access, error state, launch
// geometry).  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_ext.h>
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

// The timing events set by mla_set_launch_events for this thread, if any;
// taking them clears them.
bool take_launch_events(hipEvent_t* start, hipEvent_t* stop);

// Every kernel of the library is enqueued through here: a plain launch, or,
// when the caller armed timing events, one whose start and stop events
// bracket the kernel's own execution.
template <typename Kernel, typename... Args>
void launch(Kernel kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t stream,
            Args... args) {
  hipEvent_t e0, e1;
  if (take_launch_events(&e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool bytes16(int64_t elems, int64_t elem_bytes) { return ((elems * elem_bytes) & 15) == 0; }

// Default grid cap for grid-stride kernels: enough workgroups to keep every
// compute unit busy with several resident workgroups.
inline int64_t default_grid_cap() { return int64_t(cu_count()) * 16; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool is_fp8(int32_t dt) { return dt == MLA_KV_FP8_E4M3 || dt == MLA_KV_FP8_E5M2; }

// Element formats of a cache (and template parameter of the kernels that
// write or read one).
enum CacheFmt { kFmtBf16 = 0, kFmtE4M3 = 1, kFmtE5M2 = 2 };
inline int cache_fmt(int32_t dt) {
  return dt == MLA_KV_FP8_E4M3 ? kFmtE4M3 : dt == MLA_KV_FP8_E5M2 ? kFmtE5M2 : kFmtBf16;
}

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

// fp32 -> bf16 with the gfx950 converter (round to nearest even), two at a
// time.  Used where a NaN's payload and sign are not part of the contract.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// float64 -> bf16 bits, rounded once to nearest even (as if directly): the
// conversion to fp32 is made round-to-odd (an inexact result is truncated
// toward zero and its last bit set), so the second rounding, fp32 -> bf16,
// cannot land on a tie the first one created.  NaN -> quiet NaN with sign.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double d) {
  const float f = static_cast<float>(d);
  uint32_t u = __float_as_uint(f);
  const double back = static_cast<double>(f);
  if (back != d && d == d) {
    if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1u;  // toward zero
    u |= 1u;
  }
  return f32_to_bf16_bits(__uint_as_float(u));
}

// Rotary embedding of one lane's 4 values of a rope row, non-interleaved
// pairs (i, i + P/2) ("PR #50585 完整报告", 关键源码片段: RoPE of k_pe at the
// token's position; the formula itself is elided there):
//   first half  (x = x_i,       p = x_{i+P/2}):  y_i       = x_i cos_i - x_{i+P/2} sin_i
//   second half (x = x_{i+P/2}, p = x_i):        y_{i+P/2} = x_{i+P/2} cos_i + x_i sin_i
// rounded once to bf16.  The table holds each cos / sin as an fp32 pair
// hi + lo (hi = RN32(v), lo = RN32(v - hi): about 48 significant bits).
// Fast path, fp32 with the hi values: y32 = fma(x, c, -+ p s) is within
// B = 2^-22 (|x| + |p|) of the exact rotation (table rounding 2^-24 per
// coefficient, the product and the fma 2^-24 each).  The bf16 rounding
// boundary nearest to y32 is the midpoint of y32's bf16 interval (the other
// boundaries are a bf16 ulp away); when y32 lies farther than B from it,
// RNE(y32) is the correctly rounded result.  That test also catches the
// products nearly cancelling (then B exceeds half a bf16 ulp of y32, and no
// value is farther than that from the midpoint).  Otherwise the whole
// wavefront takes the exact path (a uniform branch, taken by about one
// wavefront in a hundred): the rotation in float64 with hi + lo, then one
// correct rounding to bf16.  In the helpers below x, p, c, s are the lane's
// 4 values, their partners and the 4 cos / sin hi values.

// One rotated value in float64 from the exact table values hi + lo (each
// operation rounded on its own, then one correct rounding to bf16).
__device__ __forceinline__ uint32_t rope1_exact(float x, float p, float ch, float cl, float sh,
                                                float sl, bool first) {
#pragma clang fp contract(off)
  const double c = static_cast<double>(ch) + static_cast<double>(cl);  // exact
  const double s = static_cast<double>(sh) + static_cast<double>(sl);  // exact
  const double u = static_cast<double>(x) * c;
  const double v = static_cast<double>(p) * s;
  return f64_to_bf16_bits(first ? u - v : u + v);
}

// The fast path of the four values: the fp32 rotations and whether every
// one of them is known to round correctly (see above).
struct Rope4Fast {
  float y[4];
  bool safe;
};
__device__ __forceinline__ Rope4Fast rope4_fast(const float* x, const float* p, const float* c,
                                                const float* s, bool first) {
  Rope4Fast r;
  r.safe = true;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float ps = p[e] * s[e];
    r.y[e] = __builtin_fmaf(x[e], c[e], first ? -ps : ps);
    const float bound = 0x1p-22f * (__builtin_fabsf(x[e]) + __builtin_fabsf(p[e]));
    const float mid = __uint_as_float((__float_as_uint(r.y[e]) & 0xFFFF0000u) | 0x8000u);
    // false for NaN (and for an infinite bound), which then takes the exact path
    r.safe = r.safe && __builtin_fabsf(r.y[e] - mid) > bound;
  }
  return r;
}

__device__ __forceinline__ uint2 rope4_exact(const float* x, const float* p, const float* c,
                                             const float* s, bool first, uint4 cl, uint4 sl) {
  const float cls[4] = {__uint_as_float(cl.x), __uint_as_float(cl.y), __uint_as_float(cl.z),
                        __uint_as_float(cl.w)};
  const float sls[4] = {__uint_as_float(sl.x), __uint_as_float(sl.y), __uint_as_float(sl.z),
                        __uint_as_float(sl.w)};
  uint32_t b[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) b[e] = rope1_exact(x[e], p[e], c[e], cls[e], s[e], sls[e], first);
  return make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
}

// lo_c / lo_s: where the lo values of the lane's angles sit in the table;
// read only when the exact path runs.
__device__ __forceinline__ uint2 rope4(const float* x, const float* p, const float* c,
                                       const float* s, bool first, const float* lo_c,
                                       const float* lo_s) {
  const Rope4Fast r = rope4_fast(x, p, c, s, first);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(!r.safe) != 0, 0))
    return rope4_exact(x, p, c, s, first, *reinterpret_cast<const uint4*>(lo_c),
                       *reinterpret_cast<const uint4*>(lo_s));
  // no NaN reaches here, so the hardware converter (RNE) serves
  return make_uint2(cvt_bf16x2(r.y[0], r.y[1]), cvt_bf16x2(r.y[2], r.y[3]));
}

// rope4 with the lo values already in registers, loaded together with the
// hi ones: for a latency-bound caller (the context epilogue) the rare exact
// path then adds no dependent load to its wavefront.
__device__ __forceinline__ uint2 rope4v(const float* x, const float* p, const float* c,
                                        const float* s, bool first, uint4 cl, uint4 sl) {
  const Rope4Fast r = rope4_fast(x, p, c, s, first);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(!r.safe) != 0, 0))
    return rope4_exact(x, p, c, s, first, cl, sl);
  return make_uint2(cvt_bf16x2(r.y[0], r.y[1]), cvt_bf16x2(r.y[2], r.y[3]));
}


// ---------------------------------------------------------------------------
// bf16 (or fp16) -> fp8 with a per-tensor dequantisation scale s:
//   code = fp8_RNE(fl32(x) / s), saturating at the format's largest finite
//   value (e4m3fn: +-448; e5m2: +-57344), NaN -> 0x7F | sign (a NaN code in
//   both formats).
// Exactness argument, step by step:
//  * quotient: r = RN(1/s) once; q0 = RN(x*r) is within one ulp of x/s, the
//    remainder x - q0*s is exact under FMA, and q = RN(q0 + rem*r) is the
//    correctly rounded x/s (Markstein).  tests/quotient_exactness.c checks
//    this on the host for every bf16 and every fp16 significand against
//    every fp32 significand of s, and for every finite bf16 value against
//    scales of every exponent: wherever the quotient can reach an fp8 code it
//    is exact for 2^-85 <= |s| < 2^126 (outside that range the remainder or
//    r leaves the normal range; such scales are a stated precondition).
//    Where the step degenerates -- x = +-0 (the sum of signed zeros
//    gives +0), x = +-Inf or an overflowing quotient (Inf - Inf gives NaN) --
//    only the sign of the final code can be wrong, and it is rewritten below.
//  * saturation: v_med3 clamps to [-max, max]; it also maps NaN onto a
//    bound, which is what turns the degenerate Inf cases into +-max.
//  * the packed converters round to nearest even in OCP e4m3fn
//    (v_cvt_pk_fp8_f32) and OCP e5m2 (v_cvt_pk_bf8_f32).
//  * sign: every code's sign bit is set to sign(x) xor sign(s) (v_perm
//    gathers the 16-bit values' high bytes, v_bfi merges them) -- exact for
//    all non-NaN inputs, including zeros, subnormal quotients and saturation.
//  * NaN inputs (rare; a branch no lane takes otherwise) get 0x7F | sign(x).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  return __builtin_fmaf(e, r, q0);
}

template <bool kE5M2>
__device__ __forceinline__ float sat_fp8(float q) {
  constexpr float kMax = kE5M2 ? 57344.0f : 448.0f;
  return __builtin_amdgcn_fmed3f(q, -kMax, kMax);
}

// Codes of 4 clamped values (byte k = value k).
template <bool kE5M2>
__device__ __forceinline__ uint32_t cvt4_raw(float a, float b, float c, float d) {
  int w;
  if constexpr (kE5M2) {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  }
  return static_cast<uint32_t>(w);
}

// Byte k of w := NaN code with the sign of x.
__device__ __forceinline__ uint32_t put_nan(uint32_t w, float x, int k) {
  const uint32_t code = 0x7Fu | ((__float_as_uint(x) >> 24) & 0x80u);
  return (w & ~(0xFFu << (8 * k))) | (code << (8 * k));
}

// IEEE fp16 halves of a word as fp32 (exact).
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// 8 16-bit values (one uint4: element 2i in the low half of word i) -> 8
// codes.  kF16 reads them as IEEE fp16, else as bf16; both formats keep the
// sign in bit 15, so the sign overwrite below serves both.  kE5M2 selects
// the e5m2 code format, else e4m3fn.
// sign_flip is 0x80808080 when s < 0, else 0.
template <bool kScaled, bool kF16 = false, bool kE5M2 = false>
__device__ __forceinline__ uint2 quant8(uint4 v, float s, float r, uint32_t sign_flip) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8], q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = kF16 ? f16_lo(w[i]) : bf16_lo(w[i]);
    f[2 * i + 1] = kF16 ? f16_hi(w[i]) : bf16_hi(w[i]);
  }
  bool nan = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    nan |= f[i] != f[i];
    q[i] = sat_fp8<kE5M2>(kScaled ? div_by_scale(f[i], s, r) : f[i]);
  }
  uint32_t c0 = cvt4_raw<kE5M2>(q[0], q[1], q[2], q[3]);
  uint32_t c1 = cvt4_raw<kE5M2>(q[4], q[5], q[6], q[7]);
  // high bytes (bit 7 = sign) of elements 0-3 and 4-7
  const uint32_t s0 = __builtin_amdgcn_perm(w[1], w[0], 0x07050301u) ^ sign_flip;
  const uint32_t s1 = __builtin_amdgcn_perm(w[3], w[2], 0x07050301u) ^ sign_flip;
  c0 = (c0 & 0x7F7F7F7Fu) | (s0 & 0x80808080u);
  c1 = (c1 & 0x7F7F7F7Fu) | (s1 & 0x80808080u);
  // A wave-uniform branch (the NaN flag voted across the wavefront) keeps
  // the patch out of the straight-line path.
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(nan) != 0, 0)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (f[k] != f[k]) c0 = put_nan(c0, f[k], k);
      if (f[k + 4] != f[k + 4]) c1 = put_nan(c1, f[k + 4], k);
    }
  }
  return make_uint2(c0, c1);
}

// 4 bf16 (one uint2: element 2i in the low half of word i) -> 4 codes.
template <bool kScaled, bool kE5M2 = false>
__device__ __forceinline__ uint32_t quant4(uint2 v, float s, float r, uint32_t sign_flip) {
  const float f[4] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
  bool nan = false;
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    nan |= f[i] != f[i];
    q[i] = sat_fp8<kE5M2>(kScaled ? div_by_scale(f[i], s, r) : f[i]);
  }
  uint32_t c = cvt4_raw<kE5M2>(q[0], q[1], q[2], q[3]);
  const uint32_t sg = __builtin_amdgcn_perm(v.y, v.x, 0x07050301u) ^ sign_flip;
  c = (c & 0x7F7F7F7Fu) | (sg & 0x80808080u);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(nan) != 0, 0)) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (f[k] != f[k]) c = put_nan(c, f[k], k);
  }
  return c;
}

// 16 16-bit values (two uint4) -> 16 codes (uint4).
template <bool kScaled, bool kF16 = false, bool kE5M2 = false>
__device__ __forceinline__ uint4 quant16(uint4 a, uint4 b, float s, float r, uint32_t flip) {
  const uint2 lo = quant8<kScaled, kF16, kE5M2>(a, s, r, flip);
  const uint2 hi = quant8<kScaled, kF16, kE5M2>(b, s, r, flip);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

__device__ __forceinline__ uint32_t sign_flip_of(float s) { return s < 0.0f ? 0x80808080u : 0u; }

// Four fp8 codes (one word; e4m3fn, or e5m2 with kE5M2) -> four fp32 values
// (exact; the NaN codes' sign is not kept -- callers rebuild those).
template <bool kE5M2>
__device__ __forceinline__ void dec4_fp8(uint32_t w, float* out) {
  float2 lo, hi;
  if constexpr (kE5M2) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), true);
    lo = make_float2(a[0], a[1]);
    hi = make_float2(b[0], b[1]);
  } else {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
    lo = make_float2(a[0], a[1]);
    hi = make_float2(b[0], b[1]);
  }
  out[0] = lo.x;
  out[1] = lo.y;
  out[2] = hi.x;
  out[3] = hi.y;
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

// Vector loads / stores.  kStream selects non-temporal (streaming) stores for
// outputs that no later step of the same kernel reads.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Every output of the library lives in device memory, so stores go through
// the global address space.  A pointer the compiler cannot trace to a kernel
// argument (a cache base read from a pointer table, an address built from
// 64-bit integer offsets) would otherwise give flat stores, and while a flat
// access is outstanding the compiler's wait for any earlier load becomes a
// wait for every outstanding memory operation, the stores' included.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* global_ptr(void* p) {
  return (__attribute__((address_space(1))) T*)(reinterpret_cast<uintptr_t>(p));
}

template <bool kStream = false>
__device__ __forceinline__ void st16(void* p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  if constexpr (kStream)
    __builtin_nontemporal_store(w, global_ptr<u32x4>(p));
  else
    *global_ptr<u32x4>(p) = w;
}
template <bool kStream = false>
__device__ __forceinline__ void st8(void* p, uint2 v) {
  const u32x2 w = {v.x, v.y};
  if constexpr (kStream)
    __builtin_nontemporal_store(w, global_ptr<u32x2>(p));
  else
    *global_ptr<u32x2>(p) = w;
}
template <bool kStream = false>
__device__ __forceinline__ void st4(void* p, uint32_t v) {
  if constexpr (kStream)
    __builtin_nontemporal_store(v, global_ptr<uint32_t>(p));
  else
    *global_ptr<uint32_t>(p) = v;
}
__device__ __forceinline__ void st2(void* p, uint16_t v) { *global_ptr<uint16_t>(p) = v; }

// Store policy per kernel (measured on MI355X): the pack and gather write
// large contiguous outputs that the next kernel of a chunk loop does not
// re-read from cache, so they stream; the insert and epilogue scatter
// 576-byte rows, where ordinary stores let the last-level cache merge lines.
constexpr bool kPackStream = true;
constexpr bool kGatherStream = true;
constexpr bool kInsertStream = false;
constexpr bool kEpiStream = false;

}  // namespace mla
