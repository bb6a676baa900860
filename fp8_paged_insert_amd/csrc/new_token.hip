// New-token epilogue: RoPE of q_pe and k_pe, the query row, the full key
// (and fp8 V), and the insert of [kv_c | rotated k_pe] into one layer's paged
// cache, in one launch.
//
// Pages: "PR #51772 完整报告", 功能与动机 (the new-token epilogue already
// quantises the query, so the chunked path must not do it again) and 关键源码
// 片段 (fused_mla_key_concat_kv_cache.py: the chunked-context pack is
// fused_mla_key_concat_kv_cache_insert without the query, the cache insert and
// RoPE, since gathered context k_pe is already rotated).  The pages name the
// op only; read as the chunked-context pack plus those three parts, each done
// as elsewhere in this library (RoPE as in the context epilogue, the key and V
// as in the pack, the cache row as in the insert).
//
// MI355X design: the op moves bytes, so there is no MFMA and no LDS.  One
// row of 16 lanes (a DPP row) handles one (token, head): it reads the query,
// k_nope and V rows and the token's k_pe, and writes the query, key and V
// rows.  Lane j owns nope / V values [8c, 8c + 8) for c = j, j + 16, ... and
// rope values [4j, 4j + 4); the rotation partner of lane j's rope values sits
// in lane j +- 8, one DPP row rotation away, and the token's cos / sin row is
// loaded once for both the query and the key rotation.  Every lane of a
// wavefront does the same work, and the four rows of a wavefront are
// consecutive heads of one token, so its loads and stores are contiguous
// runs.  Cache entries [kv_c | rotated k_pe] are tasks of their own after the
// (token, head) tasks, one 16-lane row per token, laid out like the context
// epilogue's rows.  Rotation: fp32, one rounding of x cos and a fused
// multiply-add with the partner's sin, rounded once to bf16 before any fp8
// conversion.
#include "mla_common.hpp"

namespace mla {
namespace {

constexpr int kLanes = 16;       // lanes per task: one DPP row
constexpr int kRope = 64;        // rotary width: 4 values per lane, partner 8 lanes away
constexpr int kDppRor8 = 0x128;  // lane i <- lane (i + 8) mod 16 within a DPP row
// Ordinary (not streaming) stores for every output: a 16-lane row writes a
// query or key row in two pieces (nope, then rope), and an fp8 row of 192 bytes
// shares its 128-byte lines with its neighbours, so streaming stores sent
// partial lines to HBM (11-14% extra write bytes measured); ordinary stores let
// L2 merge them (fp8 140 -> 132 us, bf16 126 -> 118 us at 8192 x 64).
constexpr bool kNtStream = false;

struct NewTokenArgs {
  const uint16_t* q_nope;
  int64_t qn_ts, qn_hs;
  const uint16_t* q_pe;
  int64_t qp_ts, qp_hs;
  const uint16_t* k_nope;
  int64_t kn_ts, kn_hs;
  const uint16_t* v;
  int64_t v_ts, v_hs;
  const uint16_t* kv_c;
  int64_t kvc_ts;
  const uint16_t* k_pe;
  int64_t kpe_ts;
  const int64_t* positions;
  const float* cos_sin;  // [max_pos, 128]: cos hi | sin hi | cos lo | sin lo of the 32 angles
  int64_t max_pos;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  const float* cache_scale;
  void* q_out;
  void* key_out;
  uint8_t* v_out;
  void* cache;
  const int64_t* slots;
  int64_t block_size, block_stride, entry_stride;  // strides in elements
  FastDiv bsize;
  FastDiv heads;
  uint32_t nope, vdim, kv_lora_rank;  // elements; multiples of 16
  uint32_t rows;                      // (token, head) tasks; the cache tasks follow
  uint32_t tasks;
  uint32_t tokens;
  // Grouped form (the MLA shape with heads a multiple of 16): wavefront
  // tasks of 16 heads of one token (row_waves of them), then cache tasks of
  // 4 tokens (one per 16-lane row), wave_tasks in all.
  uint32_t grouped, row_waves, wave_tasks;
  FastDiv hgroups;  // heads / 16
};

__device__ __forceinline__ float scale_or_one(const float* p) { return p ? p[0] : 1.0f; }

__device__ __forceinline__ int64_t entry_offset(int64_t s, const NewTokenArgs& a) {
  if (s < 0x80000000LL) {
    const uint32_t b32 = fdiv(static_cast<uint32_t>(s), a.bsize);
    return int64_t(b32) * a.block_stride +
           int64_t(static_cast<uint32_t>(s) - b32 * a.bsize.d) * a.entry_stride;
  }
  const int64_t blk = s / a.block_size;
  return blk * a.block_stride + (s - blk * a.block_size) * a.entry_stride;
}

__device__ __forceinline__ uint32_t dpp_ror8(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kDppRor8, 0xF, 0xF, false));
}

__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

// 16-byte load that does not keep its line in the caches, for the query,
// k_nope and V rows (each read once; bf16 119 -> 113 us, fp8 133 -> 132 us at
// 8192 x 64).  k_pe and the cos/sin rows, read by every head of a token, keep
// ordinary loads.
__device__ __forceinline__ uint4 ld16_once(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Lane j's rope values [4j, 4j + 4) (two bf16 words) rotated with the table
// words cv / sv of angles 4 (j mod 8) .. (tab: the lane's cos hi entries):
//   first half (j < 8)  y_i = x_i cos_i - x_{i+32} sin_i,
//   second half         y_{i+32} = x_{i+32} cos_i + x_i sin_i,
// each rounded once to bf16 (rope4).
// Every lane of the DPP row must execute it (the partner comes from lane j +- 8).
__device__ __forceinline__ uint2 rope4w(uint2 x, uint4 cv, uint4 sv, bool first, const float* tab) {
  const uint2 p = make_uint2(dpp_ror8(x.x), dpp_ror8(x.y));
  const float xf[4] = {bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y)};
  const float pf[4] = {bf16_lo(p.x), bf16_hi(p.x), bf16_lo(p.y), bf16_hi(p.y)};
  const float c[4] = {__uint_as_float(cv.x), __uint_as_float(cv.y), __uint_as_float(cv.z),
                      __uint_as_float(cv.w)};
  const float sn[4] = {__uint_as_float(sv.x), __uint_as_float(sv.y), __uint_as_float(sv.z),
                       __uint_as_float(sv.w)};
  return rope4(xf, pf, c, sn, first, tab + kRope, tab + kRope + kRope / 2);
}

// 8 bf16 -> one output chunk: 8 e4m3fn / e5m2 codes (kFmt) of x / s, or of x
// itself when !kScaled, or the 8 bf16 themselves.
template <int kFmt, bool kStream, bool kScaled = true>
__device__ __forceinline__ void put8(uint8_t* dst, uint4 x, float s, float r, uint32_t flip) {
  if constexpr (kFmt == kFmtBf16)
    st16<kStream>(dst, x);
  else
    st8<kStream>(dst, quant8<kScaled, false, kFmt == kFmtE5M2>(x, s, r, flip));
}

// 4 bf16 (one uint2) -> 4 codes or the 4 bf16 themselves.
template <int kFmt, bool kStream, bool kScaled = true>
__device__ __forceinline__ void put4(uint8_t* dst, uint2 x, float s, float r, uint32_t flip) {
  if constexpr (kFmt == kFmtBf16)
    st8<kStream>(dst, x);
  else
    st4<kStream>(dst, quant4<kScaled, kFmt == kFmtE5M2>(x, s, r, flip));
}

// kFp8: query, key and V are e4m3fn codes, else the query and key are bf16
// and there is no V output.  kScaled: the query / key / V codes are of x /
// scale (exact quotient); without it, of x itself (no scale pointers given:
// a plain cast, and three fewer ALU operations per value).  kCacheFmt: the
// cache's element format (its fp8 codes are always of x / cache_scale).
template <bool kFp8, bool kScaled, int kCacheFmt>
__global__ __launch_bounds__(256) void new_token_kernel(const NewTokenArgs a) {
  constexpr int kOut = kFp8 ? kFmtE4M3 : kFmtBf16;
  constexpr int ob = kFp8 ? 1 : 2;                          // output bytes per value
  constexpr int cb = kCacheFmt == kFmtBf16 ? 2 : 1;         // cache bytes per value
  const int j = threadIdx.x & (kLanes - 1);
  const bool first = j < kLanes / 2;
  const float qs = scale_or_one(a.q_scale), ks = scale_or_one(a.k_scale),
              vs = scale_or_one(a.v_scale);
  const float cs = kCacheFmt == kFmtBf16 ? 1.0f : scale_or_one(a.cache_scale);
  const float qr = 1.0f / qs, kr = 1.0f / ks, vr = 1.0f / vs, cr = 1.0f / cs;
  const uint32_t qf = sign_flip_of(qs), kf = sign_flip_of(ks), vf = sign_flip_of(vs),
                 cf = sign_flip_of(cs);
  const uint32_t width = a.nope + kRope;
  // ---- one token's cache entry [kv_c | rotated k_pe] (one 16-lane row; a
  // padded token, slot -1, skips the whole row)
  auto cache_row = [&](uint32_t t) {
    const int64_t slot = a.slots[t];
    if (slot < 0) return;
    const int64_t pos = min(max(a.positions[t], int64_t(0)), a.max_pos - 1);
    const float* tab = a.cos_sin + pos * (2 * kRope) + 4 * (j & 7);
    const uint4 cv = ld16(tab), sv = ld16(tab + kRope / 2);
    const uint2 kpe = ld8(a.k_pe + int64_t(t) * a.kpe_ts + 4 * j);
    const uint16_t* kc = a.kv_c + int64_t(t) * a.kvc_ts;
    uint8_t* dst = static_cast<uint8_t*>(a.cache) + entry_offset(slot, a) * cb;
    for (uint32_t c = j; c < a.kv_lora_rank / 8; c += kLanes)
      put8<kCacheFmt, kNtStream>(dst + 8 * c * cb, ld16(kc + 8 * c), cs, cr, cf);
    put4<kCacheFmt, kNtStream>(dst + (a.kv_lora_rank + 4 * j) * cb, rope4w(kpe, cv, sv, first, tab),
                               cs, cr, cf);
  };
  if (kFp8 && a.grouped) {
    // fp8 outputs, the MLA shape (nope = V width = 128), heads in groups of 16:
    // wavefront task w < row_waves covers heads [16 q, 16 q + 16) of token
    // w / G, q = w mod G (G = heads / 16); its 16-lane row r takes heads
    // 16 q + r + 4 g for g = 0..3, so each step g of the wavefront covers 4
    // consecutive heads.  The key's rope part is the token's rotated k_pe
    // for every head: each row rotates and converts it once and stores the
    // result for its 4 heads (per head, that rotation and conversion were
    // about a sixth of the fp8 forms' ALU work; with the full grid, 142.8 ->
    // 120.0 us scaled, 133.9 -> 119.6 us plain at 8192 x 64).  Wavefront tasks past
    // row_waves are cache entries, one token per row.  The bf16 form is
    // bound by HBM, not the ALU: grouped it was 2% slower, so it keeps one
    // task per row (and is compiled without this path, which would raise
    // its register count from 79 to 111).
    const uint32_t r = (threadIdx.x / kLanes) & 3;
    const uint32_t nw = (gridDim.x * blockDim.x) / 64;
    for (uint32_t w = (blockIdx.x * blockDim.x + threadIdx.x) / 64; w < a.wave_tasks; w += nw) {
      if (w >= a.row_waves) {
        const uint32_t t = (w - a.row_waves) * 4 + r;
        if (t < a.tokens) cache_row(t);
        continue;
      }
      const uint32_t t = fdiv(w, a.hgroups);
      const uint32_t h0 = (w - t * a.hgroups.d) * 16 + r;
      const int64_t pos = min(max(a.positions[t], int64_t(0)), a.max_pos - 1);
      const float* tab = a.cos_sin + pos * (2 * kRope) + 4 * (j & 7);
      const uint4 cv = ld16(tab), sv = ld16(tab + kRope / 2);
      const uint2 kpe = ld8(a.k_pe + int64_t(t) * a.kpe_ts + 4 * j);
      uint32_t kcode = 0;
      // two batches of 2 heads: a batch's loads are issued before its first
      // conversion (4 heads at once would need more than 128 VGPRs)
#pragma unroll
      for (int b = 0; b < 4; b += 2) {
        uint4 xq[2], xk[2], xv[2];
        uint2 qpe[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int64_t h = h0 + 4 * (b + g);
          xq[g] = ld16_once(a.q_nope + int64_t(t) * a.qn_ts + h * a.qn_hs + 8 * j);
          xk[g] = ld16_once(a.k_nope + int64_t(t) * a.kn_ts + h * a.kn_hs + 8 * j);
          xv[g] = ld16_once(a.v + int64_t(t) * a.v_ts + h * a.v_hs + 8 * j);
          qpe[g] = ld8(a.q_pe + int64_t(t) * a.qp_ts + h * a.qp_hs + 4 * j);
        }
        if (b == 0) kcode = quant4<kScaled, false>(rope4w(kpe, cv, sv, first, tab), ks, kr, kf);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int64_t task = int64_t(t) * a.heads.d + h0 + 4 * (b + g);
          uint8_t* qo = static_cast<uint8_t*>(a.q_out) + task * width;
          uint8_t* ko = static_cast<uint8_t*>(a.key_out) + task * width;
          put8<kFmtE4M3, kNtStream, kScaled>(qo + 8 * j, xq[g], qs, qr, qf);
          put8<kFmtE4M3, kNtStream, kScaled>(ko + 8 * j, xk[g], ks, kr, kf);
          put4<kFmtE4M3, kNtStream, kScaled>(qo + 128 + 4 * j, rope4w(qpe[g], cv, sv, first, tab),
                                             qs, qr, qf);
          st4<kNtStream>(ko + 128 + 4 * j, kcode);
          put8<kFmtE4M3, kNtStream, kScaled>(a.v_out + task * 128 + 8 * j, xv[g], vs, vr, vf);
        }
      }
    }
    return;
  }
  const uint32_t step = (gridDim.x * blockDim.x) / kLanes;
  for (uint32_t task = (blockIdx.x * blockDim.x + threadIdx.x) / kLanes; task < a.tasks;
       task += step) {
    if (task < a.rows) {
      // ---- one (token, head): query row, key row, V row
      const uint32_t t = fdiv(task, a.heads);
      const uint32_t h = task - t * a.heads.d;
      const int64_t pos = min(max(a.positions[t], int64_t(0)), a.max_pos - 1);
      const float* tab = a.cos_sin + pos * (2 * kRope) + 4 * (j & 7);
      const uint4 cv = ld16(tab), sv = ld16(tab + kRope / 2);
      const uint16_t* qn = a.q_nope + int64_t(t) * a.qn_ts + int64_t(h) * a.qn_hs;
      const uint16_t* kn = a.k_nope + int64_t(t) * a.kn_ts + int64_t(h) * a.kn_hs;
      const uint2 qpe = ld8(a.q_pe + int64_t(t) * a.qp_ts + int64_t(h) * a.qp_hs + 4 * j);
      const uint2 kpe = ld8(a.k_pe + int64_t(t) * a.kpe_ts + 4 * j);
      uint8_t* qo = static_cast<uint8_t*>(a.q_out) + int64_t(task) * width * ob;
      uint8_t* ko = static_cast<uint8_t*>(a.key_out) + int64_t(task) * width * ob;
      if (a.nope == 128 && (!kFp8 || a.vdim == 128)) {
        // The MLA shape: one nope (and V) chunk per lane, every load issued
        // before the first conversion, so a task waits on memory once (the
        // general loop below issues V's load after the query and key stores).
        const uint4 xq = ld16_once(qn + 8 * j);
        const uint4 xk = ld16_once(kn + 8 * j);
        uint4 xv = make_uint4(0, 0, 0, 0);
        if constexpr (kFp8)
          xv = ld16_once(a.v + int64_t(t) * a.v_ts + int64_t(h) * a.v_hs + 8 * j);
        put8<kOut, kNtStream, kScaled>(qo + 8 * j * ob, xq, qs, qr, qf);
        put8<kOut, kNtStream, kScaled>(ko + 8 * j * ob, xk, ks, kr, kf);
        put4<kOut, kNtStream, kScaled>(qo + (128 + 4 * j) * ob, rope4w(qpe, cv, sv, first, tab), qs,
                                         qr, qf);
        put4<kOut, kNtStream, kScaled>(ko + (128 + 4 * j) * ob, rope4w(kpe, cv, sv, first, tab), ks,
                                         kr, kf);
        if constexpr (kFp8)
          put8<kFmtE4M3, kNtStream, kScaled>(a.v_out + int64_t(task) * 128 + 8 * j, xv, vs, vr,
                                             vf);
        continue;
      }
      for (uint32_t c = j; c < a.nope / 8; c += kLanes) {
        const uint4 xq = ld16_once(qn + 8 * c);
        const uint4 xk = ld16_once(kn + 8 * c);
        put8<kOut, kNtStream, kScaled>(qo + 8 * c * ob, xq, qs, qr, qf);
        put8<kOut, kNtStream, kScaled>(ko + 8 * c * ob, xk, ks, kr, kf);
      }
      put4<kOut, kNtStream, kScaled>(qo + (a.nope + 4 * j) * ob, rope4w(qpe, cv, sv, first, tab), qs,
                                       qr, qf);
      put4<kOut, kNtStream, kScaled>(ko + (a.nope + 4 * j) * ob, rope4w(kpe, cv, sv, first, tab), ks,
                                       kr, kf);
      if constexpr (kFp8) {
        const uint16_t* vi = a.v + int64_t(t) * a.v_ts + int64_t(h) * a.v_hs;
        uint8_t* vo = a.v_out + int64_t(task) * a.vdim;
        for (uint32_t c = j; c < a.vdim / 8; c += kLanes)
          put8<kFmtE4M3, kNtStream, kScaled>(vo + 8 * c, ld16_once(vi + 8 * c), vs, vr, vf);
      }
    } else {
      cache_row(task - a.rows);
    }
  }
}

template <bool kFp8, bool kScaled>
void launch_new_token(int fmt, dim3 g, dim3 b, hipStream_t s, const NewTokenArgs& a) {
  if (fmt == kFmtE4M3)
    launch(new_token_kernel<kFp8, kScaled, kFmtE4M3>, g, b, 0, s, a);
  else if (fmt == kFmtE5M2)
    launch(new_token_kernel<kFp8, kScaled, kFmtE5M2>, g, b, 0, s, a);
  else
    launch(new_token_kernel<kFp8, kScaled, kFmtBf16>, g, b, 0, s, a);
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int32_t mla_new_token_epilogue(
    const void* q_nope, int64_t qn_tok_stride, int64_t qn_head_stride, const void* q_pe,
    int64_t qp_tok_stride, int64_t qp_head_stride, const void* k_nope, int64_t kn_tok_stride,
    int64_t kn_head_stride, const void* v, int64_t v_tok_stride, int64_t v_head_stride,
    const void* kv_c, int64_t kv_c_tok_stride, const void* k_pe, int64_t k_pe_tok_stride,
    const int64_t* positions, const float* cos_sin, int64_t max_pos, int64_t num_tokens,
    int64_t num_heads, int64_t nope, int64_t rope, int64_t vdim, int64_t kv_lora_rank,
    int32_t mode, const float* q_scale, const float* k_scale, const float* v_scale,
    void* q_out, void* key_out, void* v_out, void* cache, int32_t cache_dtype,
    const float* cache_scale, const int64_t* slot_mapping, int64_t block_size,
    int64_t block_stride, int64_t entry_stride, int64_t max_blocks, mla_stream_t stream) {
  static const char* fn = "mla_new_token_epilogue";
  clear_error();
  if (mode != MLA_PACK_KEY_BF16 && mode != MLA_PACK_KEY_V_FP8)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: mode must be KEY_BF16 or KEY_V_FP8", fn);
  const bool fp8 = mode == MLA_PACK_KEY_V_FP8;
  if (num_tokens < 0 || num_heads < 0 || nope < 0 || rope < 0 || vdim < 0 ||
      kv_lora_rank < 0 || max_blocks < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
  if (!fp8 && (v || v_out || q_scale || k_scale || v_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "%s: the bf16 mode takes no v, v_out or query/key/V scales", fn);
  if (cache) {
    const int32_t st = check_cache_dtype(fn, cache_dtype, cache_scale);
    if (st != MLA_OK) return st;
    if (!slot_mapping) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: a cache needs slot_mapping", fn);
    if (block_size <= 0 || block_stride <= 0 || entry_stride <= 0)
      return fail(MLA_ERR_INVALID_ARGUMENT, "%s: block_size and strides must be positive", fn);
    if (kv_lora_rank + rope > entry_stride)
      return fail(MLA_ERR_INVALID_ARGUMENT, "%s: a cache entry is wider than entry_stride", fn);
  } else if (slot_mapping || cache_scale) {
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: slot_mapping / cache_scale without a cache", fn);
  }
  if (num_tokens == 0) return MLA_OK;
  if (rope != kRope || nope % 16 != 0 || vdim % 16 != 0 || kv_lora_rank % 16 != 0)
    return fail(MLA_ERR_UNSUPPORTED,
                "%s: rope must be 64; nope, vdim and kv_lora_rank multiples of 16", fn);
  if (!positions || !cos_sin || max_pos <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: RoPE needs positions, cos_sin and max_pos > 0",
                fn);
  const bool rows_out = num_heads > 0;
  if (rows_out && (!q_nope || !q_pe || !k_nope || !k_pe || !q_out || !key_out ||
                   (fp8 && vdim > 0 && (!v || !v_out))))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL input or output", fn);
  if (cache && (!kv_c || !k_pe))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL kv_c or k_pe for the cache insert", fn);
  const int64_t ceb = cache ? (is_fp8(cache_dtype) ? 1 : 2) : 1;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(k_nope) || !aligned16(v) ||
      !aligned16(kv_c) || !aligned16(k_pe) || !aligned16(cos_sin) || !aligned16(q_out) ||
      !aligned16(key_out) || !aligned16(v_out) || !aligned16(cache) ||
      !bytes16(qn_tok_stride, 2) || !bytes16(qn_head_stride, 2) || !bytes16(qp_tok_stride, 2) ||
      !bytes16(qp_head_stride, 2) || !bytes16(kn_tok_stride, 2) ||
      !bytes16(kn_head_stride, 2) || !bytes16(v_tok_stride, 2) || !bytes16(v_head_stride, 2) ||
      !bytes16(kv_c_tok_stride, 2) || !bytes16(k_pe_tok_stride, 2) ||
      (cache && (!bytes16(block_stride, ceb) || !bytes16(entry_stride, ceb))))
    return fail(MLA_ERR_MISALIGNED, "%s: addresses and strides must be multiples of 16 bytes",
                fn);
  const int64_t rows = num_tokens * num_heads;
  const int64_t tasks = rows + (cache ? num_tokens : 0);
  if (tasks * kLanes >= (int64_t(1) << 31) || num_heads > 0x7FFFFFFF ||
      block_size > 0x7FFFFFFF || nope > 0xFFFF || vdim > 0xFFFF || kv_lora_rank > 0xFFFF)
    return fail(MLA_ERR_UNSUPPORTED, "%s: more than 2^27 rows; split the batch", fn);
  if (tasks == 0) return MLA_OK;
  NewTokenArgs a;
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.qn_ts = qn_tok_stride;
  a.qn_hs = qn_head_stride;
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.qp_ts = qp_tok_stride;
  a.qp_hs = qp_head_stride;
  a.k_nope = static_cast<const uint16_t*>(k_nope);
  a.kn_ts = kn_tok_stride;
  a.kn_hs = kn_head_stride;
  a.v = static_cast<const uint16_t*>(v);
  a.v_ts = v_tok_stride;
  a.v_hs = v_head_stride;
  a.kv_c = static_cast<const uint16_t*>(kv_c);
  a.kvc_ts = kv_c_tok_stride;
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.kpe_ts = k_pe_tok_stride;
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.max_pos = max_pos;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.cache_scale = cache_scale;
  a.q_out = q_out;
  a.key_out = key_out;
  a.v_out = static_cast<uint8_t*>(v_out);
  a.cache = cache;
  a.slots = slot_mapping;
  a.block_size = cache ? block_size : 1;
  a.block_stride = block_stride;
  a.entry_stride = entry_stride;
  a.bsize = make_fastdiv(static_cast<uint32_t>(a.block_size));
  a.heads = make_fastdiv(static_cast<uint32_t>(num_heads > 0 ? num_heads : 1));
  a.nope = static_cast<uint32_t>(nope);
  a.vdim = static_cast<uint32_t>(fp8 ? vdim : 0);
  a.kv_lora_rank = static_cast<uint32_t>(kv_lora_rank);
  a.rows = static_cast<uint32_t>(rows);
  a.tasks = static_cast<uint32_t>(tasks);
  a.tokens = static_cast<uint32_t>(num_tokens);
  const bool grouped = fp8 && nope == 128 && vdim == 128 && num_heads > 0 && num_heads % 16 == 0;
  a.grouped = grouped;
  a.hgroups = make_fastdiv(static_cast<uint32_t>(grouped ? num_heads / 16 : 1));
  a.row_waves = static_cast<uint32_t>(grouped ? rows / 16 : 0);
  a.wave_tasks = static_cast<uint32_t>(grouped ? rows / 16 + (cache ? ceil_div(num_tokens, 4) : 0) : 0);
  // Default grid: the full grid (one task per 16-lane row, or one grouped
  // task per wavefront) except for fp8 outputs in the ungrouped form, which
  // run 4 workgroups per CU looping over the tasks, so each wavefront's
  // per-launch set-up (the scales' reciprocals by IEEE division, when
  // scaled) is paid once per ~30 tasks.  Measured at 8192 x 64: ungrouped,
  // scaled 141.8 us on the full grid against 132.2 us, plain 131.3 against
  // 128.6 us; grouped (16 heads per task), the full grid is fastest: 120.3
  // and 120.9 us plain and scaled against 126.6 and 127.7 us at 4 per CU.
  const bool scaled = fp8 && (q_scale || k_scale || v_scale);
  const int64_t full = grouped ? ceil_div(int64_t(a.wave_tasks) * 64, 256) : ceil_div(tasks * kLanes, 256);
  const int64_t dflt = fp8 && !grouped ? std::min(full, int64_t(4) * cu_count()) : full;
  const dim3 g(max_blocks > 0 ? std::min(full, max_blocks) : dflt), b(256);
  const int fmt = cache ? cache_fmt(cache_dtype) : kFmtBf16;
  auto s = static_cast<hipStream_t>(stream);
  if (!fp8)
    launch_new_token<false, false>(fmt, g, b, s, a);
  else if (scaled)
    launch_new_token<true, true>(fmt, g, b, s, a);
  else
    launch_new_token<true, false>(fmt, g, b, s, a);
  return launch_status(fn);
}
