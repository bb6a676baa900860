// gather_pack.hip -- chunked-context gather from the paged latent cache and
// the full-key / fp8-V pack.
//
// Page: "PR #51772 完整报告" ([Attention][MLA] Fuse Kimi-K3 chunked-context
// K/V packing).  实现拆解 item 1: one kernel per chunk reads the strided
// kv_b_proj halves (k_nope, v) and the gathered k_pe directly, writes a
// contiguous key [k_nope | k_pe] (and, for fp8, a contiguous fp8 V), with a
// capped grid and a grid-stride loop for long contexts.  实现拆解 item 2: the
// context latent is gathered from the cache before kv_b_proj; item 5: with a
// plain fp8 cache the gathered latent must reach a bf16 kv_b_proj as bf16.
// 关键源码片段 (fused_mla_key_concat_kv_cache.py): output shapes and the
// bit-identity of the fp8 cast with torch's float8_e4m3fn cast.
//
// gfx950 design: both kernels walk a flat list of 16-byte output chunks, so
// every store is a full 16-byte vector and consecutive lanes write
// consecutive addresses of the contiguous outputs; loads are 16/32-byte
// vectors along the contiguous rows of the strided inputs.  The k_pe row of
// a token is read once per head from L2 (it is 128 bytes shared by H heads).
#include "mla_common.hpp"

namespace mla {
namespace {

// ----------------------------------------------------------------- gather --
struct GatherArgs {
  const uint8_t* cache;  // bytes
  const float* scale;
  const int64_t* slots;
  void* out;
  int64_t block_size, block_stride, entry_stride;  // cache elements
  int64_t width;                                    // output row length
  FastDiv per_row, bsize;
  uint32_t total;
};

// Gather kinds: a 16-bit row copy (bf16 cache), the dequantising fp8 gather
// from an e4m3fn or an e5m2 cache (16 codes in, 16 bf16 out per chunk) and
// the raw fp8 copy (16 codes of either format).
enum GatherKind { kGatherCopy16 = 0, kGatherDequant = 1, kGatherRaw8 = 2, kGatherDequantE5M2 = 3 };

// Each thread takes U chunks per pass (item, item + stride, ...): the U slot
// loads go out together, then the U cache-row loads, then the conversions,
// so the slot -> row dependence is paid once per U chunks.
template <int kKind, int U>
__global__ __launch_bounds__(256) void gather_kernel(const GatherArgs a) {
  constexpr bool kFp8 = kKind != kGatherCopy16;      // cache holds 1-byte codes
  constexpr int E = kFp8 ? 16 : 8;                   // cache elements per chunk
  constexpr int kOutBytes = kKind == kGatherRaw8 ? 1 : 2;
  constexpr bool kDequant = kKind == kGatherDequant || kKind == kGatherDequantE5M2;
  constexpr bool kE5M2 = kKind == kGatherDequantE5M2;
  const uint32_t stride = gridDim.x * blockDim.x;
  float sc = 1.0f;
  if constexpr (kDequant) sc = a.scale[0];
  for (uint32_t base = blockIdx.x * blockDim.x + threadIdx.x; base < a.total;
       base += U * stride) {
    int64_t s[U];
    uint32_t jj[U], cc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t item = base + u * stride;
      jj[u] = fdiv(item < a.total ? item : 0, a.per_row);
      cc[u] = item - jj[u] * a.per_row.d;
      s[u] = item < a.total ? a.slots[jj[u]] : 0;
    }
    uint4 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * stride < a.total) {
        int64_t blk, off;
        if (s[u] < 0x80000000LL) {
          const uint32_t b32 = fdiv(static_cast<uint32_t>(s[u]), a.bsize);
          blk = b32;
          off = static_cast<uint32_t>(s[u]) - b32 * a.bsize.d;
        } else {
          blk = s[u] / a.block_size;
          off = s[u] - blk * a.block_size;
        }
        const int64_t src_el = blk * a.block_stride + off * a.entry_stride + int64_t(cc[u]) * E;
        q[u] = kFp8 ? ld16(a.cache + src_el)
                    : ld16(reinterpret_cast<const uint16_t*>(a.cache) + src_el);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * stride >= a.total) continue;
      uint8_t* dst = static_cast<uint8_t*>(a.out) +
                     (int64_t(jj[u]) * a.width + int64_t(cc[u]) * E) * kOutBytes;
      if constexpr (kDequant) {
        const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float f[4];
          dec4_fp8<kE5M2>(w[i], f);
          // fl32(value * scale) rounded to bf16; the converter's NaN does not
          // keep the code's sign, so NaN codes are rebuilt (a rare branch).
          uint32_t lo = cvt_bf16x2(f[0] * sc, f[1] * sc);
          uint32_t hi = cvt_bf16x2(f[2] * sc, f[3] * sc);
          // NaN codes: magnitude byte 0x7F (e4m3fn) or 0x7D-0x7F (e5m2)
          constexpr uint32_t kNanBias = kE5M2 ? 0x03030303u : 0x01010101u;
          const bool nan4 = (((w[i] & 0x7F7F7F7Fu) + kNanBias) & 0x80808080u) != 0;
          if (__builtin_expect(__builtin_amdgcn_ballot_w64(nan4) != 0, 0)) {
            uint32_t b[4] = {lo & 0xFFFFu, lo >> 16, hi & 0xFFFFu, hi >> 16};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const uint32_t code = (w[i] >> (8 * k)) & 0xFFu;
              if ((code & 0x7Fu) >= (kE5M2 ? 0x7Du : 0x7Fu)) b[k] = 0x7FC0u | ((code & 0x80u) << 8);
            }
            lo = b[0] | (b[1] << 16);
            hi = b[2] | (b[3] << 16);
          }
          o[2 * i] = lo;
          o[2 * i + 1] = hi;
        }
        st16<kGatherStream>(dst, make_uint4(o[0], o[1], o[2], o[3]));
        st16<kGatherStream>(dst + 16, make_uint4(o[4], o[5], o[6], o[7]));
      } else {
        st16<kGatherStream>(dst, q[u]);
      }
    }
  }
}

// ------------------------------------------------------------------- pack --
// The outputs are cut into 16-byte chunks, numbered key chunks of every
// token first (row (t, h), chunk j), then V chunks; chunk i is written at
// byte 16 i of its output, so consecutive lanes write consecutive addresses.
// The default grid has one thread per chunk (no loop): the workgroups in
// flight then sweep the strided kv_b_proj output and the contiguous outputs
// as one advancing window, which measured faster on MI355X than a capped
// grid; a caller-given max_blocks turns the grid-stride loop on.
struct PackArgs {
  const uint16_t* k_nope;
  int64_t kn_ts, kn_hs;
  const uint16_t* k_pe;
  int64_t pe_ts;
  const uint16_t* v;
  int64_t v_ts, v_hs;
  const float* k_scale;
  const float* v_scale;
  void* key_out;
  uint8_t* v_out;
  FastDiv key_per_row;  // output chunks per key row
  FastDiv v_per_row;    // output chunks per V row (fp8 mode)
  FastDiv heads;
  uint32_t nope_chunks;  // key chunks taken from k_nope
  uint32_t key_total;    // T * H * key_per_row
  uint32_t total;        // key_total + T * H * v_per_row
};

// 16-byte load that does not keep its line in the caches: the fp8 pack reads
// every byte of the kv_b_proj output once, and in the chunk loop keeping
// those 268 MB per chunk out of the last-level cache measured 1% faster per
// step (flushed single launches: unchanged).  The bf16 pack keeps ordinary
// loads (3% slower with these).
__device__ __forceinline__ uint4 ld16_once(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Source of key chunk `item` (row (t, h) = item / key_per_row).
template <int E>
__device__ __forceinline__ const uint16_t* key_src(const PackArgs& a, uint32_t item) {
  const uint32_t row = fdiv(item, a.key_per_row);
  const uint32_t j = item - row * a.key_per_row.d;
  const uint32_t t = fdiv(row, a.heads);
  const uint32_t h = row - t * a.heads.d;
  return j < a.nope_chunks ? a.k_nope + int64_t(t) * a.kn_ts + int64_t(h) * a.kn_hs + j * E
                           : a.k_pe + int64_t(t) * a.pe_ts + (j - a.nope_chunks) * E;
}

__global__ __launch_bounds__(256) void pack_bf16_kernel(const PackArgs a) {
  constexpr int E = 8;
  uint16_t* key = static_cast<uint16_t*>(a.key_out);
  for (uint32_t item = blockIdx.x * blockDim.x + threadIdx.x; item < a.total;
       item += gridDim.x * blockDim.x)
    st16<kPackStream>(key + int64_t(item) * E, ld16(key_src<E>(a, item)));
}

// fp8 key and V.  kF16: the 16-bit inputs are IEEE fp16 (else bf16).
// kKpeRaw: k_pe holds e4m3fn codes (a_pe_ts in bytes), copied into the key's
// rope chunks unchanged.
template <bool kScaled, bool kF16, bool kKpeRaw>
__global__ __launch_bounds__(256) void pack_fp8_kernel(const PackArgs a) {
  constexpr int E = 16;
  float ks = 1.0f, vs = 1.0f;
  if constexpr (kScaled) {
    if (a.k_scale) ks = a.k_scale[0];
    if (a.v_scale) vs = a.v_scale[0];
  }
  const float kr = 1.0f / ks, vr = 1.0f / vs;
  const uint32_t kf = sign_flip_of(ks), vf = sign_flip_of(vs);
  for (uint32_t item = blockIdx.x * blockDim.x + threadIdx.x; item < a.total;
       item += gridDim.x * blockDim.x) {
    const uint16_t* src;
    uint8_t* dst;
    bool raw = false;
    const bool is_key = item < a.key_total;
    if (is_key) {
      dst = static_cast<uint8_t*>(a.key_out) + int64_t(item) * E;
      if constexpr (kKpeRaw) {
        const uint32_t row = fdiv(item, a.key_per_row);
        const uint32_t j = item - row * a.key_per_row.d;
        const uint32_t t = fdiv(row, a.heads);
        const uint32_t h = row - t * a.heads.d;
        raw = j >= a.nope_chunks;
        src = raw ? reinterpret_cast<const uint16_t*>(
                        reinterpret_cast<const uint8_t*>(a.k_pe) + int64_t(t) * a.pe_ts +
                        (j - a.nope_chunks) * E)
                  : a.k_nope + int64_t(t) * a.kn_ts + int64_t(h) * a.kn_hs + j * E;
      } else {
        src = key_src<E>(a, item);
      }
    } else {
      const uint32_t vi = item - a.key_total;
      const uint32_t row = fdiv(vi, a.v_per_row);
      const uint32_t j = vi - row * a.v_per_row.d;
      const uint32_t t = fdiv(row, a.heads);
      const uint32_t h = row - t * a.heads.d;
      src = a.v + int64_t(t) * a.v_ts + int64_t(h) * a.v_hs + j * E;
      dst = a.v_out + int64_t(vi) * E;
    }
    const uint4 x0 = ld16_once(src);
    if (kKpeRaw && raw) {
      st16<kPackStream>(dst, x0);   // 16 codes, as they are
      continue;
    }
    const uint4 x1 = ld16_once(src + 8);
    st16<kPackStream>(dst, quant16<kScaled, kF16>(x0, x1, is_key ? ks : vs, is_key ? kr : vr,
                                                  is_key ? kf : vf));
  }
}

#ifndef MLA_GATHER_UNROLL
#define MLA_GATHER_UNROLL 1
#endif
constexpr int kGatherUnroll = MLA_GATHER_UNROLL;

template <bool kScaled>
void launch_pack_fp8(bool f16, bool kpe_raw, dim3 g, dim3 b, hipStream_t s, const PackArgs& a) {
  if (f16 && kpe_raw)
    launch(pack_fp8_kernel<kScaled, true, true>, g, b, 0, s, a);
  else if (f16)
    launch(pack_fp8_kernel<kScaled, true, false>, g, b, 0, s, a);
  else if (kpe_raw)
    launch(pack_fp8_kernel<kScaled, false, true>, g, b, 0, s, a);
  else
    launch(pack_fp8_kernel<kScaled, false, false>, g, b, 0, s, a);
}

int64_t grid_for(int64_t total, int64_t max_blocks) {
  const int64_t cap = max_blocks > 0 ? max_blocks : default_grid_cap();
  return std::max<int64_t>(1, std::min<int64_t>(ceil_div(total, 256), cap));
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int32_t mla_ctx_latent_gather(const void* cache, int32_t cache_dtype,
                                         const float* cache_scale, int64_t block_size,
                                         int64_t block_stride, int64_t entry_stride,
                                         const int64_t* src_slots, int64_t num_tokens,
                                         int64_t width, int32_t out_dtype, void* out,
                                         int64_t max_blocks, mla_stream_t stream) {
  static const char* fn = "mla_ctx_latent_gather";
  clear_error();
  int32_t st;
  const bool raw = out_dtype == MLA_KV_FP8_E4M3 || out_dtype == MLA_KV_FP8_E5M2;
  if (out_dtype != MLA_KV_BF16 && !raw)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "%s: out_dtype must be bf16, or the fp8 cache's own dtype (raw codes)", fn);
  switch (cache_dtype) {
    case MLA_KV_AUTO:
    case MLA_KV_BF16:
      if (raw)
        return fail(MLA_ERR_INVALID_ARGUMENT, "%s: raw fp8 output needs an fp8 cache", fn);
      if (cache_scale)
        return fail(MLA_ERR_INVALID_ARGUMENT, "%s: a bf16 cache takes no cache_scale", fn);
      break;
    case MLA_KV_FP8_E4M3:
    case MLA_KV_FP8_E5M2:
      if (raw && out_dtype != cache_dtype)
        return fail(MLA_ERR_INVALID_ARGUMENT,
                    "%s: raw codes keep the cache's format; out_dtype must equal cache_dtype", fn);
      if (raw && cache_scale)
        return fail(MLA_ERR_INVALID_ARGUMENT,
                    "%s: the raw fp8 gather does not dequantise; pass no cache_scale", fn);
      if (!raw && !cache_scale)
        return fail(MLA_ERR_INVALID_ARGUMENT, "%s: an fp8 cache needs cache_scale", fn);
      break;
    default:
      st = check_cache_dtype(fn, cache_dtype, cache_scale);
      return st != MLA_OK ? st : fail(MLA_ERR_INVALID_ARGUMENT, "%s: bad cache dtype", fn);
  }
  if (num_tokens < 0 || width < 0 || max_blocks < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
  if (block_size <= 0 || block_stride <= 0 || entry_stride <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: block_size and strides must be positive", fn);
  if (width > entry_stride)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: width %lld exceeds entry_stride %lld", fn,
                (long long)width, (long long)entry_stride);
  if (num_tokens == 0 || width == 0) return MLA_OK;
  if (!cache || !src_slots || !out)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL cache, src_slots or out", fn);
  if (width % 16 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "%s: width must be a multiple of 16", fn);
  const bool fp8 = is_fp8(cache_dtype);
  const int64_t eb = fp8 ? 1 : 2;
  if (!aligned16(cache) || !aligned16(out) || !bytes16(block_stride, eb) ||
      !bytes16(entry_stride, eb))
    return fail(MLA_ERR_MISALIGNED, "%s: cache/out addresses and cache strides must be "
                "multiples of 16 bytes", fn);
  const int64_t E = fp8 ? 16 : 8;
  const int64_t per_row = width / E;
  const int64_t total = num_tokens * per_row;
  if (total >= (int64_t(1) << 31) || block_size > 0x7FFFFFFF)
    return fail(MLA_ERR_UNSUPPORTED, "%s: too many tokens for one launch", fn);
  GatherArgs a;
  a.cache = static_cast<const uint8_t*>(cache);
  a.scale = cache_scale;
  a.slots = src_slots;
  a.out = out;
  a.block_size = block_size;
  a.block_stride = block_stride;
  a.entry_stride = entry_stride;
  a.width = width;
  a.per_row = make_fastdiv(static_cast<uint32_t>(per_row));
  a.bsize = make_fastdiv(static_cast<uint32_t>(block_size));
  a.total = static_cast<uint32_t>(total);
  auto s = static_cast<hipStream_t>(stream);
  const int64_t blocks = grid_for(ceil_div(total, kGatherUnroll), max_blocks);
  if (raw)
    launch((gather_kernel<kGatherRaw8, kGatherUnroll>), dim3(blocks), dim3(256), 0, s, a);
  else if (cache_dtype == MLA_KV_FP8_E5M2)
    launch((gather_kernel<kGatherDequantE5M2, kGatherUnroll>), dim3(blocks), dim3(256), 0, s, a);
  else if (fp8)
    launch((gather_kernel<kGatherDequant, kGatherUnroll>), dim3(blocks), dim3(256), 0, s, a);
  else
    launch((gather_kernel<kGatherCopy16, kGatherUnroll>), dim3(blocks), dim3(256), 0, s, a);
  return launch_status(fn);
}

extern "C" int32_t mla_ctx_kv_pack(const void* k_nope, int64_t kn_tok_stride,
                                   int64_t kn_head_stride, const void* k_pe,
                                   int64_t kpe_tok_stride, const void* v,
                                   int64_t v_tok_stride, int64_t v_head_stride,
                                   int64_t num_tokens, int64_t num_heads, int64_t nope,
                                   int64_t rope, int64_t vdim, int32_t mode, int32_t src_dtype,
                                   const float* k_scale, const float* v_scale,
                                   void* key_out, void* v_out, int64_t max_blocks,
                                   mla_stream_t stream) {
  static const char* fn = "mla_ctx_kv_pack";
  clear_error();
  if (mode != MLA_PACK_KEY_BF16 && mode != MLA_PACK_KEY_V_FP8 &&
      mode != MLA_PACK_KEY_V_FP8_KPE_RAW)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: unknown mode %d", fn, mode);
  if (src_dtype != MLA_KV_BF16 && src_dtype != MLA_KV_FP16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: src_dtype must be bf16 or fp16", fn);
  const bool fp8 = mode != MLA_PACK_KEY_BF16;
  const bool kpe_raw = mode == MLA_PACK_KEY_V_FP8_KPE_RAW;
  const bool f16 = src_dtype == MLA_KV_FP16;
  if (num_tokens < 0 || num_heads < 0 || nope < 0 || rope < 0 || vdim < 0 || max_blocks < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
  if (!fp8 && (v || v_out || k_scale || v_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: the 16-bit key mode takes no v, v_out or scales",
                fn);
  if (num_tokens == 0 || num_heads == 0) return MLA_OK;
  if (nope + rope == 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: empty key rows", fn);
  if (!k_nope || (rope > 0 && !k_pe) || !key_out || (fp8 && vdim > 0 && (!v || !v_out)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL input or output", fn);
  if (nope % 16 || rope % 16 || vdim % 16)
    return fail(MLA_ERR_UNSUPPORTED, "%s: nope, rope and vdim must be multiples of 16", fn);
  if (!aligned16(k_nope) || !aligned16(k_pe) || !aligned16(key_out) || !aligned16(v) ||
      !aligned16(v_out) || !bytes16(kn_tok_stride, 2) || !bytes16(kn_head_stride, 2) ||
      !bytes16(kpe_tok_stride, kpe_raw ? 1 : 2) || !bytes16(v_tok_stride, 2) ||
      !bytes16(v_head_stride, 2))
    return fail(MLA_ERR_MISALIGNED, "%s: addresses and strides must be multiples of 16 bytes",
                fn);
  const int64_t E = fp8 ? 16 : 8;
  const int64_t key_per_row = (nope + rope) / E;
  const int64_t v_per_row = fp8 ? vdim / E : 0;
  const int64_t rows = num_tokens * num_heads;
  const int64_t key_total = rows * key_per_row;
  const int64_t total = key_total + rows * v_per_row;
  if (total >= (int64_t(1) << 31) || num_heads > 0x7FFFFFFF)
    return fail(MLA_ERR_UNSUPPORTED, "%s: more than 2^31 output chunks; split the chunk", fn);
  PackArgs a;
  a.k_nope = static_cast<const uint16_t*>(k_nope);
  a.kn_ts = kn_tok_stride;
  a.kn_hs = kn_head_stride;
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.pe_ts = kpe_tok_stride;
  a.v = static_cast<const uint16_t*>(v);
  a.v_ts = v_tok_stride;
  a.v_hs = v_head_stride;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.key_out = key_out;
  a.v_out = static_cast<uint8_t*>(v_out);
  a.key_per_row = make_fastdiv(static_cast<uint32_t>(key_per_row));
  a.v_per_row = make_fastdiv(static_cast<uint32_t>(v_per_row > 0 ? v_per_row : 1));
  a.heads = make_fastdiv(static_cast<uint32_t>(num_heads));
  a.nope_chunks = static_cast<uint32_t>(nope / E);
  a.key_total = static_cast<uint32_t>(key_total);
  a.total = static_cast<uint32_t>(total);
  auto s = static_cast<hipStream_t>(stream);
  const int64_t full = ceil_div(total, 256);
  const int64_t blocks = max_blocks > 0 ? std::min(full, max_blocks) : full;
  const bool scaled = k_scale || v_scale;
  const dim3 g(blocks), b(256);
  if (!fp8)
    launch(pack_bf16_kernel, g, b, 0, s, a);
  else if (scaled)
    launch_pack_fp8<true>(f16, kpe_raw, g, b, s, a);
  else
    launch_pack_fp8<false>(f16, kpe_raw, g, b, s, a);
  return launch_status(fn);
}
