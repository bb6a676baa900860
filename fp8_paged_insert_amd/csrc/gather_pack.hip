// gather_pack.hip -- chunked-context gather from the paged latent cache, the
// full-key / fp8-V pack, and one launch that packs chunk c while gathering
// chunk c + 1.
//
// Page: "PR #51772 完整报告" ([Attention][MLA] Fuse Kimi-K3 chunked-context
// K/V packing).  实现拆解 item 1: one kernel per chunk reads the strided
// kv_b_proj halves (k_nope, v) and the gathered k_pe directly, writes a
// contiguous key [k_nope | k_pe] (and, for fp8, a contiguous fp8 V), with a
// capped grid and a grid-stride loop for long contexts.  实现拆解 item 2: the
// context latent is gathered from the cache before kv_b_proj (and the pack
// follows kv_b_proj), chunk after chunk; item 5: with a plain fp8 cache the
// gathered latent must reach a bf16 kv_b_proj as bf16.  关键源码片段
// (fused_mla_key_concat_kv_cache.py): output shapes and the bit-identity of
// the fp8 cast with torch's float8_e4m3fn cast.
//
// gfx950 design: both kernels walk a flat list of 16-byte output chunks, so
// every store is a full 16-byte vector and consecutive lanes write
// consecutive addresses of the contiguous outputs; loads are 16/32-byte
// vectors along the contiguous rows of the strided inputs.  The k_pe row of
// a token is read once per head from L2 (it is 128 bytes shared by H heads).
#include <algorithm>

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

template <int kKind>
__device__ __forceinline__ float gather_scale(const GatherArgs& a) {
  if constexpr (kKind == kGatherDequant || kKind == kGatherDequantE5M2) return a.scale[0];
  return 1.0f;
}

// One 16-byte cache chunk (item = token * per_row + chunk) into the workspace.
template <int kKind>
__device__ __forceinline__ void gather_item(const GatherArgs& a, uint32_t item, float sc) {
  constexpr bool kFp8 = kKind != kGatherCopy16;      // cache holds 1-byte codes
  constexpr int E = kFp8 ? 16 : 8;                   // cache elements per chunk
  constexpr int kOutBytes = kKind == kGatherRaw8 ? 1 : 2;
  constexpr bool kDequant = kKind == kGatherDequant || kKind == kGatherDequantE5M2;
  constexpr bool kE5M2 = kKind == kGatherDequantE5M2;
  const uint32_t jj = fdiv(item, a.per_row);
  const uint32_t cc = item - jj * a.per_row.d;
  const int64_t s = a.slots[jj];
  int64_t blk, off;
  if (s < 0x80000000LL) {
    const uint32_t b32 = fdiv(static_cast<uint32_t>(s), a.bsize);
    blk = b32;
    off = static_cast<uint32_t>(s) - b32 * a.bsize.d;
  } else {
    blk = s / a.block_size;
    off = s - blk * a.block_size;
  }
  const int64_t src_el = blk * a.block_stride + off * a.entry_stride + int64_t(cc) * E;
  const uint4 q = kFp8 ? ld16(a.cache + src_el)
                       : ld16(reinterpret_cast<const uint16_t*>(a.cache) + src_el);
  uint8_t* dst = static_cast<uint8_t*>(a.out) + (int64_t(jj) * a.width + int64_t(cc) * E) * kOutBytes;
  if constexpr (kDequant) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
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
    st16<kGatherStream>(dst, q);
  }
}

template <int kKind>
__global__ __launch_bounds__(256) void gather_kernel(const GatherArgs a) {
  const float sc = gather_scale<kKind>(a);
  for (uint32_t item = blockIdx.x * blockDim.x + threadIdx.x; item < a.total;
       item += gridDim.x * blockDim.x)
    gather_item<kKind>(a, item, sc);
}

// ------------------------------------------------------------------- pack --
// The outputs are cut into 16-byte chunks, numbered key chunks of every
// token first (row (t, h), chunk j), then V chunks; chunk i is written at
// byte 16 i of its output, so consecutive lanes write consecutive addresses.
// The default grid has one thread per chunk (no loop): the workgroups in
// flight then sweep the strided kv_b_proj output and the contiguous outputs
// as one advancing window; a caller-given max_blocks caps the grid and each
// thread loops grid-stride.
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

// Source of key chunk `item` (row (t, h) = item / key_per_row); `rope` tells
// whether it is one of the rope chunks.
template <int E>
__device__ __forceinline__ const uint16_t* key_src(const PackArgs& a, uint32_t item, bool& rope) {
  const uint32_t row = fdiv(item, a.key_per_row);
  const uint32_t j = item - row * a.key_per_row.d;
  const uint32_t t = fdiv(row, a.heads);
  const uint32_t h = row - t * a.heads.d;
  rope = j >= a.nope_chunks;
  return rope ? a.k_pe + int64_t(t) * a.pe_ts + (j - a.nope_chunks) * E
              : a.k_nope + int64_t(t) * a.kn_ts + int64_t(h) * a.kn_hs + j * E;
}

// The 16-bit key: 8 values per chunk, copied.
struct PackBf16 {
  struct Load {
    uint4 x;
    uint32_t item;
  };
  __device__ __forceinline__ explicit PackBf16(const PackArgs&) {}
  __device__ __forceinline__ Load load(const PackArgs& a, uint32_t item) const {
    bool rope;
    return Load{ld16(key_src<8>(a, item, rope)), item};
  }
  __device__ __forceinline__ void store(const PackArgs& a, const Load& l) const {
    st16<kPackStream>(static_cast<uint16_t*>(a.key_out) + int64_t(l.item) * 8, l.x);
  }
};

// fp8 key and V: 16 values per chunk.  kF16: the 16-bit inputs are IEEE fp16
// (else bf16).  kKpeRaw: k_pe holds e4m3fn codes (pe_ts in bytes), copied
// into the key's rope chunks unchanged.
template <bool kScaled, bool kF16, bool kKpeRaw>
struct PackFp8 {
  struct Load {
    uint4 x0, x1;
    uint8_t* dst;
    bool is_key, raw;
  };
  float ks = 1.0f, vs = 1.0f, kr, vr;
  uint32_t kf, vf;
  __device__ __forceinline__ explicit PackFp8(const PackArgs& a) {
    if constexpr (kScaled) {
      if (a.k_scale) ks = a.k_scale[0];
      if (a.v_scale) vs = a.v_scale[0];
    }
    kr = 1.0f / ks;
    vr = 1.0f / vs;
    kf = sign_flip_of(ks);
    vf = sign_flip_of(vs);
  }
  __device__ __forceinline__ Load load(const PackArgs& a, uint32_t item) const {
    constexpr int E = 16;
    Load l;
    const uint16_t* src;
    l.raw = false;
    l.is_key = item < a.key_total;
    if (l.is_key) {
      l.dst = static_cast<uint8_t*>(a.key_out) + int64_t(item) * E;
      bool rope;
      src = key_src<E>(a, item, rope);
      if constexpr (kKpeRaw) {
        // a raw rope chunk: 16 one-byte codes at byte offset 16 (j - nope_chunks)
        l.raw = rope;
        if (rope) {
          const uint32_t row = fdiv(item, a.key_per_row);
          const uint32_t j = item - row * a.key_per_row.d;
          const uint32_t t = fdiv(row, a.heads);
          src = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.k_pe) +
                                                  int64_t(t) * a.pe_ts + (j - a.nope_chunks) * E);
        }
      }
    } else {
      const uint32_t vi = item - a.key_total;
      const uint32_t row = fdiv(vi, a.v_per_row);
      const uint32_t j = vi - row * a.v_per_row.d;
      const uint32_t t = fdiv(row, a.heads);
      const uint32_t h = row - t * a.heads.d;
      src = a.v + int64_t(t) * a.v_ts + int64_t(h) * a.v_hs + j * E;
      l.dst = a.v_out + int64_t(vi) * E;
    }
    l.x0 = ld16_once(src);
    l.x1 = (kKpeRaw && l.raw) ? make_uint4(0, 0, 0, 0) : ld16_once(src + 8);
    return l;
  }
  __device__ __forceinline__ void store(const PackArgs&, const Load& l) const {
    if (kKpeRaw && l.raw) {
      st16<kPackStream>(l.dst, l.x0);   // 16 codes, as they are
      return;
    }
    st16<kPackStream>(l.dst, quant16<kScaled, kF16>(l.x0, l.x1, l.is_key ? ks : vs,
                                                    l.is_key ? kr : vr, l.is_key ? kf : vf));
  }
};

// Chunks first, first + stride, ... below a.total, software-pipelined: the
// next chunk's loads are issued before the current chunk is converted and
// stored (the compiler cannot move them above that store by itself, since
// it cannot rule out aliasing), so with a capped grid a thread keeps its
// next loads in flight while it converts.
template <class Op>
__device__ __forceinline__ void pack_loop(const PackArgs& a, const Op& op, uint32_t first,
                                          uint32_t stride) {
  if (first >= a.total) return;
  auto cur = op.load(a, first);
  for (uint32_t item = first + stride; item < a.total; item += stride) {
    const auto nxt = op.load(a, item);
    op.store(a, cur);
    cur = nxt;
  }
  op.store(a, cur);
}

template <class Op>
__global__ __launch_bounds__(256) void pack_kernel(const PackArgs a) {
  const Op op(a);
  pack_loop(a, op, blockIdx.x * blockDim.x + threadIdx.x, gridDim.x * blockDim.x);
}

// -------------------------------------------------- pack c + gather c + 1 --
// Workgroups [gather_first, gather_first + gather_blocks) gather, the rest
// pack; the two sets of chunks are independent (the gather writes a
// workspace the pack does not touch), so the gather's short, latency-bound
// reads run under the pack's stream instead of in a launch of their own.
// gather_first is 0 (the gather's workgroups start first) or the number of
// pack workgroups (they start last).
template <class Op, int kKind>
__global__ __launch_bounds__(256) void pack_gather_kernel(const PackArgs a, const GatherArgs g,
                                                          uint32_t gather_first,
                                                          uint32_t gather_blocks) {
  const uint32_t gb = blockIdx.x - gather_first;  // wraps above gather_blocks when below
  if (gb < gather_blocks) {
    const float sc = gather_scale<kKind>(g);
    for (uint32_t item = gb * blockDim.x + threadIdx.x; item < g.total;
         item += gather_blocks * blockDim.x)
      gather_item<kKind>(g, item, sc);
    return;
  }
  const Op op(a);
  const uint32_t pb = blockIdx.x < gather_first ? blockIdx.x : blockIdx.x - gather_blocks;
  pack_loop(a, op, pb * blockDim.x + threadIdx.x, (gridDim.x - gather_blocks) * blockDim.x);
}

// ------------------------------------------------------- host validation --
struct PackPlan {
  PackArgs a;
  bool fp8, kpe_raw, f16, scaled;
  int64_t full_blocks;  // one thread per chunk
};

struct GatherPlan {
  GatherArgs a;
  int kind;
  int64_t blocks;  // one thread per chunk
};

// Validates the pack's arguments and fills plan; MLA_OK with plan->a.total 0
// when there is nothing to do.
int32_t plan_pack(const char* fn, const void* k_nope, int64_t kn_tok_stride,
                  int64_t kn_head_stride, const void* k_pe, int64_t kpe_tok_stride,
                  const void* v, int64_t v_tok_stride, int64_t v_head_stride,
                  int64_t num_tokens, int64_t num_heads, int64_t nope, int64_t rope,
                  int64_t vdim, int32_t mode, int32_t src_dtype, const float* k_scale,
                  const float* v_scale, void* key_out, void* v_out, int64_t max_blocks,
                  PackPlan* plan) {
  plan->a.total = 0;
  if (mode != MLA_PACK_KEY_BF16 && mode != MLA_PACK_KEY_V_FP8 &&
      mode != MLA_PACK_KEY_V_FP8_KPE_RAW)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: unknown mode %d", fn, mode);
  if (src_dtype != MLA_KV_BF16 && src_dtype != MLA_KV_FP16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: src_dtype must be bf16 or fp16", fn);
  const bool fp8 = mode != MLA_PACK_KEY_BF16;
  const bool kpe_raw = mode == MLA_PACK_KEY_V_FP8_KPE_RAW;
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
  PackArgs& a = plan->a;
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
  plan->fp8 = fp8;
  plan->kpe_raw = kpe_raw;
  plan->f16 = src_dtype == MLA_KV_FP16;
  plan->scaled = k_scale || v_scale;
  plan->full_blocks = ceil_div(total, 256);
  return MLA_OK;
}

int32_t plan_gather(const char* fn, const void* cache, int32_t cache_dtype,
                    const float* cache_scale, int64_t block_size, int64_t block_stride,
                    int64_t entry_stride, const int64_t* src_slots, int64_t num_tokens,
                    int64_t width, int32_t out_dtype, void* out, int64_t max_blocks,
                    GatherPlan* plan) {
  plan->a.total = 0;
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
  GatherArgs& a = plan->a;
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
  plan->kind = raw ? kGatherRaw8
                   : cache_dtype == MLA_KV_FP8_E5M2 ? kGatherDequantE5M2
                                                    : fp8 ? kGatherDequant : kGatherCopy16;
  plan->blocks = ceil_div(total, 256);
  return MLA_OK;
}

template <bool kScaled>
void launch_pack_fp8(const PackPlan& p, dim3 g, hipStream_t s) {
  const dim3 b(256);
  if (p.f16 && p.kpe_raw)
    launch(pack_kernel<PackFp8<kScaled, true, true>>, g, b, 0, s, p.a);
  else if (p.f16)
    launch(pack_kernel<PackFp8<kScaled, true, false>>, g, b, 0, s, p.a);
  else if (p.kpe_raw)
    launch(pack_kernel<PackFp8<kScaled, false, true>>, g, b, 0, s, p.a);
  else
    launch(pack_kernel<PackFp8<kScaled, false, false>>, g, b, 0, s, p.a);
}

template <class Op>
void launch_pack_gather(const PackPlan& p, const GatherPlan& q, int64_t pack_blocks,
                        hipStream_t s) {
  const dim3 g(static_cast<uint32_t>(pack_blocks + q.blocks)), b(256);
  const uint32_t gb = static_cast<uint32_t>(q.blocks);
  // Where the gather's workgroups go (measured on MI355X, 8192-token chunks
  // of 64 heads): first on the full pack grid (one chunk per thread), where
  // their latency-bound reads then overlap the whole pack; last on a capped
  // grid, whose workgroups loop over several chunks and would otherwise
  // start behind them.
  const uint32_t first = pack_blocks < p.full_blocks ? static_cast<uint32_t>(pack_blocks) : 0u;
  switch (q.kind) {
    case kGatherCopy16:
      launch(pack_gather_kernel<Op, kGatherCopy16>, g, b, 0, s, p.a, q.a, first, gb);
      break;
    case kGatherDequant:
      launch(pack_gather_kernel<Op, kGatherDequant>, g, b, 0, s, p.a, q.a, first, gb);
      break;
    case kGatherRaw8:
      launch(pack_gather_kernel<Op, kGatherRaw8>, g, b, 0, s, p.a, q.a, first, gb);
      break;
    default:
      launch(pack_gather_kernel<Op, kGatherDequantE5M2>, g, b, 0, s, p.a, q.a, first, gb);
      break;
  }
}

// [lo, hi) byte range touched through a strided 2-D/3-D view (elements of
// `eb` bytes): the last element's end.
struct Span {
  uintptr_t lo, hi;
};
Span span3(const void* p, int64_t eb, int64_t n0, int64_t s0, int64_t n1, int64_t s1,
           int64_t n2) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  const int64_t last = (n0 - 1) * s0 + (n1 - 1) * s1 + n2;
  return Span{lo, lo + static_cast<uintptr_t>(last * eb)};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

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
  GatherPlan q;
  const int32_t st = plan_gather(fn, cache, cache_dtype, cache_scale, block_size, block_stride,
                                 entry_stride, src_slots, num_tokens, width, out_dtype, out,
                                 max_blocks, &q);
  if (st != MLA_OK || q.a.total == 0) return st;
  const int64_t cap = max_blocks > 0 ? max_blocks : default_grid_cap();
  const dim3 g(static_cast<uint32_t>(std::max<int64_t>(1, std::min(q.blocks, cap)))), b(256);
  auto s = static_cast<hipStream_t>(stream);
  switch (q.kind) {
    case kGatherRaw8: launch(gather_kernel<kGatherRaw8>, g, b, 0, s, q.a); break;
    case kGatherDequantE5M2: launch(gather_kernel<kGatherDequantE5M2>, g, b, 0, s, q.a); break;
    case kGatherDequant: launch(gather_kernel<kGatherDequant>, g, b, 0, s, q.a); break;
    default: launch(gather_kernel<kGatherCopy16>, g, b, 0, s, q.a); break;
  }
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
  PackPlan p;
  const int32_t st = plan_pack(fn, k_nope, kn_tok_stride, kn_head_stride, k_pe, kpe_tok_stride,
                               v, v_tok_stride, v_head_stride, num_tokens, num_heads, nope, rope,
                               vdim, mode, src_dtype, k_scale, v_scale, key_out, v_out,
                               max_blocks, &p);
  if (st != MLA_OK || p.a.total == 0) return st;
  auto s = static_cast<hipStream_t>(stream);
  const int64_t blocks = max_blocks > 0 ? std::min(p.full_blocks, max_blocks) : p.full_blocks;
  const dim3 g(static_cast<uint32_t>(blocks));
  if (!p.fp8)
    launch(pack_kernel<PackBf16>, g, dim3(256), 0, s, p.a);
  else if (p.scaled)
    launch_pack_fp8<true>(p, g, s);
  else
    launch_pack_fp8<false>(p, g, s);
  return launch_status(fn);
}

extern "C" int32_t mla_ctx_kv_pack_gather(
    const void* k_nope, int64_t kn_tok_stride, int64_t kn_head_stride, const void* k_pe,
    int64_t kpe_tok_stride, const void* v, int64_t v_tok_stride, int64_t v_head_stride,
    int64_t num_tokens, int64_t num_heads, int64_t nope, int64_t rope, int64_t vdim,
    int32_t mode, int32_t src_dtype, const float* k_scale, const float* v_scale, void* key_out,
    void* v_out, const void* cache, int32_t cache_dtype, const float* cache_scale,
    int64_t block_size, int64_t block_stride, int64_t entry_stride, const int64_t* src_slots,
    int64_t gather_tokens, int64_t width, int32_t out_dtype, void* gather_out,
    int64_t max_blocks, mla_stream_t stream) {
  static const char* fn = "mla_ctx_kv_pack_gather";
  clear_error();
  PackPlan p;
  GatherPlan q;
  int32_t st = plan_pack(fn, k_nope, kn_tok_stride, kn_head_stride, k_pe, kpe_tok_stride, v,
                         v_tok_stride, v_head_stride, num_tokens, num_heads, nope, rope, vdim,
                         mode, src_dtype, k_scale, v_scale, key_out, v_out, max_blocks, &p);
  if (st != MLA_OK) return st;
  st = plan_gather(fn, cache, cache_dtype, cache_scale, block_size, block_stride, entry_stride,
                   src_slots, gather_tokens, width, out_dtype, gather_out, 0, &q);
  if (st != MLA_OK) return st;
  if (p.a.total == 0 && q.a.total == 0) return MLA_OK;
  if (p.a.total > 0 && q.a.total > 0) {
    // the gather's output must not overlap anything the pack reads or writes
    const int64_t ob = out_dtype == MLA_KV_BF16 ? 2 : 1;
    const Span w = span3(gather_out, ob, 1, 0, gather_tokens, width, width);
    const int64_t kpe_eb = p.kpe_raw ? 1 : 2;
    const int64_t key_eb = p.fp8 ? 1 : 2;
    const Span pack_spans[5] = {
        span3(k_nope, 2, num_tokens, kn_tok_stride, num_heads, kn_head_stride, nope),
        span3(k_pe, kpe_eb, 1, 0, num_tokens, kpe_tok_stride, rope),
        span3(v, 2, num_tokens, v_tok_stride, num_heads, v_head_stride, p.fp8 ? vdim : 0),
        span3(key_out, key_eb, 1, 0, num_tokens * num_heads, nope + rope, nope + rope),
        span3(v_out, 1, 1, 0, num_tokens * num_heads, vdim, p.fp8 ? vdim : 0)};
    for (int i = 0; i < 5; ++i) {
      const bool present = i < 2 || (i == 3) || (p.fp8 && vdim > 0);
      if (present && pack_spans[i].hi > pack_spans[i].lo && overlap(w, pack_spans[i]))
        return fail(MLA_ERR_INVALID_ARGUMENT,
                    "%s: gather_out overlaps an input or output of the pack", fn);
    }
    if (p.kpe_raw || p.f16)
      return fail(MLA_ERR_UNSUPPORTED,
                  "%s: the joint launch takes bf16 sources and a 16-bit k_pe; "
                  "call mla_ctx_kv_pack and mla_ctx_latent_gather", fn);
  }
  const int64_t pack_blocks = max_blocks > 0 ? std::min(p.full_blocks, max_blocks) : p.full_blocks;
  if (pack_blocks + q.blocks > 0x7FFFFFFF)
    return fail(MLA_ERR_UNSUPPORTED, "%s: too many chunks for one launch", fn);
  auto s = static_cast<hipStream_t>(stream);
  if (q.a.total == 0)
    return mla_ctx_kv_pack(k_nope, kn_tok_stride, kn_head_stride, k_pe, kpe_tok_stride, v,
                           v_tok_stride, v_head_stride, num_tokens, num_heads, nope, rope, vdim,
                           mode, src_dtype, k_scale, v_scale, key_out, v_out, max_blocks, stream);
  if (p.a.total == 0)
    return mla_ctx_latent_gather(cache, cache_dtype, cache_scale, block_size, block_stride,
                                 entry_stride, src_slots, gather_tokens, width, out_dtype,
                                 gather_out, 0, stream);
  if (!p.fp8)
    launch_pack_gather<PackBf16>(p, q, pack_blocks, s);
  else if (p.scaled)
    launch_pack_gather<PackFp8<true, false, false>>(p, q, pack_blocks, s);
  else
    launch_pack_gather<PackFp8<false, false, false>>(p, q, pack_blocks, s);
  return launch_status(fn);
}
