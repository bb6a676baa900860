// insert.hip -- grouped concat-and-cache of the MLA latent KV over all draft
// layers in one launch.
//
// Page: "PR #55356 完整报告" ([Kimi Perf] Group fp8 mla cache insertion),
// sections 功能与动机 (one launch instead of one per layer), 实现拆解 items 2-3
// (per-layer cache base addresses and scales held in device arrays; bf16 copy
// or per-layer fp8 quantisation; host checks before launch) and 关键源码片段
// (cache_kernels.cu: slot -> block / offset addressing, negative slot skips,
// kv_c at element 0 and k_pe at element kv_lora_rank of the entry).
//
// gfx950 design (not the page's one-workgroup-per-(token, layer) grid): the
// work is a flat list of 16-byte output chunks, chunk = (layer, token, j).
// Consecutive lanes take consecutive chunks of one cache entry, so every
// entry is read with coalesced 16/32-byte loads and written with 16-byte
// stores, no lane idles on the 576-element width, and one capped grid walks
// the list grid-stride for any token count.
#include "mla_common.hpp"

namespace mla {
namespace {

struct InsertArgs {
  const uint16_t* kv_c;
  int64_t kv_ls, kv_ts;
  const uint16_t* k_pe;
  int64_t pe_ls, pe_ts;
  const int64_t* cache_ptrs;
  const float* scales;
  const int64_t* slots;
  int64_t sls;
  int64_t R;  // kv_lora_rank
  int64_t block_size, block_stride, entry_stride;  // in cache elements
  FastDiv per_row;   // chunks per (layer, token) row
  FastDiv tokens;    // num_tokens
  FastDiv bsize;     // block_size (valid for slots < 2^31)
  uint32_t chunks_r;  // chunks covering kv_c
  uint32_t total;     // layers * tokens * chunks per row
};

// kFp8: 16 bf16 in -> 16 e4m3fn codes out per chunk; else 8 bf16 copied.
// Each thread takes U chunks per pass (item, item + stride, ...): the slot,
// cache-base and scale loads and the source loads of all U chunks are issued
// before the first store, so the slot -> store dependence overlaps U times.
template <bool kFp8, int U>
__global__ __launch_bounds__(256) void grouped_insert_kernel(const InsertArgs a) {
  constexpr int E = kFp8 ? 16 : 8;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t base = blockIdx.x * blockDim.x + threadIdx.x; base < a.total;
       base += U * stride) {
    int64_t s[U], col[U], cbase[U];
    float sc[U];
    uint4 v0[U], v1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t item = base + u * stride;
      if (item >= a.total) continue;
      const uint32_t row = fdiv(item, a.per_row);
      const uint32_t j = item - row * a.per_row.d;
      const uint32_t l = fdiv(row, a.tokens);
      const uint32_t t = row - l * a.tokens.d;
      s[u] = a.slots[int64_t(l) * a.sls + t];
      cbase[u] = a.cache_ptrs[l];
      if constexpr (kFp8) sc[u] = a.scales[l];
      const uint16_t* src;
      if (j < a.chunks_r) {
        col[u] = int64_t(j) * E;
        src = a.kv_c + int64_t(l) * a.kv_ls + int64_t(t) * a.kv_ts + col[u];
      } else {
        const int64_t jj = int64_t(j - a.chunks_r) * E;
        src = a.k_pe + int64_t(l) * a.pe_ls + int64_t(t) * a.pe_ts + jj;
        col[u] = a.R + jj;
      }
      v0[u] = ld16(src);
      if constexpr (kFp8) v1[u] = ld16(src + 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * stride >= a.total || s[u] < 0) continue;  // negative slot: skip
      int64_t blk, off;
      if (s[u] < 0x80000000LL) {
        const uint32_t b32 = fdiv(static_cast<uint32_t>(s[u]), a.bsize);
        blk = b32;
        off = static_cast<uint32_t>(s[u]) - b32 * a.bsize.d;
      } else {
        blk = s[u] / a.block_size;
        off = s[u] - blk * a.block_size;
      }
      const int64_t dst_off = blk * a.block_stride + off * a.entry_stride + col[u];
      if constexpr (kFp8) {
        const float rc = 1.0f / sc[u];  // IEEE division: RN(1 / scale)
        st16<kInsertStream>(reinterpret_cast<uint8_t*>(cbase[u]) + dst_off,
                            quant16<true>(v0[u], v1[u], sc[u], rc, sign_flip_of(sc[u])));
      } else {
        st16<kInsertStream>(reinterpret_cast<uint16_t*>(cbase[u]) + dst_off, v0[u]);
      }
    }
  }
}

}  // namespace

// Host validation shared with the epilogue: everything about the caches,
// slots and scales.  Returns MLA_OK or an error status.
int32_t check_insert_common(const char* fn, const int64_t* kv_cache_ptrs,
                            const float* kv_scales, const int64_t* slot_mapping,
                            int64_t num_layers, int64_t num_tokens, int64_t R, int64_t P,
                            int64_t block_size, int64_t block_stride, int64_t entry_stride,
                            int32_t dt) {
  int32_t st = check_cache_dtype(fn, dt, kv_scales);
  if (st != MLA_OK) return st;
  if (num_layers < 0 || num_tokens < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative num_layers (%lld) or num_tokens (%lld)",
                fn, (long long)num_layers, (long long)num_tokens);
  if (R <= 0 || P < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: kv_lora_rank must be > 0 and pe_dim >= 0", fn);
  if (block_size <= 0 || block_stride <= 0 || entry_stride <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "%s: block_size, block_stride and entry_stride must be positive", fn);
  if (entry_stride < R + P)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: entry_stride %lld is smaller than the entry width %lld",
                fn, (long long)entry_stride, (long long)(R + P));
  if (block_size > 1 && block_stride < (block_size - 1) * entry_stride + R + P)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: block_stride %lld lets entries of one block overlap the next",
                fn, (long long)block_stride);
  if (num_layers == 0 || num_tokens == 0) return MLA_OK;
  if (!kv_cache_ptrs || !slot_mapping)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: kv_cache_ptrs and slot_mapping must not be NULL", fn);
  const int64_t eb = is_fp8(dt) ? 1 : 2;
  if (!bytes16(block_stride, eb) || !bytes16(entry_stride, eb))
    return fail(MLA_ERR_MISALIGNED, "%s: block_stride and entry_stride must be multiples of 16 bytes", fn);
  return MLA_OK;
}

}  // namespace mla

using namespace mla;

extern "C" int32_t mla_kv_insert_grouped(
    const void* kv_c, int64_t kv_c_layer_stride, int64_t kv_c_token_stride,
    const void* k_pe, int64_t k_pe_layer_stride, int64_t k_pe_token_stride,
    const int64_t* kv_cache_ptrs, const float* kv_scales,
    const int64_t* slot_mapping, int64_t slot_layer_stride,
    int64_t num_layers, int64_t num_tokens, int64_t kv_lora_rank, int64_t pe_dim,
    int64_t block_size, int64_t block_stride, int64_t entry_stride,
    int32_t kv_cache_dtype, mla_stream_t stream) {
  static const char* fn = "mla_kv_insert_grouped";
  clear_error();
  int32_t st = check_insert_common(fn, kv_cache_ptrs, kv_scales, slot_mapping, num_layers,
                                   num_tokens, kv_lora_rank, pe_dim, block_size, block_stride,
                                   entry_stride, kv_cache_dtype);
  if (st != MLA_OK) return st;
  if (num_layers == 0 || num_tokens == 0) return MLA_OK;
  const bool fp8 = is_fp8(kv_cache_dtype);
  const int64_t E = fp8 ? 16 : 8;
  if (kv_lora_rank % 16 != 0 || pe_dim % 16 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "%s: kv_lora_rank and pe_dim must be multiples of 16", fn);
  if (!kv_c || (pe_dim > 0 && !k_pe))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: kv_c / k_pe must not be NULL", fn);
  if (!aligned16(kv_c) || !aligned16(k_pe) || !bytes16(kv_c_layer_stride, 2) ||
      !bytes16(kv_c_token_stride, 2) || !bytes16(k_pe_layer_stride, 2) ||
      !bytes16(k_pe_token_stride, 2))
    return fail(MLA_ERR_MISALIGNED,
                "%s: kv_c / k_pe addresses and strides must be multiples of 16 bytes", fn);
  const int64_t per_row = (kv_lora_rank + pe_dim) / E;
  const int64_t total = num_layers * num_tokens * per_row;
  if (num_layers > 0x7FFFFFFF || num_tokens > 0x7FFFFFFF || total >= (int64_t(1) << 31))
    return fail(MLA_ERR_UNSUPPORTED, "%s: %lld layers x %lld tokens exceed one launch", fn,
                (long long)num_layers, (long long)num_tokens);

  InsertArgs a;
  a.kv_c = static_cast<const uint16_t*>(kv_c);
  a.kv_ls = kv_c_layer_stride;
  a.kv_ts = kv_c_token_stride;
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.pe_ls = k_pe_layer_stride;
  a.pe_ts = k_pe_token_stride;
  a.cache_ptrs = kv_cache_ptrs;
  a.scales = kv_scales;
  a.slots = slot_mapping;
  a.sls = slot_layer_stride;
  a.R = kv_lora_rank;
  a.block_size = block_size;
  a.block_stride = block_stride;
  a.entry_stride = entry_stride;
  a.per_row = make_fastdiv(static_cast<uint32_t>(per_row));
  a.tokens = make_fastdiv(static_cast<uint32_t>(num_tokens));
  a.bsize = make_fastdiv(block_size < 0x7FFFFFFF ? static_cast<uint32_t>(block_size) : 1u);
  a.chunks_r = static_cast<uint32_t>(kv_lora_rank / E);
  a.total = static_cast<uint32_t>(total);

#ifndef MLA_INSERT_UNROLL
#define MLA_INSERT_UNROLL 1
#endif
  constexpr int U = MLA_INSERT_UNROLL;
#ifndef MLA_INSERT_CAP
#define MLA_INSERT_CAP 0
#endif
  const int64_t cap = MLA_INSERT_CAP > 0 ? MLA_INSERT_CAP * int64_t(cu_count())
                                         : int64_t(0x7FFFFFFF);
  const int64_t blocks = std::min<int64_t>(ceil_div(total, 256 * U), cap);
  auto s = static_cast<hipStream_t>(stream);
  if (fp8)
    launch((grouped_insert_kernel<true, U>), dim3(blocks), dim3(256), 0, s, a);
  else
    launch((grouped_insert_kernel<false, U>), dim3(blocks), dim3(256), 0, s, a);
  return launch_status(fn);
}
