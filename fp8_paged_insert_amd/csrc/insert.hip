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
// gfx950 design (not the page's one-workgroup-per-(token, layer) grid): for
// the MLA row (512 + 64) a row belongs to 16 lanes, so one wavefront moves 4
// adjacent rows with 128-256-byte contiguous accesses per instruction and
// issues all of a row's loads, slot included, before its stores; other row
// shapes take a flat list of 16-byte output chunks, one per thread.
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

// Any other row shape (kv_lora_rank and pe_dim multiples of 16): one thread
// per 16-byte output chunk.  kFmt (CacheFmt): fp8 caches take 16 bf16 in ->
// 16 e4m3fn or e5m2 codes out per
// chunk; else 8 bf16 copied.
template <int kFmt>
__global__ __launch_bounds__(256) void grouped_insert_kernel(const InsertArgs a) {
  constexpr bool kFp8 = kFmt != kFmtBf16, kE5M2 = kFmt == kFmtE5M2;
  constexpr int E = kFp8 ? 16 : 8;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t item = blockIdx.x * blockDim.x + threadIdx.x; item < a.total; item += stride) {
    const uint32_t row = fdiv(item, a.per_row);
    const uint32_t j = item - row * a.per_row.d;
    const uint32_t l = fdiv(row, a.tokens);
    const uint32_t t = row - l * a.tokens.d;
    const int64_t s = a.slots[int64_t(l) * a.sls + t];
    const int64_t cbase = a.cache_ptrs[l];
    float sc = 1.0f;
    if constexpr (kFp8) sc = a.scales[l];
    const uint16_t* src;
    int64_t col;
    if (j < a.chunks_r) {
      col = int64_t(j) * E;
      src = a.kv_c + int64_t(l) * a.kv_ls + int64_t(t) * a.kv_ts + col;
    } else {
      const int64_t jj = int64_t(j - a.chunks_r) * E;
      src = a.k_pe + int64_t(l) * a.pe_ls + int64_t(t) * a.pe_ts + jj;
      col = a.R + jj;
    }
    const uint4 v0 = ld16(src);
    uint4 v1 = v0;
    if constexpr (kFp8) v1 = ld16(src + 8);
    if (s < 0) continue;  // negative slot: skip
    int64_t blk, off;
    if (s < 0x80000000LL) {
      const uint32_t b32 = fdiv(static_cast<uint32_t>(s), a.bsize);
      blk = b32;
      off = static_cast<uint32_t>(s) - b32 * a.bsize.d;
    } else {
      blk = s / a.block_size;
      off = s - blk * a.block_size;
    }
    const int64_t dst_off = blk * a.block_stride + off * a.entry_stride + col;
    if constexpr (kFp8) {
      const float rc = 1.0f / sc;  // IEEE division: RN(1 / scale)
      st16<kInsertStream>(reinterpret_cast<uint8_t*>(cbase) + dst_off,
                          quant16<true, false, kE5M2>(v0, v1, sc, rc, sign_flip_of(sc)));
    } else {
      st16<kInsertStream>(reinterpret_cast<uint16_t*>(cbase) + dst_off, v0);
    }
  }
}

// Rows of the MLA shape (kv_lora_rank 512, pe_dim 64): a row belongs to
// kLanes lanes, lane j moving kv_c chunks j, j + kLanes, ... (8 values each)
// and k_pe[(64 / kLanes) j, (64 / kLanes) (j + 1)), so each load and store
// instruction covers 128-256 contiguous bytes of a row.  A wavefront takes
// 64 / kLanes adjacent rows and issues every load -- slot, cache base, scale
// and sources -- before its first store.
constexpr int kRowR = 512, kRowP = 64;

struct RowInsertArgs {
  const uint16_t* kv_c;
  int64_t kv_ls, kv_ts;
  const uint16_t* k_pe;
  int64_t pe_ls, pe_ts;
  const int64_t* cache_ptrs;
  const float* scales;
  const int64_t* slots;
  int64_t sls;
  int64_t block_size, block_stride, entry_stride;  // in cache elements
  FastDiv tokens, bsize;
  uint32_t rows;
};

template <int kFmt, int kLanes>
__global__ __launch_bounds__(256) void row_insert_kernel(const RowInsertArgs a) {
  constexpr bool kFp8 = kFmt != kFmtBf16, kE5M2 = kFmt == kFmtE5M2;
  constexpr int kChunks = kRowR / 8 / kLanes;  // 16-byte kv_c chunks per lane
  constexpr int kPe = kRowP / kLanes;          // k_pe values per lane (4 or 2)
  constexpr int kRowsPerWave = 64 / kLanes;
  static_assert(kPe == 4 || kPe == 2, "k_pe is moved as 4 or 2 values per lane");
  const int lane = threadIdx.x & 63;
  const int j = lane % kLanes;
  const uint32_t wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  for (uint32_t r0 = wave * kRowsPerWave; r0 < a.rows; r0 += gridDim.x * 4 * kRowsPerWave) {
    const uint32_t r = r0 + lane / kLanes;
    const uint32_t rr = min(r, a.rows - 1);   // idle lanes load in bounds
    const uint32_t l = fdiv(rr, a.tokens);
    const uint32_t t = rr - l * a.tokens.d;
    const int64_t s = a.slots[int64_t(l) * a.sls + t];
    const int64_t cb = a.cache_ptrs[l];
    float sc = 1.0f;
    if constexpr (kFp8) sc = a.scales[l];
    const uint16_t* src = a.kv_c + int64_t(l) * a.kv_ls + int64_t(t) * a.kv_ts;
    uint4 v[kChunks];
#pragma unroll
    for (int q = 0; q < kChunks; ++q) v[q] = ld16(src + 8 * (j + kLanes * q));
    const uint16_t* pesrc = a.k_pe + int64_t(l) * a.pe_ls + int64_t(t) * a.pe_ts + kPe * j;
    uint2 pe;
    if constexpr (kPe == 4) {
      pe = *reinterpret_cast<const uint2*>(pesrc);
    } else {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(pesrc);
      pe = make_uint2(w, w);
    }
    // Every load stays ahead of the slot test: without this fence the
    // compiler waits for the slot and issues the source loads in the branch.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (r >= a.rows || s < 0) continue;  // negative slot: skip
    int64_t blk, off;
    if (s < 0x80000000LL) {
      const uint32_t b32 = fdiv(static_cast<uint32_t>(s), a.bsize);
      blk = b32;
      off = static_cast<uint32_t>(s) - b32 * a.bsize.d;
    } else {
      blk = s / a.block_size;
      off = s - blk * a.block_size;
    }
    const int64_t entry = blk * a.block_stride + off * a.entry_stride;
    if constexpr (kFp8) {
      const float rc = 1.0f / sc;  // IEEE division: RN(1 / scale)
      const uint32_t flip = sign_flip_of(sc);
      uint8_t* dst = reinterpret_cast<uint8_t*>(cb) + entry;
#pragma unroll
      for (int q = 0; q < kChunks; ++q)
        st8<kInsertStream>(dst + 8 * (j + kLanes * q), quant8<true, false, kE5M2>(v[q], sc, rc, flip));
      const uint32_t c = quant4<true, kE5M2>(pe, sc, rc, flip);
      if constexpr (kPe == 4)
        st4<kInsertStream>(dst + kRowR + 4 * j, c);
      else
        st2(dst + kRowR + 2 * j, static_cast<uint16_t>(c));
    } else {
      uint16_t* dst = reinterpret_cast<uint16_t*>(cb) + entry;
#pragma unroll
      for (int q = 0; q < kChunks; ++q) st16<kInsertStream>(dst + 8 * (j + kLanes * q), v[q]);
      if constexpr (kPe == 4)
        st8<kInsertStream>(dst + kRowR + 4 * j, pe);
      else
        st4<kInsertStream>(dst + kRowR + 2 * j, pe.x);
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
  const int fmt = cache_fmt(kv_cache_dtype);
  const int64_t E = fp8 ? 16 : 8;
  if (kv_lora_rank % 16 != 0 || pe_dim % 16 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "%s: kv_lora_rank and pe_dim must be multiples of 16", fn);
  if (!kv_c || (pe_dim > 0 && !k_pe))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: kv_c / k_pe must not be NULL", fn);
  if (!aligned16(kv_c) || !bytes16(kv_c_layer_stride, 2) || !bytes16(kv_c_token_stride, 2) ||
      (pe_dim > 0 && (!aligned16(k_pe) || !bytes16(k_pe_layer_stride, 2) ||
                      !bytes16(k_pe_token_stride, 2))))
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

  auto s = static_cast<hipStream_t>(stream);
  if (kv_lora_rank == kRowR && pe_dim == kRowP) {
    // 16 lanes per row measured faster than 32 lanes, or than 16 lanes
    // moving 2 or 4 rows each, on the 5 x 16384-row workload
    constexpr int kLanes = 16;
    RowInsertArgs b;
    b.kv_c = a.kv_c;
    b.kv_ls = a.kv_ls;
    b.kv_ts = a.kv_ts;
    b.k_pe = a.k_pe;
    b.pe_ls = a.pe_ls;
    b.pe_ts = a.pe_ts;
    b.cache_ptrs = a.cache_ptrs;
    b.scales = a.scales;
    b.slots = a.slots;
    b.sls = a.sls;
    b.block_size = a.block_size;
    b.block_stride = a.block_stride;
    b.entry_stride = a.entry_stride;
    b.tokens = a.tokens;
    b.bsize = a.bsize;
    b.rows = static_cast<uint32_t>(num_layers * num_tokens);
    const int64_t blocks = ceil_div(num_layers * num_tokens, 4 * (64 / kLanes));
    if (fmt == kFmtE5M2)
      launch((row_insert_kernel<kFmtE5M2, kLanes>), dim3(blocks), dim3(256), 0, s, b);
    else if (fmt == kFmtE4M3)
      launch((row_insert_kernel<kFmtE4M3, kLanes>), dim3(blocks), dim3(256), 0, s, b);
    else
      launch((row_insert_kernel<kFmtBf16, kLanes>), dim3(blocks), dim3(256), 0, s, b);
    return launch_status(fn);
  }
  const int64_t blocks = ceil_div(total, 256);
  if (fmt == kFmtE5M2)
    launch(grouped_insert_kernel<kFmtE5M2>, dim3(blocks), dim3(256), 0, s, a);
  else if (fmt == kFmtE4M3)
    launch(grouped_insert_kernel<kFmtE4M3>, dim3(blocks), dim3(256), 0, s, a);
  else
    launch(grouped_insert_kernel<kFmtBf16>, dim3(blocks), dim3(256), 0, s, a);
  return launch_status(fn);
}
