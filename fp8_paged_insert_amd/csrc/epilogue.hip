// epilogue.hip -- fused context-KV epilogue for all draft layers in one
// launch: RMSNorm of kv_c with the layer's weight row, RoPE of k_pe at the
// token's position, bf16 rounding, fp8 (or bf16) conversion and the grouped
// paged-cache insert.
//
// Pages: "PR #50585 完整报告" ([K3 Perf] Optimize k3 dspark fused kv),
// 关键源码片段 (_precompute_fused_context_kv): the projection output is
// viewed as [num_ctx, L, 576], split into kv_c (512) and k_pe (64), RMSNorm
// uses a 2-D [L, 512] weight (one row per layer), RoPE uses the context
// positions repeated for every layer.  "PR #55356 完整报告" ([Kimi Perf]
// Group fp8 mla cache insertion), 关键源码片段 (dspark_mla.py and
// cache_kernels.cu): the normed / rotated rows then go through the grouped
// insert.
//
// gfx950 design: the pages run a permute + copy, a grouped RMSNorm, a
// flatten + RoPE and the grouped insert as separate passes over HBM; here one
// 64-lane wavefront owns one (layer, token) row end to end.  Each lane loads
// 8 kv_c values (one 16-byte load straight from the strided [T, L, 576]
// projection output, so no layer-major copy is made), the sum of squares is
// reduced across the wavefront, lanes 0-3 rotate the 64 k_pe values in
// (i, i + 32) pairs, and the row is converted and stored with 8/16-byte
// vector stores.  The token's position indexes the fp32 cos/sin table
// directly instead of a repeated-positions buffer.
#include "mla_common.hpp"

namespace mla {

int32_t check_insert_common(const char* fn, const int64_t* kv_cache_ptrs,
                            const float* kv_scales, const int64_t* slot_mapping,
                            int64_t num_layers, int64_t num_tokens, int64_t R, int64_t P,
                            int64_t block_size, int64_t block_stride, int64_t entry_stride,
                            int32_t dt);

namespace {

// -------------------------------------------------------------- rope table --
__global__ __launch_bounds__(256) void rope_table_kernel(float* out, int64_t max_pos,
                                                         int64_t rope_dim, double base) {
  const int64_t half = rope_dim / 2;
  const int64_t n = max_pos * half;
  for (int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; idx < n;
       idx += int64_t(gridDim.x) * blockDim.x) {
    const int64_t p = idx / half;
    const int64_t i = idx - p * half;
    const double theta = double(p) * pow(base, -2.0 * double(i) / double(rope_dim));
    out[p * rope_dim + i] = static_cast<float>(cos(theta));
    out[p * rope_dim + half + i] = static_cast<float>(sin(theta));
  }
}

// ---------------------------------------------------------------- epilogue --
constexpr int kR = 512;  // kv_lora_rank: lane i owns kv_c[8i, 8i + 8)
constexpr int kP = 64;   // rope dim: lane i owns k_pe[i]; lanes i and i ^ 32 pair up
#ifndef MLA_EPI_LAYERS
#define MLA_EPI_LAYERS 5
#endif
constexpr int kMaxLayers = MLA_EPI_LAYERS;  // layers one wavefront keeps in flight
constexpr int kWavesPerBlock = 4;

struct EpiArgs {
  const uint16_t* all_kv;
  int64_t kls, kts;
  const uint16_t* gamma;
  float eps;
  const int64_t* positions;
  const float* cos_sin;
  int64_t max_pos;
  const int64_t* cache_ptrs;
  const float* scales;
  const int64_t* slots;
  int64_t sls;
  int64_t block_size, block_stride, entry_stride;
  uint16_t* dbg;
  FastDiv bsize;
  uint32_t layers, tokens;
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int64_t entry_offset(int64_t s, const EpiArgs& a) {
  if (s < 0x80000000LL) {
    const uint32_t b32 = fdiv(static_cast<uint32_t>(s), a.bsize);
    return int64_t(b32) * a.block_stride +
           int64_t(static_cast<uint32_t>(s) - b32 * a.bsize.d) * a.entry_stride;
  }
  const int64_t blk = s / a.block_size;
  return blk * a.block_stride + (s - blk * a.block_size) * a.entry_stride;
}

// One wavefront owns one token and walks its layers in groups of up to
// kMaxLayers: every load of the group (the token's rows of all_kv are
// adjacent in the [T, L, 576] projection output) is issued before the first
// reduction.  RoPE pairs (i, i + 32) live in lanes i and i ^ 32, which swap
// values with one cross-half shuffle; the token's cos/sin row is read once
// (lane i holds cos_i for i < 32 and sin_{i-32} above) and shared by all
// layers.
template <bool kFp8>
__global__ __launch_bounds__(256) void epilogue_kernel(const EpiArgs a) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = threadIdx.x >> 6;
  const bool lo_half = lane < 32;
  for (uint32_t t = blockIdx.x * kWavesPerBlock + wave; t < a.tokens;
       t += gridDim.x * kWavesPerBlock) {
    const uint16_t* tok = a.all_kv + int64_t(t) * a.kts;
    // positions outside [0, max_pos) break the precondition; clamp so the
    // table read stays inside the table.
    const int64_t pos = min(max(a.positions[t], int64_t(0)), a.max_pos - 1);
    const float mine = a.cos_sin[pos * kP + lane];
    const float other = __shfl_xor(mine, 32, 64);
    const float c = lo_half ? mine : other;          // cos(theta_{lane mod 32})
    const float sn = lo_half ? -other : mine;        // -sin for the first half
    for (uint32_t l0 = 0; l0 < a.layers; l0 += kMaxLayers) {
      const int nl = min(kMaxLayers, int(a.layers - l0));
      uint4 xv[kMaxLayers], gv[kMaxLayers];
      uint32_t pe[kMaxLayers];
      int64_t sl[kMaxLayers], cb[kMaxLayers];
      float sc[kMaxLayers];
#pragma unroll
      for (int k = 0; k < kMaxLayers; ++k) {
        if (k >= nl) break;
        const uint32_t l = l0 + k;
        const uint16_t* row = tok + int64_t(l) * a.kls;
        xv[k] = ld16(row + lane * 8);
        gv[k] = ld16(a.gamma + int64_t(l) * kR + lane * 8);
        pe[k] = row[kR + lane];
        sl[k] = a.slots[int64_t(l) * a.sls + t];
        cb[k] = a.cache_ptrs[l];
        if constexpr (kFp8) sc[k] = a.scales[l];
      }
#pragma unroll
      for (int k = 0; k < kMaxLayers; ++k) {
        if (k >= nl) break;
        const uint32_t l = l0 + k;
        // ---- RMSNorm: fp32 sum of squares over the wavefront
        const uint32_t xw[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
        const uint32_t gw[4] = {gv[k].x, gv[k].y, gv[k].z, gv[k].w};
        float x[8], g[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = bf16_lo(xw[i]);
          x[2 * i + 1] = bf16_hi(xw[i]);
          g[2 * i] = bf16_lo(gw[i]);
          g[2 * i + 1] = bf16_hi(gw[i]);
        }
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(x[i], x[i], ss);
        ss = wave_sum(ss);
        const float rinv = 1.0f / __builtin_sqrtf(ss * (1.0f / kR) + a.eps);
        uint32_t yw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          yw[i] = cvt_bf16x2(x[2 * i] * rinv * g[2 * i], x[2 * i + 1] * rinv * g[2 * i + 1]);

        // ---- RoPE: y_i = x_i cos - x_{i+32} sin, y_{i+32} = x_{i+32} cos + x_i sin
        const float xp = bf16_lo(pe[k]);
        const float xq = __shfl_xor(xp, 32, 64);
        const uint32_t yp = cvt_bf16x2(xp * c + xq * sn, 0.0f) & 0xFFFFu;

        if (a.dbg) {
          uint16_t* d = a.dbg + (int64_t(l) * a.tokens + t) * (kR + kP);
          st16(d + lane * 8, make_uint4(yw[0], yw[1], yw[2], yw[3]));
          d[kR + lane] = static_cast<uint16_t>(yp);
        }
        // ---- insert (slot -> block, offset; a negative slot skips the row)
        if (sl[k] < 0) continue;
        const int64_t entry = entry_offset(sl[k], a);
        if constexpr (kFp8) {
          const float rc = 1.0f / sc[k];
          const uint32_t flip = sign_flip_of(sc[k]);
          uint8_t* dst = reinterpret_cast<uint8_t*>(cb[k]) + entry;
          st8<kEpiStream>(dst + lane * 8,
                          quant8<true>(make_uint4(yw[0], yw[1], yw[2], yw[3]), sc[k], rc, flip));
          dst[kR + lane] = static_cast<uint8_t>(quant1(bf16_lo(yp), sc[k], rc, flip));
        } else {
          uint16_t* dst = reinterpret_cast<uint16_t*>(cb[k]) + entry;
          st16<kEpiStream>(dst + lane * 8, make_uint4(yw[0], yw[1], yw[2], yw[3]));
          dst[kR + lane] = static_cast<uint16_t>(yp);
        }
      }
    }
  }
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int32_t mla_rope_cos_sin_cache(float* out, int64_t max_pos, int64_t rope_dim,
                                          double base, mla_stream_t stream) {
  static const char* fn = "mla_rope_cos_sin_cache";
  clear_error();
  if (max_pos < 0 || rope_dim <= 0 || (rope_dim & 1))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: need max_pos >= 0 and an even rope_dim > 0", fn);
  if (!(base > 0.0))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: base must be positive", fn);
  if (max_pos == 0) return MLA_OK;
  if (!out) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: out is NULL", fn);
  const int64_t n = max_pos * (rope_dim / 2);
  const int64_t blocks = std::min<int64_t>(ceil_div(n, 256), default_grid_cap());
  launch(rope_table_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, max_pos, rope_dim, base);
  return launch_status(fn);
}

extern "C" int32_t mla_ctx_kv_epilogue(
    const void* all_kv, int64_t kv_layer_stride, int64_t kv_token_stride, const void* gamma,
    float eps, const int64_t* positions, const float* cos_sin, int64_t max_pos,
    const int64_t* kv_cache_ptrs, const float* kv_scales, const int64_t* slot_mapping,
    int64_t slot_layer_stride, int64_t num_layers, int64_t num_tokens, int64_t kv_lora_rank,
    int64_t pe_dim, int64_t block_size, int64_t block_stride, int64_t entry_stride,
    int32_t kv_cache_dtype, void* dbg_rows, mla_stream_t stream) {
  static const char* fn = "mla_ctx_kv_epilogue";
  clear_error();
  int32_t st = check_insert_common(fn, kv_cache_ptrs, kv_scales, slot_mapping, num_layers,
                                   num_tokens, kv_lora_rank, pe_dim, block_size, block_stride,
                                   entry_stride, kv_cache_dtype);
  if (st != MLA_OK) return st;
  if (num_layers == 0 || num_tokens == 0) return MLA_OK;
  if (kv_lora_rank != kR || pe_dim != kP)
    return fail(MLA_ERR_UNSUPPORTED, "%s: kernel is built for kv_lora_rank 512 and pe_dim 64", fn);
  if (!all_kv || !gamma || !positions || !cos_sin)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL all_kv, gamma, positions or cos_sin", fn);
  if (max_pos <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: max_pos must be positive", fn);
  if (!(eps >= 0.0f)) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: eps must be >= 0", fn);
  if (!aligned16(all_kv) || !aligned16(gamma) || !aligned16(cos_sin) || !aligned16(dbg_rows) ||
      !bytes16(kv_layer_stride, 2) || !bytes16(kv_token_stride, 2))
    return fail(MLA_ERR_MISALIGNED, "%s: all_kv/gamma/cos_sin/dbg_rows addresses and all_kv "
                "strides must be multiples of 16 bytes", fn);
  const int64_t rows = num_layers * num_tokens;
  if (rows >= (int64_t(1) << 31) || block_size > 0x7FFFFFFF)
    return fail(MLA_ERR_UNSUPPORTED, "%s: too many rows for one launch", fn);
  EpiArgs a;
  a.all_kv = static_cast<const uint16_t*>(all_kv);
  a.kls = kv_layer_stride;
  a.kts = kv_token_stride;
  a.gamma = static_cast<const uint16_t*>(gamma);
  a.eps = eps;
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.max_pos = max_pos;
  a.cache_ptrs = kv_cache_ptrs;
  a.scales = kv_scales;
  a.slots = slot_mapping;
  a.sls = slot_layer_stride;
  a.block_size = block_size;
  a.block_stride = block_stride;
  a.entry_stride = entry_stride;
  a.dbg = static_cast<uint16_t*>(dbg_rows);
  a.bsize = make_fastdiv(static_cast<uint32_t>(block_size));
  a.layers = static_cast<uint32_t>(num_layers);
  a.tokens = static_cast<uint32_t>(num_tokens);
  const int64_t blocks =
      std::min<int64_t>(ceil_div(num_tokens, kWavesPerBlock), default_grid_cap());
  auto s = static_cast<hipStream_t>(stream);
  if (is_fp8(kv_cache_dtype))
    launch(epilogue_kernel<true>, dim3(blocks), dim3(256), 0, s, a);
  else
    launch(epilogue_kernel<false>, dim3(blocks), dim3(256), 0, s, a);
  return launch_status(fn);
}
