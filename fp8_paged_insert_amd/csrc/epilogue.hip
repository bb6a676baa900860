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
// pass reads each (layer, token) row of the strided [T, L, 576] projection
// output once (no layer-major copy) and writes its cache entry.  A row
// belongs to 16 lanes (a DPP row), 4 rows per wavefront: lane j holds the
// kv_c chunks j, j + 16, j + 32, j + 48 (8 values each) and k_pe[4j, 4j + 4),
// so every load and store instruction covers 128-256 contiguous bytes per
// row.  The sum of squares is reduced with four in-row DPP steps (no LDS
// round trip), RoPE's (i, i + 32) pairs sit in lanes j and j ^ 8 and swap
// with one DPP row rotation, and the token's position indexes the cos/sin
// table directly instead of a repeated-positions buffer.  The rotation is
// rounded once to bf16 even where its two products nearly cancel (rope4v:
// an fp32 fast path kept only where it is provably the correct rounding,
// else float64 from the table's hi + lo values).  For up to 8 layers the
// layers' RMSNorm weights are read into LDS once per workgroup
// (epilogue_lds_kernel); otherwise each row group reads its layer's weights
// from global memory (epilogue_kernel).
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
    const double c = cos(theta), s = sin(theta);
    const float ch = static_cast<float>(c), sh = static_cast<float>(s);
    float* row = out + p * 2 * rope_dim;
    row[i] = ch;
    row[half + i] = sh;
    row[rope_dim + i] = static_cast<float>(c - static_cast<double>(ch));
    row[rope_dim + half + i] = static_cast<float>(s - static_cast<double>(sh));
  }
}

// ---------------------------------------------------------------- epilogue --
constexpr int kR = 512;  // kv_lora_rank
constexpr int kP = 64;   // rope dim
constexpr int kRowLanes = 16;                       // lanes per (layer, token) row
constexpr int kRowsPerWave = 64 / kRowLanes;
constexpr int kChunks = kR / 8 / kRowLanes;         // 16-byte kv_c chunks per lane
constexpr int kPe = kP / kRowLanes;                 // k_pe values per lane
constexpr int kWavesPerBlock = 4;
constexpr int kRowsPerBlock = kRowsPerWave * kWavesPerBlock;

struct EpiArgs {
  const uint16_t* all_kv;
  int64_t kls, kts;
  const uint16_t* gamma;
  float eps;
  const int64_t* positions;
  const float* cos_sin;  // [max_pos, 2 * 64]: cos hi | sin hi | cos lo | sin lo
  int64_t max_pos;
  const int64_t* cache_ptrs;
  const float* scales;
  const int64_t* slots;
  int64_t sls;
  int64_t block_size, block_stride, entry_stride;
  uint16_t* dbg;
  FastDiv bsize, nlayers;
  uint32_t layers, tokens, rows;
};

// DPP moves inside a row of 16 lanes (every source lane is valid).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i
constexpr int kDppRor8 = 0x128;       // lane i <- lane (i + 8) mod 16

// Sum over the 16 lanes of a row; every lane gets the same bits (each step
// adds two partial sums, and fp32 addition is commutative).
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
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

// The part of a row after its loads: RoPE, RMSNorm, bf16 rounding, the
// optional debug copy of the row, fp8 (or bf16) conversion and the cache
// store.  gamma_chunk(q) yields the layer's weight chunk q of this lane.
template <int kFmt, class GammaChunk>
__device__ __forceinline__ void finish_row(const EpiArgs& a, const uint4* xv,
                                           GammaChunk gamma_chunk, uint2 pe, uint4 cv, uint4 sv,
                                           uint4 clv, uint4 slv, int64_t slot, int64_t cbase,
                                           float sc, uint32_t l, uint32_t t, bool active, int j) {
  constexpr bool kFp8 = kFmt != kFmtBf16, kE5M2 = kFmt == kFmtE5M2;
  const bool first_half = j < kRowLanes / 2;  // holds k_pe[i], i < 32
  // ---- RoPE first (its table words and partner values are dead before the
  // normed row is built): y_i = x_i cos - x_{i+32} sin, y_{i+32} = x_{i+32} cos + x_i sin
  const float xp[kPe] = {bf16_lo(pe.x), bf16_hi(pe.x), bf16_lo(pe.y), bf16_hi(pe.y)};
  const float cc[kPe] = {__uint_as_float(cv.x), __uint_as_float(cv.y), __uint_as_float(cv.z),
                         __uint_as_float(cv.w)};
  const float sn[kPe] = {__uint_as_float(sv.x), __uint_as_float(sv.y), __uint_as_float(sv.z),
                         __uint_as_float(sv.w)};
  float xq[kPe];
#pragma unroll
  for (int e = 0; e < kPe; ++e) xq[e] = dpp_f<kDppRor8>(xp[e]);
  const uint2 ype = rope4v(xp, xq, cc, sn, first_half, clv, slv);

  // ---- RMSNorm: fp32 sum of squares over the row's 16 lanes, two squares
  // per bf16 word (v_dot2c_f32_bf16: the squares of bf16 values are exact in
  // fp32), four partial sums per lane.
  float ss4[kChunks];
#pragma unroll
  for (int q = 0; q < kChunks; ++q) {
    ss4[q] = 0.0f;
    const uint32_t w[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2_t b = __builtin_bit_cast(bf16x2_t, w[i]);
      ss4[q] = __builtin_amdgcn_fdot2_f32_bf16(b, b, ss4[q], false);
    }
  }
  float ss = (ss4[0] + ss4[1]) + (ss4[2] + ss4[3]);
  ss = row_sum(ss);
  const float rinv = 1.0f / __builtin_sqrtf(ss * (1.0f / kR) + a.eps);
  uint4 y[kChunks];
#pragma unroll
  for (int q = 0; q < kChunks; ++q) {
    const uint32_t w[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
    const uint4 g = gamma_chunk(q);
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t yw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      yw[i] = cvt_bf16x2(bf16_lo(w[i]) * rinv * bf16_lo(gw[i]),
                         bf16_hi(w[i]) * rinv * bf16_hi(gw[i]));
    y[q] = make_uint4(yw[0], yw[1], yw[2], yw[3]);
  }

  if (!active) return;
  if (a.dbg) {
    uint16_t* d = a.dbg + (int64_t(l) * a.tokens + t) * (kR + kP);
#pragma unroll
    for (int q = 0; q < kChunks; ++q) st16(d + 8 * (j + kRowLanes * q), y[q]);
    st8(d + kR + kPe * j, ype);
  }
  // ---- insert (slot -> block, offset; a negative slot skips the row)
  if (slot < 0) return;
  const int64_t entry = entry_offset(slot, a);
  if constexpr (kFp8) {
    const float rc = 1.0f / sc;
    const uint32_t flip = sign_flip_of(sc);
    uint8_t* dst = reinterpret_cast<uint8_t*>(cbase) + entry;
#pragma unroll
    for (int q = 0; q < kChunks; ++q)
      st8<kEpiStream>(dst + 8 * (j + kRowLanes * q), quant8<true, false, kE5M2>(y[q], sc, rc, flip));
    st4<kEpiStream>(dst + kR + kPe * j, quant4<true, kE5M2>(ype, sc, rc, flip));
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(cbase) + entry;
#pragma unroll
    for (int q = 0; q < kChunks; ++q) st16<kEpiStream>(dst + 8 * (j + kRowLanes * q), y[q]);
    st8<kEpiStream>(dst + kR + kPe * j, ype);
  }
}

// Rows are numbered token-major (row = t * L + l), the order of the
// projection output, so the 4 rows of a wavefront are adjacent in memory.
// One row per 16-lane group per pass; the general form (any layer count).
template <int kFmt>
__global__ __launch_bounds__(256, 5) void epilogue_kernel(const EpiArgs a) {
  const int lane = threadIdx.x & 63;
  const int j = lane & (kRowLanes - 1);       // lane within the row
  const int grp = lane / kRowLanes;           // row within the wavefront
  const uint32_t wave = threadIdx.x >> 6;
  for (uint32_t r0 = (blockIdx.x * kWavesPerBlock + wave) * kRowsPerWave; r0 < a.rows;
       r0 += gridDim.x * kRowsPerBlock) {
    const uint32_t r = r0 + grp;
    const bool active = r < a.rows;
    const uint32_t rr = active ? r : a.rows - 1;   // idle lanes still load in bounds
    const uint32_t t = fdiv(rr, a.nlayers);
    const uint32_t l = rr - t * a.layers;
    const uint16_t* row = a.all_kv + int64_t(t) * a.kts + int64_t(l) * a.kls;
    const uint16_t* grow = a.gamma + int64_t(l) * kR;

    // The position is loaded first: the table read that depends on it then
    // waits only for that load (loads retire in order) and overlaps the row
    // loads instead of following them.
    // Positions outside [0, max_pos) break the precondition; clamp so the
    // table read stays inside the table.
    const int64_t pos_in = a.positions[t];
    __builtin_amdgcn_sched_barrier(0);
    uint4 xv[kChunks], gv[kChunks];
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
      xv[q] = ld16(row + 8 * (j + kRowLanes * q));
      gv[q] = ld16(grow + 8 * (j + kRowLanes * q));
    }
    const uint2 pe = *reinterpret_cast<const uint2*>(row + kR + kPe * j);
    const int64_t slot = a.slots[int64_t(l) * a.sls + t];
    const int64_t cbase = a.cache_ptrs[l];
    float sc = 1.0f;
    if constexpr (kFmt != kFmtBf16) sc = a.scales[l];
    __builtin_amdgcn_sched_barrier(0);
    const int64_t pos = min(max(pos_in, int64_t(0)), a.max_pos - 1);
    const float* cs = a.cos_sin + pos * (2 * kP) + kPe * (j & 7);
    const uint4 cv = ld16(cs);
    const uint4 sv = ld16(cs + kP / 2);
    const uint4 clv = ld16(cs + kP);
    const uint4 slv = ld16(cs + kP + kP / 2);
    // Keep every load of the row here, ahead of the first wait: without this
    // fence the compiler sinks the loads used only by the stores into the
    // store branch, after the reduction, adding memory round trips.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    finish_row<kFmt>(a, xv, [&](int q) { return gv[q]; }, pe, cv, sv, clv, slv, slot, cbase, sc,
                     l, t, active, j);
  }
}

// Form for up to kMaxLdsLayers layers: the layers' RMSNorm weights are
// copied into LDS once per workgroup, and each wavefront finishes one group
// of 4 rows.  The weight loads are issued first and the row loads right
// after them; the LDS copy and the barrier (which waits for the LDS writes
// only) come after all of the row's loads are in flight.
constexpr int kMaxLdsLayers = 8;
constexpr int kGammaChunks = kR / 8;                     // 16-byte chunks per layer
constexpr int kGammaIters = kMaxLdsLayers * kGammaChunks / 256;

template <int kFmt>
__global__ __launch_bounds__(256) void epilogue_lds_kernel(const EpiArgs a) {
  __shared__ uint4 glds[kMaxLdsLayers * kGammaChunks];
  const int lane = threadIdx.x & 63;
  const int j = lane & (kRowLanes - 1);
  const int grp = lane / kRowLanes;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t r = (blockIdx.x * kWavesPerBlock + wave) * kRowsPerWave + grp;

  const uint32_t gchunks = a.layers * kGammaChunks;
  uint4 gt[kGammaIters];
#pragma unroll
  for (int i = 0; i < kGammaIters; ++i) {
    const uint32_t c = threadIdx.x + 256u * i;
    gt[i] = ld16(a.gamma + 8 * (c < gchunks ? c : 0u));
  }
  const bool active = r < a.rows;
  const uint32_t rr = active ? r : a.rows - 1;  // idle lanes still load in bounds
  const uint32_t t = fdiv(rr, a.nlayers);
  const uint32_t l = rr - t * a.layers;
  // the position first, so that the table read waits only for it
  const int64_t pos_in = a.positions[t];
  __builtin_amdgcn_sched_barrier(0);
  const uint16_t* row = a.all_kv + int64_t(t) * a.kts + int64_t(l) * a.kls;
  uint4 xv[kChunks];
#pragma unroll
  for (int q = 0; q < kChunks; ++q) xv[q] = ld16(row + 8 * (j + kRowLanes * q));
  const uint2 pe = *reinterpret_cast<const uint2*>(row + kR + kPe * j);
  const int64_t slot = a.slots[int64_t(l) * a.sls + t];
  const int64_t cbase = a.cache_ptrs[l];
  const float sc = kFmt != kFmtBf16 ? a.scales[l] : 1.0f;
  __builtin_amdgcn_sched_barrier(0);
  // positions outside [0, max_pos) break the precondition; clamp so the
  // table read stays inside the table
  const int64_t pos = min(max(pos_in, int64_t(0)), a.max_pos - 1);
  const float* cs = a.cos_sin + pos * (2 * kP) + kPe * (j & 7);
  const uint4 cv = ld16(cs);
  const uint4 sv = ld16(cs + kP / 2);
  const uint4 clv = ld16(cs + kP);
  const uint4 slv = ld16(cs + kP + kP / 2);
  // no load may sink below this point (into the store branches)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
  for (int i = 0; i < kGammaIters; ++i) {
    const uint32_t c = threadIdx.x + 256u * i;
    if (c < gchunks) glds[c] = gt[i];
  }
  // a barrier that waits for the LDS writes only, not for the row loads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  const uint4* g = glds + l * kGammaChunks + j;
  finish_row<kFmt>(a, xv, [&](int q) { return g[kRowLanes * q]; }, pe, cv, sv, clv, slv, slot,
                   cbase, sc, l, t, active, j);
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
  if (rows >= (int64_t(1) << 31) - kRowsPerBlock || block_size > 0x7FFFFFFF)
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
  a.nlayers = make_fastdiv(static_cast<uint32_t>(num_layers));
  a.layers = static_cast<uint32_t>(num_layers);
  a.tokens = static_cast<uint32_t>(num_tokens);
  a.rows = static_cast<uint32_t>(rows);
  auto s = static_cast<hipStream_t>(stream);
  const int fmt = cache_fmt(kv_cache_dtype);
  if (num_layers <= kMaxLdsLayers) {
    const int64_t blocks = ceil_div(rows, kRowsPerBlock);  // one group of 4 rows per wavefront
    if (fmt == kFmtE5M2)
      launch(epilogue_lds_kernel<kFmtE5M2>, dim3(blocks), dim3(256), 0, s, a);
    else if (fmt == kFmtE4M3)
      launch(epilogue_lds_kernel<kFmtE4M3>, dim3(blocks), dim3(256), 0, s, a);
    else
      launch(epilogue_lds_kernel<kFmtBf16>, dim3(blocks), dim3(256), 0, s, a);
    return launch_status(fn);
  }
  const int64_t blocks = std::min<int64_t>(ceil_div(rows, kRowsPerBlock), default_grid_cap());
  if (fmt == kFmtE5M2)
    launch(epilogue_kernel<kFmtE5M2>, dim3(blocks), dim3(256), 0, s, a);
  else if (fmt == kFmtE4M3)
    launch(epilogue_kernel<kFmtE4M3>, dim3(blocks), dim3(256), 0, s, a);
  else
    launch(epilogue_kernel<kFmtBf16>, dim3(blocks), dim3(256), 0, s, a);
  return launch_status(fn);
}
