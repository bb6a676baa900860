// gemm.hip -- the fused KV-only context projection: one bf16 GEMM that
// produces the latent KV of every draft layer at once.
//
// Page: "PR #50585 完整报告" ([K3 Perf] Optimize k3 dspark fused kv),
// 功能与动机 and 实现拆解 item 2-3: a single projection hidden -> L * 576
// (MergedColumnParallelLinear over the layers' KV weights) replaces L full
// hidden -> 2112 projections whose query columns were thrown away; the
// output is then viewed as [num_ctx, L, 576].
//
// gfx950 design: Y[T, N] = X[T, K] . W[N, K]^T with bf16 operands, fp32
// accumulation in v_mfma_f32_32x32x16_bf16, one rounding to bf16.
//  * workgroup tile 256 (T) x 192 (N) x 64 (K), 4 wavefronts in a 2 x 2
//    layout, each holding 4 x 3 32x32 fp32 accumulator tiles; the default
//    problem (4096 x 7168 . 7168 x 2880) is 16 x 15 = 240 tiles, one per
//    compute unit in a single wave of the grid;
//  * both operands are K-contiguous (W is the linear layer's [out, in]
//    storage), so one 16-byte LDS read gives a lane its 8 consecutive K
//    values for either MFMA operand;
//  * LDS rows are padded to 144 bytes: 16 consecutive rows then start on
//    16 distinct 4-bank groups, so the 16-byte fragment reads of a
//    half-wavefront are conflict-free;
//  * two LDS stages; the next stage's global loads are issued into registers
//    before the current stage's MFMAs and written to the other LDS buffer
//    after them, with one barrier per stage;
//  * rows beyond T and columns beyond N are clamped on load and masked on
//    store, so any T >= 1 and any N that is a multiple of 16 work.
#include "mla_common.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 192, kBK = 64;
constexpr int kLdsRow = kBK + 8;  // bf16 elements per LDS row (144 bytes)
constexpr int kThreads = 256;
constexpr int kWaveM = 128, kWaveN = 96;   // per-wavefront tile
constexpr int kSubM = kWaveM / 32, kSubN = kWaveN / 32;
constexpr int kAChunks = kBM * kBK / 8 / kThreads;  // 16-byte loads per thread for X
constexpr int kBChunks = kBN * kBK / 8 / kThreads;  // and for W
constexpr size_t kLdsBytes = size_t(2) * (kBM + kBN) * kLdsRow * 2;

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each

struct GemmArgs {
  const uint16_t* x;
  const uint16_t* w;
  uint16_t* y;
  int64_t ldx, ldy;
  int32_t T, K, N;
  int32_t tiles_n, tiles, tiles_per_xcd;
};

__global__ __launch_bounds__(kThreads, 1) void kv_proj_kernel(const GemmArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* As = lds;                                  // [2][kBM][kLdsRow]
  uint16_t* Bs = lds + 2 * kBM * kLdsRow;              // [2][kBN][kLdsRow]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // Workgroups are dispatched round-robin over the XCDs; give XCD x the run
  // of tiles [x * per, (x + 1) * per) in row-major tile order, so the
  // workgroups sharing one L2 also share their X row blocks (for the
  // 16 x 15 tile workload: 2 tile rows per XCD, 15 workgroups per X block).
#ifndef MLA_GEMM_XCD_REMAP
#define MLA_GEMM_XCD_REMAP 1
#endif
  const int tile = MLA_GEMM_XCD_REMAP ? (blockIdx.x % kXcds) * a.tiles_per_xcd + blockIdx.x / kXcds
                                      : static_cast<int>(blockIdx.x);
  if (tile >= a.tiles) return;
  const int m0 = (tile / a.tiles_n) * kBM;
  const int n0 = (tile % a.tiles_n) * kBN;

  // this thread's global chunks: row = (tid >> 3) + 32 i, 16-byte column c
  const int c = tid & 7;
  const int r0 = tid >> 3;
  const uint16_t* xg[kAChunks];
  const uint16_t* wg[kBChunks];
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int m = min(m0 + r0 + 32 * i, a.T - 1);
    xg[i] = a.x + int64_t(m) * a.ldx + c * 8;
  }
#pragma unroll
  for (int i = 0; i < kBChunks; ++i) {
    const int n = min(n0 + r0 + 32 * i, a.N - 1);
    wg[i] = a.w + int64_t(n) * a.K + c * 8;
  }

  uint4 ra[kAChunks], rb[kBChunks];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) ra[i] = ld16(xg[i] + k0);
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) rb[i] = ld16(wg[i] + k0);
  };
  auto store_stage = [&](int buf) {
    uint16_t* as = As + buf * kBM * kLdsRow;
    uint16_t* bs = Bs + buf * kBN * kLdsRow;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i)
      *reinterpret_cast<uint4*>(as + (r0 + 32 * i) * kLdsRow + c * 8) = ra[i];
#pragma unroll
    for (int i = 0; i < kBChunks; ++i)
      *reinterpret_cast<uint4*>(bs + (r0 + 32 * i) * kLdsRow + c * 8) = rb[i];
  };

  f32x16_t acc[kSubM][kSubN];
#pragma unroll
  for (int i = 0; i < kSubM; ++i)
#pragma unroll
    for (int j = 0; j < kSubN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // fragment addressing: lane -> row (lane & 31), k group (lane >> 5) * 8
  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;

  const int stages = a.K / kBK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kb = 0; kb < stages; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < stages) load_stage((kb + 1) * kBK);
    const uint16_t* as = As + buf * kBM * kLdsRow + (wm * kWaveM + frow) * kLdsRow + fk;
    const uint16_t* bs = Bs + buf * kBN * kLdsRow + (wn * kWaveN + frow) * kLdsRow + fk;
    // fragments of k step kk + 1 are read while the MFMAs of step kk run
    bf16x8_t fa[2][kSubM], fb[2][kSubN];
    auto read_frags = [&](int slot, int kk) {
#pragma unroll
      for (int i = 0; i < kSubM; ++i)
        fa[slot][i] = *reinterpret_cast<const bf16x8_t*>(as + i * 32 * kLdsRow + kk * 16);
#pragma unroll
      for (int j = 0; j < kSubN; ++j)
        fb[slot][j] = *reinterpret_cast<const bf16x8_t*>(bs + j * 32 * kLdsRow + kk * 16);
    };
    read_frags(0, 0);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < kBK / 16) read_frags(cur ^ 1, kk + 1);
#pragma unroll
      for (int i = 0; i < kSubM; ++i)
#pragma unroll
        for (int j = 0; j < kSubN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j],
                                                              0, 0, 0);
    }
    if (kb + 1 < stages) store_stage(buf ^ 1);
    __syncthreads();
  }

  // accumulator layout: value r of lane l is C[8 (r / 4) + 4 (l / 32) + (r % 4)][l % 32]
#pragma unroll
  for (int i = 0; i < kSubM; ++i) {
#pragma unroll
    for (int j = 0; j < kSubN; ++j) {
      const int n = n0 + wn * kWaveN + j * 32 + (lane & 31);
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * kWaveM + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
        if (m < a.T)
          a.y[int64_t(m) * a.ldy + n] = static_cast<uint16_t>(cvt_bf16x2(acc[i][j][r], 0.0f));
      }
    }
  }
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" int32_t mla_ctx_kv_proj(const void* X, int64_t x_row_stride, int64_t T, int64_t K,
                                   const void* W, int64_t N, void* Y, int64_t y_row_stride,
                                   mla_stream_t stream) {
  static const char* fn = "mla_ctx_kv_proj";
  clear_error();
  if (T < 0 || K < 0 || N < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
  if (T == 0 || N == 0) return MLA_OK;
  if (!X || !W || !Y) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL operand", fn);
  if (K == 0 || K % kBK != 0 || N % 16 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "%s: K must be a positive multiple of 64 and N of 16", fn);
  if (x_row_stride < K || y_row_stride < N)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: row strides smaller than the rows", fn);
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y) || !bytes16(x_row_stride, 2) ||
      !bytes16(y_row_stride, 2))
    return fail(MLA_ERR_MISALIGNED, "%s: operands and row strides must be 16-byte aligned", fn);
  if (T > 0x7FFFFFFF - kBM || K > 0x7FFFFFFF || N > 0x7FFFFFFF - kBN)
    return fail(MLA_ERR_UNSUPPORTED, "%s: sizes beyond 2^31", fn);
  GemmArgs a;
  a.x = static_cast<const uint16_t*>(X);
  a.w = static_cast<const uint16_t*>(W);
  a.y = static_cast<uint16_t*>(Y);
  a.ldx = x_row_stride;
  a.ldy = y_row_stride;
  a.T = static_cast<int32_t>(T);
  a.K = static_cast<int32_t>(K);
  a.N = static_cast<int32_t>(N);
  a.tiles_n = static_cast<int32_t>(ceil_div(N, kBN));
  const int64_t tiles = ceil_div(T, kBM) * a.tiles_n;
  a.tiles = static_cast<int32_t>(tiles);
  a.tiles_per_xcd = static_cast<int32_t>(ceil_div(tiles, kXcds));
  const int64_t grid = int64_t(a.tiles_per_xcd) * kXcds;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kv_proj_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(kLdsBytes)) != hipSuccess)
      return fail(MLA_ERR_DEVICE, "%s: cannot reserve %zu bytes of LDS", fn, kLdsBytes);
    attr_set = true;
  }
  launch(kv_proj_kernel, dim3(grid), dim3(kThreads), kLdsBytes,
                     static_cast<hipStream_t>(stream), a);
  return launch_status(fn);
}
