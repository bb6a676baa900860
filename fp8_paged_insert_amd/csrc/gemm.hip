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
//  * operand tiles go from global memory straight into LDS with buffer loads
//    (buffer_load_dwordx4 ... lds, 1 KiB per wavefront instruction), no
//    register staging: the tile's X and W rows are buffer resources in
//    SGPRs, the K stage's byte offset is the scalar offset, and each lane's
//    offset within the tile is a constant VGPR, so a copy costs no vector
//    ALU work (as global_load_lds, each copy took a 64-bit address add, and
//    the wavefront's LDS target a v_readfirstlane; removing those made the
//    launch 5.6% faster, 141.5 -> 133.7 us); LDS rows are 128 bytes with an
//    XOR swizzle of the 16-byte chunks, so the fragment reads are
//    bank-conflict free;
//  * the X tile in a ring of three LDS buffers, the W tile in two (144 KiB),
//    and one barrier per stage, placed after the second of the four K
//    steps: the fragments of steps 2 and 3 are read before it (three
//    fragment register slots, rotating by one per stage), so stage kb's W
//    buffer is free right after it.  The copies of stage kb + 2 are spread
//    over the whole of stage kb: its 8 X copies per wavefront under steps
//    0 and 1 (into the X buffer stage kb - 1 left), its 6 W copies under
//    steps 2 and 3; the barrier waits only for stage kb + 1.  Step 3 also
//    hides the next stage's first fragment reads, and every step's MFMAs
//    hide the next step's fragment reads (the issue order is pinned with
//    sched_group_barrier).  All 14 copies under steps 2 and 3 (two
//    buffers each) measured 2% slower, under step 3 alone 10% slower;
//  * tiles are grouped per XCD so the workgroups sharing an L2 share their
//    X and W blocks;
//  * no cache-warming workgroups on the CUs the tiles leave idle: with the
//    copies spread over whole stages they made the launch 1.2 us slower
//    (earlier, with every copy after the barrier, they saved about 20 us of
//    a launch whose operands start in HBM);
//  * the finished tile is rounded to bf16 into LDS (over the stage buffers)
//    and written out in 16-byte chunks along its rows: 24 store
//    instructions per lane that cover whole 128-byte lines of Y, instead of
//    192 two-byte stores straight from the accumulator layout (which took
//    about 10 us of the launch);
//  * rows beyond T and columns beyond N are clamped on load and masked on
//    store, so any T >= 1 and any N that is a multiple of 16 work.
#include <type_traits>
#include "mla_common.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBM = 256, kBN = 192, kBK = 64;
constexpr int kThreads = 256;
constexpr int kRowBytes = kBK * 2;                      // one tile row of K values in LDS
constexpr int kXStageBytes = kBM * kRowBytes;          // one stage of the X tile
constexpr int kWStageBytes = kBN * kRowBytes;          // one stage of the W tile
constexpr int kXBufs = 3, kWBufs = 2;
constexpr int kWBase = kXBufs * kXStageBytes;
constexpr size_t kLdsBytes = size_t(kXBufs) * kXStageBytes + size_t(kWBufs) * kWStageBytes;
constexpr int kWaveM = 128, kWaveN = 96;                // per-wavefront tile
constexpr int kSubM = kWaveM / 32, kSubN = kWaveN / 32;
constexpr int kOutRow = kBN * 2 + 16;  // bytes per output-tile row in LDS (padded)
static_assert(size_t(kBM) * kOutRow <= kLdsBytes, "the output tile fits over the stages");
constexpr int kDppSwapPairs = 0xB1;     // DPP quad_perm [1, 0, 3, 2]: lanes 2c <-> 2c + 1
constexpr int kXBlocks = kBM / 8 / 4;  // 1 KiB (8-row) LDS blocks of X each wavefront fills
constexpr int kWBlocks = kBN / 8 / 4;  // and of W

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedLdsRead = 0x100;

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kMaxLdsDevices = 64;  // devices whose LDS attribute is remembered
constexpr int kGroupRows = 4;


struct GemmArgs {
  const uint16_t* x;
  const uint16_t* w;
  uint16_t* y;
  int64_t ldx, ldy;
  int32_t T, K, N;
  int32_t tiles_n, tiles, tiles_per_xcd;
};

// The 16-byte chunk c of tile row r sits in LDS slot c ^ swz(r) of that row.
// Rows are 128 bytes, so without the swizzle the fragment reads (32 rows,
// one chunk each) would all hit the same 4 banks; with it, any 8 consecutive
// rows, and the 8 even or the 8 odd rows of any 16, cover 8 distinct slots.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Buffer resource over a tile's rows: base address, no stride, a 2 GiB
// range (the host keeps every offset a tile uses below 2^31 bytes), and the
// gfx9 data-format word.
constexpr int kBufferConfig = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, 0x7FFFFFFF,
                                           kBufferConfig);
}

// One wavefront-wide direct copy of 16 bytes per lane from a tile into LDS:
// lane l reads at byte voff (its own) + soff (uniform) of the resource, and
// its bytes land at dst + 16 l (dst is wavefront-uniform).
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t res, uint32_t voff,
                                            uint32_t soff, uint8_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_void_t*)dst, 16, voff, soff, 0, 0);
}

__global__ __launch_bounds__(kThreads, 1) void kv_proj_kernel(const GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];   // [3][kBM rows], then [2][kBN rows], of 128 B

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets in SGPRs
  const int wm = wave >> 1, wn = wave & 1;
  // Workgroups are dispatched round-robin over the XCDs.  Tiles are
  // numbered in groups of kGroupRows tile rows, column by column inside a
  // group, and XCD x takes the run [x * per, (x + 1) * per) of that order:
  // the workgroups sharing one L2 then cover a compact block of tiles (for
  // the 16 x 15 tile workload: 4 tile rows by 7 or 8 tile columns), which
  // reads fewer distinct X and W bytes per L2 than whole tile rows would.
  const int t = (blockIdx.x % kXcds) * a.tiles_per_xcd + blockIdx.x / kXcds;
  if (t >= a.tiles) return;
  const int tiles_m = a.tiles / a.tiles_n;
  const int group = t / (kGroupRows * a.tiles_n);
  const int in_group = t - group * kGroupRows * a.tiles_n;
  const int group_rows = min(kGroupRows, tiles_m - group * kGroupRows);
  const int m0 = (group * kGroupRows + in_group % group_rows) * kBM;
  const int n0 = (in_group / group_rows) * kBN;

  // Loading: each 1 KiB block of a stage holds 8 tile rows; lane l of the
  // copy fills slot (l & 7) of row (l >> 3), so it fetches chunk
  // (l & 7) ^ swz(row).  Rows beyond T or N are clamped (masked on store).
  // Offsets are in bytes from the tile's first X / W row.
  const __amdgpu_buffer_rsrc_t xres = tile_rsrc(a.x + int64_t(m0) * a.ldx);
  const __amdgpu_buffer_rsrc_t wres = tile_rsrc(a.w + int64_t(n0) * a.K);
  uint32_t xoffb[kXBlocks], woffb[kWBlocks];
#pragma unroll
  for (int i = 0; i < kXBlocks; ++i) {
    const int r = (wave * kXBlocks + i) * 8 + (lane >> 3);
    const int m = min(m0 + r, a.T - 1);
    xoffb[i] = static_cast<uint32_t>((int64_t(m - m0) * a.ldx + ((lane & 7) ^ swz(r)) * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < kWBlocks; ++i) {
    const int r = (wave * kWBlocks + i) * 8 + (lane >> 3);
    const int n = min(n0 + r, a.N - 1);
    woffb[i] = static_cast<uint32_t>((int64_t(n - n0) * a.K + ((lane & 7) ^ swz(r)) * 8) * 2);
  }
  // copies of stage kb: X blocks [c0, c1) into X buffer xb, W blocks
  // [c0, c1) into W buffer wb
  auto issue_x = [&](int kb, int xb, int c0, int c1) {
    uint8_t* base = lds + xb * kXStageBytes;
#pragma unroll
    for (int i = c0; i < c1; ++i)
      copy_to_lds(xres, xoffb[i], kb * (kBK * 2), base + (wave * kXBlocks + i) * 1024);
  };
  auto issue_w = [&](int kb, int wb, int c0, int c1) {
    uint8_t* base = lds + kWBase + wb * kWStageBytes;
#pragma unroll
    for (int i = c0; i < c1; ++i)
      copy_to_lds(wres, woffb[i], kb * (kBK * 2), base + (wave * kWBlocks + i) * 1024);
  };
  static_assert(kXBlocks == 8 && kWBlocks == 6, "copies are issued 4 + 4 + 3 + 3 per stage");

  f32x16_t acc[kSubM][kSubN];
#pragma unroll
  for (int i = 0; i < kSubM; ++i)
#pragma unroll
    for (int j = 0; j < kSubN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Fragments: lane l takes tile row (l & 31) of a 32-row block and the
  // 8 K values of chunk 2 kk + (l >> 5).
  const int hi = lane >> 5;
  auto frag_off = [&](int row, int kk) {
    return row * kRowBytes + (((2 * kk + hi) ^ swz(row)) << 4);
  };
  int xoff[kSubM][kBK / 16], xoff2[kSubM][kBK / 16], woff[kSubN][kBK / 16];
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
#pragma unroll
    for (int i = 0; i < kSubM; ++i) {
      xoff[i][kk] = frag_off(wm * kWaveM + i * 32 + (lane & 31), kk);
      xoff2[i][kk] = xoff[i][kk] + 2 * kXStageBytes;
    }
#pragma unroll
    for (int j = 0; j < kSubN; ++j)
      woff[j][kk] = kWBase + frag_off(wn * kWaveN + j * 32 + (lane & 31), kk);
  }

  // Pipeline, per stage kb computed from X buffer kb % 3 and W buffer
  // kb % 2, with three fragment register slots rotating by one per stage:
  //   step 0: MFMAs, step 1's fragments and 4 of stage kb + 2's X copies
  //           (into X buffer (kb + 2) % 3) under them;
  //   step 1: MFMAs, steps 2 and 3's fragments and the other 4 X copies
  //           under them;
  //   barrier: stage kb + 1 has landed everywhere (only the 8 X copies
  //           just issued may be in flight) and no wavefront reads stage
  //           kb any more;
  //   steps 2, 3: MFMAs with 3 of stage kb + 2's W copies (into W buffer
  //           kb % 2) under each, and stage kb + 1's step-0 fragments read
  //           under step 3.
  // X buffer (kb + 2) % 3 held stage kb - 1, whose last reads returned
  // before the previous barrier, so the X copies may start before this
  // stage's barrier.
  const int stages = a.K / kBK;
  bf16x8_t fa[3][kSubM], fb[3][kSubN];
  // X fragment i of X buffer xb, W fragment j of W buffer wb.  The K loop
  // is unrolled by six stages, so both buffer indices are compile-time
  // constants, and every read's buffer base fits the ds_read immediate
  // (below 64 KiB): X buffers 0 and 1 directly, X buffer 2 through xoff2
  // (its base folded in), the W buffers through woff (the W region's base
  // folded in).  No read needs a vector add (0.6% faster than one add per
  // read of X buffer 2 and of every W buffer).
  auto xfrag = [&](int xb, int i, int kk) {
    return xb == 2 ? *reinterpret_cast<const bf16x8_t*>(lds + xoff2[i][kk])
                   : *reinterpret_cast<const bf16x8_t*>(lds + xb * kXStageBytes + xoff[i][kk]);
  };
  auto wfrag = [&](int wb, int j, int kk) {
    return *reinterpret_cast<const bf16x8_t*>(lds + wb * kWStageBytes + woff[j][kk]);
  };
  auto read_frags = [&](int slot, int xb, int wb, int kk) {
#pragma unroll
    for (int i = 0; i < kSubM; ++i) fa[slot][i] = xfrag(xb, i, kk);
#pragma unroll
    for (int j = 0; j < kSubN; ++j) fb[slot][j] = wfrag(wb, j, kk);
  };
  // fragment q of a step: X fragments 0..3, then W fragments 4..6
  auto read_one = [&](int slot, int q, int xb, int wb, int kk) {
    if (q < kSubM)
      fa[slot][q] = xfrag(xb, q, kk);
    else
      fb[slot][q - kSubM] = wfrag(wb, q - kSubM, kk);
  };
  auto mfma_step = [&](int slot) {
#pragma unroll
    for (int i = 0; i < kSubM; ++i)
#pragma unroll
      for (int j = 0; j < kSubN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j],
                                                            0, 0, 0);
  };
  constexpr int kFrags = kSubM + kSubN;          // fragment reads per step
  constexpr int kMfma = kSubM * kSubN;           // MFMAs per step
  static_assert(kFrags == 7 && kMfma == 12, "schedule below is for 7 reads / 12 MFMAs");

  issue_x(0, 0, 0, kXBlocks);
  issue_w(0, 0, 0, kWBlocks);
  issue_x(min(1, stages - 1), 1, 0, kXBlocks);
  issue_w(min(1, stages - 1), 1, 0, kWBlocks);
  __builtin_amdgcn_s_waitcnt(0x0F7E);  // vmcnt(14): stage 0 has landed
  __syncthreads();
  read_frags(0, 0, 0, 0);
  auto do_stage = [&](auto R, int kb) {
    constexpr int r = decltype(R)::value;
    constexpr int sa = r % 3, sb = (r + 1) % 3, sc = (r + 2) % 3;
    constexpr int xbuf = r % 3, wbuf = r % 2;
    const int ahead = min(kb + 2, stages - 1);
    constexpr int xnext = (r + 2) % 3;
    // step 0
    read_frags(sb, xbuf, wbuf, 1);
    issue_x(ahead, xnext, 0, 4);
    mfma_step(sa);
#pragma unroll
    for (int q = 0; q < kFrags; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 1, 0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    // step 1
    // program order = issue order: the copies write LDS, so the compiler
    // keeps them in place relative to the fragment reads
#pragma unroll
    for (int q = 0; q < 4; ++q) read_one(sc, q, xbuf, wbuf, 2);
#pragma unroll
    for (int q = 4; q < 7; ++q) {
      read_one(sc, q, xbuf, wbuf, 2);
      issue_x(ahead, xnext, q, q + 1);
    }
    read_one(sa, 0, xbuf, wbuf, 3);
    issue_x(ahead, xnext, 7, 8);
#pragma unroll
    for (int q = 1; q < 7; ++q) read_one(sa, q, xbuf, wbuf, 3);
    mfma_step(sb);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 2, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    }
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // stage kb + 1 has landed: only stage kb + 2's X copies (the last 8
    // issued) may still be in flight
    // and the fragment reads of stage kb have returned; a bare barrier, since
    // __syncthreads() would also wait for those X copies
    __builtin_amdgcn_s_waitcnt(0x0078);  // vmcnt(8) lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    // step 2
    issue_w(ahead, wbuf, 0, 3);
    mfma_step(sc);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMfma - 3, 0);
    __builtin_amdgcn_sched_barrier(0);
    // step 3
    read_frags(sb, (r + 1) % 3, (r + 1) % 2, 0);
    issue_w(ahead, wbuf, 3, 6);
    mfma_step(sa);
#pragma unroll
    for (int q = 0; q < 7; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 1, 0);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  using R0 = std::integral_constant<int, 0>;
  using R1 = std::integral_constant<int, 1>;
  using R2 = std::integral_constant<int, 2>;
  using R3 = std::integral_constant<int, 3>;
  using R4 = std::integral_constant<int, 4>;
  using R5 = std::integral_constant<int, 5>;
  for (int kb = 0; kb < stages; kb += 6) {
    do_stage(R0{}, kb);
    if (kb + 1 < stages) do_stage(R1{}, kb + 1);
    if (kb + 2 < stages) do_stage(R2{}, kb + 2);
    if (kb + 3 < stages) do_stage(R3{}, kb + 3);
    if (kb + 4 < stages) do_stage(R4{}, kb + 4);
    if (kb + 5 < stages) do_stage(R5{}, kb + 5);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the repeated copies have landed
  __syncthreads();                      // and no wavefront reads a stage any more

  // Output: the workgroup's bf16 tile is assembled in LDS (kBM rows of
  // kOutRow bytes, over the stage buffers), then written out in 16-byte
  // chunks, consecutive lanes along a row, so every store instruction covers
  // whole 128-byte lines of Y.  Accumulator value r of lane l is
  // C[8 (r / 4) + 4 (l / 32) + (r % 4)][l % 32] of its 32 x 32 tile: values r
  // and r + 1 (r even) are rows R and R + 1 of one column.  Lanes 2c and
  // 2c + 1 swap their rounded pairs, so the even lane holds row R and the odd
  // lane row R + 1 of columns 2c and 2c + 1: one 4-byte LDS write each.
  const int odd = lane & 1;
#pragma unroll
  for (int i = 0; i < kSubM; ++i) {
#pragma unroll
    for (int j = 0; j < kSubN; ++j) {
      const int col = wn * kWaveN + j * 32 + (lane & 31) - odd;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const uint32_t own = cvt_bf16x2(acc[i][j][r], acc[i][j][r + 1]);
        const uint32_t other = static_cast<uint32_t>(
            __builtin_amdgcn_update_dpp(0, static_cast<int>(own), kDppSwapPairs, 0xF, 0xF, false));
        const uint32_t word = odd ? __builtin_amdgcn_perm(own, other, 0x07060302u)
                                  : __builtin_amdgcn_perm(other, own, 0x05040100u);
        const int row = wm * kWaveM + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4) + odd;
        *reinterpret_cast<uint32_t*>(lds + row * kOutRow + col * 2) = word;
      }
    }
  }
  __syncthreads();
  constexpr int kRowChunks = kBN * 2 / 16;
#pragma unroll 4
  for (int c = tid; c < kBM * kRowChunks; c += kThreads) {
    const int row = c / kRowChunks, ch = c - row * kRowChunks;
    const int m = m0 + row, n = n0 + ch * 8;
    // N is a multiple of 16: a chunk of 8 columns is wholly inside or outside
    if (m < a.T && n < a.N)
      st16(a.y + int64_t(m) * a.ldy + n, *reinterpret_cast<const uint4*>(lds + row * kOutRow + ch * 16));
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
  // a tile's copies address its rows by 32-bit byte offsets below 2^31,
  // checked in elements below 2^30 (the stride first, so nothing overflows);
  // an X tile spans at least as much as a W tile (kBM > kBN, x_row_stride >= K)
  constexpr int64_t kTileSpan = int64_t(1) << 30;
  if (x_row_stride >= kTileSpan / (kBM - 1) || (kBM - 1) * x_row_stride + K >= kTileSpan)
    return fail(MLA_ERR_UNSUPPORTED, "%s: a %d-row tile of X would span 2 GiB or more", fn, kBM);
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
  const int64_t grid = int64_t(a.tiles_per_xcd) * kXcds;  // blocks past the tiles return
  // The LDS reservation is a per-device attribute of the kernel: set it once
  // on each device the projection runs on.
  static int attr_set[kMaxLdsDevices] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(MLA_ERR_DEVICE, "%s: no current HIP device", fn);
  if (dev >= kMaxLdsDevices || !__atomic_load_n(&attr_set[dev], __ATOMIC_ACQUIRE)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kv_proj_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(kLdsBytes)) != hipSuccess)
      return fail(MLA_ERR_DEVICE, "%s: cannot reserve %zu bytes of LDS", fn, kLdsBytes);
    if (dev < kMaxLdsDevices) __atomic_store_n(&attr_set[dev], 1, __ATOMIC_RELEASE);
  }
  launch(kv_proj_kernel, dim3(grid), dim3(kThreads), kLdsBytes,
                     static_cast<hipStream_t>(stream), a);
  return launch_status(fn);
}
