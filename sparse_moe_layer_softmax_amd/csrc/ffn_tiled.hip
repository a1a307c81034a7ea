// ffn_tiled.hip -- LDS-tiled MFMA grouped GEMM for many rows per expert (prefill), and the
// dense fp32-output GEMM of the router at large T.
//
// Hy3 deep-dive (happyrock.cloud) `MoEFeedForward` (SwiGLU expert FFN) and Hy4 config
// walkthrough (lshu.cn), section "MoE routed experts" (swiglu_limit, silu); Hy3 explainer
// (tqpw.cn) section 2.1: each expert runs on the rows routed to it.
#include <algorithm>

#include "ffn_kernels.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------------------------
// Kernel "tiled": BM = 256 rows x 256 weight rows per workgroup (gate/up: 128 gate rows and the
// 128 matching up rows), four wavefronts of 128 x 128, each 4 x 4 MFMA 32x32x16 fragments with
// fp32 accumulators in AGPRs. Per CU this is the largest tile the register file holds, and it
// halves the operand bytes per FLOP of a 128-row tile: the global->LDS fill rate of a CU, not
// the MFMA rate, is what bounds this kernel.
//  - K is staged BK = 32 at a time through a 4-stage LDS ring (128 KB) filled by direct
//    global->LDS loads (global_load_lds_dwordx4, no VGPR staging). Each K-tile is consumed in
//    two phases around one workgroup barrier, so that no fragment read sits right behind a
//    barrier; the next K-tile's DMA instructions are spread between the MFMAs and the
//    instruction order is pinned with sched_group_barrier.
//  - LDS rows are XOR-swizzled by 16-byte chunk (swz) so MFMA operand reads are conflict free
//    on the 64-bank LDS.
//  - The main loop is specialised on the number of 32-row fragments of a wavefront that hold
//    rows of the group (MIV), so partly filled tiles skip MFMAs without branching in the loop.
//  - Work items are ordered inside XCD-contiguous slices of the real work list (its size comes
//    from the device-side tile count, so spare grid slots do not unbalance the XCDs); inside a
//    group the work runs in bands of up to kBand row tiles, n-blocks outer and the band's row
//    tiles inner, so workgroups running together on an XCD share one weight tile (same
//    n-block) and the band's activation rows through L2, and a group with at most kBand row
//    tiles reads each of its weight tiles from HBM once.
//  - bf16 results are staged through LDS and written as whole 16-byte row segments.
constexpr int kTN = 256;  // weight rows per tile (gate/up: 128 gate + 128 up)
constexpr int kXcds = 8;
constexpr int kBand = 8;

template <int BM, int BK, int S>
constexpr size_t tiled_smem() { return sizeof(uint16_t) * S * (BM + kTN) * BK; }

// The configuration used for large row counts.
constexpr int kBM = 256, kBK = 32, kStages = 4;

// LDS element offset of (row, k) in a [rows][BK] bf16 stage. The 16-byte chunks of a row are
// XOR-swizzled so that the MFMA operand reads (16 consecutive rows at one logical chunk per
// 16-lane group) hit 16 distinct 16-byte slots of a 256-byte window (64 banks): for 128-byte rows
// the slot is the chunk ^ (row % 8) ^ ((row / 8) % 2); for 64-byte rows, chunk ^ ((row / 4) % 4).
template <int BK>
__device__ __forceinline__ int swz(int row, int k) {
  if (BK == 64) return row * 64 + (((k >> 3) ^ (row & 7) ^ ((row >> 3) & 1)) << 3) + (k & 7);
  return row * 32 + (((k >> 3) ^ ((row >> 2) & 3)) << 3) + (k & 7);
}

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left at their maxima.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Workgroup barrier without the memory fence of __syncthreads (which would also wait for every
// in-flight global->LDS load). Callers order their own LDS traffic with wait_vmcnt and the data
// dependencies of the LDS reads; the empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void lds_dma16(const uint16_t* g, uint16_t* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}

// EPI = kEpiSwiglu: gate/up rows interleaved, h = bf16(silu(clamp g) * clamp u);
// kEpiBf16: plain bf16 output (down projection); kEpiF32: fp32 output (router logits).
// p.tiles == nullptr selects dense mode: one group of rows [0, rows_max) in BM-row tiles.
// Main loop and epilogue of one tile; MIV = live 32-row fragments of this wavefront (0..BM/64).
template <int EPI, int BM, int BK, int S, int MIV>
__device__ __forceinline__ void tiled_main(const GroupedParams& p, int g, int nb, int r0, int r1) {
  constexpr bool GATED = EPI == kEpiSwiglu;
  constexpr int MI = BM / 64;         // 32-row fragments per wavefront
  constexpr int kStageA = BM * BK, kStageB = kTN * BK;  // bf16 elements
  constexpr int RPB = 512 / BK;       // rows per 1 KB DMA block
  constexpr int CPR = BK / 8;         // 16-byte chunks per row
  constexpr int NA = BM / RPB / 4;    // DMA instructions per wave per K-tile, A
  constexpr int NB = kTN / RPB / 4;   // ... B
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sA = smem;                // [S][BM][BK]
  uint16_t* sB = smem + S * kStageA;  // [S][256][BK]
  const int Kd = p.Kd;
  const int tid = threadIdx.x;
  // wavefront index as a scalar: the LDS destinations of the DMA (M0) are then pure SALU math
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- DMA assignment. A 1 KB LDS block holds RPB rows of BK elements; lane i fills its
  // 16-byte slot i: row i/CPR of the block, physical chunk i%CPR, which holds the logical chunk
  // that swz() places there. Wave w fills blocks w, w+4, w+8, ...
  const int lrow = lane / CPR;
  int lchunk;
  if (BK == 64)
    lchunk = (lane & 7) ^ lrow ^ (wave & 1);  // block w+4i: (row/8)%2 == w%2
  else
    lchunk = (lane & 3) ^ ((lane >> 4) & 3);  // (row/4)%4 == lane/16 inside a 16-row block
  uint32_t aoff[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = r0 + (wave + 4 * i) * RPB + lrow;
    int src = 0;
    if (r < r1) src = r < p.n_ident ? r : p.gather[r - p.n_ident] / p.topk;
    if (static_cast<unsigned>(src) >= static_cast<unsigned>(p.a_rows)) src = 0;
    aoff[i] = static_cast<uint32_t>(src) * Kd + lchunk * 8;
  }
  const size_t wst = static_cast<size_t>(p.N) * Kd;
  const uint16_t* W0 = g < p.g_split ? p.W0a + g * wst : p.W0b + (g - p.g_split) * wst;
  const uint16_t* W1 = W0;
  if (GATED) W1 = g < p.g_split ? p.W1a + g * wst : p.W1b + (g - p.g_split) * wst;
  const uint16_t* bsrc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int b = (wave + 4 * i) * RPB + lrow;  // weight-tile row 0..255
    int row;
    const uint16_t* Wm = W0;
    if (GATED) {
      // wave column wn = b/128 holds h columns nb*128 + wn*64 + [0,64): fragments 0,1 are the gate
      // rows, fragments 2,3 the matching up rows
      const int q = (b & 127) >> 5;
      row = nb * 128 + (b >> 7) * 64 + (q & 1) * 32 + (b & 31);
      Wm = q < 2 ? W0 : W1;
    } else {
      row = nb * kTN + b;
    }
    bsrc[i] = Wm + static_cast<size_t>(row) * Kd + lchunk * 8;
  }

  f32x16_t acc[MIV > 0 ? MIV : 1][4];
#pragma unroll
  for (int i = 0; i < (MIV > 0 ? MIV : 1); ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = Kd / BK;
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  // LDS offset of this lane's fragment row fr at K-step ks inside a 32-row-aligned block: the
  // swizzle term depends only on fr (the block bases are multiples of 32 rows), so one offset
  // per K-step serves every fragment of every stage.
  int lds_off[BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) lds_off[ks] = swz<BK>(fr, ks * 16 + fk);
  constexpr int PER = NA + NB;
  u32x4_t af[2][MIV > 0 ? MIV : 1], bf[2][4];
  auto fetch = [&](int stage, int ks, int set) {
    const uint16_t* a = sA + stage * kStageA + wm * (BM / 2) * BK;
    const uint16_t* b = sB + stage * kStageB + wn * 128 * BK;
#pragma unroll
    for (int i = 0; i < MIV; ++i)
      af[set][i] = *reinterpret_cast<const u32x4_t*>(&a[i * 32 * BK + lds_off[ks]]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[set][j] = *reinterpret_cast<const u32x4_t*>(&b[j * 32 * BK + lds_off[ks]]);
  };
  if constexpr (S == 2) {
    // Two-stage ring with whole 128-byte row segments per DMA instruction (BK = 64): iteration kt
    // waits for tile kt, passes the barrier (every wavefront is then done with the other stage),
    // and fills the other stage with tile kt+1 while it computes tile kt; the DMA instructions
    // are spread one per few MFMAs. Past the end of K the last tile is reloaded (never read).
    constexpr int KS = BK / 16;
    constexpr int kMf = KS * MIV * 4;                     // MFMAs per K-tile
    constexpr int kStepD = kMf >= PER ? kMf / PER : 1;    // one DMA every kStepD MFMAs
    static_assert(MIV == 0 || kMf % PER == 0, "DMA spread must divide the MFMAs");
#pragma unroll
    for (int d = 0; d < PER; ++d) {
      if (d < NA)
        lds_dma16(p.A + aoff[d], sA + (wave + 4 * d) * 512);
      else
        lds_dma16(bsrc[d - NA], sB + (wave + 4 * (d - NA)) * 512);
    }
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<0>();  // tile kt has landed
      barrier_no_fence();
      const int kn = min(kt + 1, nk - 1);
      const int sn = (kt + 1) & 1;
      auto dma = [&](int d) {
        if (d < NA)
          lds_dma16(p.A + aoff[d] + kn * BK, sA + sn * kStageA + (wave + 4 * d) * 512);
        else
          lds_dma16(bsrc[d - NA] + kn * BK, sB + sn * kStageB + (wave + 4 * (d - NA)) * 512);
      };
      if (MIV == 0) {
#pragma unroll
        for (int d = 0; d < PER; ++d) dma(d);
        continue;
      }
      fetch(kt & 1, 0, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) fetch(kt & 1, ks + 1, (ks + 1) & 1);
#pragma unroll
        for (int i = 0; i < MIV; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = mfma32x32x16(af[ks & 1][i], bf[ks & 1][j], acc[i][j]);
            const int m = (ks * MIV + i) * 4 + j + 1;
            if (m % kStepD == 0 && m / kStepD <= PER) dma(m / kStepD - 1);
          }
      }
      constexpr int kFrag = MIV + 4;
      constexpr int kMfs = MIV * 4;
      __builtin_amdgcn_sched_group_barrier(0x100, kFrag, 0);
#pragma unroll
      for (int m = 0; m < kMf; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (m / kMfs + 1 < KS && m % kMfs < kFrag) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if ((m + 1) % kStepD == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
  } else {
    // Software pipeline (BK = 32, two K-steps per K-tile). Iteration kt runs in two phases split
    // by the workgroup barrier:
    //   A: MFMAs of K-step 0 of tile kt; read tile kt's K-step-1 fragments; half of the DMA of
    //      tile kt+S-1 (into the stage tile kt-1 used, free since the barrier of iteration kt-1);
    //   wait until tile kt+1 has landed and this wavefront's fragment reads are complete; barrier;
    //   B: MFMAs of K-step 1 of tile kt; read tile kt+1's K-step-0 fragments; the other half of
    //      the DMA.
    // No fragment read waits right behind a barrier. Past the end of K every DMA reloads the last
    // tile into the free stage (never read, except by the final prefetch whose values are unused),
    // so each wait is a constant count and the phases have no branches.
    static_assert(BK == 32, "the two-phase pipeline assumes two K-steps per K-tile");
    constexpr int HALF = PER / 2;
    for (int t = 0; t < S - 1; ++t) {
      const int kt_src = min(t, nk - 1);
  #pragma unroll
      for (int d = 0; d < PER; ++d) {
        if (d < NA)
          lds_dma16(p.A + aoff[d] + kt_src * BK, sA + t * kStageA + (wave + 4 * d) * 512);
        else
          lds_dma16(bsrc[d - NA] + kt_src * BK, sB + t * kStageB + (wave + 4 * (d - NA)) * 512);
      }
    }
    wait_vmcnt<(S - 2) * PER>();  // tile 0 has landed
    barrier_no_fence();
    if (MIV > 0) fetch(0, 0, 0);
    constexpr int kMf = MIV * 4;                        // MFMAs per K-step
    constexpr int kStepH = kMf >= HALF ? kMf / HALF : 1;  // one DMA every kStepH MFMAs
    static_assert(MIV == 0 || kMf % HALF == 0, "DMA spread must divide the MFMAs");
    constexpr int kFrag = MIV + 4;                      // fragment reads per K-step
    for (int kt = 0; kt < nk; ++kt) {
      const int kn = min(kt + S - 1, nk - 1);
      const int sn = (kt + S - 1) % S;
      auto dma = [&](int d) {
        if (d < NA)
          lds_dma16(p.A + aoff[d] + kn * BK, sA + sn * kStageA + (wave + 4 * d) * 512);
        else
          lds_dma16(bsrc[d - NA] + kn * BK, sB + sn * kStageB + (wave + 4 * (d - NA)) * 512);
      };
      // ---- phase A
      if (MIV > 0) {
        fetch(kt % S, 1, 1);
  #pragma unroll
        for (int i = 0; i < MIV; ++i)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = mfma32x32x16(af[0][i], bf[0][j], acc[i][j]);
            const int m = i * 4 + j + 1;
            if (m % kStepH == 0 && m / kStepH <= HALF) dma(m / kStepH - 1);
          }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  #pragma unroll
        for (int m = 1; m < kMf; ++m) {
          if (m - 1 < kFrag) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (m % kStepH == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        if (kMf - 1 < kFrag) __builtin_amdgcn_sched_group_barrier(0x100, kFrag - (kMf - 1), 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      } else {
  #pragma unroll
        for (int d = 0; d < HALF; ++d) dma(d);
      }
      wait_vmcnt<(S - 3) * PER + HALF>();  // tile kt+1 has landed
      wait_lgkmcnt0();  // this wavefront's fragment reads of the stage are complete
      barrier_no_fence();
      // ---- phase B
      if (MIV > 0) {
        fetch((kt + 1) % S, 0, 0);
  #pragma unroll
        for (int i = 0; i < MIV; ++i)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = mfma32x32x16(af[1][i], bf[1][j], acc[i][j]);
            const int m = i * 4 + j + 1;
            if (m % kStepH == 0 && m / kStepH <= HALF) dma(HALF + m / kStepH - 1);
          }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  #pragma unroll
        for (int m = 1; m < kMf; ++m) {
          if (m - 1 < kFrag) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (m % kStepH == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        if (kMf - 1 < kFrag) __builtin_amdgcn_sched_group_barrier(0x100, kFrag - (kMf - 1), 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      } else {
  #pragma unroll
        for (int d = HALF; d < PER; ++d) dma(d);
      }
    }
  }

  // ---- epilogue: lane holds rows 8*(v/4) + 4*(lane/32) + v%4 of each 32x32 block, column lane%32
  if (EPI == kEpiF32) {
#pragma unroll
    for (int i = 0; i < MIV; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = r0 + wm * (BM / 2) + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r >= r1) continue;
        float* o = p.out_f32 + static_cast<size_t>(r) * p.N;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[nb * kTN + wn * 128 + j * 32 + fr] = acc[i][j][v];
      }
    return;
  }
  // bf16 outputs go through LDS so that global stores are whole 16-byte row segments. Each
  // wavefront owns a [MIV*32][C] bf16 slice of the (now idle) stage ring; its 16-byte chunks are
  // XOR-swizzled by row so the column-wise fragment writes spread over the banks.
  constexpr int C = GATED ? 64 : 128;  // output columns of this wavefront
  constexpr int CH = C / 8;            // 16-byte chunks per row
  __syncthreads();                     // every wavefront is done with the stage ring
  uint16_t* ep = smem + wave * (BM / 2) * C;
  auto eoff = [&](int row, int col) { return row * C + ((((col >> 3) ^ row) & (CH - 1)) << 3) + (col & 7); };
#pragma unroll
  for (int i = 0; i < MIV; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (GATED) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          ep[eoff(row, j * 32 + fr)] = f32_to_bf16(clamped_swiglu(acc[i][j][v], acc[i][j + 2][v], p.limit));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) ep[eoff(row, j * 32 + fr)] = f32_to_bf16(acc[i][j][v]);
      }
    }
    // one fragment row at a time: keeps the scheduler from reading every accumulator out of the
    // AGPRs at once
    __builtin_amdgcn_sched_barrier(0);
  }
  // the slice is private to this wavefront; its LDS accesses complete in order
  const int col0 = GATED ? nb * 128 + wn * 64 : nb * kTN + wn * 128;
  const int rbase = r0 + wm * (BM / 2);
  constexpr int RPI = 64 / CH;  // rows per store instruction
#pragma unroll
  for (int it = 0; it < MIV * 32 / RPI; ++it) {
    const int row = it * RPI + lane / CH;
    const int ch = lane % CH;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&ep[row * C + (((ch ^ row) & (CH - 1)) << 3)]);
    if (rbase + row < r1)
      *reinterpret_cast<u32x4_t*>(p.out + static_cast<size_t>(rbase + row) * p.N + col0 + ch * 8) = v;
  }
}


template <int EPI, int BM, int BK, int S>
__global__ __launch_bounds__(256, 1) void ffn_tiled_kernel(GroupedParams p, int nblk) {
  constexpr int MI = BM / 64;  // 32-row fragments per wavefront

  // ---- work item: XCD-contiguous slices of the work list (band order inside each group)
  const bool dense = p.tiles == nullptr;
  const int n_tiles = dense ? (p.rows_max + BM - 1) / BM : p.tiles[0];
  const int total = n_tiles * nblk;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int w = (blockIdx.x % kXcds) * per_xcd + slot;
  if (w >= total) return;
  // the group's items occupy nblk x its tile range of the work list
  const int ts = w / nblk;
  const int g = dense ? 0 : p.tiles[1 + ts];
  const int first = dense ? 0 : p.tiles[1 + 2 * p.max_tiles + ts];
  const int mt = dense ? n_tiles : p.tiles[1 + 3 * p.max_tiles + ts];
  const int u = w - first * nblk;
  const int band = u / (kBand * nblk);
  const int band_tiles = min(kBand, mt - band * kBand);
  if (band_tiles <= 0) return;  // only with a malformed (truncated) tile table
  const int v = u - band * kBand * nblk;
  const int nb = v / band_tiles;
  const int tile = first + band * kBand + (v - nb * band_tiles);
  if (tile >= n_tiles) return;
  const int r0 = dense ? tile * BM : p.tiles[1 + p.max_tiles + tile];
  const int r_end = dense ? p.rows_max : p.offsets[g + 1];
  const int r1 = min(min(r0 + BM, r_end), p.rows_max);
  if (r0 < 0 || r1 <= r0) return;

  const int wm = (threadIdx.x >> 6) >> 1;
  // 32-row fragments of this wavefront that hold rows of the group (uniform per wavefront); the
  // main loop is specialised on it so that no branch sits between the MFMAs
  const int miv = min(MI, max(0, (r1 - (r0 + wm * (BM / 2)) + 31) / 32));
  switch (miv) {
    case 0: tiled_main<EPI, BM, BK, S, 0>(p, g, nb, r0, r1); break;
    case 1: tiled_main<EPI, BM, BK, S, 1>(p, g, nb, r0, r1); break;
    case 2: tiled_main<EPI, BM, BK, S, (2 <= MI ? 2 : MI)>(p, g, nb, r0, r1); break;
    case 3: tiled_main<EPI, BM, BK, S, (3 <= MI ? 3 : MI)>(p, g, nb, r0, r1); break;
    default: tiled_main<EPI, BM, BK, S, MI>(p, g, nb, r0, r1); break;
  }
}


// One-time opt-in to the large dynamic LDS allocation of a tiled kernel instantiation.
template <int EPI, int BM, int BK, int S>
hipError_t tiled_prepare() {
  static bool done = false;
  if (done) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&ffn_tiled_kernel<EPI, BM, BK, S>),
      hipFuncAttributeMaxDynamicSharedMemorySize, tiled_smem<BM, BK, S>());
  if (e == hipSuccess) done = true;
  return e;
}

template <int EPI, int BM, int BK, int S>
hipError_t tiled_launch(const GroupedParams& p, int nblk, int n_tiles_max, hipStream_t stream) {
  const hipError_t e = tiled_prepare<EPI, BM, BK, S>();
  if (e != hipSuccess) return e;
  const int grid = (n_tiles_max * nblk + kXcds - 1) / kXcds * kXcds;
  const auto kernel = ffn_tiled_kernel<EPI, BM, BK, S>;
  constexpr size_t smem = tiled_smem<BM, BK, S>();
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), smem, stream, p, nblk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tiled(Epilogue epi, const GroupedParams& p, int max_tiles, hipStream_t stream) {
  static_assert(kBM == kTiledRows, "row tile of the tiled kernel");
  switch (epi) {
    case kEpiSwiglu: return tiled_launch<kEpiSwiglu, kBM, kBK, kStages>(p, p.N / 128, max_tiles, stream);
    case kEpiBf16: return tiled_launch<kEpiBf16, kBM, kBK, kStages>(p, p.N / kTN, max_tiles, stream);
    default: return tiled_launch<kEpiF32, kBM, kBK, kStages>(p, p.N / kTN, max_tiles, stream);
  }
}

bool dense_gemm_f32_supported(int N, int Kd) { return N == kTN && Kd % kBK == 0; }

hipError_t launch_dense_gemm_f32(const uint16_t* A, int rows, const uint16_t* W, int N, int Kd,
                                 float* out, hipStream_t stream) {
  GroupedParams p{};
  p.A = A;
  p.a_rows = rows;
  p.n_ident = 0x7fffffff;
  p.rows_max = rows;
  p.tiles = nullptr;  // dense mode
  p.W0a = p.W0b = W;
  p.g_split = 0;
  p.out_f32 = out;
  p.N = N;
  p.Kd = Kd;
  return launch_tiled(kEpiF32, p, (rows + kBM - 1) / kBM, stream);
}

}  // namespace moe
