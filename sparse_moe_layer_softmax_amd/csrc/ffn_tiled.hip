// ffn_tiled.hip -- LDS-tiled MFMA grouped GEMM for many rows per expert (prefill), and the
// dense fp32-output GEMM of the router at large T.
//
// Hy3 deep-dive (happyrock.cloud) `MoEFeedForward` (SwiGLU expert FFN) and Hy4 config
// walkthrough (lshu.cn), section "MoE routed experts" (swiglu_limit, silu); Hy3 explainer
// (tqpw.cn) section 2.1: each expert runs on the rows routed to it.
#include <algorithm>
#include <atomic>

#include "ffn_kernels.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------------------------
// Kernel "tiled": a workgroup computes a 320-row x 256-weight-row output tile (gate/up: 128 gate
// rows and the 128 matching up rows) with eight wavefronts, two per SIMD. Wavefront w owns rows
// 160*(w/4) .. +160 and weight rows 64*(w%4) .. +64 of the tile: 5 x 2 MFMA 32x32x16 fragments,
// 160 fp32 accumulators per lane.
//  - The operand bytes a CU moves into LDS per FLOP, (BM + BN) / (BM * BN), bound this kernel
//    (the global->LDS fill path, not the MFMAs, is the limit), so the tile is as large as the
//    register file of two wavefronts per SIMD allows. 320 rows also fit a whole expert at the
//    prefill shape (about T*k/E = 256 rows each, never more than ~310) in one row tile.
//  - K is staged 64 at a time through a two-stage LDS ring (2 x 72 KB) filled by direct
//    global->LDS loads (global_load_lds_dwordx4, no VGPR staging). Weight tiles load
//    non-temporal when their group has a single row tile and under the default cache policy when
//    several row tiles read them. One such instruction moves 1 KB: 8 rows of 128 bytes, whole L2
//    lines. The DMA of K-tile kt+1 is issued at the start of K-tile kt, so it has a whole K-tile
//    of compute to land.
//  - Each wavefront loads the activation rows of its own live 32-row fragments (one instruction
//    per fragment) and an eighth of the weight tile, so rows past the end of a group cost neither
//    DMA nor MFMA: ragged expert tails are cheap.
//  - Ping-pong: the two wavefronts of a SIMD alternate between a memory phase (issue DMA, read the
//    fragments of a 32-wide K slice from LDS into VGPRs) and a compute phase (20 MFMAs on
//    fragments already in registers, nothing else). Workgroup barriers separate the phases; the
//    second half of the wavefronts starts one phase late, so while one wavefront of a SIMD
//    computes, the other one moves data, and a stall of the memory pipeline (DMA issue
//    back-pressure, LDS latency) never holds up the MFMA issue of the computing wavefront.
//  - LDS rows are XOR-swizzled by 16-byte chunk (swz) so MFMA operand reads are conflict free
//    on the 64-bank LDS.
//  - The main loop is specialised on the number of 32-row fragments of a wavefront that hold
//    rows of the group (MIV), so partly filled tiles skip MFMAs and DMA without branching in the
//    loop.
//  - Work items are ordered inside XCD-contiguous slices of the real work list (its size comes
//    from the device-side tile count, so spare grid slots do not unbalance the XCDs); inside a
//    group the work runs in bands of up to kBand row tiles, n-blocks outer and the band's row
//    tiles inner, so workgroups running together on an XCD share one weight tile (same
//    n-block) and the band's activation rows through L2, and a group with at most kBand row
//    tiles reads each of its weight tiles from HBM once.
//  - bf16 results are staged through LDS and written as whole 16-byte row segments.
//  - kEpiBf16T (the backward's data gradients, out = A W with W stored [K][N]): the weight tile
//    is moved into LDS as it lies in memory, [64 k][256 n], and each MFMA B operand is put
//    together by two LDS transpose reads (ds_read_b64_tr_b16), so the weights need no
//    transposed copy in HBM.
constexpr int kThreads = 512;
constexpr int kBM = 320;  // rows per tile
constexpr int kMI = 5;    // 32-row fragments per wavefront (160 rows: half the tile)
constexpr int kTN = 256;  // weight rows per tile (gate/up: 128 gate + 128 up)
constexpr int kBK = 64;   // K per stage
constexpr int kStages = 2;
constexpr int kXcds = 8;
constexpr int kBand = 8;
constexpr int kStageA = kBM * kBK, kStageB = kTN * kBK;  // bf16 elements per stage
constexpr int kStageB8 = kTN * kBK;                      // bytes per FP8 weight stage
constexpr int kStagesB8 = 3;  // FP8 weight stages: K-tile kt+2 is fetched during K-tile kt
constexpr size_t kSmemRing = sizeof(uint16_t) * kStages * (kStageA + kStageB);
// MX scale stages: per K-tile one dword (4 E8M0 bytes) per tile row and per weight row
constexpr int kScaleStage = kBM + kTN;
// after the ring: the W8A8 row scales of the tile, or the two MX scale stages
constexpr size_t kSmem = kSmemRing + sizeof(uint32_t) * (2 * kScaleStage > kBM ? 2 * kScaleStage : kBM);
constexpr int kDmaB = kTN / 8 / 8;  // weight-tile DMA instructions per wavefront per K-tile

// LDS element offset of (row, k) in a [rows][64] bf16 stage. The eight 16-byte chunks of a row
// are XOR-swizzled (slot = chunk ^ (row % 8) ^ ((row / 8) % 2)) so that an MFMA operand read (32
// consecutive rows at one logical chunk per 32-lane half) puts the 16 lanes of each pass on 16
// distinct 16-byte bank groups of the 64-bank LDS.
__device__ __forceinline__ int swz(int row, int k) {
  return row * kBK + (((k >> 3) ^ (row & 7) ^ ((row >> 3) & 1)) << 3) + (k & 7);
}

// Weight stage of kEpiBf16T: [64 k][256 n] bf16 as the weight lies in memory. The 32 16-byte
// chunks of row k sit at slot chunk ^ tsw(k). A transpose read serves a 16-lane group 4 k-rows
// x 16 columns; one instruction covers 8 k-rows (k % 4 all four values, k / 8 both parities)
// and 4 consecutive chunks, and tsw sends those 16 (row, chunk) pairs to 16 distinct 16-byte
// bank groups however the hardware pairs the lane groups.
__device__ __forceinline__ int tsw(int k) { return ((k & 3) << 2) ^ (((k >> 3) & 1) << 1); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// LDS transpose read of 4 16-bit values. In each group of 16 lanes, lane i returns element
// i % 4 of the 8 bytes addressed by lanes 4r + i / 4 of its group, r = 0..3, in that order:
// with lane 4r + q pointing at row r, columns 4q..4q+3 of a 4 x 16 block, lane i gets column i.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* l) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(l));
  return __builtin_bit_cast(u32x2_t, v);
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
// in-flight global->LDS load). Callers order their own LDS traffic with wait_vmcnt /
// wait_lgkmcnt0; the empty asm statements keep the compiler from moving memory accesses across
// the barrier and the scheduling barriers keep it from moving anything else (MFMAs) across.
__device__ __forceinline__ void barrier_no_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Global->LDS DMA of 16 bytes per lane. STREAM marks the load non-temporal (cache policy NT): used
// for the weight tiles of a group with a single row tile, which no other workgroup reads and
// which would otherwise displace the activation rows that the group's column blocks re-read from
// L2.
template <bool STREAM = false>
__device__ __forceinline__ void lds_dma16(const uint16_t* g, uint16_t* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, STREAM ? 2 : 0);
}

// The same DMA through a buffer descriptor: address = descriptor base + voff (per lane) + soff
// (uniform), 32-bit byte offsets. The per-lane address is one register instead of a 64-bit pair,
// which leaves the main loop about 20 more registers; the fill runs 5-8% faster than in the 64-bit
// form at the prefill and long-prefill shapes.
template <bool STREAM = false>
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              uint16_t* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)l, 16, voff, soff, 0,
                                           STREAM ? 2 : 0);
}

// Raw (unstrided, untyped) buffer descriptor over `bytes` bytes from `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// EPI = kEpiSwiglu: gate/up rows interleaved, h = bf16(silu(clamp g) * clamp u);
// kEpiBf16: plain bf16 output (down projection); kEpiF32: fp32 output (router logits).
// p.tiles == nullptr selects dense mode: one group of rows [0, rows_max) in kBM-row tiles.
// Main loop and epilogue of one tile over the nk K-tiles from K-tile kb (fp32 output: into the
// partial-sum plane split); MIV = live 32-row fragments of this wavefront (0..5). BUF: the DMA
// goes through buffer descriptors, which the host selects when the activation operand and every
// weight matrix hold at most 4 GiB (each is then addressed by 32-bit byte offsets); otherwise
// through 64-bit addresses.
template <int EPI, int MIV, bool BUF>
__device__ __forceinline__ void tiled_main(const GroupedParams& p, int g, int nb, int r0, int r1,
                                           int kb, int nk, int split, bool b_shared) {
  constexpr bool W8 = EPI == kEpiSwiglu8 || EPI == kEpiBf16_8;     // FP8 weights, bf16 activations
  constexpr bool MX = EPI == kEpiSwigluMx || EPI == kEpiBf16Mx;     // ... with MX block scales
  constexpr bool A8 = EPI == kEpiSwiglu88 || EPI == kEpiBf16_88 || MX;  // FP8 weights and activations
  constexpr bool BT = EPI == kEpiBf16T;  // weights [Kd][N], read with the LDS transpose read
  constexpr bool GATED = EPI == kEpiSwiglu || EPI == kEpiSwigluBwd || EPI == kEpiSwiglu8 ||
                         EPI == kEpiSwiglu88 || EPI == kEpiSwigluSave || EPI == kEpiSwigluMx;
  constexpr int MV = MIV > 0 ? MIV : 1;  // array extent
  // DMA instructions of this wavefront that may still be in flight when a K-tile's operands
  // must have landed: FP8 weight tiles run one K-tile further ahead (the next-but-one tile's)
  constexpr int kLead = W8 ? 2 : 0;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sA = smem;                      // [2][320][64]
  uint16_t* sB = smem + kStages * kStageA;  // [2][256][64] bf16, or [2][256][64] bytes (W8)
  uint8_t* sB8 = reinterpret_cast<uint8_t*>(sB);
  const int Kd = p.Kd;
  const int tid = threadIdx.x;
  // wavefront index as a scalar: the LDS destinations of the DMA (M0) are then pure SALU math
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = wave >> 2;    // rows 160*half .. +160 of the tile; also the ping-pong group
  const int quarter = wave & 3;  // weight rows 64*quarter .. +64 of the tile
  if constexpr (A8 && !MX) {  // the activation-row scale of every tile row (0 past the group's end)
    float* srow = reinterpret_cast<float*>(smem + kSmemRing / sizeof(uint16_t));
    if (tid < kBM) {
      const int r = r0 + tid;
      float sa = 0.f;
      if (r < r1) {
        int src = r < p.n_ident ? r : p.gather[r - p.n_ident] / p.topk;
        if (static_cast<unsigned>(src) >= static_cast<unsigned>(p.a_rows)) src = 0;
        sa = p.a_scale[src];
      }
      srow[tid] = sa;
    }
    __syncthreads();
  }

  // ---- DMA assignment. A 1 KB block holds 8 rows of 64 elements; lane i fills its 16-byte slot
  // i: row i/8 of the block, physical chunk i%8, which holds the logical chunk that swz() places
  // there. A stage: the wavefront (half, quarter) fills blocks 20*half + quarter + 4i, i < MIV,
  // which together with the other quarters of its half are exactly the rows of its live
  // fragments (fragment i = blocks 20*half + 4i .. +4). B stage: wavefront w fills blocks w+8i.
  // Every block index used here is congruent to the quarter mod 2, so a row's (row / 8) % 2 is
  // quarter % 2, and its row % 8 is lane / 8.
  // Activation rows are addressed in 16-byte units by a 32-bit offset from A, so any row of an
  // operand of up to 64 GiB is reachable (row * Kd passes 2^32 elements for the activations of a
  // long prefill, e.g. h [T + T*K, I]); the host rejects larger operands.
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow ^ (quarter & 1);
  uint32_t a16[MV];
#pragma unroll
  for (int i = 0; i < MIV; ++i) {
    const int r = r0 + (20 * half + quarter + 4 * i) * 8 + lrow;
    int src = 0;
    if (r < r1) src = r < p.n_ident ? r : p.gather[r - p.n_ident] / p.topk;
    if (static_cast<unsigned>(src) >= static_cast<unsigned>(p.a_rows)) src = 0;
    a16[i] = static_cast<uint32_t>((static_cast<size_t>(src) * Kd + lchunk * 8) >> 3);
  }
  const size_t wst = static_cast<size_t>(p.N) * Kd;
  const uint16_t* W0 = g < p.g_split ? p.W0a + g * wst : p.W0b + (g - p.g_split) * wst;
  const uint16_t* W1 = W0;
  if (GATED) W1 = g < p.g_split ? p.W1a + g * wst : p.W1b + (g - p.g_split) * wst;
  // weight-tile row b (0..255) -> weight matrix row; gated: the wavefront with quarter q holds
  // h columns nb*128 + q*32 + [0,32), its fragment 0 the gate rows, fragment 1 the up rows
  auto wrow = [&](int b) { return GATED ? nb * 128 + (b >> 6) * 32 + (b & 31) : nb * kTN + b; };
  // the weight rows a wavefront moves all come from one matrix: block w + 8i holds tile rows
  // 8(w + 8i) .. +8, whose 32-row fragment index is (w >> 2) + 2i, so for gate/up the half of
  // the wavefront picks gate (0) or up (1). Block i's weight rows are block 0's plus 32i (gate/up:
  // wrow(b + 64i) = wrow(b) + 32i) or plus 64i (down), so one row address and a uniform step
  // address all of them.
  const uint16_t* Wb = GATED && half ? W1 : W0;
  const size_t bstep = static_cast<size_t>(GATED ? 32 : 64) * Kd;
  // weight rows likewise in 16-byte units from Wb (the weight gradients' B operands, [N][K] with
  // K about 9T, pass 2^32 elements at long prefills)
  uint32_t b16 = 0;
  if (!W8 && !BT) b16 = static_cast<uint32_t>((static_cast<size_t>(wrow(wave * 8 + lrow)) * Kd + lchunk * 8) >> 3);
  // (built in both forms, used only by the buffer form, where both sizes fit 32 bits)
  const __amdgpu_buffer_rsrc_t rA =
      raw_rsrc(p.A, static_cast<uint32_t>(static_cast<size_t>(p.a_rows) * Kd * sizeof(uint16_t)));
  const __amdgpu_buffer_rsrc_t rB = raw_rsrc(Wb, static_cast<uint32_t>(wst * sizeof(uint16_t)));
  // W8: a B stage is [256 rows][64 codes]; a 1 KB DMA block holds 16 rows. Lane i fills row
  // i/4 of the block, physical 16-byte chunk i%4, which holds logical chunk
  // (i%4) ^ ((row / 4) % 4); wavefront w fills blocks w + 8i, i < 2.
  // The matrix of block w + 8i, (w + 8i) / 2 mod 2 for gate/up, is uniform over the wavefront.
  // Buffer form: byte offsets qoff8[i] from that matrix (N * Kd bytes).
  const uint8_t* bsrc8[2];
  uint32_t qoff8[2] = {0, 0};
  __amdgpu_buffer_rsrc_t rQ[2] = {rB, rB};
  if constexpr (W8) {
    const uint8_t* Q0 = g < p.g_split ? p.Q0a + g * wst : p.Q0b + (g - p.g_split) * wst;
    const uint8_t* Q1 = Q0;
    if (GATED) Q1 = g < p.g_split ? p.Q1a + g * wst : p.Q1b + (g - p.g_split) * wst;
    const int lc8 = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int b = (wave + 8 * i) * 16 + (lane >> 2);
      const bool up = GATED && (((wave + 8 * i) >> 1) & 1);
      const uint8_t* Qm = up ? Q1 : Q0;
      bsrc8[i] = Qm + static_cast<size_t>(wrow(b)) * Kd + kb * kBK + lc8 * 16;
      qoff8[i] = static_cast<uint32_t>(static_cast<size_t>(wrow(b)) * Kd + lc8 * 16);
      rQ[i] = raw_rsrc(Qm, static_cast<uint32_t>(wst));
    }
  }
  // BT: a B stage is [64 k][256 n]; a 1 KB DMA block holds 2 k-rows of 32 chunks. Lane i fills
  // row i / 32 of block w + 8i', physical chunk i % 32, which holds logical chunk
  // (i % 32) ^ tsw(row); the wavefront's four blocks lie 16 rows apart, which tsw ignores.
  const uint16_t* V0 = nullptr;
  const uint16_t* V1 = nullptr;
  uint32_t btoff = 0;  // within 16 k-rows of one K-tile: < 16 N
  __amdgpu_buffer_rsrc_t rV0 = rB, rV1 = rB;
  if constexpr (BT) {
    const size_t s0 = static_cast<size_t>(p.k_w0) * p.N, s1 = static_cast<size_t>(Kd - p.k_w0) * p.N;
    V0 = g < p.g_split ? p.W0a + g * s0 : p.W0b + (g - p.g_split) * s0;
    V1 = g < p.g_split ? p.W1a + g * s1 : p.W1b + (g - p.g_split) * s1;
    const int row = 2 * wave + (lane >> 5);
    btoff = static_cast<uint32_t>(row) * p.N + nb * kTN + (((lane & 31) ^ tsw(row)) << 3);
    rV0 = raw_rsrc(V0, static_cast<uint32_t>(s0 * sizeof(uint16_t)));
    rV1 = raw_rsrc(V1, static_cast<uint32_t>(s1 * sizeof(uint16_t)));
  }
  auto dma_a = [&](int kt, int stage) {
    if constexpr (BUF) {
      const uint32_t k2 = static_cast<uint32_t>((kb + kt) * kBK) * sizeof(uint16_t);
#pragma unroll
      for (int i = 0; i < MIV; ++i)
        lds_dma16_buf(rA, a16[i] * 16u, k2, sA + stage * kStageA + (20 * half + quarter + 4 * i) * 512);
    } else {
#pragma unroll
      for (int i = 0; i < MIV; ++i)
        lds_dma16(reinterpret_cast<const uint16_t*>(reinterpret_cast<const u32x4_t*>(p.A) + a16[i]) +
                      (kb + kt) * kBK,
                  sA + stage * kStageA + (20 * half + quarter + 4 * i) * 512);
    }
  };
  auto dma_b = [&](int kt, int stage) {
    if constexpr (BT) {
      const int k0 = (kb + kt) * kBK;  // first weight row of the K-tile (one matrix per K-tile)
      if constexpr (BUF) {
        const bool lo = k0 < p.k_w0;
        const uint32_t so = static_cast<uint32_t>(static_cast<size_t>(lo ? k0 : k0 - p.k_w0) * p.N * sizeof(uint16_t));
#pragma unroll
        for (int i = 0; i < kDmaB; ++i)
          lds_dma16_buf<true>(lo ? rV0 : rV1, btoff * 2u, so + static_cast<uint32_t>(i * 16 * p.N * sizeof(uint16_t)),
                              sB + stage * kStageB + (wave + 8 * i) * 512);
      } else {
        const uint16_t* src = k0 < p.k_w0 ? V0 + static_cast<size_t>(k0) * p.N
                                          : V1 + static_cast<size_t>(k0 - p.k_w0) * p.N;
#pragma unroll
        for (int i = 0; i < kDmaB; ++i)
          lds_dma16<true>(src + btoff + i * 16 * p.N, sB + stage * kStageB + (wave + 8 * i) * 512);
      }
    } else if constexpr (W8) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(sB8 + stage * kStageB8 + (wave + 8 * i) * 1024);
        if constexpr (BUF) {
          if (b_shared)
            lds_dma16_buf(rQ[i], qoff8[i], static_cast<uint32_t>((kb + kt) * kBK), dst);
          else
            lds_dma16_buf<true>(rQ[i], qoff8[i], static_cast<uint32_t>((kb + kt) * kBK), dst);
        } else {
          if (b_shared)
            lds_dma16(reinterpret_cast<const uint16_t*>(bsrc8[i] + kt * kBK), dst);
          else
            lds_dma16<true>(reinterpret_cast<const uint16_t*>(bsrc8[i] + kt * kBK), dst);
        }
      }
    } else if constexpr (BUF) {
      const uint32_t k2 = static_cast<uint32_t>((kb + kt) * kBK) * sizeof(uint16_t);
      if (b_shared) {
#pragma unroll
        for (int i = 0; i < kDmaB; ++i)
          lds_dma16_buf(rB, b16 * 16u, static_cast<uint32_t>(i * bstep * sizeof(uint16_t)) + k2,
                        sB + stage * kStageB + (wave + 8 * i) * 512);
      } else {
#pragma unroll
        for (int i = 0; i < kDmaB; ++i)
          lds_dma16_buf<true>(rB, b16 * 16u, static_cast<uint32_t>(i * bstep * sizeof(uint16_t)) + k2,
                              sB + stage * kStageB + (wave + 8 * i) * 512);
      }
    } else {
      if (b_shared) {
#pragma unroll
        for (int i = 0; i < kDmaB; ++i)
          lds_dma16(reinterpret_cast<const uint16_t*>(reinterpret_cast<const u32x4_t*>(Wb + i * bstep) + b16) +
                        (kb + kt) * kBK,
                    sB + stage * kStageB + (wave + 8 * i) * 512);
      } else {
#pragma unroll
        for (int i = 0; i < kDmaB; ++i)
          lds_dma16<true>(reinterpret_cast<const uint16_t*>(reinterpret_cast<const u32x4_t*>(Wb + i * bstep) + b16) +
                              (kb + kt) * kBK,
                          sB + stage * kStageB + (wave + 8 * i) * 512);
      }
    }
  };

  // MX: the K-tile's scale dwords into scale stage `stage` (after the ring): tile rows (wavefront
  // 0: rows 0-255, wavefront 1: rows 256-319, 16 lanes) and weight rows (wavefront 2; gate/up:
  // gate rows in lanes 0-31, up rows in lanes 32-63). Each lane moves the dwords of 4 rows.
  uint32_t* sS = reinterpret_cast<uint32_t*>(smem + kSmemRing / sizeof(uint16_t));
  const uint8_t* Xg = nullptr;
  const uint8_t* Xu = nullptr;
  if constexpr (MX) {
    const size_t xst = static_cast<size_t>(Kd / kBK) * p.N * sizeof(uint32_t);  // bytes per matrix
    Xg = g < p.g_split ? p.X0a + g * xst : p.X0b + (g - p.g_split) * xst;
    Xu = GATED ? (g < p.g_split ? p.X1a + g * xst : p.X1b + (g - p.g_split) * xst) : Xg;
  }
  auto dma_s = [&](int kt, int stage) {
    if constexpr (MX) {
      const size_t kk = static_cast<size_t>(kb + kt);
      uint32_t* dst = sS + stage * kScaleStage;
      if (wave == 0 || (wave == 1 && lane < (kBM - 256) / 4)) {
        const uint8_t* src = p.a_mx + ((kk * p.a_mx_rows + r0 + 256 * wave) * 4 + lane * 16);
        lds_dma16(reinterpret_cast<const uint16_t*>(src), reinterpret_cast<uint16_t*>(dst + 256 * wave));
      } else if (wave == 2) {
        const size_t plane = kk * p.N;
        const uint8_t* src = GATED ? (lane < 32 ? Xg : Xu) + (plane + nb * 128 + (lane & 31) * 4) * 4
                                   : Xg + (plane + nb * kTN + lane * 4) * 4;
        lds_dma16(reinterpret_cast<const uint16_t*>(src), reinterpret_cast<uint16_t*>(dst + kBM));
      }
    }
  };
  // MX: this K-tile's scale dwords of the lane's A rows and weight rows, shifted so that byte 0
  // holds the scale the lane supplies in the current slice h: lane half q gives the scale of the
  // slice's block q, block 2h + q of the K-tile
  uint32_t dsa[MV], dsb[2];

  f32x16_t acc[MV][2];
#pragma unroll
  for (int i = 0; i < MV; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int fr = lane & 31, fk = (lane >> 5) * 8;
  // LDS offset of this lane's fragment row fr at 16-wide K-step ks inside a 32-row-aligned
  // block: the swizzle term depends only on fr (row bases are multiples of 32), so one offset
  // per K-step serves every fragment and stage.
  // W8 takes a different one-to-one assignment of K elements to lanes, the same for A and B:
  // K-step ks of slice h reads elements 32h + 16q + 8ks + [0, 8) (q = lane / 32), so that one
  // 16-byte LDS read returns a lane's codes for both K-steps of the slice.
  int lds_off[kBK / 16];
  if constexpr (!A8) {
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks)
      lds_off[ks] = W8 ? swz(fr, 32 * (ks >> 1) + 2 * fk + 8 * (ks & 1)) : swz(fr, ks * 16 + fk);
  }
  // W8 B read: row quarter*64 + 32j + fr, logical chunk 2h + q of the 64-byte row
  const int boff8 = ((fr >> 2) & 3);
  // BT B read of fragment j at K-step ks: lane group G = lane / 16 covers columns
  // quarter*64 + 32j + 16(G % 2) + [0, 16) and k-rows 16ks + 8(G / 2) + [0, 8) in two reads of
  // 4 rows; lane 4r + q of a group points at row r, columns 4q..4q+3 of its 4 x 16 block. The
  // k-row's tsw term is the same for every ks and both reads.
  int bt_rd[2] = {0, 0};
  if constexpr (BT) {
    const int G = lane >> 4, q = lane & 15;
    const int kr = 8 * (G >> 1) + (q >> 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n0 = quarter * 64 + 32 * j + 16 * (G & 1) + 4 * (q & 3);
      bt_rd[j] = kr * kTN + (((n0 >> 3) ^ tsw(kr)) << 3) + (n0 & 7);
    }
  }
  u32x4_t af[2][MV], bf[2][2];
  u32x8_t af8[MV], bf8[2];  // W8A8: one 32-code operand per fragment, its two 16-byte halves
  // fragments of the 32-wide K slice h of a stage
  auto fetch = [&](int stage, int bstage, int h) {
    const uint16_t* a = sA + stage * kStageA + half * 160 * kBK;
    const uint16_t* b = sB + stage * kStageB + quarter * 64 * kBK;
    if constexpr (A8) {
      // h is not a compile-time constant here (the slice loop is not unrolled): the two offsets
      // (those of K-steps 2h and 2h + 1) are computed, not looked up in lds_off, whose dynamic
      // indexing would put it in scratch memory and which would hold four more registers
      // lane half q: bytes 0-15 = codes 64h + 16q + [0, 16), bytes 16-31 = codes 64h + 32 + 16q +
      // [0, 16); the MFMA's first 32-code block is bytes 0-15 of both halves, its second bytes
      // 16-31 (the layout of its MX block scales)
      const int o0 = swz(fr, 32 * h + fk), o1 = swz(fr, 32 * h + 16 + fk);
#pragma unroll
      for (int i = 0; i < MIV; ++i) {
        af8[i].lo = *reinterpret_cast<const u32x4_t*>(&a[i * 32 * kBK + o0]);
        af8[i].hi = *reinterpret_cast<const u32x4_t*>(&a[i * 32 * kBK + o1]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf8[j].lo = *reinterpret_cast<const u32x4_t*>(&b[j * 32 * kBK + o0]);
        bf8[j].hi = *reinterpret_cast<const u32x4_t*>(&b[j * 32 * kBK + o1]);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < MIV; ++i) {
      af[0][i] = *reinterpret_cast<const u32x4_t*>(&a[i * 32 * kBK + lds_off[2 * h]]);
      af[1][i] = *reinterpret_cast<const u32x4_t*>(&a[i * 32 * kBK + lds_off[2 * h + 1]]);
    }
    if constexpr (BT) {
      const uint16_t* bt = sB + bstage * kStageB;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int o = bt_rd[j] + (32 * h + 16 * kk) * kTN;
          const u32x2_t lo = lds_read_tr16(bt + o), hi = lds_read_tr16(bt + o + 4 * kTN);
          bf[kk][j] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        }
    } else if (W8) {
      const uint8_t* b8 = sB8 + bstage * kStageB8 + quarter * 64 * 64;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4_t c = *reinterpret_cast<const u32x4_t*>(
            b8 + (j * 32 + fr) * 64 + (((2 * h + (lane >> 5)) ^ boff8) << 4));
        bf[0][j] = e4m3x8_to_bf16(c[0], c[1]);
        bf[1][j] = e4m3x8_to_bf16(c[2], c[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf[0][j] = *reinterpret_cast<const u32x4_t*>(&b[j * 32 * kBK + lds_off[2 * h]]);
        bf[1][j] = *reinterpret_cast<const u32x4_t*>(&b[j * 32 * kBK + lds_off[2 * h + 1]]);
      }
    }
  };

  // ---- pipeline. Phases alternate memory (M) and compute (C), each covering a 32-wide K slice
  // (two per K-tile); every phase ends at a workgroup barrier. Half 0 runs M C M C ...; half 1
  // runs the same one phase later, so the halves are always in opposite phases. The first M of
  // K-tile kt issues this wavefront's DMA of K-tile kt+1 into the other stage (both halves
  // finished reading K-tile kt-1 from it before the barrier that opened this M); every M reads
  // the fragments of its slice. K-tile kt+1 must have landed before the barrier that opens half
  // 0's first M of it: each wavefront waits for all of its DMA there (half 0 at the end of the
  // last C of K-tile kt, half 1 at the end of its last M). Past the end of K the DMA reloads the
  // last K-tile into the free stage (never read). Every wavefront passes 2 + 4*nk barriers.
  // nk == 0 (an empty K range, uniform over the workgroup): no DMA, no barrier, zero result
  if (nk > 0) {
    dma_a(0, 0);
    dma_b(0, 0);
    dma_s(0, 0);
    if (W8) dma_b(min(1, nk - 1), 1);
    wait_vmcnt<kLead>();
    barrier_no_fence();
    if (half == 1) barrier_no_fence();
    // one memory phase and one compute phase of 32-wide K slice h of K-tile kt
    auto phase = [&](int kt, int h) {
      // ---- memory phase
      if (MIV > 0) fetch(kt & 1, W8 ? kt % kStagesB8 : kt & 1, h);
      if (MX && MIV > 0) {  // the K-tile's scale dwords, read with the slice-0 fragments
        if (h == 0) {
          const uint32_t* ss = sS + (kt & 1) * kScaleStage;
#pragma unroll
          for (int i = 0; i < MIV; ++i) dsa[i] = ss[half * 160 + i * 32 + fr];
#pragma unroll
          for (int j = 0; j < 2; ++j) dsb[j] = ss[kBM + (GATED ? j * 128 + quarter * 32 + fr : quarter * 64 + j * 32 + fr)];
        }
      }
      if (h == 0) {
        dma_s(min(kt + 1, nk - 1), (kt + 1) & 1);
        dma_a(min(kt + 1, nk - 1), (kt + 1) & 1);
        if (W8) dma_b(min(kt + 2, nk - 1), (kt + 2) % kStagesB8);
        else dma_b(min(kt + 1, nk - 1), (kt + 1) & 1);
      }
      if (half == 1 && h == 1) wait_vmcnt<kLead>();
      wait_lgkmcnt0();
      if (MX && MIV > 0) {  // byte 0 <- the scale of block 2h + (lane half) of the K-tile
        const int sh = h == 0 ? 8 * (lane >> 5) : 16;
#pragma unroll
        for (int i = 0; i < MIV; ++i) dsa[i] >>= sh;
#pragma unroll
        for (int j = 0; j < 2; ++j) dsb[j] >>= sh;
      }
      barrier_no_fence();
      // ---- compute phase
      if (MIV > 0) {
        __builtin_amdgcn_s_setprio(1);
        if constexpr (MX) {  // one scaled FP8 MFMA covers the slice's two blocks
#pragma unroll
          for (int i = 0; i < MIV; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x64_fp8_mx(af8[i], bf8[j], acc[i][j], dsa[i], dsb[j]);
        } else if constexpr (A8) {  // one FP8 MFMA covers the slice's 64 codes
#pragma unroll
          for (int i = 0; i < MIV; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x64_fp8(af8[i], bf8[j], acc[i][j]);
        } else {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < MIV; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j)
                acc[i][j] = mfma32x32x16(af[ks][i], bf[ks][j], acc[i][j]);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      if (half == 0 && h == 1) wait_vmcnt<kLead>();
      barrier_no_fence();
    };
    for (int kt = 0; kt < nk; ++kt) {
      if constexpr (A8) {  // not unrolled: keeps the FP8 operands within the registers
#pragma clang loop unroll(disable)
        for (int h = 0; h < 2; ++h) phase(kt, h);
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) phase(kt, h);
      }
    }
    if (half == 0) barrier_no_fence();
  }

  // ---- epilogue: lane holds rows 8*(v/4) + 4*(lane/32) + v%4 of each 32x32 block, column lane%32
  const int rbase = r0 + half * 160;
  if (W8 || (A8 && !MX)) {  // per-row weight scales of this lane's two columns multiply the fp32 sums
    const size_t so = static_cast<size_t>(g < p.g_split ? g : g - p.g_split) * p.N;
    const float* S0 = (g < p.g_split ? p.S0a : p.S0b) + so;
    const float* S1 = GATED ? (g < p.g_split ? p.S1a : p.S1b) + so : S0;
    float sc[2];
    if (GATED) {
      sc[0] = S0[nb * 128 + quarter * 32 + fr];
      sc[1] = S1[nb * 128 + quarter * 32 + fr];
    } else {
      sc[0] = S0[nb * kTN + quarter * 64 + fr];
      sc[1] = S0[nb * kTN + quarter * 64 + 32 + fr];
    }
#pragma unroll
    for (int i = 0; i < MIV; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] *= sc[j];
  }
  if (EPI == kEpiF32) {
    // fp32 results go through LDS so that global stores are whole 16-byte row segments (a
    // quarter of the store instructions of per-lane 4-byte stores). Each wavefront stages one
    // 32-row x 64-column fragment row at a time in two private 8 KB buffers of the (now idle)
    // stage ring, used by alternate fragment rows; the 16-byte chunks are XOR-swizzled by bit 2
    // of the row, so the two lane halves of a column write (rows 4 apart) use different banks.
    __syncthreads();  // every DMA has landed and every wavefront left the ring
    const size_t plane = static_cast<size_t>(p.rows_max) * p.N;
    float* ob = p.out_f32 + split * plane;
    if (p.k_tiles && split >= p.g_split) ob = p.out_f32_b + (split - p.g_split) * plane;
    const int col0 = nb * kTN + quarter * 64;
    auto foff = [](int row, int col) {
      return row * 64 + (((col >> 2) ^ (((row >> 2) & 1) << 3)) << 2) + (col & 3);
    };
#pragma unroll
    for (int i = 0; i < MIV; ++i) {
      float* ep = reinterpret_cast<float*>(smem) + (wave * 2 + (i & 1)) * 32 * 64;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
#pragma unroll
        for (int j = 0; j < 2; ++j) ep[foff(row, j * 32 + fr)] = acc[i][j][v];
      }
      // the buffers are private to this wavefront and its LDS accesses complete in order
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = it * 4 + (lane >> 4);
        const int ch = lane & 15;
        const f32x4_t val = *reinterpret_cast<const f32x4_t*>(&ep[foff(row, ch * 4)]);
        const int r = rbase + i * 32 + row;
        // non-temporal: nothing in this kernel reads the planes back, and the weight gradients
        // write far more than the L2 holds
        if (r < r1)
          __builtin_nontemporal_store(val, reinterpret_cast<f32x4_t*>(ob + static_cast<size_t>(r) * p.N + col0 + ch * 4));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  if (EPI == kEpiSwigluBwd) {
    // g = acc[i][0], u = acc[i][1] at intermediate column c; the clamp passes the gradient on
    // [-L, L]. Lanes store 32 consecutive columns of a row (64-byte segments).
    const int c = nb * 128 + quarter * 32 + fr;
    const float L = p.limit;
    const size_t ld = 2 * static_cast<size_t>(p.N);
#pragma unroll
    for (int i = 0; i < MIV; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = rbase + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r >= r1) continue;
        float dg, du;
        swiglu_bwd(acc[i][0][v], acc[i][1][v], bf16_to_f32(p.dh[static_cast<size_t>(r) * p.N + c]),
                   L, dg, du);
        p.out[r * ld + c] = f32_to_bf16(dg);
        p.out[r * ld + p.N + c] = f32_to_bf16(du);
      }
    return;
  }
  // bf16 outputs go through LDS so that global stores are whole 16-byte row segments. Each
  // wavefront owns two [32][C] bf16 buffers of the (now idle) stage ring, used by alternate
  // fragment rows; their 16-byte chunks are XOR-swizzled by row so the column-wise fragment
  // writes spread over the banks.
  constexpr int C = GATED ? 32 : 64;  // output columns of this wavefront
  constexpr int CH = C / 8;           // 16-byte chunks per row
  constexpr int RPI = 64 / CH;        // rows per store instruction
  __syncthreads();                    // every DMA has landed and every wavefront left the ring
  const int col0 = GATED ? nb * 128 + quarter * 32 : nb * kTN + quarter * 64;
  auto eoff = [&](int row, int col) { return row * C + ((((col >> 3) ^ row) & (CH - 1)) << 3) + (col & 7); };
#pragma unroll
  for (int i = 0; i < MIV; ++i) {
    if constexpr (A8 && !MX) {  // the scale of each output row's activation row (staged in LDS)
      const float* srow = reinterpret_cast<const float*>(smem + kSmemRing / sizeof(uint16_t));
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4_t sa = *reinterpret_cast<const f32x4_t*>(
            &srow[half * 160 + i * 32 + 8 * g4 + 4 * (lane >> 5)]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j][4 * g4 + k] *= sa[k];
      }
    }
    uint16_t* ep = smem + (wave * 2 + (i & 1)) * 32 * C;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (GATED) {
        ep[eoff(row, fr)] = f32_to_bf16(clamped_swiglu(acc[i][0][v], acc[i][1][v], p.limit));
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) ep[eoff(row, j * 32 + fr)] = f32_to_bf16(acc[i][j][v]);
      }
    }
    // the buffers are private to this wavefront and its LDS accesses complete in order
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int row = it * RPI + lane / CH;
      const int ch = lane % CH;
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(&ep[row * C + (((ch ^ row) & (CH - 1)) << 3)]);
      const int r = rbase + i * 32 + row;
      if (r < r1) *reinterpret_cast<u32x4_t*>(p.out + static_cast<size_t>(r) * p.N + col0 + ch * 8) = val;
      if constexpr (MX && GATED) {
        // the four lanes of a row hold its 32 columns col0.. (block `quarter` of 128-column plane
        // nb): h's MX codes and scale byte for the down projection, from the bf16 values just
        // stored
        if (p.mx_hq) {
          uint2 codes;
          const int sc = mx_quant8(val, &codes);
          if (r < r1) {
            *reinterpret_cast<uint2*>(p.mx_hq + static_cast<size_t>(r) * p.N + col0 + ch * 8) = codes;
            if (ch == 0) p.mx_hs[(static_cast<size_t>(nb) * p.mx_h_rows + r) * 4 + quarter] = static_cast<uint8_t>(sc);
          }
        }
      }
    }
    // one fragment row at a time: keeps the scheduler from reading every accumulator at once
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (EPI == kEpiSwigluSave) {
    // the fp32 gate and up sums: each fragment row (32 rows x 32 gate + 32 up columns) goes
    // through a private 8 KB LDS buffer, as in the fp32 epilogue, for 16-byte row stores
    __syncthreads();  // every wavefront has left its bf16 staging buffers
    const int c0 = nb * 128 + quarter * 32;
    const size_t ldg = 2 * static_cast<size_t>(p.N);
    auto foff = [](int row, int col) {
      return row * 64 + (((col >> 2) ^ (((row >> 2) & 1) << 3)) << 2) + (col & 3);
    };
#pragma unroll
    for (int i = 0; i < MIV; ++i) {
      float* fp = reinterpret_cast<float*>(smem) + (wave * 2 + (i & 1)) * 32 * 64;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
#pragma unroll
        for (int j = 0; j < 2; ++j) fp[foff(row, j * 32 + fr)] = acc[i][j][v];
      }
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = it * 4 + (lane >> 4);
        const int ch = lane & 15;  // chunks 0..7: gate columns, 8..15: up columns
        const f32x4_t val = *reinterpret_cast<const f32x4_t*>(&fp[foff(row, ch * 4)]);
        const int r = rbase + i * 32 + row;
        const int col = ch < 8 ? c0 + ch * 4 : p.N + c0 + (ch - 8) * 4;
        if (r < r1)
          __builtin_nontemporal_store(val, reinterpret_cast<f32x4_t*>(p.gu + static_cast<size_t>(r) * ldg + col));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}


template <int EPI, bool BUF>
__global__ __launch_bounds__(kThreads, 1) void ffn_tiled_kernel(GroupedParams p, int nblk) {
  // ---- work item: XCD-contiguous slices of the work list (band order inside each group)
  const bool dense = p.tiles == nullptr;
  const int n_tiles = dense ? (p.rows_max + kBM - 1) / kBM : p.tiles[0];
  const int splits = dense && p.k_splits > 1 ? p.k_splits : 1;
  const int total = n_tiles * nblk * splits;
  // Work item of this workgroup. Normally XCD-contiguous slices of the list (workgroup i runs on
  // XCD i % 8), so that the workgroups of one XCD share operands through its L2. With per-split K
  // ranges (one split per expert, weight gradients) the splits differ in length by orders of
  // magnitude and the long ones are adjacent, so there the items go round-robin over the XCDs in
  // list order: the long splits (the list's first) spread over the whole GPU and start first.
  int ws;
  if (p.k_tiles) {
    ws = blockIdx.x;
  } else {
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    if (slot >= per_xcd) return;
    ws = (blockIdx.x % kXcds) * per_xcd + slot;
  }
  if (ws >= total) return;
  // dense mode: the K splits of one output tile are adjacent items. With per-split K-tile ranges
  // (k_tiles: one output matrix per split, over its own rows of K) the splits are outermost.
  int split, w;
  if (p.k_tiles) {
    split = ws / (n_tiles * nblk);
    w = ws - split * (n_tiles * nblk);
  } else {
    split = ws % splits;
    w = ws / splits;
  }
  const int nk = p.k_tiles ? p.k_tiles[2 * split + 1] : p.Kd / kBK / splits;  // K-tiles of this item
  const int kb = p.k_tiles ? p.k_tiles[2 * split] : split * nk;                // its first K-tile
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
  const int r0 = dense ? tile * kBM : p.tiles[1 + p.max_tiles + tile];
  const int r_end = dense ? p.rows_max : p.offsets[g + 1];
  const int r1 = min(min(r0 + kBM, r_end), p.rows_max);
  if (r0 < 0 || r1 <= r0) return;

  const int half = (threadIdx.x >> 6) >> 2;
  // weight tiles that several row tiles of the group read stay in L2 under the default policy; a group with one row tile streams its weights past L2 (non-temporal), so that they do
  // not evict the activation rows its column blocks share
  const bool b_shared = mt > 1;
  // 32-row fragments of this wavefront that hold rows of the group (uniform per wavefront); the
  // main loop is specialised on it so that no branch sits between the MFMAs. Every
  // specialisation passes the same barriers.
  const int miv = min(kMI, max(0, (r1 - (r0 + half * 160) + 31) / 32));
  switch (miv) {
    case 0: tiled_main<EPI, 0, BUF>(p, g, nb, r0, r1, kb, nk, split, b_shared); break;
    case 1: tiled_main<EPI, 1, BUF>(p, g, nb, r0, r1, kb, nk, split, b_shared); break;
    case 2: tiled_main<EPI, 2, BUF>(p, g, nb, r0, r1, kb, nk, split, b_shared); break;
    case 3: tiled_main<EPI, 3, BUF>(p, g, nb, r0, r1, kb, nk, split, b_shared); break;
    case 4: tiled_main<EPI, 4, BUF>(p, g, nb, r0, r1, kb, nk, split, b_shared); break;
    default: tiled_main<EPI, 5, BUF>(p, g, nb, r0, r1, kb, nk, split, b_shared); break;
  }
}


// Opt-in to the large dynamic LDS allocation of a tiled kernel instantiation. Calls may come
// from several host threads at once (one per stream): the flag is atomic, and a repeated opt-in
// by two first callers is harmless (the attribute is simply set twice to the same value).
template <int EPI, bool BUF>
hipError_t tiled_prepare() {
  static std::atomic<bool> done{false};
  if (done.load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_tiled_kernel<EPI, BUF>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kSmem);
  if (e == hipSuccess) done.store(true, std::memory_order_release);
  return e;
}

template <int EPI, bool BUF>
hipError_t tiled_launch_form(const GroupedParams& p, int nblk, int n_tiles_max, hipStream_t stream) {
  const hipError_t e = tiled_prepare<EPI, BUF>();
  if (e != hipSuccess) return e;
  const int items = n_tiles_max * nblk * (p.tiles == nullptr && p.k_splits > 1 ? p.k_splits : 1);
  const int grid = (items + kXcds - 1) / kXcds * kXcds;
  const auto kernel = ffn_tiled_kernel<EPI, BUF>;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), kSmem, stream, p, nblk);
  return hipGetLastError();
}

// The buffer-descriptor form when the activation operand and each weight matrix hold at most
// 4 GiB (32-bit byte offsets reach all of them), else the 64-bit-address form.
template <int EPI>
hipError_t tiled_launch(const GroupedParams& p, int nblk, int n_tiles_max, hipStream_t stream) {
  constexpr bool W8 = EPI == kEpiSwiglu8 || EPI == kEpiBf16_8;
  const size_t lim = 0xFFFFFFFFull;
  const bool a_fits = static_cast<size_t>(p.a_rows) * p.Kd * sizeof(uint16_t) <= lim;
  // one weight matrix: [N][Kd] (bf16 or FP8 codes), or for the transposed form [Kd][N] per group
  // split in two at k_w0
  const bool b_fits = static_cast<size_t>(p.N) * p.Kd * (W8 ? 1 : sizeof(uint16_t)) <= lim;
  if (a_fits && b_fits) return tiled_launch_form<EPI, true>(p, nblk, n_tiles_max, stream);
  return tiled_launch_form<EPI, false>(p, nblk, n_tiles_max, stream);
}

}  // namespace

hipError_t launch_tiled(Epilogue epi, const GroupedParams& p, int max_tiles, hipStream_t stream) {
  static_assert(kBM == kTiledRows, "row tile of the tiled kernel");
  switch (epi) {
    case kEpiSwiglu: return tiled_launch<kEpiSwiglu>(p, p.N / 128, max_tiles, stream);
    case kEpiSwigluBwd: return tiled_launch<kEpiSwigluBwd>(p, p.N / 128, max_tiles, stream);
    case kEpiSwigluSave: return tiled_launch<kEpiSwigluSave>(p, p.N / 128, max_tiles, stream);
    case kEpiSwiglu8: return tiled_launch<kEpiSwiglu8>(p, p.N / 128, max_tiles, stream);
    case kEpiBf16_8: return tiled_launch<kEpiBf16_8>(p, p.N / kTN, max_tiles, stream);
    case kEpiSwiglu88: return tiled_launch<kEpiSwiglu88>(p, p.N / 128, max_tiles, stream);
    case kEpiBf16_88: return tiled_launch<kEpiBf16_88>(p, p.N / kTN, max_tiles, stream);
    case kEpiSwigluMx: return tiled_launch<kEpiSwigluMx>(p, p.N / 128, max_tiles, stream);
    case kEpiBf16Mx: return tiled_launch<kEpiBf16Mx>(p, p.N / kTN, max_tiles, stream);
    case kEpiBf16: return tiled_launch<kEpiBf16>(p, p.N / kTN, max_tiles, stream);
    case kEpiBf16T: return tiled_launch<kEpiBf16T>(p, p.N / kTN, max_tiles, stream);
    default: return tiled_launch<kEpiF32>(p, p.N / kTN, max_tiles, stream);
  }
}

bool dense_gemm_f32_supported(int N, int Kd) { return N == kTN && Kd % kBK == 0; }

// The most K splits (a divisor of the K-tile count, at most 16) that keep one output tile per
// split item within one wave of workgroups on 256 CUs.
int dense_gemm_splits(int rows, int Kd) {
  const int tiles = (rows + kBM - 1) / kBM;
  const int nkt = Kd / kBK;
  int best = 1;
  for (int s = 2; s <= 16 && s <= nkt; ++s)
    if (nkt % s == 0 && tiles * s <= 256) best = s;
  return best;
}

hipError_t launch_dense_gemm_f32(const uint16_t* A, int rows, const uint16_t* W, int N, int Kd,
                                 int splits, float* out, hipStream_t stream) {
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
  p.k_splits = splits;
  return launch_tiled(kEpiF32, p, (rows + kBM - 1) / kBM, stream);
}

}  // namespace moe
