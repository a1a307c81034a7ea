// ffn.hip -- grouped SwiGLU expert FFN over variable-length row groups.
//
// Hy3 deep-dive (happyrock.cloud) `MoEFeedForward`: y = down(silu(gate x) * up x) with
// bias-free projections of shapes [I,H], [I,H], [H,I]. Hy4 config walkthrough (lshu.cn),
// section "MoE routed experts": swiglu_limit 10 clips the SwiGLU activations to +-10 (read here
// as clamping the gate and up pre-activations), hidden_act silu. Hy3 explainer (tqpw.cn)
// section 2.1: every expert runs on the rows routed to it.
//
// Rows arrive grouped (one group per expert, optionally the shared expert as group 0). A tile
// table built on the device maps workgroup -> (group, first row), so the grid is sized from
// host-known bounds and no host synchronisation is needed; spare workgroups exit at once.
//
// Kernel "skinny": tiles of up to 64 rows (MFMA 16x16x32, 16-row sub-blocks; only the occupied
// sub-blocks are computed). Each wavefront owns 16 output columns of the gate AND the up
// projection (so the SwiGLU epilogue pairs them in registers), or 32 columns of the down
// projection. Weight fragments are loaded straight from HBM with 16-byte loads in MFMA operand
// order: this is the weight-streaming path for small row counts per expert.
//
// Kernel "tiled" (below): the MFMA-bound path for large row counts.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSkinnyRows = 64;

struct GroupedParams {
  const uint16_t* A;        // activation rows: x [T, Kd] (gate/up) or h [rows, Kd] (down)
  int32_t a_rows;           // rows of A (bounds the gathered row index)
  const int32_t* gather;    // row_to_slot
  int32_t n_ident;          // rows below this read A row r itself
  int32_t topk;
  int32_t rows_max;         // output rows; no row at or beyond it is read or written
  const int32_t* offsets;   // [G+1]
  const int32_t* tiles;     // tile table
  int32_t max_tiles;
  const uint16_t* W0a;      // gate (gated) or down weights for groups < g_split
  const uint16_t* W0b;      // ... for groups >= g_split
  const uint16_t* W1a;      // up weights (gated only)
  const uint16_t* W1b;
  int32_t g_split;
  uint16_t* out;            // [rows, N] bf16
  float* out_f32;           // [rows, N] fp32 (router logits)
  int32_t N;                // output columns (I for gate/up, H for down)
  int32_t Kd;               // reduction length (H for gate/up, I for down)
  float limit;
};

__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                          int G, int bm, int max_tiles,
                                                          int32_t* __restrict__ tiles) {
  __shared__ int base[1025];
  // G <= 1024 groups; ntiles per group then an exclusive scan (one thread, fixed order)
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int n = offsets[g + 1] - offsets[g];
    base[g] = n > 0 ? (n + bm - 1) / bm : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int g = 0; g < G; ++g) {
      const int c = base[g];
      base[g] = acc;
      acc += c;
    }
    base[G] = acc;
    tiles[0] = acc < max_tiles ? acc : max_tiles;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int r0 = offsets[g];
    const int nt = base[g + 1] - base[g];
    for (int i = 0; i < nt; ++i) {
      const int ti = base[g] + i;
      if (ti < max_tiles) {
        tiles[1 + ti] = g;
        tiles[1 + max_tiles + ti] = r0 + i * bm;
        tiles[1 + 2 * max_tiles + ti] = base[g];  // first tile of the group
        tiles[1 + 3 * max_tiles + ti] = nt;       // tiles of the group
      }
    }
  }
}

__global__ void single_group_offsets_kernel(int32_t* offsets, int rows) {
  offsets[0] = 0;
  offsets[1] = rows;
}

template <bool GATED, int NS>
__device__ __forceinline__ void skinny_tile(const GroupedParams& p, int g, int r0, int r1,
                                            int col0) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int Kd = p.Kd;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  const uint16_t* ap[NS];
  bool av[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int r = r0 + 16 * s + lr;
    av[s] = r < r1;
    int src = 0;
    if (av[s]) src = r < p.n_ident ? r : p.gather[r - p.n_ident] / p.topk;
    if (static_cast<unsigned>(src) >= static_cast<unsigned>(p.a_rows)) {  // malformed gather
      av[s] = false;
      src = 0;
    }
    ap[s] = p.A + static_cast<size_t>(src) * Kd + lk;
  }

  const size_t wst = static_cast<size_t>(p.N) * Kd;
  const uint16_t* W0 = g < p.g_split ? p.W0a + g * wst : p.W0b + (g - p.g_split) * wst;
  const uint16_t* b0;
  const uint16_t* b1;
  if (GATED) {
    const uint16_t* W1 = g < p.g_split ? p.W1a + g * wst : p.W1b + (g - p.g_split) * wst;
    b0 = W0 + static_cast<size_t>(col0 + lr) * Kd + lk;
    b1 = W1 + static_cast<size_t>(col0 + lr) * Kd + lk;
  } else {
    b0 = W0 + static_cast<size_t>(col0 + lr) * Kd + lk;
    b1 = W0 + static_cast<size_t>(col0 + 16 + lr) * Kd + lk;
  }

  f32x4_t acc0[NS], acc1[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    acc0[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc1[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  constexpr int U = 4;
  for (int k = 0; k < Kd; k += 32 * U) {
    u32x4_t bb0[U], bb1[U], aa[NS][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bb0[u] = ld16(b0 + k + 32 * u);
      bb1[u] = ld16(b1 + k + 32 * u);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int u = 0; u < U; ++u) aa[s][u] = av[s] ? ld16(ap[s] + k + 32 * u) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        acc0[s] = mfma16x16x32(aa[s][u], bb0[u], acc0[s]);
        acc1[s] = mfma16x16x32(aa[s][u], bb1[u], acc1[s]);
      }
  }

#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = r0 + 16 * s + 4 * (lane >> 4) + v;
      if (r < r1) {
        uint16_t* o = p.out + static_cast<size_t>(r) * p.N;
        if (GATED) {
          o[col0 + lr] = f32_to_bf16(clamped_swiglu(acc0[s][v], acc1[s][v], p.limit));
        } else {
          o[col0 + lr] = f32_to_bf16(acc0[s][v]);
          o[col0 + 16 + lr] = f32_to_bf16(acc1[s][v]);
        }
      }
    }
}

template <bool GATED>
__global__ __launch_bounds__(256) void ffn_skinny_kernel(GroupedParams p) {
  const int tile = blockIdx.x;
  if (tile >= p.tiles[0]) return;
  const int g = p.tiles[1 + tile];
  const int r0 = p.tiles[1 + p.max_tiles + tile];
  const int r1 = min(min(r0 + kSkinnyRows, p.offsets[g + 1]), p.rows_max);
  if (r0 < 0 || r1 <= r0) return;
  const int wave = threadIdx.x >> 6;
  const int col0 = GATED ? blockIdx.y * 64 + wave * 16 : blockIdx.y * 128 + wave * 32;
  switch ((r1 - r0 + 15) >> 4) {
    case 1: skinny_tile<GATED, 1>(p, g, r0, r1, col0); break;
    case 2: skinny_tile<GATED, 2>(p, g, r0, r1, col0); break;
    case 3: skinny_tile<GATED, 3>(p, g, r0, r1, col0); break;
    case 4: skinny_tile<GATED, 4>(p, g, r0, r1, col0); break;
    default: break;
  }
}


// ---------------------------------------------------------------------------------------------
// Kernel "tiled": BM rows x 256 weight rows per workgroup, four wavefronts of (BM/2) x 128 on
// MFMA 32x32x16 (BM/64 x 4 fragments each). K is staged BK at a time through a ring of STAGES
// LDS buffers filled by direct global->LDS loads (global_load_lds_dwordx4: no VGPR staging), so
// STAGES-1 K-tiles are in flight while one is consumed. With BM = 256 a K-tile brings 32 bytes
// per 1024 MFMA FLOPs into LDS, half the operand traffic of BM = 128, which is what the
// global->LDS fill rate of a CU allows. A wavefront skips the MFMAs of 32-row fragments that lie
// past the group's last row. Work items are ordered inside XCD-contiguous slices of the real work list (its size
// comes from the device-side tile count, so spare grid slots do not unbalance the XCDs); inside
// a group the work runs in bands of up to kBand row tiles, n-blocks outer and the band's row
// tiles inner, so workgroups running together on an XCD share one weight tile (same n-block)
// and the band's activation rows through L2, and a group with at most kBand row tiles reads
// each of its weight tiles from HBM once.
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

// Wait until at most `tiles` K-tiles of PER loads each are still in flight.
template <int PER>
__device__ __forceinline__ void wait_tiles(int tiles) {
  switch (tiles) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<PER>(); break;
    case 2: wait_vmcnt<2 * PER>(); break;
    case 3: wait_vmcnt<3 * PER>(); break;
    case 4: wait_vmcnt<4 * PER>(); break;
    default: wait_vmcnt<5 * PER>(); break;
  }
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

enum Epilogue { kEpiSwiglu = 0, kEpiBf16 = 1, kEpiF32 = 2 };

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
  const int wave = tid >> 6, lane = tid & 63;
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

  // DMA instruction d (0..NA+NB-1) of K-tile kt
  auto issue_one = [&](int kt, int d) {
    const int st = kt % S;
    const int k0 = kt * BK;
    if (d < NA)
      lds_dma16(p.A + aoff[d] + k0, sA + st * kStageA + (wave + 4 * d) * 512);
    else
      lds_dma16(bsrc[d - NA] + k0, sB + st * kStageB + (wave + 4 * (d - NA)) * 512);
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int d = 0; d < NA + NB; ++d) issue_one(kt, d);
  };

  f32x16_t acc[MIV > 0 ? MIV : 1][4];
#pragma unroll
  for (int i = 0; i < (MIV > 0 ? MIV : 1); ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = Kd / BK;
  for (int t = 0; t < S - 1 && t < nk; ++t) issue(t);
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  // LDS offset of this lane's fragment row fr at K-step ks inside a 32-row-aligned block: the
  // swizzle term depends only on fr (the block bases are multiples of 32 rows), so one offset
  // per K-step serves every fragment of every stage.
  int lds_off[BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) lds_off[ks] = swz<BK>(fr, ks * 16 + fk);
  // The next K-tile's DMA instructions are spread between the MFMAs (one every kStep MFMAs) so
  // that issuing them never leaves the MFMA pipe idle.
  constexpr int kMfmaPerTile = (BK / 16) * MIV * 4;
  constexpr int kStep = kMfmaPerTile >= NA + NB ? kMfmaPerTile / (NA + NB) : 1;
  static_assert(MIV == 0 || kMfmaPerTile % (NA + NB) == 0, "DMA spread must divide the MFMAs");
  // Every iteration issues exactly one K-tile of DMA: past the end it reloads the last tile into
  // the free stage (never read), so exactly S-2 later tiles are in flight at each wait and the
  // loop body has no branch (which lets the instruction order below be pinned).
  for (int t = nk; t < S - 1; ++t) issue(nk - 1);  // K shorter than the ring
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<(S - 2) * (NA + NB)>();  // K-tile kt has landed
    barrier_no_fence();
    const int kn = min(kt + S - 1, nk - 1);  // tile loaded into the stage consumed in kt-1
    const int sn = (kt + S - 1) % S;
    auto issue_next = [&](int d) {
      if (d < NA)
        lds_dma16(p.A + aoff[d] + kn * BK, sA + sn * kStageA + (wave + 4 * d) * 512);
      else
        lds_dma16(bsrc[d - NA] + kn * BK, sB + sn * kStageB + (wave + 4 * (d - NA)) * 512);
    };
    if (MIV == 0) {
#pragma unroll
      for (int d = 0; d < NA + NB; ++d) issue_next(d);
      continue;
    }
    const uint16_t* a = sA + (kt % S) * kStageA + wm * (BM / 2) * BK;
    const uint16_t* b = sB + (kt % S) * kStageB + wn * 128 * BK;
    // fragments of K-step ks+1 are read while the MFMAs of K-step ks run
    u32x4_t af[2][MIV > 0 ? MIV : 1], bf[2][4];
    auto fetch = [&](int ks, int set) {
#pragma unroll
      for (int i = 0; i < MIV; ++i)
        af[set][i] = *reinterpret_cast<const u32x4_t*>(&a[i * 32 * BK + lds_off[ks]]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[set][j] = *reinterpret_cast<const u32x4_t*>(&b[j * 32 * BK + lds_off[ks]]);
    };
    fetch(0, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) fetch(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < MIV; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = mfma32x32x16(af[ks & 1][i], bf[ks & 1][j], acc[i][j]);
          const int m = (ks * MIV + i) * 4 + j + 1;  // MFMAs issued so far in this K-tile
          if (m % kStep == 0 && m / kStep <= NA + NB) issue_next(m / kStep - 1);
        }
    }
    // Pin the order: K-step 0's fragment reads; then each MFMA followed by one of the next
    // K-step's fragment reads (while any remain) and, every kStep MFMAs, one DMA instruction.
    constexpr int kFrag = MIV + 4;           // fragment reads per K-step
    constexpr int kMfmaStep = MIV * 4;       // MFMAs per K-step
    __builtin_amdgcn_sched_group_barrier(0x100, kFrag, 0);
#pragma unroll
    for (int m = 0; m < kMfmaPerTile; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      const int in_step = m % kMfmaStep;
      if (m / kMfmaStep + 1 < BK / 16 && in_step < kFrag) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if ((m + 1) % kStep == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
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

size_t tile_table_bytes(int max_tiles) { return sizeof(int32_t) * (1 + 4 * static_cast<size_t>(max_tiles)); }

int max_tiles_for(int rows_max, int n_groups, int bm) { return (rows_max + bm - 1) / bm + n_groups; }

hipError_t launch_single_group_offsets(int32_t* offsets, int rows, hipStream_t stream) {
  hipLaunchKernelGGL(single_group_offsets_kernel, dim3(1), dim3(1), 0, stream, offsets, rows);
  return hipGetLastError();
}

hipError_t launch_ffn(const FfnProblem& q, hipStream_t stream, hipEvent_t const* ev) {
  auto mark = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord(ev[i], stream);
  };
  // Few rows per group (decode): stream the weights. Many rows per group: LDS-tiled MFMA.
  const bool tiled = q.rows_max >= 64 * q.n_groups;
  const int bm = tiled ? kBM : kSkinnyRows;
  const int max_tiles = max_tiles_for(q.rows_max, q.n_groups, bm);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, stream, q.offsets, q.n_groups, bm,
                     max_tiles, q.tiles);
  mark(0);

  GroupedParams p{};
  p.gather = q.gather;
  p.rows_max = q.rows_max;
  p.n_ident = q.n_ident;
  p.topk = q.topk;
  p.offsets = q.offsets;
  p.tiles = q.tiles;
  p.max_tiles = max_tiles;
  p.g_split = q.g_split;
  p.limit = q.limit;

  // gate/up + clamped SwiGLU -> h
  p.A = q.x;
  p.a_rows = q.T;
  p.W0a = q.gate_a;
  p.W0b = q.gate_b;
  p.W1a = q.up_a;
  p.W1b = q.up_b;
  p.out = q.h;
  p.N = q.I;
  p.Kd = q.H;
  if (tiled) {
    const hipError_t e = tiled_launch<kEpiSwiglu, kBM, kBK, kStages>(p, q.I / 128, max_tiles, stream);
    if (e != hipSuccess) return e;
  }
  else
    hipLaunchKernelGGL(ffn_skinny_kernel<true>, dim3(max_tiles, q.I / 64), dim3(256), 0, stream, p);
  mark(1);

  // down -> y (h rows are already in row order: identity gather)
  p.A = q.h;
  p.a_rows = q.rows_max;
  p.n_ident = 0x7fffffff;
  p.gather = nullptr;
  p.W0a = q.down_a;
  p.W0b = q.down_b;
  p.W1a = p.W1b = nullptr;
  p.out = q.y;
  p.N = q.H;
  p.Kd = q.I;
  if (tiled) {
    const hipError_t e = tiled_launch<kEpiBf16, kBM, kBK, kStages>(p, q.H / kTN, max_tiles, stream);
    if (e != hipSuccess) return e;
  }
  else
    hipLaunchKernelGGL(ffn_skinny_kernel<false>, dim3(max_tiles, q.H / 128), dim3(256), 0, stream, p);
  mark(2);
  return hipGetLastError();
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
  return tiled_launch<kEpiF32, kBM, kBK, kStages>(p, N / kTN, (rows + kBM - 1) / kBM, stream);
}

}  // namespace moe
