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
// Kernel "tiled2" (below): the MFMA-bound path for large row counts.
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


constexpr int kTileK = 64;   // reduction elements per LDS stage

// LDS element offset of (row, k) inside a [rows][64] bf16 stage. 16-byte chunks are XOR-swizzled
// with (row % 8) ^ ((row / 8) % 2), so the MFMA operand reads (16 consecutive rows at one chunk)
// touch 16 distinct 16-byte slots of every 256-byte window: free of bank conflicts on the 64-bank
// LDS, and on a 32-bank one (8 consecutive rows are distinct too).
__device__ __forceinline__ int swz(int row, int k) {
  return row * kTileK + (((k >> 3) ^ (row & 7) ^ ((row >> 3) & 1)) << 3) + (k & 7);
}

// ---------------------------------------------------------------------------------------------
// Kernel "tiled2": 128 rows x 256 weight rows per workgroup, four wavefronts of 64 x 128
// (2 x 4 MFMA 32x32x16 fragments: 0.75 KB of LDS reads per MFMA), K staged 64 at a time through a
// three-stage LDS ring filled by direct global->LDS loads (global_load_lds_dwordx4: no VGPR
// staging), so two K-tiles are in flight while a third is consumed. Work items are ordered
// n-block fastest inside a row tile (the gathered rows are reused by consecutive workgroups) and
// each XCD takes one contiguous slice of the real work list (its L2 then holds the slice's
// weights and rows); the slice size comes from the device-side tile count, so spare grid slots
// do not unbalance the XCDs. Inside a group the work runs in bands of up to kBand row tiles:
// n-blocks outer, the band's row tiles inner. Workgroups running together on an XCD then share
// one weight tile (same n-block) and the band's activation rows through L2, and a group with at
// most kBand row tiles reads each of its weight tiles from HBM once.
constexpr int kT2M = 128;
constexpr int kT2N = 256;
constexpr int kT2K = 64;
constexpr int kT2Stages = 3;
constexpr int kT2StageA = kT2M * kT2K;  // bf16 elements
constexpr int kT2StageB = kT2N * kT2K;
constexpr int kXcds = 8;
constexpr int kBand = 8;
constexpr size_t kT2Smem = sizeof(uint16_t) * kT2Stages * (kT2StageA + kT2StageB);

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
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
// p.tiles == nullptr selects dense mode: one group of rows [0, rows_max) in 128-row tiles.
template <int EPI>
__global__ __launch_bounds__(256, 1) void ffn_tiled2_kernel(GroupedParams p, int nblk) {
  constexpr bool GATED = EPI == kEpiSwiglu;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sA = smem;                                // [stages][128*64]
  uint16_t* sB = smem + kT2Stages * kT2StageA;        // [stages][256*64]

  // ---- work item: XCD-contiguous slices of the work list (band order inside each group)
  const bool dense = p.tiles == nullptr;
  const int n_tiles = dense ? (p.rows_max + kT2M - 1) / kT2M : p.tiles[0];
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
  const int r0 = dense ? tile * kT2M : p.tiles[1 + p.max_tiles + tile];
  const int r_end = dense ? p.rows_max : p.offsets[g + 1];
  const int r1 = min(min(r0 + kT2M, r_end), p.rows_max);
  if (r0 < 0 || r1 <= r0) return;

  const int Kd = p.Kd;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- DMA assignment. A 1 KB LDS block holds 8 rows x 128 B; lane i fills slot i, i.e. row
  // i/8 of the block and physical chunk i%8, which holds the logical chunk given by swz().
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow ^ (wave & 1);  // blocks wave+4i: row/8 odd iff wave odd
  // A: blocks wave, wave+4, wave+8, wave+12 (rows 8*block + lrow)
  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + (wave + 4 * i) * 8 + lrow;
    int src = 0;
    if (r < r1) src = r < p.n_ident ? r : p.gather[r - p.n_ident] / p.topk;
    if (static_cast<unsigned>(src) >= static_cast<unsigned>(p.a_rows)) src = 0;
    aoff[i] = static_cast<uint32_t>(src) * Kd + lchunk * 8;
  }
  // B: blocks wave + 4*i, i < 8 (weight-tile rows 8*block + lrow)
  const size_t wst = static_cast<size_t>(p.N) * Kd;
  const uint16_t* W0 = g < p.g_split ? p.W0a + g * wst : p.W0b + (g - p.g_split) * wst;
  const uint16_t* W1 = W0;
  if (GATED) W1 = g < p.g_split ? p.W1a + g * wst : p.W1b + (g - p.g_split) * wst;
  const uint16_t* bsrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = (wave + 4 * i) * 8 + lrow;  // 0..255
    int row;
    const uint16_t* Wm = W0;
    if (GATED) {
      // wave column wn = b/128 holds h columns nb*128 + wn*64 + [0,64): fragments 0,1 are the gate
      // rows, fragments 2,3 the matching up rows
      const int q = (b & 127) >> 5;
      row = nb * 128 + (b >> 7) * 64 + (q & 1) * 32 + (b & 31);
      Wm = q < 2 ? W0 : W1;
    } else {
      row = nb * kT2N + b;
    }
    bsrc[i] = Wm + static_cast<size_t>(row) * Kd + lchunk * 8;
  }

  auto issue = [&](int kt) {
    const int st = kt % kT2Stages;
    const int k0 = kt * kT2K;
    uint16_t* a = sA + st * kT2StageA;
    uint16_t* b = sB + st * kT2StageB;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(p.A + aoff[i] + k0, a + (wave + 4 * i) * 512);
#pragma unroll
    for (int i = 0; i < 8; ++i) lds_dma16(bsrc[i] + k0, b + (wave + 4 * i) * 512);
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = Kd / kT2K;
  issue(0);
  if (nk > 1) issue(1);
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    // K-tile kt has landed once at most one later tile (12 loads) is still in flight
    if (kt + 1 < nk) wait_vmcnt<12>(); else wait_vmcnt<0>();
    barrier_no_fence();
    if (kt + 2 < nk) issue(kt + 2);
    const uint16_t* a = sA + (kt % kT2Stages) * kT2StageA;
    const uint16_t* b = sB + (kt % kT2Stages) * kT2StageB;
    // fragments of K-step ks+1 are read while the MFMAs of K-step ks run
    u32x4_t af[2][2], bf[2][4];
    auto fetch = [&](int ks, int set) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[set][i] = *reinterpret_cast<const u32x4_t*>(&a[swz(wm * 64 + i * 32 + fr, ks * 16 + fk)]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[set][j] = *reinterpret_cast<const u32x4_t*>(&b[swz(wn * 128 + j * 32 + fr, ks * 16 + fk)]);
    };
    fetch(0, 0);
#pragma unroll
    for (int ks = 0; ks < kT2K / 16; ++ks) {
      if (ks + 1 < kT2K / 16) fetch(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(af[ks & 1][i], bf[ks & 1][j], acc[i][j]);
    }
  }

  // ---- epilogue
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = r0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (r >= r1) continue;
      if (EPI == kEpiSwiglu) {
        uint16_t* o = p.out + static_cast<size_t>(r) * p.N;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          o[nb * 128 + wn * 64 + j * 32 + fr] =
              f32_to_bf16(clamped_swiglu(acc[i][j][v], acc[i][j + 2][v], p.limit));
      } else if (EPI == kEpiBf16) {
        uint16_t* o = p.out + static_cast<size_t>(r) * p.N;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[nb * kT2N + wn * 128 + j * 32 + fr] = f32_to_bf16(acc[i][j][v]);
      } else {
        float* o = p.out_f32 + static_cast<size_t>(r) * p.N;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[nb * kT2N + wn * 128 + j * 32 + fr] = acc[i][j][v];
      }
    }
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
  const int bm = tiled ? kT2M : kSkinnyRows;
  const int max_tiles = max_tiles_for(q.rows_max, q.n_groups, bm);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, stream, q.offsets, q.n_groups, bm,
                     max_tiles, q.tiles);
  mark(0);
    if (tiled) {
    static bool attr_set = false;  // per process; the attribute is a property of the kernel
    if (!attr_set) {
      hipError_t e1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_tiled2_kernel<kEpiSwiglu>),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, kT2Smem);
      hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_tiled2_kernel<kEpiBf16>),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, kT2Smem);
      if (e1 != hipSuccess) return e1;
      if (e2 != hipSuccess) return e2;
      attr_set = true;
    }
  }

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
    const int nblk = q.I / 128;
    const int grid = (max_tiles * nblk + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(ffn_tiled2_kernel<kEpiSwiglu>, dim3(grid), dim3(256), kT2Smem, stream, p, nblk);
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
    const int nblk = q.H / kT2N;
    const int grid = (max_tiles * nblk + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(ffn_tiled2_kernel<kEpiBf16>, dim3(grid), dim3(256), kT2Smem, stream, p, nblk);
  }
  else
    hipLaunchKernelGGL(ffn_skinny_kernel<false>, dim3(max_tiles, q.H / 128), dim3(256), 0, stream, p);
  mark(2);
  return hipGetLastError();
}

bool dense_gemm_f32_supported(int N, int Kd) { return N == kT2N && Kd % kT2K == 0; }

hipError_t launch_dense_gemm_f32(const uint16_t* A, int rows, const uint16_t* W, int N, int Kd,
                                 float* out, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_tiled2_kernel<kEpiF32>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kT2Smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
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
  const int nblk = N / kT2N;
  const int n_tiles = (rows + kT2M - 1) / kT2M;
  const int grid = (n_tiles * nblk + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(ffn_tiled2_kernel<kEpiF32>, dim3(grid), dim3(256), kT2Smem, stream, p, nblk);
  return hipGetLastError();
}

}  // namespace moe
