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
// Kernel "tiled": 128-row x 128-column tiles, K staged through LDS 64 at a time (double
// buffered, one barrier per K step), four wavefronts of 64x64 on MFMA 32x32x16. The LDS rows
// are XOR-swizzled by 16-byte chunk so the MFMA operand reads are bank-conflict free. For the
// gate/up projection the 128 weight rows of a tile are 64 gate rows and the 64 matching up rows,
// interleaved by 32 so that each wavefront's accumulators hold matching gate and up columns and
// the SwiGLU epilogue stays in registers. This is the MFMA-bound path for large row counts.
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
  uint16_t* out;            // [rows, N]
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


constexpr int kTileM = 128;  // rows per tile
constexpr int kTileN = 128;  // weight rows per tile (gate/up: 64 gate + 64 up)
constexpr int kTileK = 64;   // reduction elements per LDS stage

// LDS element offset of (row, k) inside a [rows][64] bf16 stage, 16-byte chunks XOR-swizzled.
__device__ __forceinline__ int swz(int row, int k) {
  return row * kTileK + ((((k >> 3) ^ (row & 7))) << 3) + (k & 7);
}

template <bool GATED>
__global__ __launch_bounds__(256, 2) void ffn_tiled_kernel(GroupedParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kTileM * kTileK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kTileN * kTileK];

  const int tile = blockIdx.x;
  if (tile >= p.tiles[0]) return;
  const int g = p.tiles[1 + tile];
  const int r0 = p.tiles[1 + p.max_tiles + tile];
  const int r1 = min(min(r0 + kTileM, p.offsets[g + 1]), p.rows_max);
  if (r0 < 0 || r1 <= r0) return;
  const int Kd = p.Kd;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global -> LDS assignment: thread loads 16-byte chunk (tid & 7) of rows (tid >> 3) + 32 i
  const int lch = tid & 7;
  const uint16_t* ga[4];
  bool gav[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + (tid >> 3) + 32 * i;
    gav[i] = r < r1;
    int src = 0;
    if (gav[i]) src = r < p.n_ident ? r : p.gather[r - p.n_ident] / p.topk;
    if (static_cast<unsigned>(src) >= static_cast<unsigned>(p.a_rows)) {
      gav[i] = false;
      src = 0;
    }
    ga[i] = p.A + static_cast<size_t>(src) * Kd + lch * 8;
  }
  const size_t wst = static_cast<size_t>(p.N) * Kd;
  const uint16_t* W0 = g < p.g_split ? p.W0a + g * wst : p.W0b + (g - p.g_split) * wst;
  const uint16_t* W1 = nullptr;
  if (GATED) W1 = g < p.g_split ? p.W1a + g * wst : p.W1b + (g - p.g_split) * wst;
  const uint16_t* gb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = (tid >> 3) + 32 * i;  // B tile row
    if (GATED) {
      const int w = b & 63;
      const int col = blockIdx.y * 64 + (b >> 6) * 32 + (w & 31);
      gb[i] = (w < 32 ? W0 : W1) + static_cast<size_t>(col) * Kd + lch * 8;
    } else {
      gb[i] = W0 + static_cast<size_t>(blockIdx.y * kTileN + b) * Kd + lch * 8;
    }
  }
  int soff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) soff[i] = swz((tid >> 3) + 32 * i, lch * 8);

  const u32x4_t zero = {0u, 0u, 0u, 0u};
  u32x4_t ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = gav[i] ? ld16(ga[i] + k0) : zero;
      rb[i] = ld16(gb[i] + k0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4_t*>(&sA[buf][soff[i]]) = ra[i];
      *reinterpret_cast<u32x4_t*>(&sB[buf][soff[i]]) = rb[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = Kd / kTileK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kTileK);
#pragma unroll
    for (int ks = 0; ks < kTileK / 16; ++ks) {
      u32x4_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const u32x4_t*>(&sA[buf][swz(wm * 64 + i * 32 + fr, ks * 16 + fk)]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const u32x4_t*>(&sB[buf][swz(wn * 64 + j * 32 + fr, ks * 16 + fk)]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 8*(v/4) + 4*(lane/32) + v%4 of each 32x32 block, column lane%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = r0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (r >= r1) continue;
      uint16_t* o = p.out + static_cast<size_t>(r) * p.N;
      if (GATED) {
        o[blockIdx.y * 64 + wn * 32 + fr] = f32_to_bf16(clamped_swiglu(acc[i][0][v], acc[i][1][v], p.limit));
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) o[blockIdx.y * kTileN + wn * 64 + j * 32 + fr] = f32_to_bf16(acc[i][j][v]);
      }
    }
}

}  // namespace

size_t tile_table_bytes(int max_tiles) { return sizeof(int32_t) * (1 + 2 * static_cast<size_t>(max_tiles)); }

int max_tiles_for(int rows_max, int n_groups, int bm) { return (rows_max + bm - 1) / bm + n_groups; }

hipError_t launch_single_group_offsets(int32_t* offsets, int rows, hipStream_t stream) {
  hipLaunchKernelGGL(single_group_offsets_kernel, dim3(1), dim3(1), 0, stream, offsets, rows);
  return hipGetLastError();
}

hipError_t launch_ffn(const FfnProblem& q, hipStream_t stream, hipEvent_t const* ev) {
  auto mark = [&](int i) {
    if (ev && ev[i]) hipEventRecord(ev[i], stream);
  };
  // Few rows per group (decode): stream the weights. Many rows per group: LDS-tiled MFMA.
  const bool tiled = q.rows_max >= 64 * q.n_groups;
  const int bm = tiled ? kTileM : kSkinnyRows;
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
  if (tiled)
    hipLaunchKernelGGL(ffn_tiled_kernel<true>, dim3(max_tiles, q.I / 64), dim3(256), 0, stream, p);
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
  if (tiled)
    hipLaunchKernelGGL(ffn_tiled_kernel<false>, dim3(max_tiles, q.H / kTileN), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(ffn_skinny_kernel<false>, dim3(max_tiles, q.H / 128), dim3(256), 0, stream, p);
  mark(2);
  return hipGetLastError();
}

}  // namespace moe
