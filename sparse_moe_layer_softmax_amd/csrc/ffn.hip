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
// Two kernels: ffn_skinny.hip (weight streaming, few rows per expert) and ffn_tiled.hip
// (LDS-tiled MFMA, many rows per expert). This file builds the tile table and dispatches.
#include "ffn_kernels.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                          int G, int bm, int max_tiles,
                                                          int32_t* __restrict__ tiles) {
  __shared__ int base[1025];
  __shared__ int wsum[4];
  // G <= 1024 groups, four consecutive ones per thread: tiles per group, then an exclusive
  // integer scan (lanes by shuffles, wavefronts through LDS)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int n4[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * tid + i;
    const int n = g < G ? offsets[g + 1] - offsets[g] : 0;
    n4[i] = n > 0 ? (n + bm - 1) / bm : 0;
    sum += n4[i];
  }
  int inc = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int b = inc - sum;
  for (int j = 0; j < w; ++j) b += wsum[j];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * tid + i;
    if (g < G) base[g] = b;
    b += n4[i];
  }
  if (tid == 0) {
    const int acc = wsum[0] + wsum[1] + wsum[2] + wsum[3];
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

}  // namespace

size_t tile_table_bytes(int max_tiles) { return sizeof(int32_t) * (1 + 4 * static_cast<size_t>(max_tiles)); }

int max_tiles_for(int rows_max, int n_groups, int bm) { return (rows_max + bm - 1) / bm + n_groups; }

hipError_t launch_build_tiles(const int32_t* offsets, int n_groups, int bm, int max_tiles,
                              int32_t* tiles, hipStream_t stream) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, stream, offsets, n_groups, bm,
                     max_tiles, tiles);
  return hipGetLastError();
}

hipError_t launch_single_group_offsets(int32_t* offsets, int rows, hipStream_t stream) {
  hipLaunchKernelGGL(single_group_offsets_kernel, dim3(1), dim3(1), 0, stream, offsets, rows);
  return hipGetLastError();
}

hipError_t launch_ffn(const FfnProblem& q, hipStream_t stream, hipEvent_t const* ev) {
  auto mark = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord(ev[i], stream);
  };
  // Few rows per group (decode): stream the weights. Many rows per group: LDS-tiled MFMA. Both
  // kernels have an FP8-weight form.
  const bool tiled = q.gu || q.rows_max >= 64 * q.n_groups;
  const bool small = !tiled && q.rows_max <= kSkinnyRowsSmall * q.n_groups;
  const int bm = tiled ? kTiledRows : (small ? kSkinnyRowsSmall : kSkinnyRows);
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

  // gate/up + clamped SwiGLU -> h. W8A8: x quantised per row first; the tiled kernel then
  // moves the codes as pairs (Kd = H / 2), the skinny kernel reads them as bytes.
  hipError_t e = hipSuccess;
  if (q.mx) {
    e = launch_quant_mx(q.x, q.T, q.H, nullptr, q.xq, q.xs, q.mx_rows, q.s2r, q.topk, q.n_ident,
                        stream);
    if (e != hipSuccess) return e;
  } else if (q.a8) {
    e = launch_quant_rows(q.x, q.T, q.H, nullptr, q.xq, q.sx, stream);
    if (e != hipSuccess) return e;
  }
  p.A = q.a8 ? reinterpret_cast<const uint16_t*>(q.xq) : q.x;
  p.a_scale = q.sx;
  p.a_rows = q.T;
  p.W0a = q.gate_a;
  p.W0b = q.gate_b;
  p.W1a = q.up_a;
  p.W1b = q.up_b;
  p.Q0a = q.qgate_a;
  p.Q0b = q.qgate_b;
  p.Q1a = q.qup_a;
  p.Q1b = q.qup_b;
  p.S0a = q.sgate_a;
  p.S0b = q.sgate_b;
  p.S1a = q.sup_a;
  p.S1b = q.sup_b;
  if (q.a8) {  // the codes take the bf16 weights' places
    p.W0a = reinterpret_cast<const uint16_t*>(q.qgate_a);
    p.W0b = reinterpret_cast<const uint16_t*>(q.qgate_b);
    p.W1a = reinterpret_cast<const uint16_t*>(q.qup_a);
    p.W1b = reinterpret_cast<const uint16_t*>(q.qup_b);
  }
  if (q.mx) {
    p.X0a = q.xgate_a;
    p.X0b = q.xgate_b;
    p.X1a = q.xup_a;
    p.X1b = q.xup_b;
    p.a_mx = q.xs;
    p.a_mx_rows = q.mx_rows;
  }
  p.out = q.h;
  p.N = q.I;
  p.Kd = q.a8 && tiled ? q.H / 2 : q.H;
  if (q.mx && tiled) {  // the tiled epilogue quantises h for the down projection itself
    p.mx_hq = q.hq;
    p.mx_hs = q.hs;
    p.mx_h_rows = q.mx_rows;
  }
  p.gu = q.gu;
  if (q.gu && (q.w8 || q.a8)) return hipErrorInvalidValue;
  if (tiled)
    e = launch_tiled(q.mx ? kEpiSwigluMx
                          : q.a8 ? kEpiSwiglu88 : (q.w8 ? kEpiSwiglu8 : (q.gu ? kEpiSwigluSave : kEpiSwiglu)),
                     p, max_tiles, stream);
  else
    e = launch_skinny(true, q.w8, q.a8, p, max_tiles, bm, stream, q.mx);
  if (e != hipSuccess) return e;
  mark(1);

  // down -> y (h rows are already in row order: identity gather); W8A8: the valid h rows
  // (offsets[G] of them) quantised per row first; MX: quantised by blocks, in the tiled
  // gate/up epilogue or here after the weight-streaming kernel
  p.mx_hq = nullptr;
  p.mx_hs = nullptr;
  if (q.mx && !tiled) {
    e = launch_quant_mx(q.h, q.rows_max, q.I, q.offsets + q.n_groups, q.hq, q.hs, q.mx_rows,
                        nullptr, 0, 0, stream);
    if (e != hipSuccess) return e;
  } else if (q.a8 && !q.mx) {
    e = launch_quant_rows(q.h, q.rows_max, q.I, q.offsets + q.n_groups, q.hq, q.sh, stream);
    if (e != hipSuccess) return e;
  }
  p.A = q.a8 ? reinterpret_cast<const uint16_t*>(q.hq) : q.h;
  p.a_scale = q.sh;
  p.a_rows = q.rows_max;
  p.n_ident = 0x7fffffff;
  p.gather = nullptr;
  p.W0a = q.down_a;
  p.W0b = q.down_b;
  p.W1a = p.W1b = nullptr;
  p.Q0a = q.qdown_a;
  p.Q0b = q.qdown_b;
  p.Q1a = p.Q1b = nullptr;
  p.S0a = q.sdown_a;
  p.S0b = q.sdown_b;
  p.S1a = p.S1b = nullptr;
  if (q.a8) {
    p.W0a = reinterpret_cast<const uint16_t*>(q.qdown_a);
    p.W0b = reinterpret_cast<const uint16_t*>(q.qdown_b);
  }
  if (q.mx) {
    p.X0a = q.xdown_a;
    p.X0b = q.xdown_b;
    p.X1a = p.X1b = nullptr;
    p.a_mx = q.hs;
  }
  p.out = q.y;
  p.N = q.H;
  p.Kd = q.a8 && tiled ? q.I / 2 : q.I;
  if (tiled)
    e = launch_tiled(q.mx ? kEpiBf16Mx : q.a8 ? kEpiBf16_88 : (q.w8 ? kEpiBf16_8 : kEpiBf16), p,
                     max_tiles, stream);
  else
    e = launch_skinny(false, q.w8, q.a8, p, max_tiles, bm, stream, q.mx);
  if (e != hipSuccess) return e;
  mark(2);
  return hipGetLastError();
}

}  // namespace moe
