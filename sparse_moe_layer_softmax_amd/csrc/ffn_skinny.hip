// ffn_skinny.hip -- weight-streaming grouped SwiGLU FFN kernel for few rows per expert.
//
// Hy3 deep-dive (happyrock.cloud) `MoEFeedForward`: y = down(silu(gate x) * up x), bias-free
// projections; Hy4 config walkthrough (lshu.cn), section "MoE routed experts": swiglu_limit
// clamps the gate and up pre-activations, hidden_act silu.
//
// Row tiles of up to 64 rows (MFMA 16x16x32 in 16-row sub-blocks; only the occupied sub-blocks
// are computed). Each wavefront owns 16 output columns of the gate AND the up projection (so the
// SwiGLU epilogue pairs them in registers), or 32 columns of the down projection. Weight
// fragments are loaded straight from HBM with 16-byte loads in MFMA operand order: at a few rows
// per expert (decode) the layer is a weight stream and this kernel runs at HBM speed.
#include "ffn_kernels.h"
#include "moe_device.h"

namespace moe {
namespace {

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


}  // namespace

hipError_t launch_skinny(bool gated, const GroupedParams& p, int max_tiles, hipStream_t stream) {
  if (gated)
    hipLaunchKernelGGL(ffn_skinny_kernel<true>, dim3(max_tiles, p.N / 64), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(ffn_skinny_kernel<false>, dim3(max_tiles, p.N / 128), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
