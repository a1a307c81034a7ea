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
//
// W8 form (FP8 expert weights, E4M3 codes with one fp32 scale per weight row): each lane loads
// 16 codes at a time, converts them exactly to bf16 in registers (every E4M3 value is a bf16
// value) and runs the same bf16 MFMAs; the row scales multiply the fp32 sums in the epilogue.
// Within a 128-element K block, lane group g (lane / 16) takes 16-code chunks g and g + 4 of
// each weight row, and MFMA u of the block reads elements 16g + 64(u/2) + 8(u%2) + [0, 8) of
// both operands: any one-to-one assignment of K elements to MFMA lanes gives the same dot
// product, and this one gives every lane two whole 16-byte weight loads per block.
#include "ffn_kernels.h"
#include "moe_device.h"

namespace moe {
namespace {

// Eight E4M3 codes (two dwords, code 0 in the low byte) -> the eight bf16 of one MFMA operand.
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return r;
}

__device__ __forceinline__ u32x4_t ld16b(const uint8_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

template <bool GATED, int NS, bool W8>
__device__ __forceinline__ void skinny_tile(const GroupedParams& p, int g, int r0, int r1,
                                            int col0) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15;
  const int lk = W8 ? (lane >> 4) * 16 : (lane >> 4) * 8;  // this lane's first K element
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
  // weight rows of this lane's two B fragments (gate and up, or down columns col0 and col0 + 16)
  const size_t row0 = static_cast<size_t>(col0 + lr) * Kd + lk;
  const size_t row1 = static_cast<size_t>(GATED ? col0 + lr : col0 + 16 + lr) * Kd + lk;
  const uint16_t* b0 = nullptr;
  const uint16_t* b1 = nullptr;
  const uint8_t* q0 = nullptr;
  const uint8_t* q1 = nullptr;
  if (W8) {
    const uint8_t* Q0 = g < p.g_split ? p.Q0a + g * wst : p.Q0b + (g - p.g_split) * wst;
    const uint8_t* Q1 = Q0;
    if (GATED) Q1 = g < p.g_split ? p.Q1a + g * wst : p.Q1b + (g - p.g_split) * wst;
    q0 = Q0 + row0;
    q1 = Q1 + row1;
  } else {
    const uint16_t* W0 = g < p.g_split ? p.W0a + g * wst : p.W0b + (g - p.g_split) * wst;
    const uint16_t* W1 = W0;
    if (GATED) W1 = g < p.g_split ? p.W1a + g * wst : p.W1b + (g - p.g_split) * wst;
    b0 = W0 + row0;
    b1 = W1 + row1;
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
    if (W8) {
      const u32x4_t c0 = ld16b(q0 + k), c1 = ld16b(q0 + k + 64);
      const u32x4_t d0 = ld16b(q1 + k), d1 = ld16b(q1 + k + 64);
      bb0[0] = e4m3x8_to_bf16(c0[0], c0[1]);
      bb0[1] = e4m3x8_to_bf16(c0[2], c0[3]);
      bb0[2] = e4m3x8_to_bf16(c1[0], c1[1]);
      bb0[3] = e4m3x8_to_bf16(c1[2], c1[3]);
      bb1[0] = e4m3x8_to_bf16(d0[0], d0[1]);
      bb1[1] = e4m3x8_to_bf16(d0[2], d0[3]);
      bb1[2] = e4m3x8_to_bf16(d1[0], d1[1]);
      bb1[3] = e4m3x8_to_bf16(d1[2], d1[3]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bb0[u] = ld16(b0 + k + 32 * u);
        bb1[u] = ld16(b1 + k + 32 * u);
      }
    }
    // activations at the same K elements as the weight operands of MFMA u
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ko = W8 ? 64 * (u >> 1) + 8 * (u & 1) : 32 * u;
        aa[s][u] = av[s] ? ld16(ap[s] + k + ko) : zero;
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        acc0[s] = mfma16x16x32(aa[s][u], bb0[u], acc0[s]);
        acc1[s] = mfma16x16x32(aa[s][u], bb1[u], acc1[s]);
      }
  }

  // FP8: per-row weight scales of this lane's two output columns
  float sc0 = 1.f, sc1 = 1.f;
  if (W8) {
    const size_t so = static_cast<size_t>(g < p.g_split ? g : g - p.g_split) * p.N;
    const float* S0 = (g < p.g_split ? p.S0a : p.S0b) + so;
    const float* S1 = S0;
    if (GATED) S1 = (g < p.g_split ? p.S1a : p.S1b) + so;
    sc0 = S0[col0 + lr];
    sc1 = S1[GATED ? col0 + lr : col0 + 16 + lr];
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = r0 + 16 * s + 4 * (lane >> 4) + v;
      if (r < r1) {
        uint16_t* o = p.out + static_cast<size_t>(r) * p.N;
        const float a0 = W8 ? acc0[s][v] * sc0 : acc0[s][v];
        const float a1 = W8 ? acc1[s][v] * sc1 : acc1[s][v];
        if (GATED) {
          o[col0 + lr] = f32_to_bf16(clamped_swiglu(a0, a1, p.limit));
        } else {
          o[col0 + lr] = f32_to_bf16(a0);
          o[col0 + 16 + lr] = f32_to_bf16(a1);
        }
      }
    }
}

template <bool GATED, bool W8>
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
    case 1: skinny_tile<GATED, 1, W8>(p, g, r0, r1, col0); break;
    case 2: skinny_tile<GATED, 2, W8>(p, g, r0, r1, col0); break;
    case 3: skinny_tile<GATED, 3, W8>(p, g, r0, r1, col0); break;
    case 4: skinny_tile<GATED, 4, W8>(p, g, r0, r1, col0); break;
    default: break;
  }
}


}  // namespace

hipError_t launch_skinny(bool gated, bool w8, const GroupedParams& p, int max_tiles, hipStream_t stream) {
  const dim3 grid(max_tiles, gated ? p.N / 64 : p.N / 128);
  if (gated && w8)
    hipLaunchKernelGGL((ffn_skinny_kernel<true, true>), grid, dim3(256), 0, stream, p);
  else if (gated)
    hipLaunchKernelGGL((ffn_skinny_kernel<true, false>), grid, dim3(256), 0, stream, p);
  else if (w8)
    hipLaunchKernelGGL((ffn_skinny_kernel<false, true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((ffn_skinny_kernel<false, false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
