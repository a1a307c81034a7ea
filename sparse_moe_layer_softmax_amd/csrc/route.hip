// route.hip -- router projection, softmax, top-k, renormalisation and routed scaling.
//
// Hy4 deep-dive (happyrock.cloud) `MoERouter`: a bias-free linear gate hidden -> experts,
// softmax over the experts, top-k. Hy3 deep-dive `SparseMoERouter.forward`: the selected
// probabilities are renormalised to sum to one. Hy4 config walkthrough (lshu.cn), section "MoE
// routed experts": norm_topk_prob true, routed_scaling_factor 2.827 scales the routed output.
//
// Two kernels:
//  1. route_gemm: x [T,H] . Wr[E,H]^T on MFMA 16x16x32 bf16 with fp32 accumulation. The hidden
//     dimension is split S ways when T is small so that enough workgroups stream Wr; each
//     split writes its own fp32 partial [S,T,E] (no atomics). For T >= 1024 and E = 256 the
//     LDS-tiled MFMA kernel of the expert FFN computes the logits instead, with its own split
//     of the hidden dimension into S partial planes.
//  2. route_topk: one wavefront per token. Sums the S partials in split order, adds the bias
//     and, in training, the caller's score noise (Hy4 deep-dive `MoERouter`: noise on the scores
//     before the softmax), stores the logits, then selects the top-k by (logit descending, expert ascending) with
//     wavefront arg-max reductions. Because the renormalised weight p_j / sum_top p_i equals
//     e^{l_j - l_max} / sum_top e^{l_i - l_max}, only the k selected exponentials are needed
//     when norm_topk_prob is set; otherwise the full softmax denominator is reduced.
#include <float.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteTokTile = 64;  // tokens per workgroup (4 waves x 16)
constexpr int kRouteExpTile = 32;  // experts per workgroup (2 MFMA column blocks)

__global__ __launch_bounds__(256) void route_gemm_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wr,
                                                         float* __restrict__ part, int T,
                                                         int H, int E, int kc) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouteTokTile + wave * 16;
  const int e0 = blockIdx.y * kRouteExpTile;
  const int k0 = blockIdx.z * kc;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int ta = t0 + lr;
  const bool av = ta < T;
  const int eb0 = e0 + lr, eb1 = e0 + 16 + lr;
  const bool bv0 = eb0 < E, bv1 = eb1 < E;
  const uint16_t* ap = x + static_cast<size_t>(av ? ta : 0) * H + k0 + lk;
  const uint16_t* bp0 = wr + static_cast<size_t>(bv0 ? eb0 : 0) * H + k0 + lk;
  const uint16_t* bp1 = wr + static_cast<size_t>(bv1 ? eb1 : 0) * H + k0 + lk;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kc; k += 128) {
    u32x4_t a[4], b0[4], b1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = av ? ld16(ap + k + 32 * u) : zero;
      b0[u] = bv0 ? ld16(bp0 + k + 32 * u) : zero;
      b1[u] = bv1 ? ld16(bp1 + k + 32 * u) : zero;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc0 = mfma16x16x32(a[u], b0[u], acc0);
      acc1 = mfma16x16x32(a[u], b1[u], acc1);
    }
  }
  float* out = part + static_cast<size_t>(blockIdx.z) * T * E;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = t0 + 4 * (lane >> 4) + v;
    if (t < T) {
      if (bv0) out[static_cast<size_t>(t) * E + eb0] = acc0[v];
      if (bv1) out[static_cast<size_t>(t) * E + eb1] = acc1[v];
    }
  }
}

// Total order used by the selection: larger value first, lower expert id among equal values.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// BATCH: partial planes whose loads one lane issues together (per expert of its four). Few
// tokens (decode) leave the GPU mostly idle, so a deep batch hides the load latency within the
// wavefront; many tokens hide it across wavefronts, and a shallow batch keeps the register
// count (and so the occupancy) low.
template <int BATCH>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ part, int S, const float* __restrict__ bias,
    const float* __restrict__ noise, float* __restrict__ logits, float* __restrict__ topk_w, int32_t* __restrict__ topk_idx,
    int T, int E, int K, int norm_topk, float scale) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const size_t plane = static_cast<size_t>(T) * E;
  // each lane sums the S partials of its experts e = lane + 64q in split order; the loads of a
  // batch of BATCH splits for all four experts are issued together so their latencies overlap
  // (lanes past E read expert 0's column and discard it)
  // (-0 + p == p for every p, so starting from -0 keeps the split-order sum exact)
  const float* src[4];
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    src[q] = part + static_cast<size_t>(t) * E + (e < E ? e : 0);
    v[q] = -0.f;
  }
  int z = 0;
  for (; z + BATCH <= S; z += BATCH) {
    float pz[4][BATCH];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < BATCH; ++u) pz[q][u] = src[q][(z + u) * plane];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < BATCH; ++u) v[q] += pz[q][u];
  }
  for (; z < S; ++z)
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += src[q][z * plane];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    if (e < E) {
      float s = v[q];
      if (bias) s += bias[e];
      if (noise) s += noise[static_cast<size_t>(t) * E + e];
      v[q] = s;
      if (logits) logits[static_cast<size_t>(t) * E + e] = s;
    } else {
      v[q] = -FLT_MAX;
    }
  }
  // k rounds of wavefront arg-max. Lane j keeps the j-th selection.
  uint32_t taken = 0;
  float my_val = 0.f, lmax = 0.f;
  int my_idx = 0;
  for (int j = 0; j < K; ++j) {
    float bv = -FLT_MAX;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (e < E && !((taken >> q) & 1u) && better(v[q], e, bv, bi)) {
        bv = v[q];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (j == 0) lmax = bv;
    if (lane == j) {
      my_val = bv;
      my_idx = bi;
    }
  }
  // Numerators e^{l_j - l_max} for the selected slots.
  const float ex = lane < K ? expf(my_val - lmax) : 0.f;
  float denom;
  if (norm_topk) {
    denom = ex;
  } else {
    denom = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + 64 * q < E) denom += expf(v[q] - lmax);
  }
  // xor butterfly: every lane ends with the same, order-fixed sum
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) denom += __shfl_xor(denom, off);
  if (lane < K) {
    topk_w[static_cast<size_t>(t) * K + lane] = scale * ex / denom;
    topk_idx[static_cast<size_t>(t) * K + lane] = my_idx;
  }
}

}  // namespace

// Large T with a 256-wide expert dimension: the tiled MFMA kernel computes the logits in one
// pass (no hidden split).
static bool route_tiled(int T, int H, int E) { return T >= 1024 && dense_gemm_f32_supported(E, H); }

int route_splits(int T, int H, int E) {
  if (route_tiled(T, H, E)) return dense_gemm_splits(T, H);
  const int tiles = ((T + kRouteTokTile - 1) / kRouteTokTile) * ((E + kRouteExpTile - 1) / kRouteExpTile);
  const int kmax = H / 128;  // each split covers a multiple of 128 hidden elements
  int best = 1;
  for (int s = 1; s <= kmax && s <= 64; ++s) {
    if (kmax % s) continue;
    best = s;
    if (tiles * s >= 512) break;
  }
  return best;
}

hipError_t launch_route(const moe_shape& s, const uint16_t* x, const uint16_t* w_router,
                        const float* bias, const float* noise, float* logits, float* topk_w,
                        int32_t* topk_idx, float* partials, int S, hipStream_t stream) {
  if (route_tiled(s.T, s.H, s.E)) {
    const hipError_t e = launch_dense_gemm_f32(x, s.T, w_router, s.E, s.H, S, partials, stream);
    if (e != hipSuccess) return e;
  } else {
    dim3 g1((s.T + kRouteTokTile - 1) / kRouteTokTile, (s.E + kRouteExpTile - 1) / kRouteExpTile, S);
    hipLaunchKernelGGL(route_gemm_kernel, g1, dim3(256), 0, stream, x, w_router, partials, s.T,
                       s.H, s.E, s.H / S);
  }
  if (s.T < 1024)
    hipLaunchKernelGGL(route_topk_kernel<16>, dim3((s.T + 3) / 4), dim3(256), 0, stream, partials,
                       S, bias, noise, logits, topk_w, topk_idx, s.T, s.E, s.K, s.norm_topk_prob,
                       s.routed_scaling);
  else
    hipLaunchKernelGGL(route_topk_kernel<2>, dim3((s.T + 3) / 4), dim3(256), 0, stream, partials,
                       S, bias, noise, logits, topk_w, topk_idx, s.T, s.E, s.K, s.norm_topk_prob,
                       s.routed_scaling);
  return hipGetLastError();
}

}  // namespace moe
