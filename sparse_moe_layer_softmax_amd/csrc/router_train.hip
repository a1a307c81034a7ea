// router_train.hip -- training-side router statistics.
//
// Hy3 deep-dive (happyrock.cloud) `SparseMoERouter`, training branch and its load-balancing
// loss: P_e is the token mean of the routing probabilities, f_e the share of the T*K top-k
// selections that chose expert e, and the loss is E * sum_e P_e f_e; the expert-count and
// token-count buffers move as exponential moving averages (decay 0.9 on the page).
//
// Two kernels and no floating-point atomics, so every run gives the same bits:
//  1. stats_partial: blocks of kStatTok tokens. A wavefront takes one token at a time: softmax
//     over the E logits (wavefront max, exponentials, fixed-shape butterfly sum) and the
//     probabilities added to per-lane accumulators in token order. The four wavefronts' sums are
//     added in wavefront order into one partial row per block. Selection counts per block come
//     from LDS integer atomics (exact in any order).
//  2. stats_final: one workgroup. Thread e adds the partial rows in block order and forms P_e,
//     f_e and the EMA updates; a fixed-shape tree over e gives the loss.
#include <cfloat>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kStatTok = 64;  // tokens per partial-sum block

__global__ __launch_bounds__(256) void stats_partial_kernel(const float* __restrict__ logits,
                                                            const int32_t* __restrict__ topk_idx,
                                                            int T, int E, int K,
                                                            float* __restrict__ part_p,
                                                            int32_t* __restrict__ part_c) {
  __shared__ float wsum[4][256];
  __shared__ int cnt[256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int e = threadIdx.x; e < 256; e += 256) cnt[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kStatTok;
  const int t1 = min(t0 + kStatTok, T);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int t = t0 + wave; t < t1; t += 4) {
    const float* l = logits + static_cast<size_t>(t) * E;
    float v[4];
    float m = -FLT_MAX;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      v[q] = e < E ? l[e] : -FLT_MAX;
      m = fmaxf(m, v[q]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float ex[4];
    float z = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ex[q] = lane + 64 * q < E ? expf(v[q] - m) : 0.f;
      z += ex[q];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += ex[q] / z;
  }
  // selection counts of this block's tokens (ids outside [0, E) are not counted)
  for (int i = threadIdx.x; i < (t1 - t0) * K; i += 256) {
    const int e = topk_idx[static_cast<size_t>(t0) * K + i];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&cnt[e], 1);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) wsum[wave][lane + 64 * q] = acc[q];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    part_p[static_cast<size_t>(blockIdx.x) * E + e] = ((wsum[0][e] + wsum[1][e]) + wsum[2][e]) + wsum[3][e];
    part_c[static_cast<size_t>(blockIdx.x) * E + e] = cnt[e];
  }
}

__global__ __launch_bounds__(256) void stats_final_kernel(
    const float* __restrict__ part_p, const int32_t* __restrict__ part_c, int nb, int T, int E,
    int K, float decay, float* __restrict__ prob_mean, float* __restrict__ load_frac,
    float* __restrict__ aux_loss, float* __restrict__ ema_counts, float* __restrict__ ema_tokens) {
  __shared__ float prod[256];
  const int e = threadIdx.x;
  float pf = 0.f;
  if (e < E) {
    float sp = 0.f;
    int c = 0;  // at most T*K selections
    for (int b = 0; b < nb; ++b) {
      sp += part_p[static_cast<size_t>(b) * E + e];
      c += part_c[static_cast<size_t>(b) * E + e];
    }
    const float P = sp / static_cast<float>(T);
    const float f = static_cast<float>(c) / static_cast<float>(T * K);  // both exact integers
    prob_mean[e] = P;
    load_frac[e] = f;
    pf = P * f;
    if (ema_counts) ema_counts[e] = decay * ema_counts[e] + (1.f - decay) * static_cast<float>(c);
  }
  prod[e] = pf;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if (e < off) prod[e] += prod[e + off];
    __syncthreads();
  }
  if (e == 0) {
    *aux_loss = prod[0] * static_cast<float>(E);
    if (ema_tokens) *ema_tokens = decay * *ema_tokens + (1.f - decay) * static_cast<float>(T);
  }
}

}  // namespace

int router_stats_blocks(int T) { return (T + kStatTok - 1) / kStatTok; }

hipError_t launch_router_stats(const moe_shape& s, const float* logits, const int32_t* topk_idx,
                               float* part_p, int32_t* part_c, float decay, float* prob_mean,
                               float* load_frac, float* aux_loss, float* ema_counts,
                               float* ema_tokens, hipStream_t stream) {
  if (s.E > 256 || s.T < 1) return hipErrorInvalidValue;
  const int nb = router_stats_blocks(s.T);
  hipLaunchKernelGGL(stats_partial_kernel, dim3(nb), dim3(256), 0, stream, logits, topk_idx, s.T,
                     s.E, s.K, part_p, part_c);
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(256), 0, stream, part_p, part_c, nb, s.T,
                     s.E, s.K, decay, prob_mean, load_frac, aux_loss, ema_counts, ema_tokens);
  return hipGetLastError();
}

}  // namespace moe
