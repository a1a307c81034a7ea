// combine.hip -- weighted, atomic-free combine of the routed rows and the shared expert row.
//
// Hy4 deep-dive (happyrock.cloud) `MoELayer.forward`: the routed output accumulates
// weight * expert(x) over the token's top-k experts and the shared expert's output is added
// (routed_output + shared_output). Hy4 config walkthrough (lshu.cn), section "MoE routed
// experts": routed_scaling_factor scales the routed part only (already folded into topk_w).
//
// One workgroup per token (H / 8 threads, up to 1024; wider rows in 2048-column blocks), so each
// gathered row is read whole by one workgroup; each thread owns 8 consecutive columns (16-byte
// loads and stores). The sum runs in fp32 in slot order j = 0..K-1, then the shared row, and is
// rounded to bf16 once, so the result does not depend on scheduling.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(1024) void combine_kernel(
    const uint16_t* __restrict__ y_routed, const float* __restrict__ topk_w,
    const int32_t* __restrict__ slot_to_row, const uint16_t* __restrict__ y_shared,
    uint16_t* __restrict__ out, int H, int K) {
  const int t = blockIdx.x;
  const int c = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (c >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j = 0; j < K; ++j) {
    const int row = slot_to_row[static_cast<size_t>(t) * K + j];
    if (row < 0) continue;  // dropped by capacity
    const float w = topk_w[static_cast<size_t>(t) * K + j];
    const u32x4_t v = ld16(y_routed + static_cast<size_t>(row) * H + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += w * __uint_as_float(v[i] << 16);
      acc[2 * i + 1] += w * __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  if (y_shared) {
    const u32x4_t v = ld16(y_shared + static_cast<size_t>(t) * H + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(v[i] << 16);
      acc[2 * i + 1] += __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
  *reinterpret_cast<u32x4_t*>(out + static_cast<size_t>(t) * H + c) = o;
}

}  // namespace

hipError_t launch_combine(const moe_shape& s, const uint16_t* y_routed, const float* topk_w,
                          const int32_t* slot_to_row, const uint16_t* y_shared, uint16_t* out,
                          hipStream_t stream) {
  // one workgroup per token when its row fits (H / 8 <= 1024 threads): each gathered row is then
  // read whole by one workgroup
  const int threads = s.H / 8 <= 1024 ? s.H / 8 : kCombineThreads;
  const int cols_per_block = threads * 8;
  dim3 grid(s.T, (s.H + cols_per_block - 1) / cols_per_block);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(threads), 0, stream, y_routed, topk_w,
                     slot_to_row, y_shared, out, s.H, s.K);
  return hipGetLastError();
}

}  // namespace moe
