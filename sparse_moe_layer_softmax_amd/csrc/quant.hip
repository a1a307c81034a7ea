// quant.hip -- per-row dynamic FP8 (OCP E4M3) quantisation of bf16 activation rows, for the
// W8A8 form of the expert FFN.
//
// The pages deploy the model from an FP8 checkpoint (Tencent Hunyuan Hy4 Preview deep technical
// analysis, deployment commands) without defining the format. Each row v gets
//   amax = max |v|,  scale = amax / 448,  code = E4M3_RNE(clamp(v * (448 / amax), +-448))
// (both divisions correctly rounded fp32, the product one fp32 multiply), so the row is
// scale * e4m3(code) to within half an E4M3 step. An all-zero row, and a row so small that
// 448 / amax overflows fp32 (amax below 448 / FLT_MAX, about 1.3e-36), is quantised unscaled:
// scale 1 and code = E4M3_RNE(v), which is a zero code for every such value.
//
// One wavefront per row, two passes over it (the second one hits L2): the absolute maximum by
// a wavefront max-reduction (exact, order-free), then eight values per lane and step turned
// into codes by the hardware conversion v_cvt_pk_fp8_f32 (nearest-even) and stored as one
// 8-byte segment per lane.
#include <float.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float clamp448(float q) { return fminf(fmaxf(q, -448.f), 448.f); }

// four codes (bytes 0..3 = a, b, c, d)
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
  return static_cast<uint32_t>(w);
}

__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ v, int rows,
                                                         int cols, const int32_t* __restrict__ rows_dev,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n = rows_dev ? min(rows, *rows_dev) : rows;
  if (r >= n) return;
  const uint16_t* vr = v + static_cast<size_t>(r) * cols;
  float amax = 0.f;
  for (int c = lane * 8; c < cols; c += 512) {
    const u32x4_t t = ld16(vr + c);
#pragma unroll
    for (int d = 0; d < 4; ++d) amax = fmaxf(amax, fmaxf(fabsf(bf_lo(t[d])), fabsf(bf_hi(t[d]))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  float inv = 1.f, scale = 1.f;
  if (amax > 0.f) {
    const float q = __fdiv_rn(448.f, amax);
    if (q <= FLT_MAX) {  // else (+inf) the row is below what a scaled E4M3 code can reach
      inv = q;
      scale = __fdiv_rn(amax, 448.f);
    }
  }
  if (lane == 0) scales[r] = scale;
  uint8_t* cr = codes + static_cast<size_t>(r) * cols;
  for (int c = lane * 8; c < cols; c += 512) {
    const u32x4_t t = ld16(vr + c);
    uint2 o;
    o.x = pack4(bf_lo(t[0]) * inv, bf_hi(t[0]) * inv, bf_lo(t[1]) * inv, bf_hi(t[1]) * inv);
    o.y = pack4(bf_lo(t[2]) * inv, bf_hi(t[2]) * inv, bf_lo(t[3]) * inv, bf_hi(t[3]) * inv);
    *reinterpret_cast<uint2*>(cr + c) = o;
  }
}

}  // namespace

hipError_t launch_quant_rows(const uint16_t* v, int rows, int cols, const int32_t* rows_dev,
                             uint8_t* codes, float* scales, hipStream_t stream) {
  if (rows < 1) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, v, rows,
                     cols, rows_dev, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
