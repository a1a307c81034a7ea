// quant.hip -- dynamic FP8 (OCP E4M3) quantisation of bf16 activation rows: per row (one fp32
// scale, the W8A8 form of the expert FFN) or per 32-element block (one E8M0 scale, the MX form).
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

// MX (OCP Microscaling) block quantisation. Per 32 consecutive elements of a row the E8M0 scale
// byte is s = max(E - 8, 0), E the biased fp32 exponent field of the block's absolute maximum:
// floor(log2(amax)) - 8 + 127 for a normal amax, clamped at 0 (2^-127), which also covers an
// amax that is zero or subnormal. The codes are E4M3_RNE(clamp(v * 2^(127 - s), +-448)); the
// power of two is a normal fp32 value (s <= 246 for bf16 input), so the product is exact unless
// it falls below the fp32 normal range, where the E4M3 code is zero either way.
// (The block step itself is mx_quant8, which the tiled gate/up epilogue also applies to h as it
// writes it; this kernel quantises x, and h after the weight-streaming kernel.)
// One wavefront per row; a lane takes 8 consecutive elements, so a block is 4 lanes and a
// 128-element K-tile (one dword of 4 scale bytes) 16 lanes. The codes keep the source row
// order; the scale dwords go to planes [cols / 128][plane_rows] of the GEMM that reads them:
//   s2r == NULL: source row r is GEMM row r;
//   else (x before the gate/up GEMM): source row t is GEMM row t when n_ident > 0 (the shared
//   expert's identity rows) and GEMM row n_ident + s2r[t * K + k] for each kept slot k.
__global__ __launch_bounds__(256) void quant_mx_kernel(const uint16_t* __restrict__ v, int rows,
                                                       int cols, const int32_t* __restrict__ rows_dev,
                                                       uint8_t* __restrict__ codes,
                                                       uint32_t* __restrict__ scales, int plane_rows,
                                                       const int32_t* __restrict__ s2r, int K,
                                                       int n_ident) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n = rows_dev ? min(rows, *rows_dev) : rows;
  if (r >= n) return;
  const uint16_t* vr = v + static_cast<size_t>(r) * cols;
  uint8_t* cr = codes + static_cast<size_t>(r) * cols;
  // the token's GEMM rows of its K slots (K <= 64), one per lane, loaded once for all columns
  const int slot_row = s2r && lane < K ? s2r[static_cast<size_t>(r) * K + lane] : -1;
  for (int c = lane * 8; c < cols; c += 512) {
    const u32x4_t t = ld16(vr + c);
    uint2 o;
    const int s = mx_quant8(t, &o);
    *reinterpret_cast<uint2*>(cr + c) = o;
    // the K-tile's four scale bytes, blocks in order, from lanes 0, 4, 8, 12 of the 16-lane group
    const int g0 = lane & ~15;
    const uint32_t dw = static_cast<uint32_t>(__shfl(s, g0)) | (static_cast<uint32_t>(__shfl(s, g0 + 4)) << 8) |
                        (static_cast<uint32_t>(__shfl(s, g0 + 8)) << 16) |
                        (static_cast<uint32_t>(__shfl(s, g0 + 12)) << 24);
    const size_t plane = static_cast<size_t>((c - (lane & 15) * 8) / 128) * plane_rows;
    if (!s2r) {
      if ((lane & 15) == 0) scales[plane + r] = dw;
    } else {
      if ((lane & 15) == 0 && n_ident > 0) scales[plane + r] = dw;
      for (int k = 0; k < K; ++k) {  // the token's kept slots (row -1: dropped)
        const int j = __shfl(slot_row, k);
        if ((lane & 15) == 0 && j >= 0) scales[plane + n_ident + j] = dw;
      }
    }
  }
}

}  // namespace

hipError_t launch_quant_mx(const uint16_t* v, int rows, int cols, const int32_t* rows_dev,
                           uint8_t* codes, uint8_t* scales, int plane_rows, const int32_t* s2r,
                           int K, int n_ident, hipStream_t stream) {
  if (rows < 1) return hipSuccess;
  if (s2r && (K < 1 || K > 64)) return hipErrorInvalidValue;  // one slot per lane of a wavefront
  hipLaunchKernelGGL(quant_mx_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, v, rows, cols,
                     rows_dev, codes, reinterpret_cast<uint32_t*>(scales), plane_rows, s2r, K, n_ident);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* v, int rows, int cols, const int32_t* rows_dev,
                             uint8_t* codes, float* scales, hipStream_t stream) {
  if (rows < 1) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, v, rows,
                     cols, rows_dev, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
