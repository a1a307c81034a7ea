// moe_device.h -- gfx950 device helpers shared by the MoE kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace moe {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// 16-byte global load (8 bf16).
__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%16][8*(l/16) + 0..7] and B[8*(l/16) + 0..7][l%16] and holds
// D[4*(l/16) + v][l%16] for v = 0..3.
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D(32x32) += A(32x16) * B(16x32). Lane l supplies A[l%32][8*(l/32) + 0..7] and
// B[8*(l/32) + 0..7][l%32]; holds D[8*(v/4) + 4*(l/32) + v%4][l%32] for v = 0..15.
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Gradients of the clamped SwiGLU h = silu(clamp(g, +-L)) * clamp(u, +-L) at the fp32 sums g, u
// given dh (no clamp for L <= 0): dg = dh clamp(u) silu'(clamp g), passed only where
// -L <= g <= L, and du = dh silu(clamp g), passed only where -L <= u <= L. One definition for
// every kernel that forms them, so they agree bit for bit.
__device__ __forceinline__ void swiglu_bwd(float gv, float uv, float dhv, float L, float& dg,
                                           float& du) {
  const float gc = L > 0.f ? fminf(fmaxf(gv, -L), L) : gv;
  const float uc = L > 0.f ? fminf(fmaxf(uv, -L), L) : uv;
  const float sg = 1.f / (1.f + expf(-gc));
  const bool pg = !(L > 0.f) || (gv >= -L && gv <= L);
  const bool pu = !(L > 0.f) || (uv >= -L && uv <= L);
  dg = pg ? dhv * uc * (sg * (1.f + gc * (1.f - sg))) : 0.f;
  du = pu ? dhv * (gc * sg) : 0.f;
}

typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));

// D(32x32) += A(32x64) * B(64x32) on FP8 E4M3 codes (the gfx950 FP8 MFMA; the block scales it
// takes are 1.0, E8M0 127). Lane l supplies 32 codes of row l%32 of A and of column l%32 of B,
// and D is laid out as for mfma32x32x16. The two lane halves and the 32 byte positions each
// stand for one K index, the same for A and B, so any one-to-one placement of the 64 K values
// on (lane half, byte) that A and B share gives the same product.
__device__ __forceinline__ f32x16_t mfma32x32x64_fp8(u32x8_t a, u32x8_t b, f32x16_t c) {
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8_t, a),
                                                         __builtin_bit_cast(i32x8_t, b), c, 0, 0,
                                                         0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
}

// The same product with MX block scales. The instruction's first 32-code block of row r (of A;
// column r of B) is bytes 0-15 of lanes r and r + 32, its second block bytes 16-31 of both; lane
// r supplies the first block's E8M0 byte and lane r + 32 the second's, in bits 7:0 of sa (A) and
// sb (B). A probe on the GPU fixed this layout (one-hot codes against distinct per-lane scales).
__device__ __forceinline__ f32x16_t mfma32x32x64_fp8_mx(u32x8_t a, u32x8_t b, f32x16_t c, uint32_t sa,
                                                       uint32_t sb) {
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8_t, a),
                                                         __builtin_bit_cast(i32x8_t, b), c, 0, 0, 0,
                                                         static_cast<int>(sa), 0, static_cast<int>(sb));
}

// Eight OCP E4M3 codes (two dwords, code 0 in the low byte) -> the eight bf16 of one MFMA
// operand. Exact: every E4M3 value is a bf16 value (the gfx950 scaled convert, scale 1).
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return r;
}

// The same with an MX block scale: the eight bf16 of e4m3(code) * 2^(s - 127) for the E8M0 byte
// s, exact while the product stays within bf16's normal range (s from 10 to 245 for any code).
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16_mx(uint32_t lo, uint32_t hi, uint32_t s) {
  const uint32_t b = s & 0xFFu;
  const float sc = __uint_as_float(b ? b << 23 : 0x00400000u);  // 2^(b - 127)
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true));
  return r;
}

// silu(clamp(g)) * clamp(u): the SwiGLU activation with swiglu_limit applied to both
// pre-activations (limit <= 0 disables the clamp).
__device__ __forceinline__ float clamped_swiglu(float g, float u, float limit) {
  if (limit > 0.f) {
    g = fminf(fmaxf(g, -limit), limit);
    u = fminf(fmaxf(u, -limit), limit);
  }
  return g / (1.f + __expf(-g)) * u;
}

// ---- FP8 (OCP E4M3) encoding of bf16 values, shared by the quantisers and the fused epilogue
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float clamp448(float q) { return fminf(fmaxf(q, -448.f), 448.f); }

// four codes (bytes 0..3 = a, b, c, d): E4M3 nearest-even of each value clamped to +-448
// (v_cvt_pk_fp8_f32)
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
  return static_cast<uint32_t>(w);
}

// MX (OCP MXFP8) block quantisation, for a lane holding 8 of a 32-element block's bf16 values
// (t: four dwords, element 0 in the low half of t[0]) in a group of 4 lanes (lane ^ 1, lane ^ 2)
// that holds the block. Returns the block's E8M0 byte s = max(E(amax) - 8, 0), E the biased
// fp32 exponent of the block's largest magnitude (a zero block: 0), and the lane's 8 codes
// E4M3_RNE(clamp(v * 2^(127 - s), +-448)) in *codes; every step is exact but the final rounding.
__device__ __forceinline__ int mx_quant8(const u32x4_t& t, uint2* codes) {
  float amax = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) amax = fmaxf(amax, fmaxf(fabsf(bf_lo(t[d])), fabsf(bf_hi(t[d]))));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int s = max(static_cast<int>((__float_as_uint(amax) >> 23) & 0xFF) - 8, 0);
  const float f = __uint_as_float(static_cast<uint32_t>(254 - s) << 23);  // 2^(127 - s)
  codes->x = pack4(bf_lo(t[0]) * f, bf_hi(t[0]) * f, bf_lo(t[1]) * f, bf_hi(t[1]) * f);
  codes->y = pack4(bf_lo(t[2]) * f, bf_hi(t[2]) * f, bf_lo(t[3]) * f, bf_hi(t[3]) * f);
  return s;
}

}  // namespace moe
