// backward.hip -- backward pass of the MoE layer (training).
//
// The router is trained on the pages (Hy3 deep-dive `SparseMoERouter` training branch with its
// load-balancing loss; Hy4 deep-dive `MoERouter` scores noise) but no backward is printed, so
// this differentiates the forward in reverse:
//   combine   dy_row = w_j * dout[t] (bf16); d w_j = <dout[t], y_row>          combine_bwd
//   down      dh = dy Wd (bf16)                                                 gemm kDh
//   SwiGLU    g, u recomputed (x Wg^T, x Wu^T); dg = dh clamp(u) silu'(clamp g) [|g| <= L],
//             du = dh silu(clamp g) [|u| <= L] (bf16)                           gemm kGu
//   gate/up   dx_row = dg Wg + du Wu (bf16)                                     gemm kDx
//   weights   dWd = dy^T h, dWg = dg^T x, dWu = du^T x (fp32, per expert)     gemm kWd, kWgu
//   routing   d logits through renormalisation, scaling and softmax, plus the load-balancing
//             loss term (its f held fixed); dWr = dl^T x, dx_router = dl Wr    router_bwd, f32 gemm
//   dx        the token's routed rows in slot order, the shared row, the router term  dx_sum
// The shared expert is group 0 of the grouped GEMMs (identity rows), as in the forward.
//
// One MFMA kernel serves the five grouped products. Tiles of 128x128 outputs, K staged 32 at
// a time through a double-buffered LDS pair [128][40] (operand rows with K contiguous, padded
// so that the 16-byte fragment reads of 16 lanes hit distinct bank groups); 4 wavefronts of
// 64x64 (2x2 MFMA 32x32x16). Operands whose source is K-contiguous are copied row-wise with
// 16-byte loads; operands whose source is contiguous along M or N (the data-gradient weights
// and both operands of the weight gradients, which reduce over rows) are transposed on their
// way into LDS. The next K tile's global loads are in flight while the current one computes.
// Everything runs in a fixed order: no floating-point atomics.
#include <cfloat>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 32, kLd = kBK + 8;  // LDS row stride in bf16
enum Mode { kDh = 0, kGu = 1, kDx = 2, kWd = 3, kWgu = 4 };

struct GemmP {
  const int32_t* offsets;  // [G+1] group row offsets (shared group first when present)
  int g_split;             // groups below it use the *_a (shared expert) operands
  const int32_t* tiles;
  int max_tiles;
  const int32_t* gather;   // row_to_slot
  int n_ident, topk, rows_max, H, I;
  const uint16_t* x;       // [T, H]
  const uint16_t* dy;      // [rows, H]
  const uint16_t* h;       // [rows, I] forward
  const uint16_t* dh;      // [rows, I]
  const uint16_t* dgu;     // [rows, 2I] = [dg | du]
  uint16_t* out16;         // kDh: dh, kGu: dgu, kDx: dx_rows
  const uint16_t *wg_a, *wg_b, *wu_a, *wu_b, *wd_a, *wd_b;
  float *gwg_a, *gwg_b, *gwu_a, *gwu_b, *gwd_a, *gwd_b;
  float limit;
};

__device__ __forceinline__ int x_row(const GemmP& p, int r) {
  return r < p.n_ident ? r : p.gather[r - p.n_ident] / p.topk;
}

// 8 bf16 values of a 16-byte chunk written down a column of the [rows][kLd] LDS tile.
__device__ __forceinline__ void lds_column8(uint16_t* l, int outer0, int k, u32x4_t v) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    l[(outer0 + 2 * d) * kLd + k] = static_cast<uint16_t>(v[d] & 0xffffu);
    l[(outer0 + 2 * d + 1) * kLd + k] = static_cast<uint16_t>(v[d] >> 16);
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(GemmP p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][(kBM + kBN) * kLd];
  constexpr bool GK = MODE == kWd || MODE == kWgu;  // grouped over K: weight gradients
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int g, m0, m_end, k_lo, k_hi;
  const int n0 = blockIdx.y * kBN;
  if (!GK) {
    const int tile = blockIdx.x;
    if (tile >= p.tiles[0]) return;
    g = p.tiles[1 + tile];
    m0 = p.tiles[1 + p.max_tiles + tile];
    m_end = min(p.offsets[g + 1], p.rows_max);
    if (m0 < 0 || m0 >= m_end) return;
    k_lo = 0;
    k_hi = MODE == kDx ? 2 * p.I : p.H;
  } else {
    g = blockIdx.z;
    m0 = blockIdx.x * kBM;
    m_end = MODE == kWd ? p.H : 2 * p.I;
    k_lo = p.offsets[g];
    k_hi = min(p.offsets[g + 1], p.rows_max);
  }
  const bool sh = g < p.g_split;
  const size_t IH = static_cast<size_t>(p.I) * p.H;
  const size_t eo = sh ? 0 : static_cast<size_t>(g - p.g_split) * IH;
  const uint16_t* Wg = (sh ? p.wg_a : p.wg_b) + eo;
  const uint16_t* Wu = (sh ? p.wu_a : p.wu_b) + eo;
  const uint16_t* Wd = (sh ? p.wd_a : p.wd_b) + eo;
  const int I2 = 2 * p.I;

  // ---- global loads of one K tile (two 16-byte chunks of A and two of B per thread)
  u32x4_t ra[2], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      if (!GK) {
        // A rows (K contiguous): row idx/4, chunk idx%4
        const int row = idx >> 2, ch = idx & 3, m = m0 + row, k = k0 + 8 * ch;
        if (m < m_end) {
          if (MODE == kDh) ra[i] = ld16(p.dy + static_cast<size_t>(m) * p.H + k);
          if (MODE == kGu) ra[i] = ld16(p.x + static_cast<size_t>(x_row(p, m)) * p.H + k);
          if (MODE == kDx) ra[i] = ld16(p.dgu + static_cast<size_t>(m) * I2 + k);
        } else {
          ra[i] = z;
        }
        if (MODE == kGu) {  // B rows (K contiguous): 64 gate rows then the same 64 up rows
          const int n = idx >> 2, c = n0 / 2 + (n & 63);
          rb[i] = ld16((n < 64 ? Wg : Wu) + static_cast<size_t>(c) * p.H + k0 + 8 * ch);
        } else {  // B contiguous along N: k row idx/16, 8 columns at 8*(idx%16)
          const int kr = idx >> 4, nc = n0 + 8 * (idx & 15), k = k0 + kr;
          if (MODE == kDh) rb[i] = ld16(Wd + static_cast<size_t>(k) * p.I + nc);
          if (MODE == kDx)
            rb[i] = k < p.I ? ld16(Wg + static_cast<size_t>(k) * p.H + nc)
                            : ld16(Wu + static_cast<size_t>(k - p.I) * p.H + nc);
        }
      } else {
        // both operands contiguous along M / N, K = layer rows of the group
        const int kr = idx >> 4, c8 = 8 * (idx & 15), r = k0 + kr;
        if (r < k_hi) {
          if (MODE == kWd) {
            ra[i] = ld16(p.dy + static_cast<size_t>(r) * p.H + m0 + c8);
            rb[i] = ld16(p.h + static_cast<size_t>(r) * p.I + n0 + c8);
          } else {
            ra[i] = ld16(p.dgu + static_cast<size_t>(r) * I2 + m0 + c8);
            rb[i] = ld16(p.x + static_cast<size_t>(x_row(p, r)) * p.H + n0 + c8);
          }
        } else {
          ra[i] = z;
          rb[i] = z;
        }
      }
    }
  };
  auto store = [&](uint16_t* l) {
    uint16_t* la = l;
    uint16_t* lb = l + kBM * kLd;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      if (!GK) {
        *reinterpret_cast<u32x4_t*>(la + (idx >> 2) * kLd + 8 * (idx & 3)) = ra[i];
        if (MODE == kGu)
          *reinterpret_cast<u32x4_t*>(lb + (idx >> 2) * kLd + 8 * (idx & 3)) = rb[i];
        else
          lds_column8(lb, 8 * (idx & 15), idx >> 4, rb[i]);
      } else {
        lds_column8(la, 8 * (idx & 15), idx >> 4, ra[i]);
        lds_column8(lb, 8 * (idx & 15), idx >> 4, rb[i]);
      }
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = (k_hi - k_lo + kBK - 1) / kBK;
  if (nk > 0) {
    load(k_lo);
    store(lds[0]);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
      if (t + 1 < nk) load(k_lo + (t + 1) * kBK);
      const uint16_t* la = lds[t & 1];
      const uint16_t* lb = la + kBM * kLd;
#pragma unroll
      for (int kk = 0; kk < kBK; kk += 16) {
        u32x4_t af[2], bf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          af[i] = *reinterpret_cast<const u32x4_t*>(la + (wm * 64 + i * 32 + (lane & 31)) * kLd + kk + 8 * (lane >> 5));
          bf[i] = *reinterpret_cast<const u32x4_t*>(lb + (wn * 64 + i * 32 + (lane & 31)) * kLd + kk + 8 * (lane >> 5));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(af[i], bf[j], acc[i][j]);
      }
      if (t + 1 < nk) store(lds[(t + 1) & 1]);
      __syncthreads();
    }
  }

  // ---- epilogue. Lane l of fragment (i, j) holds rows 8(v/4) + 4(l/32) + v%4, column l%32.
  if (MODE == kGu) {
    // gate (wn = 0) and up (wn = 1) of the same columns meet through LDS
    float* ex = reinterpret_cast<float*>(&lds[0][0]);  // [2 wm][64][64] fp32 = 32 KB
    __syncthreads();
    if (wn == 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            ex[(wm * 64 + row) * 64 + j * 32 + (lane & 31)] = acc[i][j][v];
          }
    }
    __syncthreads();
    if (wn == 0) {
      const float L = p.limit;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            const int m = m0 + wm * 64 + row;
            if (m >= m_end) continue;
            const int c = n0 / 2 + j * 32 + (lane & 31);  // intermediate column
            const float gv = acc[i][j][v];
            const float uv = ex[(wm * 64 + row) * 64 + j * 32 + (lane & 31)];
            const float gc = L > 0.f ? fminf(fmaxf(gv, -L), L) : gv;
            const float uc = L > 0.f ? fminf(fmaxf(uv, -L), L) : uv;
            const float sg = 1.f / (1.f + expf(-gc));
            const float dhv = bf16_to_f32(p.dh[static_cast<size_t>(m) * p.I + c]);
            const bool pg = !(L > 0.f) || (gv >= -L && gv <= L);
            const bool pu = !(L > 0.f) || (uv >= -L && uv <= L);
            const float dg = pg ? dhv * uc * (sg * (1.f + gc * (1.f - sg))) : 0.f;
            const float du = pu ? dhv * (gc * sg) : 0.f;
            p.out16[static_cast<size_t>(m) * I2 + c] = f32_to_bf16(dg);
            p.out16[static_cast<size_t>(m) * I2 + p.I + c] = f32_to_bf16(du);
          }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (m >= m_end) continue;
        const float a = acc[i][j][v];
        if (MODE == kDh) p.out16[static_cast<size_t>(m) * p.I + n] = f32_to_bf16(a);
        if (MODE == kDx) p.out16[static_cast<size_t>(m) * p.H + n] = f32_to_bf16(a);
        if (MODE == kWd) ((sh ? p.gwd_a : p.gwd_b) + eo)[static_cast<size_t>(m) * p.I + n] = a;
        if (MODE == kWgu) {
          if (m < p.I)
            ((sh ? p.gwg_a : p.gwg_b) + eo)[static_cast<size_t>(m) * p.H + n] = a;
          else
            ((sh ? p.gwu_a : p.gwu_b) + eo)[static_cast<size_t>(m - p.I) * p.H + n] = a;
        }
      }
}

// Routed-row gradients dy = w * dout (bf16), the shared rows' dy = dout, and the routing-weight
// gradients <dout[t], y_row> (one wavefront per token, lane-order partial sums, fixed butterfly).
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const uint16_t* __restrict__ dout, const float* __restrict__ topk_w,
    const int32_t* __restrict__ slot_to_row, const uint16_t* __restrict__ y, int n_ident, int T,
    int K, int H, uint16_t* __restrict__ dy, float* __restrict__ d_topk_w) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const uint16_t* go = dout + static_cast<size_t>(t) * H;
  if (n_ident > 0)
    for (int c = lane * 8; c < H; c += 512)
      *reinterpret_cast<u32x4_t*>(dy + static_cast<size_t>(t) * H + c) = ld16(go + c);
  for (int j = 0; j < K; ++j) {
    const size_t s = static_cast<size_t>(t) * K + j;
    const int r = slot_to_row[s];
    if (r < 0) {
      if (lane == 0) d_topk_w[s] = 0.f;
      continue;
    }
    const float w = topk_w[s];
    const uint16_t* yr = y + static_cast<size_t>(n_ident + r) * H;
    uint16_t* dr = dy + static_cast<size_t>(n_ident + r) * H;
    float acc = 0.f;
    for (int c = lane * 8; c < H; c += 512) {
      const u32x4_t a = ld16(go + c), b = ld16(yr + c);
      u32x4_t o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float g0 = bf16_to_f32(static_cast<uint16_t>(a[d] & 0xffffu));
        const float g1 = bf16_to_f32(static_cast<uint16_t>(a[d] >> 16));
        acc += g0 * bf16_to_f32(static_cast<uint16_t>(b[d] & 0xffffu));
        acc += g1 * bf16_to_f32(static_cast<uint16_t>(b[d] >> 16));
        o[d] = pack_bf16x2(w * g0, w * g1);
      }
      *reinterpret_cast<u32x4_t*>(dr + c) = o;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) d_topk_w[s] = acc;
  }
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Selections per expert (integer atomics: exact in any order).
__global__ void count_kernel(const int32_t* __restrict__ topk_idx, int n, int E,
                             int32_t* __restrict__ cnt) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const int e = topk_idx[i];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&cnt[e], 1);
  }
}

// Logit gradients of one token per wavefront: the routing-weight gradients through the
// renormalisation and scaling to the selected probabilities, the loss term to every
// probability, then the softmax.
__global__ __launch_bounds__(256) void router_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ d_topk_w, const int32_t* __restrict__ cnt, int T, int E, int K,
    int norm, float scale, float d_aux, float* __restrict__ dl) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const float* l = logits + static_cast<size_t>(t) * E;
  float p[4];
  float m = -FLT_MAX;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    p[q] = lane + 64 * q < E ? l[lane + 64 * q] : -FLT_MAX;
    m = fmaxf(m, p[q]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float z = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    p[q] = lane + 64 * q < E ? expf(p[q] - m) : 0.f;
    z += p[q];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
#pragma unroll
  for (int q = 0; q < 4; ++q) p[q] /= z;
  // lane j < K: selection j's expert, weight gradient and probability
  const int my_e = lane < K ? topk_idx[static_cast<size_t>(t) * K + lane] : 0;
  const float my_dw = lane < K ? d_topk_w[static_cast<size_t>(t) * K + lane] : 0.f;
  float my_p = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float v = __shfl(p[q], my_e & 63);
    if ((my_e >> 6) == q) my_p = v;
  }
  if (lane >= K) my_p = 0.f;
  float coef;
  if (norm) {
    float Z = my_p, ws = my_dw * my_p;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      Z += __shfl_xor(Z, off);
      ws += __shfl_xor(ws, off);
    }
    coef = scale / Z * my_dw - scale / (Z * Z) * ws;
  } else {
    coef = scale * my_dw;
  }
  float dp[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < K; ++j) {
    const int ej = __shfl(my_e, j);
    const float cj = __shfl(coef, j);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + 64 * q == ej) dp[q] += cj;
  }
  const float tk = static_cast<float>(T) * static_cast<float>(K);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (d_aux != 0.f && lane + 64 * q < E)
      dp[q] += d_aux * static_cast<float>(E) * (static_cast<float>(cnt[lane + 64 * q]) / tk) /
               static_cast<float>(T);
  float dot = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) dot += p[q] * dp[q];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (lane + 64 * q < E) dl[static_cast<size_t>(t) * E + lane + 64 * q] = p[q] * (dp[q] - dot);
}

// C[M,N] (fp32, row-major) = sum_k A(m,k) B(k,n), A fp32 at A[m*sam + k*sak], B bf16 at
// B[k*sbk + n*sbn]: the router's small products in fp32. 64x64 tiles, K in steps of 16.
__global__ __launch_bounds__(256) void f32_gemm_kernel(const float* __restrict__ A, long sam,
                                                       long sak, const uint16_t* __restrict__ B,
                                                       long sbk, long sbn, int M, int N, int K,
                                                       float* __restrict__ C) {
  __shared__ float As[16][65], Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = threadIdx.x; i < 16 * 64; i += 256) {
      const int kk = i >> 6, o = i & 63;
      const int k = k0 + kk;
      As[kk][o] = (k < K && m0 + o < M) ? A[(m0 + o) * sam + k * sak] : 0.f;
      Bs[kk][o] = (k < K && n0 + o < N) ? bf16_to_f32(B[k * sbk + (n0 + o) * sbn]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] += As[kk][ty * 4 + a] * Bs[kk][tx * 4 + b];
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int m = m0 + ty * 4 + a, n = n0 + tx * 4 + b;
      if (m < M && n < N) C[static_cast<size_t>(m) * N + n] = acc[a][b];
    }
}

// dx[t] = bf16( sum_j dx_row(t,j) (slot order, kept slots) + dx_shared[t] + dx_router[t] ).
__global__ __launch_bounds__(256) void dx_sum_kernel(const uint16_t* __restrict__ dx_rows,
                                                     const float* __restrict__ dx_router,
                                                     const int32_t* __restrict__ slot_to_row,
                                                     int n_ident, int T, int K, int H,
                                                     uint16_t* __restrict__ dx) {
  const int chunks = H / 8;
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long>(T) * chunks) return;
  const int t = static_cast<int>(idx / chunks), c = static_cast<int>(idx % chunks) * 8;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint16_t* row) {
    const u32x4_t v = ld16(row + c);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      s[2 * d] += bf16_to_f32(static_cast<uint16_t>(v[d] & 0xffffu));
      s[2 * d + 1] += bf16_to_f32(static_cast<uint16_t>(v[d] >> 16));
    }
  };
  for (int j = 0; j < K; ++j) {
    const int r = slot_to_row[static_cast<size_t>(t) * K + j];
    if (r >= 0) add(dx_rows + static_cast<size_t>(n_ident + r) * H);
  }
  if (n_ident > 0) add(dx_rows + static_cast<size_t>(t) * H);
  const float* dr = dx_router + static_cast<size_t>(t) * H + c;
  u32x4_t o;
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(s[2 * d] + dr[2 * d], s[2 * d + 1] + dr[2 * d + 1]);
  *reinterpret_cast<u32x4_t*>(dx + static_cast<size_t>(t) * H + c) = o;
}

template <int MODE>
hipError_t gemm(const GemmP& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_gemm_kernel<MODE>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int backward_tile_rows() { return kBM; }

hipError_t launch_layer_backward(const BwdProblem& b, hipStream_t stream) {
  const moe_shape& s = b.s;
  const int T = s.T, H = s.H, E = s.E, K = s.K, I = s.I;
  const int n_ident = b.shared ? T : 0;
  const int G = E + (b.shared ? 1 : 0);
  const int rows_max = n_ident + T * K;
  if (H % kBN || I % 64 || (2 * I) % kBM || H % kBM || G > 1024) return hipErrorInvalidValue;
  hipError_t e;
  // 1. combine backward
  hipLaunchKernelGGL(combine_bwd_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, b.dout,
                     b.topk_w, b.slot_to_row, b.y, n_ident, T, K, H, b.dy, b.d_topk_w);
  // 2. tile table of 128-row tiles over the groups
  const int max_tiles = max_tiles_for(rows_max, G, kBM);
  if ((e = launch_build_tiles(b.grp_offsets, G, kBM, max_tiles, b.tiles, stream)) != hipSuccess) return e;
  GemmP p{};
  p.offsets = b.grp_offsets;
  p.g_split = b.shared ? 1 : 0;
  p.tiles = b.tiles;
  p.max_tiles = max_tiles;
  p.gather = b.row_to_slot;
  p.n_ident = n_ident;
  p.topk = K;
  p.rows_max = rows_max;
  p.H = H;
  p.I = I;
  p.x = b.x;
  p.dy = b.dy;
  p.h = b.h;
  p.dh = b.dh;
  p.dgu = b.dgu;
  p.wg_a = b.s_gate;
  p.wu_a = b.s_up;
  p.wd_a = b.s_down;
  p.wg_b = b.w_gate;
  p.wu_b = b.w_up;
  p.wd_b = b.w_down;
  p.gwg_a = b.d_s_gate;
  p.gwu_a = b.d_s_up;
  p.gwd_a = b.d_s_down;
  p.gwg_b = b.d_w_gate;
  p.gwu_b = b.d_w_up;
  p.gwd_b = b.d_w_down;
  p.limit = s.swiglu_limit;
  // 3. dh = dy Wd;  4. dg, du with g, u recomputed;  5. dx rows = dg Wg + du Wu
  p.out16 = b.dh;
  if ((e = gemm<kDh>(p, dim3(max_tiles, I / kBN), stream)) != hipSuccess) return e;
  p.out16 = b.dgu;
  if ((e = gemm<kGu>(p, dim3(max_tiles, 2 * I / kBN), stream)) != hipSuccess) return e;
  p.out16 = b.dx_rows;
  if ((e = gemm<kDx>(p, dim3(max_tiles, H / kBN), stream)) != hipSuccess) return e;
  // 6. weight gradients, one output per group (zero for a group without rows)
  if ((e = gemm<kWd>(p, dim3(H / kBM, I / kBN, G), stream)) != hipSuccess) return e;
  if ((e = gemm<kWgu>(p, dim3(2 * I / kBM, H / kBN, G), stream)) != hipSuccess) return e;
  // 7. router: selections per expert, logit gradients, dWr = dl^T x, dx_router = dl Wr
  hipLaunchKernelGGL(zero_i32_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, b.cnt, E);
  hipLaunchKernelGGL(count_kernel, dim3((T * K + 255) / 256), dim3(256), 0, stream, b.topk_idx,
                     T * K, E, b.cnt);
  hipLaunchKernelGGL(router_bwd_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, b.logits,
                     b.topk_idx, b.d_topk_w, b.cnt, T, E, K, s.norm_topk_prob, s.routed_scaling,
                     b.d_aux, b.d_logits);
  hipLaunchKernelGGL(f32_gemm_kernel, dim3((H + 63) / 64, (E + 63) / 64), dim3(256), 0, stream,
                     b.d_logits, 1L, static_cast<long>(E), b.x, static_cast<long>(H), 1L, E, H, T,
                     b.d_w_router);
  hipLaunchKernelGGL(f32_gemm_kernel, dim3((H + 63) / 64, (T + 63) / 64), dim3(256), 0, stream,
                     b.d_logits, static_cast<long>(E), 1L, b.w_router, static_cast<long>(H), 1L, T,
                     H, E, b.dx_router);
  // 8. dx
  const long nthr = static_cast<long>(T) * (H / 8);
  hipLaunchKernelGGL(dx_sum_kernel, dim3(static_cast<unsigned>((nthr + 255) / 256)), dim3(256), 0,
                     stream, b.dx_rows, b.dx_router, b.slot_to_row, n_ident, T, K, H, b.d_x);
  return hipGetLastError();
}

}  // namespace moe
