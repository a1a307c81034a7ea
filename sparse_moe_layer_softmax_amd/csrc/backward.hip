// backward.hip -- backward pass of the MoE layer (training).
//
// The router is trained on the pages (Hy3 deep-dive `SparseMoERouter` training branch with its
// load-balancing loss; Hy4 deep-dive `MoERouter` scores noise) but no backward is printed, so
// this differentiates the forward in reverse:
//   combine   dy_row = w_j * dout[t] (bf16); d w_j = <dout[t], y_row>          combine_bwd
//   down      dh = dy Wd (bf16)                                  tiled kernel, Wd as stored
//   SwiGLU    g, u recomputed (x Wg^T, x Wu^T); dg = dh clamp(u) silu'(clamp g) [|g| <= L],
//             du = dh silu(clamp g) [|u| <= L] (bf16)           tiled kernel, backward epilogue
//   gate/up   dx_row = dg Wg + du Wu (bf16)                      tiled kernel, Wg, Wu as stored
//   weights   dWd = dy^T h, dWg = dg^T x, dWu = du^T x (fp32, per expert)
//                                   tiled kernel over row-contiguous (transposed) operands
//   routing   d logits through renormalisation, scaling and softmax, plus the load-balancing
//             loss term (its f held fixed); dWr = dl^T x, dx_router = dl Wr    router_bwd, f32 gemm
//   dx        the token's routed rows in slot order, the shared row, the router term  dx_sum
// The shared expert is group 0 of the grouped products (identity rows), as in the forward.
//
// Every MFMA product runs on the forward's LDS-tiled kernel (ffn_tiled.hip). The data gradients
// read the weights as they are stored (reduction dimension = weight rows) through the kernel's
// LDS transpose-read form. The weight gradients reduce over the rows of each expert: their operands (dy, h,
// [dg | du], the gathered x) are transposed so that each expert's rows form one contiguous,
// 64-aligned K range, and the tiled kernel runs in dense mode with one K range and one fp32
// output matrix per expert (an expert without rows gets zeros).
// Everything runs in a fixed order: no floating-point atomics.
#include <cfloat>

#include "ffn_kernels.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kKT = 64;  // rows per K-tile of the weight gradients (the tiled kernel's K step)

// Weight-gradient operands with the layer rows (their reduction dimension) contiguous:
// dst[c][t * 64 + j] = src[row(r0_t + j)][c] for the rows of K-tile t of the tile table (rows
// past the group's end read as 0), so each group's rows start at a multiple of 64.
// row(r) = r, or with gather the token of layer row r (identity rows first). A workgroup moves
// 64 rows x kKtCols columns (C a multiple of kKtCols) through LDS, 512 bytes of each source row.
constexpr int kKtCols = 256;
__global__ __launch_bounds__(256) void ktile_transpose_kernel(
    const uint16_t* __restrict__ src, int C, const int32_t* __restrict__ tiles, int max_tiles,
    const int32_t* __restrict__ offsets, int rows_max, const int32_t* __restrict__ gather,
    int n_ident, int topk, int ld_dst, uint16_t* __restrict__ dst) {
  // row pitch kKtCols + 2 (129 dwords): the column gathers below hit distinct banks
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][kKtCols + 2];
  const int t = blockIdx.y;
  if (t >= tiles[0]) return;
  const int g = tiles[1 + t], r0 = tiles[1 + max_tiles + t];
  const int r_end = min(offsets[g + 1], rows_max);
  const int c0 = blockIdx.x * kKtCols;
  // in: thread (a, b) moves columns 8b..8b+8 of tile rows a + 8p, p < 8 (16-byte loads)
  const int a = threadIdx.x >> 5, b = threadIdx.x & 31;
#pragma unroll
  for (int pass = 0; pass < 8; ++pass) {
    const int i = pass * 8 + a;
    const int r = r0 + i;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r < r_end) {
      const int sr = gather ? (r < n_ident ? r : gather[r - n_ident] / topk) : r;
      v = ld16(src + static_cast<size_t>(sr) * C + c0 + 8 * b);
    }
    uint32_t* tp = reinterpret_cast<uint32_t*>(&tile[i][8 * b]);
#pragma unroll
    for (int m = 0; m < 4; ++m) tp[m] = v[m];
  }
  __syncthreads();
  // out: thread (o, q) writes elements 8q..8q+8 of output rows (source columns) c0 + o + 32p
  const int q = threadIdx.x & 7, o0 = threadIdx.x >> 3;
#pragma unroll
  for (int pass = 0; pass < 8; ++pass) {
    const int o = pass * 32 + o0;
    u32x4_t w;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      w[m] = static_cast<uint32_t>(tile[8 * q + 2 * m][o]) |
             (static_cast<uint32_t>(tile[8 * q + 2 * m + 1][o]) << 16);
    *reinterpret_cast<u32x4_t*>(dst + static_cast<size_t>(c0 + o) * ld_dst +
                                static_cast<size_t>(t) * kKT + 8 * q) = w;
  }
}

// kt[2g], kt[2g+1]: first K-tile and K-tile count of group g (the tile table's order). One
// workgroup of 256 threads, four consecutive groups per thread (G <= 1024): counts, then an
// exclusive integer scan (lanes by shuffles, wavefronts through LDS).
__global__ __launch_bounds__(256) void group_ktiles_kernel(const int32_t* __restrict__ offsets, int G,
                                                           int32_t* __restrict__ kt) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int c4[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * tid + i;
    c4[i] = g < G ? (offsets[g + 1] - offsets[g] + kKT - 1) / kKT : 0;
    sum += c4[i];
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
    if (g < G) {
      kt[2 * g] = b;
      kt[2 * g + 1] = c4[i];
    }
    b += c4[i];
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

// dg, du (bf16, [rows][2I]: dg in columns [0, I), du in [I, 2I)) from the forward's fp32 gate and
// up sums gu (same layout) and dh [rows][I]; four columns per thread. Rows at or past *rows_dev
// (the layer's row count) are left untouched.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ gu,
                                                         const uint16_t* __restrict__ dh,
                                                         const int32_t* __restrict__ rows_dev,
                                                         int rows_max, int I, float L,
                                                         uint16_t* __restrict__ dgu) {
  const int per_row = I / 4;
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long>(rows_max) * per_row) return;
  const int r = static_cast<int>(idx / per_row), c = static_cast<int>(idx % per_row) * 4;
  if (r >= *rows_dev) return;
  const size_t ld = 2 * static_cast<size_t>(I);
  const f32x4_t g = *reinterpret_cast<const f32x4_t*>(gu + r * ld + c);
  const f32x4_t u = *reinterpret_cast<const f32x4_t*>(gu + r * ld + I + c);
  const uint2 d = *reinterpret_cast<const uint2*>(dh + static_cast<size_t>(r) * I + c);
  const float dhv[4] = {bf16_to_f32(static_cast<uint16_t>(d.x & 0xffffu)),
                        bf16_to_f32(static_cast<uint16_t>(d.x >> 16)),
                        bf16_to_f32(static_cast<uint16_t>(d.y & 0xffffu)),
                        bf16_to_f32(static_cast<uint16_t>(d.y >> 16))};
  float dg[4], du[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) swiglu_bwd(g[q], u[q], dhv[q], L, dg[q], du[q]);
  *reinterpret_cast<uint2*>(dgu + r * ld + c) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
  *reinterpret_cast<uint2*>(dgu + r * ld + I + c) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Selections per expert (integer atomics: exact in any order). Each workgroup counts a chunk of
// kCountChunk selections into an LDS histogram and adds its nonzero bins to cnt, so a skewed
// routing (one expert selected by every token) does not serialise on one global counter.
constexpr int kCountChunk = 4096;
__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ topk_idx, int n,
                                                    int E, int32_t* __restrict__ cnt) {
  __shared__ int32_t hist[1024];  // E <= 1024
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int i0 = blockIdx.x * kCountChunk, i1 = min(n, i0 + kCountChunk);
  for (int i = i0 + threadIdx.x; i < i1; i += blockDim.x) {
    const int e = topk_idx[i];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    if (hist[e]) atomicAdd(&cnt[e], hist[e]);
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

// C[M,N] (fp32, row-major) = sum_k A(m,k) B(k,n): the router's products in fp32. A is fp32 with
// A(m,k) = A[m*lda + k] (AK) or A[k*lda + m]; B is bf16 [K][N] with row pitch ldb (N a multiple of
// 128, ldb of 8). 128x128 tiles, K in steps of 16 through a double-buffered LDS tile. Thread
// (tx, ty) of the 16x16 grid owns rows ty*4 + {0..3} and 64 + ty*4 + {0..3} and columns
// tx*4 + {0..3} and 64 + tx*4 + {0..3}, so each k costs it four 16-byte LDS reads for 64 FMAs.
// Each output sums its k in increasing order. With gridDim.z > 1, workgroup z reduces the K
// range [z*kc, z*kc + kc) into plane z of C (M*N each).
template <bool AK>
__global__ __launch_bounds__(256) void f32_gemm_kernel(const float* __restrict__ A, long lda,
                                                       const uint16_t* __restrict__ B, long ldb,
                                                       int M, int N, int K, int kc,
                                                       float* __restrict__ C) {
  constexpr int TM = 128, TN = 128, BK = 16, PM = TM + 4;  // PM: A rows padded (AK stores)
  __shared__ __attribute__((aligned(16))) float As[2][BK][PM];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK][TN];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int kb = blockIdx.z * kc, ke = min(K, kb + kc);
  C += static_cast<size_t>(blockIdx.z) * M * N;
  // A element i of this thread: AK, 16 lanes read 16 consecutive k of a row; else consecutive
  // lanes read consecutive m of a k-row. B: one 16-byte load of 8 bf16 per thread.
  auto a_mk = [&](int i, int& m, int& k) {
    if (AK) {
      k = tid & 15;
      m = (tid >> 4) + 16 * i;
    } else {
      m = tid & 127;
      k = (tid >> 7) + 2 * i;
    }
  };
  float ra[8];
  u32x4_t rb;
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int m, k;
      a_mk(i, m, k);
      const int gm = m0 + m, gk = k0 + k;
      ra[i] = gm < M && gk < ke ? (AK ? A[gm * lda + gk] : A[gk * lda + gm]) : 0.f;
    }
    const int gk = k0 + (tid >> 4);
    rb = gk < ke ? ld16(B + gk * ldb + n0 + (tid & 15) * 8) : u32x4_t{0u, 0u, 0u, 0u};
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int m, k;
      a_mk(i, m, k);
      As[buf][k][m] = ra[i];
    }
    float* bp = &Bs[buf][tid >> 4][(tid & 15) * 8];
    f32x4_t lo, hi;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      lo[2 * q] = bf16_to_f32(static_cast<uint16_t>(rb[q] & 0xffffu));
      lo[2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(rb[q] >> 16));
      hi[2 * q] = bf16_to_f32(static_cast<uint16_t>(rb[q + 2] & 0xffffu));
      hi[2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(rb[q + 2] >> 16));
    }
    *reinterpret_cast<f32x4_t*>(bp) = lo;
    *reinterpret_cast<f32x4_t*>(bp + 4) = hi;
  };
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;
  if (nk > 0) {
    load(kb);
    store(0);
  }
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    const int cur = t & 1;
    if (t + 1 < nk) load(kb + (t + 1) * BK);
#pragma unroll 2
    for (int kk = 0; kk < BK; ++kk) {
      const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(&As[cur][kk][ty * 4]);
      const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(&As[cur][kk][64 + ty * 4]);
      const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(&Bs[cur][kk][tx * 4]);
      const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(&Bs[cur][kk][64 + tx * 4]);
      const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    // the other buffer was last read in step t - 1, which every thread finished before the
    // barrier that ended it
    if (t + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + (i < 4 ? ty * 4 + i : 64 + ty * 4 + i - 4);
    if (m >= M) continue;
    float* c = C + static_cast<size_t>(m) * N + n0 + tx * 4;
    *reinterpret_cast<f32x4_t*>(c) = f32x4_t{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    *reinterpret_cast<f32x4_t*>(c + 64) = f32x4_t{acc[i][4], acc[i][5], acc[i][6], acc[i][7]};
  }
}

// out[i] = sum over the S planes in order (plane stride n).
__global__ __launch_bounds__(256) void sum_planes_kernel(const float* __restrict__ part, int S,
                                                         long n, float* __restrict__ out) {
  const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = part[i];
  for (int z = 1; z < S; ++z) s += part[z * n + i];
  out[i] = s;
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

}  // namespace

hipError_t launch_layer_backward(const BwdProblem& b, hipStream_t stream) {
  const moe_shape& s = b.s;
  const int T = s.T, H = s.H, E = s.E, K = s.K, I = s.I;
  const int n_ident = b.shared ? T : 0;
  const int G = E + (b.shared ? 1 : 0);
  const int rows_max = n_ident + T * K;
  if (H % 256 || I % 256 || G > 1024) return hipErrorInvalidValue;
  hipError_t e;
  // 1. combine backward
  hipLaunchKernelGGL(combine_bwd_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, b.dout,
                     b.topk_w, b.slot_to_row, b.y, n_ident, T, K, H, b.dy, b.d_topk_w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 2. dh = dy Wd, 3. dg, du with g, u recomputed, 4. dx rows = dg Wg + du Wu: the tiled kernel
  const int mt = max_tiles_for(rows_max, G, kTiledRows);
  if ((e = launch_build_tiles(b.grp_offsets, G, kTiledRows, mt, b.tiles_tiled, stream)) != hipSuccess)
    return e;
  {
    GroupedParams q{};
    q.A = b.dy;
    q.a_rows = rows_max;
    q.n_ident = 0x7fffffff;  // rows are already in layer order
    q.rows_max = rows_max;
    q.offsets = b.grp_offsets;
    q.tiles = b.tiles_tiled;
    q.max_tiles = mt;
    q.W0a = b.s_down;  // Wd [H][I]: the reduction runs over its rows
    q.W0b = b.w_down;
    q.k_w0 = H;
    q.g_split = b.shared ? 1 : 0;
    q.out = b.dh;
    q.N = I;
    q.Kd = H;
    if ((e = launch_tiled(kEpiBf16T, q, mt, stream)) != hipSuccess) return e;
  }
  if (b.gu) {
    // g and u as the forward stored them: dg and du elementwise
    const long n = static_cast<long>(rows_max) * (I / 4);
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       stream, b.gu, b.dh, b.grp_offsets + G, rows_max, I, s.swiglu_limit, b.dgu);
  } else {
    // g and u recomputed by the tiled forward kernel, whose epilogue forms dg and du
    GroupedParams q{};
    q.A = b.x;
    q.a_rows = T;
    q.gather = b.row_to_slot;
    q.n_ident = n_ident;
    q.topk = K;
    q.rows_max = rows_max;
    q.offsets = b.grp_offsets;
    q.tiles = b.tiles_tiled;
    q.max_tiles = mt;
    q.W0a = b.s_gate;
    q.W0b = b.w_gate;
    q.W1a = b.s_up;
    q.W1b = b.w_up;
    q.g_split = b.shared ? 1 : 0;
    q.out = b.dgu;
    q.N = I;
    q.Kd = H;
    q.limit = s.swiglu_limit;
    q.dh = b.dh;
    if ((e = launch_tiled(kEpiSwigluBwd, q, mt, stream)) != hipSuccess) return e;
  }
  {
    GroupedParams q{};
    q.A = b.dgu;
    q.a_rows = rows_max;
    q.n_ident = 0x7fffffff;
    q.rows_max = rows_max;
    q.offsets = b.grp_offsets;
    q.tiles = b.tiles_tiled;
    q.max_tiles = mt;
    q.W0a = b.s_gate;  // reduction rows [0, I): Wg [I][H] against dg, [I, 2I): Wu against du
    q.W0b = b.w_gate;
    q.W1a = b.s_up;
    q.W1b = b.w_up;
    q.k_w0 = I;
    q.g_split = b.shared ? 1 : 0;
    q.out = b.dx_rows;
    q.N = H;
    q.Kd = 2 * I;
    if ((e = launch_tiled(kEpiBf16T, q, mt, stream)) != hipSuccess) return e;
  }
  // 5. weight gradients, one output matrix per group (zero for a group without rows): the
  // operands transposed so that each group's rows are a contiguous, 64-aligned K range, then the
  // tiled kernel in dense mode with one K range and one output plane per group
  {
    const int mtk = max_tiles_for(rows_max, G, kKT);
    const int ldk = mtk * kKT;
    if ((e = launch_build_tiles(b.grp_offsets, G, kKT, mtk, b.ktiles, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(group_ktiles_kernel, dim3(1), dim3(256), 0, stream, b.grp_offsets, G, b.kt);
    auto ktr = [&](const uint16_t* src, int C, const int32_t* gather, uint16_t* dst) {
      hipLaunchKernelGGL(ktile_transpose_kernel, dim3(C / kKtCols, mtk), dim3(256), 0, stream, src, C,
                         b.ktiles, mtk, b.grp_offsets, rows_max, gather, n_ident, K, ldk, dst);
    };
    ktr(b.dy, H, nullptr, b.dyT);
    ktr(b.h, I, nullptr, b.hT);
    ktr(b.dgu, 2 * I, nullptr, b.dguT);
    ktr(b.x, H, b.row_to_slot, b.xgT);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    auto wgrad = [&](const uint16_t* A, int M, const uint16_t* B, int N, float* out_shared,
                     float* out_routed) {
      GroupedParams q{};
      q.A = A;
      q.a_rows = M;
      q.n_ident = 0x7fffffff;
      q.rows_max = M;
      q.tiles = nullptr;  // dense mode
      q.W0a = q.W0b = B;
      q.g_split = b.shared ? 1 : 0;
      q.out_f32 = out_shared;
      q.out_f32_b = out_routed;
      q.N = N;
      q.Kd = ldk;
      q.k_splits = G;
      q.k_tiles = b.kt;
      return launch_tiled(kEpiF32, q, (M + kTiledRows - 1) / kTiledRows, stream);
    };
    if ((e = wgrad(b.dyT, H, b.hT, I, b.d_s_down, b.d_w_down)) != hipSuccess) return e;
    if ((e = wgrad(b.dguT, I, b.xgT, H, b.d_s_gate, b.d_w_gate)) != hipSuccess) return e;
    if ((e = wgrad(b.dguT + static_cast<size_t>(I) * ldk, I, b.xgT, H, b.d_s_up, b.d_w_up)) != hipSuccess)
      return e;
  }
  // 6. router: selections per expert, logit gradients, dWr = dl^T x, dx_router = dl Wr
  hipLaunchKernelGGL(zero_i32_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, b.cnt, E);
  hipLaunchKernelGGL(count_kernel, dim3((T * K + kCountChunk - 1) / kCountChunk), dim3(256), 0,
                     stream, b.topk_idx, T * K, E, b.cnt);
  hipLaunchKernelGGL(router_bwd_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, b.logits,
                     b.topk_idx, b.d_topk_w, b.cnt, T, E, K, s.norm_topk_prob, s.routed_scaling,
                     b.d_aux, b.d_logits);
  const int rs = router_splits(T);
  const int rkc = (T + rs - 1) / rs;
  hipLaunchKernelGGL(f32_gemm_kernel<false>, dim3(H / 128, (E + 127) / 128, rs), dim3(256), 0,
                     stream, b.d_logits, static_cast<long>(E), b.x, static_cast<long>(H), E, H, T,
                     rkc, rs > 1 ? b.router_part : b.d_w_router);
  if (rs > 1) {
    const long n = static_cast<long>(E) * H;
    hipLaunchKernelGGL(sum_planes_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                       0, stream, b.router_part, rs, n, b.d_w_router);
  }
  hipLaunchKernelGGL(f32_gemm_kernel<true>, dim3(H / 128, (T + 127) / 128), dim3(256), 0, stream,
                     b.d_logits, static_cast<long>(E), b.w_router, static_cast<long>(H), T, H, E, E,
                     b.dx_router);
  // 7. dx
  const long nthr = static_cast<long>(T) * (H / 8);
  hipLaunchKernelGGL(dx_sum_kernel, dim3(static_cast<unsigned>((nthr + 255) / 256)), dim3(256), 0,
                     stream, b.dx_rows, b.dx_router, b.slot_to_row, n_ident, T, K, H, b.d_x);
  return hipGetLastError();
}

}  // namespace moe
