// ffn_skinny.hip -- weight-streaming grouped SwiGLU FFN kernel for few rows per expert.
//
// Hy3 deep-dive (happyrock.cloud) `MoEFeedForward`: y = down(silu(gate x) * up x), bias-free
// projections; Hy4 config walkthrough (lshu.cn), section "MoE routed experts": swiglu_limit
// clamps the gate and up pre-activations, hidden_act silu.
//
// Row tiles of up to 64 rows (MFMA 16x16x32 in 16-row sub-blocks; only the occupied sub-blocks
// are computed). Each wavefront owns 16 output columns of the gate AND the up projection (so the
// SwiGLU epilogue pairs them in registers), or 32 columns of the down projection. Weight
// fragments come straight from HBM into registers, each load instruction reading whole 128-byte
// lines of 8 weight rows non-temporally, and a DPP row rotate moves every chunk to the lane whose
// MFMA operand holds it: at a few rows per expert (decode) the layer is a weight stream and this
// kernel runs at HBM speed.
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

// Weight loads bypass cache retention: each weight line is read once per launch.
constexpr bool kWeightNT = true;

__device__ __forceinline__ u32x4_t ldw(const uint8_t* p) {
  const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
  if (kWeightNT) return __builtin_nontemporal_load(q);
  return *q;
}

// One 128-byte line of each of a fragment's 16 weight rows, as two loads: L0 (this lane's chunk
// in fragment rows 0-7) and L1 (rows 8-15, hoff bytes on).
struct LineRaw {
  u32x4_t l0, l1;
};

__device__ __forceinline__ LineRaw load_line(const uint8_t* p, size_t hoff) {
  return LineRaw{ldw(p), ldw(p + hoff)};
}

// Hands every lane r (= lane % 16) its own row's chunks G (f0) and G + 4 (f1). Lanes r < 8 of a
// 16-lane row hold their chunk G in L0 and receive chunk G + 4 from lane r + 8's L0; lanes r >= 8
// hold chunk G + 4 in L1 and receive chunk G from lane r - 8's L1. row_ror:8 (DPP control 0x128)
// pairs r with r + 8 mod 16; the bank mask picks the receiving half (banks 0-1: r < 8, banks 2-3:
// r >= 8).
__device__ __forceinline__ void exchange_line(const LineRaw& w, u32x4_t& f0, u32x4_t& f1) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f0[d] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        static_cast<int>(w.l0[d]), static_cast<int>(w.l1[d]), 0x128, 0xF, 0xC, false));
    f1[d] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        static_cast<int>(w.l1[d]), static_cast<int>(w.l0[d]), 0x128, 0xF, 0x3, false));
  }
}

template <bool GATED, int NS, bool W8, bool A8, bool MX = false>
__device__ __forceinline__ void skinny_tile(const GroupedParams& p, int g, int r0, int r1,
                                            int col0) {
  static_assert(!A8 || W8, "FP8 activations come with FP8 weights");
  static_assert(!MX || A8, "MX block scales come with FP8 activations");
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15;
  const int lk = W8 ? (lane >> 4) * 16 : (lane >> 4) * 8;  // this lane's first K element
  const int Kd = p.Kd;

  // activation row of tile row r (identity rows first, then gathered tokens); -1 if malformed
  auto source = [&](int r) {
    const int src = r < p.n_ident ? r : p.gather[r - p.n_ident] / p.topk;
    return static_cast<unsigned>(src) < static_cast<unsigned>(p.a_rows) ? src : -1;
  };
  // lanes of rows past the tile load the tile's first row (a segment the same instruction
  // already reads) and mask it to zero, rather than a fixed row that every workgroup would hit
  const int src0 = max(source(r0), 0);
  const uint16_t* ap[NS];
  const uint8_t* ap8[NS];  // A8: this lane's codes of each row (lk is then a byte offset too)
  bool av[NS];
  u32x4_t am[NS];  // all ones for rows of the tile, zero past it
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int r = r0 + 16 * s + lr;
    av[s] = r < r1;
    int src = src0;
    if (av[s]) {
      src = source(r);
      if (src < 0) {  // malformed gather
        av[s] = false;
        src = src0;
      }
    }
    ap[s] = p.A + static_cast<size_t>(src) * Kd + lk;
    ap8[s] = reinterpret_cast<const uint8_t*>(p.A) + static_cast<size_t>(src) * Kd + lk;
    const uint32_t m = av[s] ? ~0u : 0u;
    am[s] = u32x4_t{m, m, m, m};
  }

  // Weight fragments. Each 16-row B fragment is read in 128-byte lines: load L0 covers rows 0-7
  // of the fragment, load L1 rows 8-15, every row with one whole line (lanes r and r + 8 of each
  // 16-lane row take its 16-byte chunks G and G + 4, G = lane / 16). A rotate by 8 inside each
  // 16-lane row then hands every lane r its own row's chunks G and G + 4, which is what MFMA
  // operands u (even) and u + 1 need. Whole-line loads let the weights stream non-temporally.
  const int lo8 = lr & 7;
  const size_t rowb = W8 ? static_cast<size_t>(Kd) : 2 * static_cast<size_t>(Kd);  // row bytes
  const size_t wst = static_cast<size_t>(p.N) * rowb;                            // matrix bytes
  const size_t cb = 16 * ((lane >> 4) + 4 * (lr >> 3));
  const uint8_t* M0;
  const uint8_t* M1;
  if (W8) {
    M0 = g < p.g_split ? p.Q0a + g * wst : p.Q0b + (g - p.g_split) * wst;
    M1 = GATED ? (g < p.g_split ? p.Q1a + g * wst : p.Q1b + (g - p.g_split) * wst) : M0;
  } else {
    const uint8_t* W0a = reinterpret_cast<const uint8_t*>(p.W0a);
    const uint8_t* W0b = reinterpret_cast<const uint8_t*>(p.W0b);
    M0 = g < p.g_split ? W0a + g * wst : W0b + (g - p.g_split) * wst;
    M1 = M0;
    if (GATED) {
      const uint8_t* W1a = reinterpret_cast<const uint8_t*>(p.W1a);
      const uint8_t* W1b = reinterpret_cast<const uint8_t*>(p.W1b);
      M1 = g < p.g_split ? W1a + g * wst : W1b + (g - p.g_split) * wst;
    }
  }
  // this lane's L0 address in the fragment of gate (or down columns col0..) and of up (or down
  // columns col0 + 16..); L1 is 8 rows further
  const uint8_t* w0 = M0 + static_cast<size_t>(col0 + lo8) * rowb + cb;
  const uint8_t* w1 = M1 + static_cast<size_t>(GATED ? col0 + lo8 : col0 + 16 + lo8) * rowb + cb;
  const size_t hoff = 8 * rowb;
  // MX: this lane's weight-scale dwords (4 E8M0 bytes per 128-code K-tile) of its gate (or down
  // column col0 + lr) row and its up (or down column col0 + 16 + lr) row, planes of N dwords
  const uint32_t* xs0 = nullptr;
  const uint32_t* xs1 = nullptr;
  if constexpr (MX) {
    const size_t xst = static_cast<size_t>(Kd / 128) * p.N;  // dwords per matrix
    const uint32_t* X0 = reinterpret_cast<const uint32_t*>(g < p.g_split ? p.X0a : p.X0b) +
                         (g < p.g_split ? g : g - p.g_split) * xst;
    const uint32_t* X1 = GATED ? reinterpret_cast<const uint32_t*>(g < p.g_split ? p.X1a : p.X1b) +
                                     (g < p.g_split ? g : g - p.g_split) * xst
                               : X0;
    xs0 = X0 + col0 + lr;
    xs1 = X1 + (GATED ? col0 + lr : col0 + 16 + lr);
  }

  f32x4_t acc0[NS], acc1[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    acc0[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc1[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  constexpr int U = 4;
  // one iteration covers 128 K elements: two 128-byte lines of each bf16 weight row, one line of
  // each FP8 row
  // The next iteration's weight lines are loaded before this iteration's MFMAs (the last
  // iteration reloads its own lines, which stay in bounds and go unused).
  constexpr int LN = W8 ? 1 : 2;
  constexpr size_t KB = W8 ? 128 : 256;  // weight bytes per row and iteration
  LineRaw r0w[LN], r1w[LN];
#pragma unroll
  for (int ln = 0; ln < LN; ++ln) {
    r0w[ln] = load_line(w0 + 128 * ln, hoff);
    r1w[ln] = load_line(w1 + 128 * ln, hoff);
  }
  uint32_t c0s = 0, c1s = 0;  // MX: the current K-tile's weight-scale dwords
  if constexpr (MX) {
    c0s = xs0[0];
    c1s = xs1[0];
  }
  for (int k = 0; k < Kd; k += 128) {
    const size_t kb = W8 ? static_cast<size_t>(k) : 2 * static_cast<size_t>(k);
    const size_t kn = k + 128 < Kd ? kb + KB : kb;
    LineRaw n0w[LN], n1w[LN];
#pragma unroll
    for (int ln = 0; ln < LN; ++ln) {
      n0w[ln] = load_line(w0 + kn + 128 * ln, hoff);
      n1w[ln] = load_line(w1 + kn + 128 * ln, hoff);
    }
    uint32_t n0s = 0, n1s = 0;  // MX: the next K-tile's weight-scale dwords
    if constexpr (MX) {
      const size_t kt1 = static_cast<size_t>(k + 128 < Kd ? k / 128 + 1 : k / 128) * p.N;
      n0s = xs0[kt1];
      n1s = xs1[kt1];
    }
    // MX: chunk G of a row is block G / 2 of the K-tile, chunk G + 4 block 2 + G / 2
    const int gb = (lane >> 4) >> 1;
    // activations at the same K elements as the weight operands of MFMA u; rows past the tile
    // read a valid row and are masked to zero, so the loads need no branch
    u32x4_t aa[NS][U];
    if (MX) {  // as A8, each 16-code chunk decoded with its block's scale byte
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int r = av[s] ? r0 + 16 * s + lr : r0;
        const uint32_t sd = reinterpret_cast<const uint32_t*>(p.a_mx)[static_cast<size_t>(k / 128) * p.a_mx_rows + r];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4_t t = *reinterpret_cast<const u32x4_t*>(ap8[s] + k + 64 * c);
          const uint32_t sb = sd >> (8 * (gb + 2 * c));
          aa[s][2 * c] = e4m3x8_to_bf16_mx(t[0], t[1], sb) & am[s];
          aa[s][2 * c + 1] = e4m3x8_to_bf16_mx(t[2], t[3], sb) & am[s];
        }
      }
    } else if (A8) {  // 16 codes per load: elements 16g + 64c + [0, 16) feed MFMAs 2c and 2c + 1
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4_t t = *reinterpret_cast<const u32x4_t*>(ap8[s] + k + 64 * c);
          aa[s][2 * c] = e4m3x8_to_bf16(t[0], t[1]) & am[s];
          aa[s][2 * c + 1] = e4m3x8_to_bf16(t[2], t[3]) & am[s];
        }
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int ko = W8 ? 64 * (u >> 1) + 8 * (u & 1) : 32 * u;
          const u32x4_t t = ld16(ap[s] + k + ko);
          aa[s][u] = t & am[s];
        }
    }
    u32x4_t f0[2 * LN], f1[2 * LN];  // [2 * line + half]: chunk G (half 0) or G + 4 (half 1)
#pragma unroll
    for (int ln = 0; ln < LN; ++ln) {
      exchange_line(r0w[ln], f0[2 * ln], f0[2 * ln + 1]);
      exchange_line(r1w[ln], f1[2 * ln], f1[2 * ln + 1]);
      r0w[ln] = n0w[ln];
      r1w[ln] = n1w[ln];
    }
    u32x4_t bb0[U], bb1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (MX) {  // chunk half u/2 is block gb + 2 (u/2) of the K-tile
        const u32x4_t& c = f0[u >> 1];
        const u32x4_t& d = f1[u >> 1];
        const int sh = 8 * (gb + 2 * (u >> 1));
        bb0[u] = e4m3x8_to_bf16_mx(c[2 * (u & 1)], c[2 * (u & 1) + 1], c0s >> sh);
        bb1[u] = e4m3x8_to_bf16_mx(d[2 * (u & 1)], d[2 * (u & 1) + 1], c1s >> sh);
      } else if (W8) {  // MFMA u takes codes 8(u%2)..+8 of chunk half u/2
        const u32x4_t& c = f0[u >> 1];
        const u32x4_t& d = f1[u >> 1];
        bb0[u] = e4m3x8_to_bf16(c[2 * (u & 1)], c[2 * (u & 1) + 1]);
        bb1[u] = e4m3x8_to_bf16(d[2 * (u & 1)], d[2 * (u & 1) + 1]);
      } else {
        bb0[u] = f0[u];
        bb1[u] = f1[u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        acc0[s] = mfma16x16x32(aa[s][u], bb0[u], acc0[s]);
        acc1[s] = mfma16x16x32(aa[s][u], bb1[u], acc1[s]);
      }
    if constexpr (MX) {
      c0s = n0s;
      c1s = n1s;
    }
  }

  // FP8: per-row weight scales of this lane's two output columns
  float sc0 = 1.f, sc1 = 1.f;
  if (W8 && !MX) {
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
        float a0 = W8 ? acc0[s][v] * sc0 : acc0[s][v];
        float a1 = W8 ? acc1[s][v] * sc1 : acc1[s][v];
        if (A8 && !MX) {  // the activation row's scale (rows of the tile hold their own source row)
          const int sr = source(r);
          const float sa = sr >= 0 ? p.a_scale[sr] : 0.f;
          a0 *= sa;
          a1 *= sa;
        }
        if (GATED) {
          o[col0 + lr] = f32_to_bf16(clamped_swiglu(a0, a1, p.limit));
        } else {
          o[col0 + lr] = f32_to_bf16(a0);
          o[col0 + 16 + lr] = f32_to_bf16(a1);
        }
      }
    }
}

// MAXNS: the most 16-row sub-blocks a tile may hold (the tile table's row tile is 16 * MAXNS).
// The register count follows the largest sub-block count compiled in, so a table of 16-row tiles
// with MAXNS = 1 runs at several times the occupancy of the 64-row form.
template <bool GATED, bool W8, bool A8 = false, int MAXNS = 4, bool MX = false>
__global__ __launch_bounds__(256) void ffn_skinny_kernel(GroupedParams p) {
  const int tile = blockIdx.x;
  if (tile >= p.tiles[0]) return;
  const int g = p.tiles[1 + tile];
  const int r0 = p.tiles[1 + p.max_tiles + tile];
  const int r1 = min(min(r0 + 16 * MAXNS, p.offsets[g + 1]), p.rows_max);
  if (r0 < 0 || r1 <= r0) return;
  const int wave = threadIdx.x >> 6;
  const int col0 = GATED ? blockIdx.y * 64 + wave * 16 : blockIdx.y * 128 + wave * 32;
  switch ((r1 - r0 + 15) >> 4) {
    case 1: skinny_tile<GATED, 1, W8, A8, MX>(p, g, r0, r1, col0); break;
    case 2: if constexpr (MAXNS >= 2) skinny_tile<GATED, 2, W8, A8, MX>(p, g, r0, r1, col0); break;
    case 3: if constexpr (MAXNS >= 3) skinny_tile<GATED, 3, W8, A8, MX>(p, g, r0, r1, col0); break;
    case 4: if constexpr (MAXNS >= 4) skinny_tile<GATED, 4, W8, A8, MX>(p, g, r0, r1, col0); break;
    default: break;
  }
}


}  // namespace

template <int MAXNS>
static void skinny_dispatch(bool gated, bool w8, bool a8, bool mx, const GroupedParams& p, dim3 grid,
                            hipStream_t stream) {
  if (mx && gated)
    hipLaunchKernelGGL((ffn_skinny_kernel<true, true, true, MAXNS, true>), grid, dim3(256), 0, stream, p);
  else if (mx)
    hipLaunchKernelGGL((ffn_skinny_kernel<false, true, true, MAXNS, true>), grid, dim3(256), 0, stream, p);
  else if (a8 && gated)
    hipLaunchKernelGGL((ffn_skinny_kernel<true, true, true, MAXNS>), grid, dim3(256), 0, stream, p);
  else if (a8)
    hipLaunchKernelGGL((ffn_skinny_kernel<false, true, true, MAXNS>), grid, dim3(256), 0, stream, p);
  else if (gated && w8)
    hipLaunchKernelGGL((ffn_skinny_kernel<true, true, false, MAXNS>), grid, dim3(256), 0, stream, p);
  else if (gated)
    hipLaunchKernelGGL((ffn_skinny_kernel<true, false, false, MAXNS>), grid, dim3(256), 0, stream, p);
  else if (w8)
    hipLaunchKernelGGL((ffn_skinny_kernel<false, true, false, MAXNS>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((ffn_skinny_kernel<false, false, false, MAXNS>), grid, dim3(256), 0, stream, p);
}

hipError_t launch_skinny(bool gated, bool w8, bool a8, const GroupedParams& p, int max_tiles,
                         int tile_rows, hipStream_t stream, bool mx) {
  const dim3 grid(max_tiles, gated ? p.N / 64 : p.N / 128);
  if (tile_rows == 16)
    skinny_dispatch<1>(gated, w8, a8, mx, p, grid, stream);
  else
    skinny_dispatch<4>(gated, w8, a8, mx, p, grid, stream);
  return hipGetLastError();
}

}  // namespace moe
