// ffn_kernels.h -- grouped-GEMM kernels of the expert FFN (internal; shared by ffn*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Operands of one grouped projection (gate/up with the SwiGLU epilogue, or down).
struct GroupedParams {
  const uint16_t* A;        // activation rows: x [T, Kd] (gate/up) or h [rows, Kd] (down)
  int32_t a_rows;           // rows of A (bounds the gathered row index)
  const int32_t* gather;    // row_to_slot
  int32_t n_ident;          // rows below this read A row r itself
  int32_t topk;
  int32_t rows_max;         // output rows; no row at or beyond it is read or written
  const int32_t* offsets;   // [G+1]
  const int32_t* tiles;     // tile table
  int32_t max_tiles;
  const uint16_t* W0a;      // gate (gated) or down weights for groups < g_split
  const uint16_t* W0b;      // ... for groups >= g_split
  const uint16_t* W1a;      // up weights (gated only)
  const uint16_t* W1b;
  // FP8 weights (the weight-streaming kernel's W8 form): E4M3 codes laid out like W*, and one fp32
  // scale per weight row (Sa: [N] for groups < g_split, Sb: [groups, N] for the others)
  const uint8_t* Q0a;
  const uint8_t* Q0b;
  const uint8_t* Q1a;
  const uint8_t* Q1b;
  const float* S0a;
  const float* S0b;
  const float* S1a;
  const float* S1b;
  int32_t g_split;
  uint16_t* out;            // [rows, N] bf16
  float* out_f32;           // [rows, N] fp32 (router logits); with k_splits > 1, k_splits such planes
  int32_t k_splits;         // dense mode only: the reduction is split into this many K ranges (0 = 1)
  int32_t N;                // output columns (I for gate/up, H for down)
  int32_t Kd;               // reduction length (H for gate/up, I for down)
  float limit;
  const uint16_t* dh;       // kEpiSwigluBwd: [rows, N] bf16 gradient of h
  // dense mode with per-split K ranges (weight gradients): split s reduces K-tiles
  // [k_tiles[2s], k_tiles[2s] + k_tiles[2s+1]) into its own fp32 output plane; planes of
  // splits >= g_split go to out_f32_b (at split - g_split)
  const int32_t* k_tiles;
  float* out_f32_b;
  // FP8 activations (W8A8): A holds E4M3 codes, one fp32 scale per A row (indexed like A's rows)
  const float* a_scale;
  // kEpiBf16T: the weights are stored [Kd][N] (N contiguous). Rows k < k_w0 of a group's weight
  // are row k of its W0* matrix ([k_w0][N] per group), the others row k - k_w0 of its W1*
  // matrix ([Kd - k_w0][N] per group). A multiple of 64.
  int32_t k_w0;
  // kEpiSwigluSave: [rows, 2N] fp32, the gate sums in columns [0, N) and the up sums in [N, 2N)
  float* gu;
  // MX block scales (kEpiSwigluMx / kEpiBf16Mx and the skinny kernel's MX form), one E8M0 byte
  // per 32 codes along K. Weights: like Q*, one [K/128][N][4] array per matrix (K in codes), the
  // *b arrays stacked per group. Activations: planes [K/128][a_mx_rows][4] indexed by GEMM row.
  const uint8_t* X0a;
  const uint8_t* X0b;
  const uint8_t* X1a;
  const uint8_t* X1b;
  const uint8_t* a_mx;
  int32_t a_mx_rows;
  // kEpiSwigluMx, when mx_hq is set: h also leaves the epilogue MX-quantised, as codes
  // [rows, N] and scale bytes in planes [N/128][mx_h_rows][4] by row (the down GEMM's a_mx)
  uint8_t* mx_hq;
  uint8_t* mx_hs;
  int32_t mx_h_rows;
};


// Weight-streaming kernel for few rows per group (ffn_skinny.hip): row tiles of kSkinnyRows, or
// of kSkinnyRowsSmall when the groups hold at most that many rows on average (decode): a
// narrower tile lets the kernel run at a higher occupancy, at the price of re-reading the weights
// of a group once per extra tile.
constexpr int kSkinnyRows = 64;
constexpr int kSkinnyRowsSmall = 16;
// gated: gate/up + SwiGLU over N = I columns (64 per workgroup); else down (128 per workgroup).
// w8: the weights are the FP8 Q*/S* operands. a8 (with w8): A holds E4M3 codes [rows, Kd] with
// one fp32 scale per row in a_scale.
// mx (with a8): MX block scales (X*, a_mx) in place of the per-row ones.
hipError_t launch_skinny(bool gated, bool w8, bool a8, const GroupedParams& p, int max_tiles,
                         int tile_rows, hipStream_t stream, bool mx = false);

// LDS-tiled MFMA kernel for many rows per group (ffn_tiled.hip): row tiles of kTiledRows.
constexpr int kTiledRows = 320;
// kEpiSwigluBwd: gate/up recomputed for the backward pass; with dh it writes dg and du
// (the clamped SwiGLU's derivative) into out [rows, 2N] as [dg | du].
// kEpiSwiglu8 / kEpiBf16_8: kEpiSwiglu / kEpiBf16 with FP8 weights (the Q* codes and S* row
// scales of GroupedParams).
// kEpiSwiglu88 / kEpiBf16_88: FP8 weights and FP8 activations (W8A8): A and W0*/W1* hold E4M3
// codes, Kd counts pairs of codes (K / 2, so the byte tiles move exactly as bf16 tiles do), the
// products run on the FP8 MFMA, and the S* weight-row scales times a_scale of the row multiply
// the fp32 sums.
// kEpiBf16T: kEpiBf16 over weights stored with the output columns contiguous ([Kd][N], see
// k_w0), as the data gradients of the backward pass read them: out = A W. The weight tile lands
// in LDS as it lies in memory and the MFMA operands are read from it with the LDS transpose read.
// kEpiSwigluSave: kEpiSwiglu that also stores the fp32 gate and up sums (gu), which the
// backward pass then reads instead of recomputing them.
// kEpiSwigluMx / kEpiBf16Mx: the W8A8 forms with MX block scales (X*, a_mx) in place of the
// per-row ones: each MFMA applies the E8M0 scales of its 32-code blocks, so the fp32 sums need
// no scale in the epilogue.
enum Epilogue { kEpiSwiglu = 0, kEpiBf16 = 1, kEpiF32 = 2, kEpiSwigluBwd = 3, kEpiSwiglu8 = 4,
                kEpiBf16_8 = 5, kEpiSwiglu88 = 6, kEpiBf16_88 = 7, kEpiBf16T = 8,
                kEpiSwigluSave = 9, kEpiSwigluMx = 10, kEpiBf16Mx = 11 };
hipError_t launch_tiled(Epilogue epi, const GroupedParams& p, int max_tiles, hipStream_t stream);

}  // namespace moe
