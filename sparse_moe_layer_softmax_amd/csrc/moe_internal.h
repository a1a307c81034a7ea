// moe_internal.h -- host-side launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

// ---- router (route.hip)
// Split of the hidden dimension used by the router GEMM (a divisor of H/128).
int route_splits(int T, int H, int E);
// partials: [S, T, E] fp32 scratch. noise ([T,E] fp32, added to the logits) and logits may be
// NULL.
hipError_t launch_route(const moe_shape& s, const uint16_t* x, const uint16_t* w_router,
                        const float* bias, const float* noise, float* logits, float* topk_w,
                        int32_t* topk_idx, float* partials, int S, hipStream_t stream);

// ---- training-side router statistics (router_train.hip)
// Blocks of the partial-sum pass (part_p [n, E] fp32 and part_c [n, E] int32 scratch).
int router_stats_blocks(int T);
hipError_t launch_router_stats(const moe_shape& s, const float* logits, const int32_t* topk_idx,
                               float* part_p, int32_t* part_c, float decay, float* prob_mean,
                               float* load_frac, float* aux_loss, float* ema_counts,
                               float* ema_tokens, hipStream_t stream);

// ---- dispatch (permute.hip)
// Slots handled by one dispatch block, and the number of blocks.
int permute_chunk(int TK);
int permute_blocks(int TK);
// block_counts/block_base: [nblk, E] int32 scratch each.
// ext_offsets (may be NULL): [E+2] = {0, n_ident, n_ident + offsets[0..E]} where n_ident
// rows of identity (shared expert) precede the routed rows; written when n_ident > 0.
hipError_t launch_permute(const moe_shape& s, const int32_t* topk_idx, int32_t* counts,
                          int32_t* offsets, int32_t* row_to_slot, int32_t* slot_to_row,
                          int32_t* block_counts, int32_t* block_base, int32_t* ext_offsets,
                          int n_ident, hipStream_t stream);

// ---- grouped FFN (ffn.hip)
// Tile table: tiles[0] = number of tiles, tiles[1 + i] = group, tiles[1 + max + i] = first row.
size_t tile_table_bytes(int max_tiles);
int max_tiles_for(int rows_max, int n_groups, int bm);
// Tile table of bm-row tiles over the groups of offsets [n_groups + 1] (at most max_tiles).
hipError_t launch_build_tiles(const int32_t* offsets, int n_groups, int bm, int max_tiles,
                              int32_t* tiles, hipStream_t stream);
// Writes {0, rows} into offsets[0..1] (a one-group offsets array on the device).
hipError_t launch_single_group_offsets(int32_t* offsets, int rows, hipStream_t stream);

struct FfnProblem {
  const uint16_t* x;          // [T, H] activations
  int32_t T;
  const int32_t* gather;      // row_to_slot (NULL: no gathered rows)
  int32_t n_ident;            // rows r < n_ident read x row r; others x row gather[r-n_ident]/K
  int32_t topk;               // K
  const int32_t* offsets;     // [G+1] group row offsets on the device
  int32_t n_groups;           // G
  int32_t rows_max;           // bound on offsets[G]
  int32_t g_split;            // groups < g_split take the *_a weights, others *_b
  const uint16_t *gate_a, *gate_b, *up_a, *up_b, *down_a, *down_b;
  // FP8 expert weights (w8): E4M3 codes in place of the bf16 weights above, with one fp32 scale
  // per weight row (scale_* of the *_a weights is [N], of the *_b weights [G - g_split, N]).
  bool w8;
  const uint8_t *qgate_a, *qgate_b, *qup_a, *qup_b, *qdown_a, *qdown_b;
  const float *sgate_a, *sgate_b, *sup_a, *sup_b, *sdown_a, *sdown_b;
  int32_t H, I;
  float limit;
  uint16_t* h;                // [rows_max, I]
  uint16_t* y;                // [rows_max, H]
  int32_t* tiles;             // tile table scratch (tile_table_bytes(max_tiles_for(...)))
  // FP8 activations (a8, with w8): x [T, H] and h [rows_max, I] are quantised per row to E4M3
  // codes (xq, hq) with one fp32 scale per row (sx, sh) before the projection that reads them
  bool a8;
  uint8_t* xq;
  float* sx;
  uint8_t* hq;
  float* sh;
  // MX block scales (mx, with w8 and a8): the weights' E8M0 bytes in place of the fp32 row
  // scales, one [K/128][N][4] array per matrix (xgate_* etc., stacked per group as the codes);
  // x and h quantised per 32-element block into xq / hq with their scale planes xs
  // ([H/128][mx_rows][4]) and hs ([I/128][mx_rows][4]) indexed by GEMM row, mx_rows at least
  // rows_max + kTiledRows. s2r: slot_to_row, which places the x scales of a token's slots.
  bool mx;
  const uint8_t *xgate_a, *xgate_b, *xup_a, *xup_b, *xdown_a, *xdown_b;
  uint8_t* xs;
  uint8_t* hs;
  int32_t mx_rows;
  const int32_t* s2r;
  // bf16 weights only: when set, the gate/up projection also stores its fp32 gate and up sums,
  // [rows_max, 2I] (gate in columns [0, I), up in [I, 2I)), and both projections take the tiled
  // kernel, whatever the rows per group, so that the sums are the ones the backward's recompute
  // would form
  float* gu;
};
// ev (may be NULL): three events recorded after the tile table, the gate/up GEMM and the
// down GEMM (each entry may be NULL).
hipError_t launch_ffn(const FfnProblem& p, hipStream_t stream, hipEvent_t const* ev = nullptr);

// Per-row dynamic E4M3 quantisation (quant.hip): codes [rows, cols], scales [rows]; rows at or
// past *rows_dev (when given) are left untouched. cols a multiple of 8.
hipError_t launch_quant_rows(const uint16_t* v, int rows, int cols, const int32_t* rows_dev,
                             uint8_t* codes, float* scales, hipStream_t stream);
// MX block quantisation (quant.hip): codes [rows, cols] in source row order; one E8M0 byte per
// 32 elements, stored as planes [cols / 128][plane_rows][4] indexed by GEMM row: source row r
// itself (s2r NULL), or for tokens: row t when n_ident > 0 and n_ident + s2r[t*K + k] for each
// kept slot. cols a multiple of 128; rows at or past *rows_dev (when given) are skipped.
hipError_t launch_quant_mx(const uint16_t* v, int rows, int cols, const int32_t* rows_dev,
                           uint8_t* codes, uint8_t* scales, int plane_rows, const int32_t* s2r,
                           int K, int n_ident, hipStream_t stream);

// Dense C[rows, N] (fp32) = A[rows, Kd] . W[N, Kd]^T on the tiled MFMA kernel (router logits
// at large T). Supported when N == 256 and Kd % 64 == 0. The reduction is split into
// dense_gemm_splits(rows, Kd) K ranges so that the launch fills the GPU; split s writes its
// partial sums to out + s*rows*N (fp32, no atomics), and the caller adds the planes in order.
bool dense_gemm_f32_supported(int N, int Kd);
int dense_gemm_splits(int rows, int Kd);
hipError_t launch_dense_gemm_f32(const uint16_t* A, int rows, const uint16_t* W, int N, int Kd,
                                 int splits, float* out, hipStream_t stream);

// ---- backward pass (backward.hip)
struct BwdProblem {
  moe_shape s;
  bool shared;
  // inputs: layer weights and the forward's saved tensors (rows: shared rows first, then the
  // routed rows grouped by expert; grp_offsets = {0, T, T + offsets} or offsets)
  const uint16_t *x, *w_router, *w_gate, *w_up, *w_down, *s_gate, *s_up, *s_down;
  const float *logits, *topk_w;
  const int32_t *topk_idx, *row_to_slot, *slot_to_row, *grp_offsets;
  const uint16_t *h, *y, *dout;
  float d_aux;
  // scratch
  uint16_t *dy, *dh, *dgu, *dx_rows;  // [rows, H], [rows, I], [rows, 2I], [rows, H]
  float* dx_router;                   // [T, H]
  int32_t* cnt;                       // [E]
  int32_t* tiles_tiled;               // tile table of the tiled forward kernel's row tile
  // weight-gradient operands with the rows contiguous (ld = backward_ktile_ld(rows, G)):
  uint16_t *dyT, *hT, *dguT, *xgT;    // [H][ld], [I][ld], [2I][ld], [H][ld]
  int32_t *ktiles, *kt;               // K-tile table of 64-row tiles, [2G] per-group ranges
  float* router_part;
  const float* gu;                    // the forward's fp32 gate/up sums [rows, 2I], or NULL (recompute)                 // [router_splits(T), E, H] fp32 partial planes of dWr
  // outputs
  float *d_topk_w, *d_logits;         // [T, K], [T, E]
  uint16_t* d_x;                      // [T, H]
  float *d_w_router, *d_w_gate, *d_w_up, *d_w_down, *d_s_gate, *d_s_up, *d_s_down;
};
hipError_t launch_layer_backward(const BwdProblem& b, hipStream_t stream);
// Row stride of the transposed weight-gradient operands, and the K-tile table's tile bound.
inline int backward_ktiles(int rows_max, int n_groups) { return max_tiles_for(rows_max, n_groups, 64); }
// The router weight gradient dWr = dlogits^T x reduces over all T tokens with only E/128 x H/128
// output tiles; it is split into this many token ranges of at least 1024 (at most 16), each with
// its own fp32 partial plane, summed in order afterwards.
inline int router_splits(int T) { return T <= 1024 ? 1 : (T + 1023) / 1024 < 16 ? (T + 1023) / 1024 : 16; }

// ---- combine (combine.hip)
hipError_t launch_combine(const moe_shape& s, const uint16_t* y_routed, const float* topk_w,
                          const int32_t* slot_to_row, const uint16_t* y_shared, uint16_t* out,
                          hipStream_t stream);

}  // namespace moe
