/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts FFN layer forward.
 *
 * The layer (Hy4 preview shape: hidden 6144, 256 routed experts, top-8, one always-on shared
 * expert, expert intermediate 2048, routed_scaling_factor 2.827, swiglu_limit 10, silu, bf16):
 *
 *   logits = x Wr^T (+ b)                        router projection
 *   p = softmax(logits); top-k; w = s * p_top / sum(p_top)     routing weights
 *   dispatch (t, j) slots to their experts (stable, optional per-expert capacity)
 *   y_e = Wd_e ( silu(clamp(Wg_e x)) * clamp(Wu_e x) )        SwiGLU expert FFN
 *   out = sum_j w_j y_{e_j} + y_shared                         combine
 *
 * Sources, cited by page title and section:
 *  - "Tencent Hunyuan Hy4 Preview deep technical analysis" (happyrock.cloud): the `MoERouter`
 *    sketch (bias-free linear gate, softmax, top-k) and `MoELayer` (256 routed experts, one
 *    shared expert always run, routed output plus shared output).
 *  - "Tencent Hunyuan Hy3 official release deep analysis" (happyrock.cloud): `SparseMoERouter`
 *    (token flattening, softmax, top-k, renormalisation of the selected probabilities,
 *    capacity_factor) and `MoEFeedForward` (SwiGLU: down(silu(gate x) * up x), no biases).
 *  - "Hy4 preview config.json deep interpretation" (lshu.cn), section "MoE routed experts":
 *    n_routed_experts 256, num_experts_per_tok 8, n_shared_experts 1, moe_intermediate_size
 *    2048, norm_topk_prob true, routed_scaling_factor 2.827, swiglu_limit 10; section
 *    "length, vocabulary and training details": hidden_act silu, dtype bfloat16.
 *  - Hy3 sparse-MoE explainer (tqpw.cn), section 2.1: expert-major dispatch, each expert run on
 *    the rows routed to it, then aggregation.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (HBM), row-major, densely packed. bf16 tensors are
 *    passed as their 16-bit patterns (uint16_t). The `moe_shape` is a HOST pointer.
 *  - The caller owns every buffer, including the workspace. The library never allocates,
 *    frees, synchronises, or reads device memory from the host.
 *  - Each call only enqueues kernels on `stream` (0 = the null stream) and returns; results are
 *    visible after the caller synchronises that stream. Calls are stateless; concurrent calls
 *    on different streams need separate workspaces.
 *  - Every argument check runs on the host before any launch; on error nothing is enqueued.
 *    Faults inside kernels surface at the caller's next synchronisation (HIP convention).
 *  - Inputs must be finite. Results are deterministic: the same inputs give the same bits.
 *  - Supported shapes: 1 <= K <= 16, K <= E <= 256, H and I multiples of 256, T >= 1 with
 *    T*(K+1) < 2^31, and every operand that the LDS-tiled MFMA kernel reads at most 64 GiB
 *    (it addresses rows in 16-byte units with 32-bit offsets): x [T,H], one expert matrix
 *    [I,H], and the layer rows h [T*(K+1), I] (moe_expert_ffn: [rows_max, I]). At the Hy4 shape
 *    that allows T <= 1,864,135. moe_layer_backward also needs dy [rows,H], [dg|du] [rows,2I]
 *    and its row-contiguous copies [H][ld], [2I][ld] (ld about the layer row count plus 64 per
 *    expert) within 64 GiB: T <= 619,548 at the Hy4 shape. Others return MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* NULL required pointer, non-positive size, K > E, ... */
#define MOE_ERR_UNSUPPORTED (-2) /* shape outside the supported set listed above          */
#define MOE_ERR_WORKSPACE (-3)   /* ws_bytes smaller than the matching *_workspace_size     */
#define MOE_ERR_HIP (-4)         /* a kernel launch failed (hipGetLastError)                */
#define MOE_ERR_SCRATCH (-5)     /* moe_layer_forward_noalloc: workspace over its scratch   */

/* Layer shape and constants (Hy4 config walkthrough, section "MoE routed experts"). */
typedef struct moe_shape {
  int32_t T;              /* tokens = batch * sequence (the Hy3 router flattens them)       */
  int32_t H;              /* hidden size (6144)                                              */
  int32_t E;              /* routed experts (256)                                            */
  int32_t K;              /* experts per token, top-k (8)                                    */
  int32_t I;              /* expert intermediate size (2048); the shared expert's too        */
  int32_t n_shared;       /* shared experts: 0 or 1                                          */
  int32_t norm_topk_prob; /* 1: renormalise the k selected probabilities to sum 1            */
  float routed_scaling;   /* s, multiplies every routed weight (2.827); never the shared one */
  float swiglu_limit;     /* L: gate and up pre-activations clamped to [-L, L]; <= 0 = off   */
  int32_t capacity;       /* per-expert capacity C (slots beyond it are dropped); <= 0 = off */
} moe_shape;

/* Human-readable text for a return code (static storage). */
const char* moe_strerror(int code);

/* ---------------------------------------------------------------- router: moe_route
 * Router projection, softmax over the E experts, top-k, renormalisation and routed scaling
 * (Hy4 deep-dive `MoERouter.forward`; Hy3 deep-dive `SparseMoERouter.forward`; Hy4 config
 * walkthrough `norm_topk_prob`, `routed_scaling_factor`).
 *   x        [T,H] bf16           tokens
 *   w_router [E,H] bf16           gate weight in nn.Linear (out, in) layout
 *   bias     [E]   fp32 or NULL   optional additive logit bias (the pages' router has none)
 *   logits   [T,E] fp32 or NULL   out: logits = x w_router^T + bias, fp32 accumulation
 *   topk_w   [T,K] fp32           out: w_j = s * p_j / sum_{i<K} p_i   (s * p_j without renorm)
 *   topk_idx [T,K] int32          out: expert ids by logit descending; equal logits -> lower id
 * Selection compares the fp32 logits (-0.0 == +0.0), so it is exact given the logits.
 * ws: moe_route_workspace_size(shape) bytes, 256-byte aligned.                              */
size_t moe_route_workspace_size(const moe_shape* shape);
int moe_route(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router,
              const float* bias, float* logits, float* topk_w, int32_t* topk_idx, void* ws,
              size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- router, training: moe_route_train
 * moe_route in training mode, plus the router statistics of the training branch.
 *   noise [T,E] fp32 or NULL   added to the logits before the softmax and the top-k (Hy4
 *                               deep-dive `MoERouter`: N(0, 0.01^2) scores noise in training;
 *                               the caller draws it, so runs are reproducible)
 *   logits, topk_w, topk_idx    as in moe_route (logits include the noise; NULL logits are kept
 *                               in the workspace)
 * Statistics (Hy3 deep-dive `SparseMoERouter`, training branch and load-balancing loss):
 *   prob_mean [E] fp32 out      P_e = (1/T) sum_t softmax(logits[t])[e]
 *   load_frac [E] fp32 out      f_e = #{(t,j): topk_idx[t,j] = e} / (T*K), before any capacity
 *   aux_loss  [1] fp32 out      E * sum_e P_e f_e
 *   ema_counts [E] fp32 in/out or NULL   ema_decay * ema + (1 - ema_decay) * count_e
 *   ema_tokens [1] fp32 in/out or NULL   ema_decay * ema + (1 - ema_decay) * T
 *   ema_decay                   in [0, 1] (0.9 on the page), else MOE_ERR_INVALID_ARG
 * Reductions run in a fixed order: the same inputs give the same bits on every run.
 * ws: moe_route_train_workspace_size(shape) bytes, 256-byte aligned.                          */
size_t moe_route_train_workspace_size(const moe_shape* shape);
int moe_route_train(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router,
                    const float* bias, const float* noise, float* logits, float* topk_w,
                    int32_t* topk_idx, float* prob_mean, float* load_frac, float* aux_loss,
                    float* ema_counts, float* ema_tokens, float ema_decay, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- dispatch: moe_permute
 * Token-to-expert dispatch (Hy3 explainer 2.1: the rows of each expert gathered together).
 * A slot is (t, j), id s = t*K + j. Rows are grouped by expert, ascending expert id; inside an
 * expert, ascending slot id (a stable counting sort). With capacity C > 0 only the first C
 * slots of each expert (in slot order) are kept.
 *   topk_idx    [T*K]  int32 in   expert of each slot (0 <= id < E)
 *   counts      [E]    int32 out  kept rows per expert
 *   offsets     [E+1]  int32 out  exclusive prefix sum of counts; offsets[E] = R kept rows
 *   row_to_slot [T*K]  int32 out  slot id of row r for r < R; -1 for R <= r < T*K
 *   slot_to_row [T*K]  int32 out  row of slot s, -1 if dropped
 * ws: moe_permute_workspace_size(shape) bytes.                                              */
size_t moe_permute_workspace_size(const moe_shape* shape);
int moe_permute(const moe_shape* shape, const int32_t* topk_idx, int32_t* counts,
                int32_t* offsets, int32_t* row_to_slot, int32_t* slot_to_row, void* ws,
                size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- experts: moe_expert_ffn
 * Grouped SwiGLU FFN over variable-length row groups (Hy3 deep-dive `MoEFeedForward`; clamp
 * from the Hy4 config walkthrough's swiglu_limit; silu from hidden_act):
 *   for group g and row r in [group_offsets[g], group_offsets[g+1]):
 *     a = x[token(r)],  token(r) = row_to_slot[r] / K   (row_to_slot != NULL)
 *                       token(r) = r                     (row_to_slot == NULL)
 *     h[r] = bf16( silu(clamp(a Wg_g^T, L)) * clamp(a Wu_g^T, L) )     fp32 accumulate
 *     y[r] = bf16( h[r] Wd_g^T )                                        fp32 accumulate
 *   n_groups       G >= 1 (E for the routed experts, 1 for the shared expert)
 *   rows_max       upper bound on group_offsets[G] (T*K routed, T shared); sizes the grid
 *   x              [T,H] bf16
 *   row_to_slot    [rows_max] int32 or NULL (identity: row r is token r, rows_max <= T)
 *   group_offsets  [G+1] int32 on the device, non-decreasing, group_offsets[0] = 0, or NULL
 *                  meaning one group of rows_max rows
 *   w_gate, w_up   [G,I,H] bf16;  w_down [G,H,I] bf16
 *   h              [rows_max,I] bf16 out, or NULL (then kept in the workspace)
 *   y              [rows_max,H] bf16 out; rows >= group_offsets[G] are left untouched
 * ws: moe_expert_ffn_workspace_size(shape, G, rows_max) bytes.                              */
size_t moe_expert_ffn_workspace_size(const moe_shape* shape, int32_t n_groups, int32_t rows_max);
int moe_expert_ffn(const moe_shape* shape, int32_t n_groups, int32_t rows_max,
                   const uint16_t* x, const int32_t* row_to_slot, const int32_t* group_offsets,
                   const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                   uint16_t* h, uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- combine: moe_combine
 * Weighted combine (Hy4 deep-dive `MoELayer.forward`: routed_output + shared_output):
 *   out[t] = bf16( sum_{j<K, slot_to_row[t*K+j] >= 0} topk_w[t,j] * y_routed[slot_to_row[t*K+j]]
 *                  + y_shared[t] )
 * summed in fp32 in slot order j = 0..K-1, the shared row last; no atomics.
 *   y_routed    [R,H] bf16,  topk_w [T,K] fp32,  slot_to_row [T*K] int32
 *   y_shared    [T,H] bf16 or NULL,   out [T,H] bf16                                       */
int moe_combine(const moe_shape* shape, const uint16_t* y_routed, const float* topk_w,
                const int32_t* slot_to_row, const uint16_t* y_shared, uint16_t* out,
                hipStream_t stream);

/* ---------------------------------------------------------------- whole layer
 * moe_route -> moe_permute -> routed + shared expert FFN (one grouped launch per projection,
 * the shared expert is one more group) -> moe_combine, all on `stream`, no host sync.
 *   x [T,H], w_router [E,H], bias [E] fp32 or NULL,
 *   w_gate/w_up [E,I,H], w_down [E,H,I]           routed experts
 *   s_gate/s_up [I,H], s_down [H,I]               shared expert (NULL iff n_shared == 0)
 *   out [T,H] bf16
 * The intermediates stay in the workspace; moe_layer_workspace_layout gives their byte
 * offsets so a caller may read them after the stream completes.
 * ws: moe_layer_workspace_size(shape) bytes, 256-byte aligned.                              */
typedef struct moe_layer_ws_layout {
  size_t logits;      /* [T,E] fp32                                      */
  size_t topk_w;      /* [T,K] fp32                                      */
  size_t topk_idx;    /* [T,K] int32                                     */
  size_t counts;      /* [E] int32                                       */
  size_t offsets;     /* [E+1] int32                                     */
  size_t row_to_slot; /* [T*K] int32                                     */
  size_t slot_to_row; /* [T*K] int32                                     */
  size_t h;           /* [T + T*K, I] bf16: shared rows first, then routed rows */
  size_t y;           /* [T + T*K, H] bf16: same row order as h          */
  size_t total;       /* bytes                                           */
} moe_layer_ws_layout;

size_t moe_layer_workspace_size(const moe_shape* shape);
int moe_layer_workspace_layout(const moe_shape* shape, moe_layer_ws_layout* layout);
int moe_layer_forward(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router,
                      const float* bias, const uint16_t* w_gate, const uint16_t* w_up,
                      const uint16_t* w_down, const uint16_t* s_gate, const uint16_t* s_up,
                      const uint16_t* s_down, uint16_t* out, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* Same as moe_layer_forward, and records caller-created HIP events on `stream` at the phase
 * boundaries below (any entry may be NULL; `phase_events` itself may be NULL). For timing
 * single kernels with hipEventElapsedTime; the computation is identical to moe_layer_forward.
 *   [0] start  [1] after routing  [2] after dispatch  [3] after the tile table
 *   [4] after the gate/up grouped GEMM  [5] after the down grouped GEMM  [6] after combine   */
#define MOE_LAYER_PHASE_EVENTS 7
int moe_layer_forward_profiled(const moe_shape* shape, const uint16_t* x,
                               const uint16_t* w_router, const float* bias,
                               const uint16_t* w_gate, const uint16_t* w_up,
                               const uint16_t* w_down, const uint16_t* s_gate,
                               const uint16_t* s_up, const uint16_t* s_down, uint16_t* out,
                               void* ws, size_t ws_bytes, hipStream_t stream,
                               hipEvent_t const* phase_events);

/* ---------------------------------------------------------------- FP8 expert weights
 * The pages deploy the model from an FP8 checkpoint ("Tencent Hunyuan Hy4 Preview deep
 * technical analysis", deployment commands; Hy4 config walkthrough, dtype notes) but define no
 * weight format. Format used here: each expert weight matrix (routed and shared gate, up, down)
 * is stored as OCP FP8 E4M3 codes (uint8, same [rows, cols] layout as the bf16 weights) plus
 * one fp32 scale per row (output channel); the weight value is scale[row] * e4m3(code). The
 * router weights, activations and every stored intermediate stay bf16 exactly as in the bf16
 * entry points, whose definitions these follow; the codes must not be NaN (0x7F, 0xFF).
 * Each projection is computed as scale[col] * sum_k a[k] * e4m3(code[col,k]) with the products
 * summed in fp32, then rounded where the bf16 path rounds.
 *
 * moe_expert_ffn_fp8: moe_expert_ffn with
 *   w_gate, w_up [G,I,H] E4M3 codes, w_gate_scale, w_up_scale [G,I] fp32,
 *   w_down [G,H,I] E4M3 codes, w_down_scale [G,H] fp32.
 * ws: moe_expert_ffn_workspace_size(shape, G, rows_max) bytes (the same as for bf16).           */
int moe_expert_ffn_fp8(const moe_shape* shape, int32_t n_groups, int32_t rows_max,
                       const uint16_t* x, const int32_t* row_to_slot,
                       const int32_t* group_offsets, const uint8_t* w_gate,
                       const float* w_gate_scale, const uint8_t* w_up, const float* w_up_scale,
                       const uint8_t* w_down, const float* w_down_scale, uint16_t* h,
                       uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward_profiled with FP8 expert weights:
 *   w_gate, w_up [E,I,H] codes + [E,I] scales;  w_down [E,H,I] codes + [E,H] scales
 *   s_gate, s_up [I,H] codes + [I] scales;      s_down [H,I] codes + [H] scales (all NULL iff
 *                                               n_shared == 0)
 * Workspace, layout, outputs and phase_events (may be NULL) as for the bf16 layer.            */
int moe_layer_forward_fp8(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router,
                          const float* bias, const uint8_t* w_gate, const float* w_gate_scale,
                          const uint8_t* w_up, const float* w_up_scale, const uint8_t* w_down,
                          const float* w_down_scale, const uint8_t* s_gate,
                          const float* s_gate_scale, const uint8_t* s_up,
                          const float* s_up_scale, const uint8_t* s_down,
                          const float* s_down_scale, uint16_t* out, void* ws, size_t ws_bytes,
                          hipStream_t stream, hipEvent_t const* phase_events);

/* ---------------------------------------------------------------- FP8 activations too (W8A8)
 * The same FP8 deployment (the pages name an FP8 checkpoint and no format), with the FP8
 * matrix cores doing the products: the activations entering each expert projection are also
 * OCP E4M3, quantised per row on the fly (dynamic, one fp32 scale per row):
 *   amax = max_c |v[c]|,  scale = amax / 448,  code[c] = E4M3_RNE(clamp(v[c] * (448 / amax), +-448))
 * with both divisions correctly rounded fp32 and the product one fp32 multiply; an all-zero row
 * gets scale 1 and zero codes. A projection is then
 *   (sum_k e4m3(a_code[k]) * e4m3(w_code[k])) * w_scale[col] * a_scale[row]
 * with the code products summed in fp32, rounded where the bf16 path rounds (h, y, out).
 *
 * moe_quantize_rows_e4m3: that quantisation on its own.
 *   x [rows, cols] bf16 (16-byte aligned),  codes [rows, cols] uint8 (8-byte aligned),
 *   scales [rows] fp32;  rows >= 1, cols a positive multiple of 8.
 * Returns MOE_ERR_INVALID_ARG for a NULL pointer, bad sizes or bad alignment.              */
int moe_quantize_rows_e4m3(const uint16_t* x, int32_t rows, int32_t cols, uint8_t* codes,
                           float* scales, hipStream_t stream);

/* moe_layer_forward_w8a8: moe_layer_forward_fp8 (same arguments, same outputs) in the W8A8 form:
 * x is quantised once per token (the shared expert reads the same codes) before the gate/up
 * projections, and the h rows once each before the down projections. The router and the
 * combine stay as in the bf16 layer.
 * ws: moe_layer_w8a8_workspace_size(shape) bytes, 256-byte aligned. Its first part has the
 * layout moe_layer_workspace_layout gives; the quantised activations follow at the offsets
 * moe_layer_w8a8_workspace_layout gives, readable after the stream completes.              */
typedef struct moe_layer_a8_ws_layout {
  size_t xq;      /* [T,H] E4M3 codes of x                                        */
  size_t x_scale; /* [T] fp32                                                     */
  size_t hq;      /* [T + T*K, I] E4M3 codes of h, rows as in h (valid rows only) */
  size_t h_scale; /* [T + T*K] fp32                                               */
  size_t total;   /* bytes of the whole workspace                                 */
} moe_layer_a8_ws_layout;

size_t moe_layer_w8a8_workspace_size(const moe_shape* shape);
int moe_layer_w8a8_workspace_layout(const moe_shape* shape, moe_layer_a8_ws_layout* layout);
int moe_layer_forward_w8a8(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router,
                           const float* bias, const uint8_t* w_gate, const float* w_gate_scale,
                           const uint8_t* w_up, const float* w_up_scale, const uint8_t* w_down,
                           const float* w_down_scale, const uint8_t* s_gate,
                           const float* s_gate_scale, const uint8_t* s_up,
                           const float* s_up_scale, const uint8_t* s_down,
                           const float* s_down_scale, uint16_t* out, void* ws, size_t ws_bytes,
                           hipStream_t stream, hipEvent_t const* phase_events);

/* ---------------------------------------------------- MX block-scaled FP8 weights and activations
 * The same FP8 deployment with per-block scales, in the OCP Microscaling (MX v1.0) MXFP8 form
 * that the gfx950 scaled FP8 matrix instructions apply natively: one E8M0 scale byte s (value
 * 2^(s - 127), s = 255 not allowed) per 32 consecutive elements along the reduction dimension,
 * elements OCP E4M3. Scale arrays are K-tile-major: for a matrix [N][K] (K a multiple of 128)
 * the byte of row n, block b is at  ((b / 4) * N + n) * 4 + b % 4,  i.e. [K/128][N][4] (routed
 * experts: E such arrays back to back, like the codes).
 * The activations entering each expert projection are quantised per row and block on the fly:
 *   shared = floor(log2(amax)) - 8 clamped to [-127, 127] (amax: the block's largest |v|; an
 *   all-zero block takes -127), s = shared + 127,  code = E4M3_RNE(clamp(v / 2^shared, +-448)).
 * A projection is sum_k e4m3(a)2^(sa-127) e4m3(w)2^(sw-127) with fp32 accumulation, rounded
 * where the bf16 path rounds (h, y, out). The weight-streaming path (few rows per expert) decodes
 * each code times its scale to bf16, exact for scale bytes 10..245.
 *
 * moe_quantize_rows_mx: that quantisation on its own.
 *   x [rows, cols] bf16 (16-byte aligned), codes [rows, cols] uint8 (8-byte aligned),
 *   scales [cols/128][rows][4] bytes (4-byte aligned); rows >= 1, cols a positive multiple of 128.
 * Returns MOE_ERR_INVALID_ARG for a NULL pointer, bad sizes or bad alignment.
 *
 * moe_layer_forward_mx: moe_layer_forward_fp8 with MX weights (each fp32 scale array replaced by
 * its E8M0 byte array) and MX activations; outputs as moe_layer_forward.
 * ws: moe_layer_mx_workspace_size(shape) bytes, 256-byte aligned. Its first part has the layout
 * moe_layer_workspace_layout gives; the quantised activations follow at the offsets of
 * moe_layer_mx_workspace_layout. Their scales are planes [K/128][scale_rows][4] indexed by the
 * row of the projection's grouped GEMM (shared-expert rows [0, T) first when n_shared = 1, then
 * the routed rows in slot_to_row order).                                                       */
typedef struct moe_layer_mx_ws_layout {
  size_t xq;         /* [T,H] E4M3 codes of x (token order)                              */
  size_t x_scale;    /* [H/128][scale_rows][4] E8M0 bytes of x, by gate/up GEMM row      */
  size_t hq;         /* [T + T*K, I] E4M3 codes of h, rows as in h (valid rows only)     */
  size_t h_scale;    /* [I/128][scale_rows][4] E8M0 bytes of h, by row of h              */
  size_t scale_rows; /* rows of a scale plane: T*K (+ T with a shared expert) + 320       */
  size_t total;      /* bytes of the whole workspace                                     */
} moe_layer_mx_ws_layout;

int moe_quantize_rows_mx(const uint16_t* x, int32_t rows, int32_t cols, uint8_t* codes,
                         uint8_t* scales, hipStream_t stream);
size_t moe_layer_mx_workspace_size(const moe_shape* shape);
int moe_layer_mx_workspace_layout(const moe_shape* shape, moe_layer_mx_ws_layout* layout);
int moe_layer_forward_mx(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router,
                         const float* bias, const uint8_t* w_gate, const uint8_t* w_gate_scale,
                         const uint8_t* w_up, const uint8_t* w_up_scale, const uint8_t* w_down,
                         const uint8_t* w_down_scale, const uint8_t* s_gate,
                         const uint8_t* s_gate_scale, const uint8_t* s_up,
                         const uint8_t* s_up_scale, const uint8_t* s_down,
                         const uint8_t* s_down_scale, uint16_t* out, void* ws, size_t ws_bytes,
                         hipStream_t stream, hipEvent_t const* phase_events);

/* ================================================================ backward pass (training)
 * The routers on the pages are trained (Hy3 deep-dive `SparseMoERouter`: training branch with a
 * load-balancing loss and count EMAs; Hy4 deep-dive `MoERouter`: noise on the scores in
 * training). The pages print no backward; this is the derivative of moe_layer_forward:
 *   combine   dy_row = bf16(w_j dout[t]) for each kept slot; d w_j = <dout[t], y_row>
 *   down      dh = bf16(dy Wd)
 *   SwiGLU    g = x Wg^T, u = x Wu^T in fp32 (stored by moe_layer_forward_train, or recomputed);
 *             dg = bf16(dh clamp(u) silu'(clamp g) [-L <= g <= L]),
 *             du = bf16(dh silu(clamp g) [-L <= u <= L]) (no masks for L <= 0)
 *   gate/up   dx_row = bf16(dg Wg + du Wu)
 *   weights   dWd = dy^T h, dWg = dg^T x, dWu = du^T x per expert (and the shared expert, whose
 *             dy is dout), fp32 sums over the expert's rows; an expert without rows gets zeros
 *   routing   d logits through the renormalisation and routed scaling (top-k choice fixed) and
 *             the softmax, plus d_aux times the gradient of E sum_e P_e f_e with f held fixed
 *             (f counted from the top-k indices, before capacity); dWr = dl^T x (fp32),
 *             dx_router = dl Wr (fp32)
 *   dx        bf16( sum over the token's kept slots in slot order of dx_row, + the shared
 *             row's dx_row, + dx_router )
 * Inputs: the layer's bf16 weights (FP8 weights are not supported here), x, and the workspace
 * of a moe_layer_forward or moe_layer_forward_train call with the same shape and inputs
 * (fwd_ws, its logits, routing, dispatch, h and y are read), d_out [T,H] bf16, d_aux (0 for no
 * loss term). gu: the gate/up sums that moe_layer_forward_train stored (16-byte aligned), or
 * NULL to recompute them; the result is the same either way.
 * Outputs: d_x [T,H] bf16; d_w_router [E,H], d_w_gate/d_w_up [E,I,H], d_w_down [E,H,I] fp32;
 * d_s_gate/d_s_up [I,H], d_s_down [H,I] fp32 (NULL iff n_shared = 0); d_topk_w [T,K] and
 * d_logits [T,E] fp32 or NULL (then kept in the workspace). d_out and d_x 16-byte aligned.
 * Every reduction runs in a fixed order: the same inputs give the same bits on every run.
 * ws: moe_layer_backward_workspace_size(shape) bytes, 256-byte aligned.                        */
typedef struct moe_bwd_ws_layout {
  size_t dy;        /* [T + T*K, H] bf16: output gradient per layer row (shared rows first)  */
  size_t dh;        /* [T + T*K, I] bf16                                                       */
  size_t dgu;       /* [T + T*K, 2I] bf16: dg in columns [0, I), du in [I, 2I)                 */
  size_t dx_rows;   /* [T + T*K, H] bf16: per-row input gradient                               */
  size_t dx_router; /* [T, H] fp32                                                             */
  size_t d_topk_w;  /* [T, K] fp32 (used when the caller passes no d_topk_w)                   */
  size_t d_logits;  /* [T, E] fp32 (used when the caller passes no d_logits)                   */
  size_t total;     /* bytes                                                                   */
} moe_bwd_ws_layout;
size_t moe_layer_backward_workspace_size(const moe_shape* shape);
int moe_layer_backward_workspace_layout(const moe_shape* shape, moe_bwd_ws_layout* layout);
int moe_layer_backward(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router,
                       const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                       const uint16_t* s_gate, const uint16_t* s_up, const uint16_t* s_down,
                       const void* fwd_ws, size_t fwd_ws_bytes, const float* gu,
                       const uint16_t* d_out, float d_aux, uint16_t* d_x, float* d_w_router,
                       float* d_w_gate, float* d_w_up, float* d_w_down, float* d_s_gate,
                       float* d_s_up, float* d_s_down, float* d_topk_w, float* d_logits, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It takes no workspace: the
 * layer's workspace lives in a static device array of moe_layer_noalloc_scratch_bytes() bytes
 * (64 MiB) that the library holds on every GPU it runs on until the process ends (the Hy4 decode
 * batch, T = 64, needs about 12 MiB; T up to 416 fits at the Hy4 shape). Arguments, layout
 * and results as moe_layer_forward (the same kernels, so the same bits). The call allocates and
 * frees nothing; its first call on a device looks up that device's array address
 * (hipGetSymbolAddress) once. It uses the array of the CURRENT device: a non-null stream must
 * belong to it (else MOE_ERR_INVALID_ARG). MOE_ERR_SCRATCH when moe_layer_workspace_size(shape)
 * exceeds the array. Nothing in the array needs to start at zero, and each call overwrites what
 * the previous one left. Every call on one GPU shares its array: calls that overlap in time on
 * one GPU (different streams, or host threads) race and give undefined results; serialise them
 * (one stream, or events).                                                                        */
size_t moe_layer_noalloc_scratch_bytes(void);
int moe_layer_forward_noalloc(const moe_shape* shape, const uint16_t* x,
                              const uint16_t* w_router, const float* bias,
                              const uint16_t* w_gate, const uint16_t* w_up,
                              const uint16_t* w_down, const uint16_t* s_gate,
                              const uint16_t* s_up, const uint16_t* s_down, uint16_t* out,
                              hipStream_t stream);

/* The forward of a training step: moe_layer_forward, which also stores for moe_layer_backward
 * the fp32 gate and up sums g = x Wg^T, u = x Wu^T of every layer row (the pre-activation
 * values of the SwiGLU step above; Hy3 deep-dive `MoEFeedForward`, Hy4 config walkthrough
 * "MoE routed experts"). The backward then reads them and skips recomputing the gate/up GEMM.
 * gu: [T + T*K, 2I] fp32, device, 16-byte aligned, caller-owned: row r (layer order, shared rows
 * first, as in the workspace's h) holds g in columns [0, I) and u in [I, 2I); rows past the
 * layer's row count (capacity drops) are not written. The gate/up and down projections always
 * run on the LDS-tiled MFMA kernel here, whatever the rows per expert, so the stored sums are the
 * ones the backward's recompute forms, bit for bit. Everything else, workspace included, as
 * moe_layer_forward; NULL gu is MOE_ERR_INVALID_ARG.                                            */
int moe_layer_forward_train(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router,
                            const float* bias, const uint16_t* w_gate, const uint16_t* w_up,
                            const uint16_t* w_down, const uint16_t* s_gate, const uint16_t* s_up,
                            const uint16_t* s_down, uint16_t* out, float* gu, void* ws,
                            size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
