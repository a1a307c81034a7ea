/*
 * moe_oracle.h -- plain, slow CPU reference for the sparse MoE FFN layer forward.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library. It shares no code, header, table or helper with the
 * HIP library: it has its own bf16 rounding, its own loops, and accumulates every dot
 * product sequentially in double precision.
 *
 * Sources (web pages; cited by title and section):
 *  [Hy4-deep-dive]  "Tencent Hunyuan Hy4 Preview deep technical analysis" (happyrock.cloud blog),
 *                   code sketches `MoERouter` and `MoELayer`.
 *  [Hy3-deep-dive]  "Tencent Hunyuan Hy3 official release deep analysis" (happyrock.cloud blog),
 *                   `SparseMoERouter.forward`, `MoEFeedForward.forward`, Go `computeConfidence`.
 *  [Hy4-config]     "Hy4 preview config.json deep interpretation" (lshu.cn), sections
 *                   "MoE routed experts: 256 choose 8" and "length, vocabulary and training details".
 *  [Hy3-explainer]  Hy3 sparse-MoE explainer (tqpw.cn), section 2.1 "basic working principle of MoE".
 *
 * Conventions: bf16 tensors are passed as raw uint16 bit patterns, row-major, host memory.
 * Every function is deterministic for any OpenMP thread count (each output element is
 * produced by one thread with a fixed sequential summation order).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Round a double to the nearest bf16 value, ties to even (IEEE RNE); overflow -> inf,
 * NaN -> canonical quiet NaN 0x7FC0. Single rounding from the double value. */
uint16_t oracle_bf16_from_double(double v);
/* Exact widening of a bf16 bit pattern. */
double oracle_double_from_bf16(uint16_t b);

/* Router projection, [Hy4-deep-dive] `MoERouter.gate` (a bias-free linear map hidden -> experts)
 * and [Hy3-deep-dive] `self.gate(x_flat)`. logits[t,e] = fp32( sum_h x[t,h]*wr[e,h] ) + bias[e],
 * the sum taken in double in ascending h and rounded to fp32, the bias added in fp32.
 * bias may be NULL (the pages' router has none).
 * Only tokens listed in `tokens` (n_tok entries) are computed when tokens != NULL; their rows
 * of `logits` (full [T,E] array) are written, the rest are untouched. */
void oracle_router_logits(int T, int H, int E, const uint16_t* x, const uint16_t* wr,
                          const float* bias, const int32_t* tokens, int n_tok, float* logits);

/* Softmax over the experts, top-k, optional renormalisation, routed scaling.
 * [Hy4-deep-dive] `torch.topk(F.softmax(scores), k)`; [Hy3-deep-dive] renormalisation of the
 * selected probabilities; [Hy4-config] `norm_topk_prob: true`, `routed_scaling_factor: 2.827`.
 * Selection takes the k largest fp32 logits (softmax is strictly increasing, so this is the
 * same set as the k largest probabilities), ordered by value descending and, for equal values,
 * by expert index ascending; -0.0 and +0.0 are equal. Logits must be finite.
 * w[t,j] = fp32( scale * p_j / sum_{i in top-k} p_i ) when norm_topk != 0, else fp32(scale*p_j).
 * probs (may be NULL) receives the full double softmax [T,E]. */
void oracle_route_from_logits(int T, int E, int K, int norm_topk, double scale,
                              const float* logits, int32_t* topk_idx, float* topk_w,
                              double* probs);

/* Token-to-expert dispatch: a stable counting sort of slot ids s = t*K + j by expert,
 * [Hy3-explainer] 2.1 (per-expert gather `x[expert_mask]`). capacity > 0 keeps the first
 * `capacity` slots of each expert in ascending slot order and drops the rest.
 * counts[E] kept per expert, offsets[E+1] exclusive scan, row_to_slot[T*K] (rows >= offsets[E]
 * are set to -1), slot_to_row[T*K] (-1 for dropped slots). */
void oracle_dispatch(int T, int K, int E, int capacity, const int32_t* topk_idx,
                     int32_t* counts, int32_t* offsets, int32_t* row_to_slot,
                     int32_t* slot_to_row);

/* SwiGLU gate/up half of one expert on n gathered rows, [Hy3-deep-dive] `MoEFeedForward`
 * (gate_proj, up_proj, silu) with the [Hy4-config] `swiglu_limit` clamp of both pre-activations:
 * g = fp32( sum_h x*wg[i,h] ), u = fp32( sum_h x*wu[i,h] ) (sums in double, then rounded to
 * fp32), g,u clamped to [-limit, limit] when limit > 0, h[r,i] = bf16( g/(1+exp(-g)) * u ) with
 * the SwiGLU in double. wg, wu are [I,H]; x_rows is [n,H]. */
void oracle_gateup_rows(int n, int H, int I, double limit, const uint16_t* x_rows,
                        const uint16_t* wg, const uint16_t* wu, uint16_t* h);

/* Down projection of one expert, [Hy3-deep-dive] `down_proj`:
 * y[r,c] = bf16( fp32( sum_i h[r,i]*wd[c,i] ) ) (the sum in double), wd is [H,I], h is [n,I]. */
void oracle_down_rows(int n, int H, int I, const uint16_t* h, const uint16_t* wd, uint16_t* y);

/* Weighted combine, [Hy4-deep-dive] `MoELayer.forward` (routed sum plus shared expert output):
 * out[t,c] = bf16( sum_{j<K, slot_to_row[t*K+j] >= 0} w[t,j]*y[row,c] + y_shared[t,c] ), summed in
 * double in slot order, the shared term last. y_shared may be NULL. */
void oracle_combine(int T, int K, int H, const float* topk_w, const int32_t* slot_to_row,
                    const uint16_t* y_routed, const uint16_t* y_shared, uint16_t* out);

/* Whole layer, sparse evaluation (steps above in order). The routed expert weights are
 * wg,wu [E,I,H] and wd [E,H,I]; the shared expert's are sg,su [I,H], sd [H,I] (NULL = none).
 * When use_logits != 0, `logits` is taken as input and the router projection is skipped;
 * otherwise it is written. All outputs are caller-owned host arrays:
 * topk_idx/topk_w [T,K], counts [E], offsets [E+1], row_to_slot/slot_to_row [T*K],
 * h_routed [T*K,I], y_routed [T*K,H] (rows >= offsets[E] untouched), h_shared [T,I],
 * y_shared [T,H], out [T,H]. h_* and y_shared may be NULL when not wanted. */
void oracle_layer_forward(int T, int H, int E, int K, int I, int norm_topk, double scale,
                          double limit, int capacity, const uint16_t* x, const uint16_t* wr,
                          const float* bias, const uint16_t* wg, const uint16_t* wu,
                          const uint16_t* wd, const uint16_t* sg, const uint16_t* su,
                          const uint16_t* sd, int use_logits, float* logits, int32_t* topk_idx,
                          float* topk_w, int32_t* counts, int32_t* offsets,
                          int32_t* row_to_slot, int32_t* slot_to_row, uint16_t* h_routed,
                          uint16_t* y_routed, uint16_t* h_shared, uint16_t* y_shared,
                          uint16_t* out);

/* Dense brute force (small inputs only): every expert evaluated on every token, then masked
 * by the kept top-k assignment, [Hy4-deep-dive] token loop `routed[b,s] += w * expert(x)`.
 * Takes the routing (topk_idx, topk_w, slot_to_row kept mask) as input, no permutation. */
void oracle_layer_dense(int T, int H, int E, int K, int I, double limit, const uint16_t* x,
                        const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                        const uint16_t* sg, const uint16_t* su, const uint16_t* sd,
                        const int32_t* topk_idx, const float* topk_w,
                        const int32_t* slot_to_row, uint16_t* out);

/* ---- FP8 expert weights. The pages deploy an FP8 checkpoint but define no format; the reading
 * used here: every expert weight matrix ([Hy4-config] shapes) is stored as OCP FP8 E4M3 codes
 * (uint8, row-major) with one fp32 scale per row (output channel), the weight value being
 * scale[row] * e4m3(code). Router weights and activations stay bf16. */

/* Exact value of an E4M3 code: sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
 * holds subnormals m * 2^-9; S.1111.111 is NaN (no infinities; largest finite 448). */
double oracle_double_from_e4m3(uint8_t code);

/* oracle_gateup_rows / oracle_down_rows with FP8 weights: qg, qu [I,H] codes with scales cg, cu
 * [I]; qd [H,I] codes with scales cd [H]. Dot products in double over w = scale * e4m3(code). */
void oracle_gateup_rows_fp8(int n, int H, int I, double limit, const uint16_t* x_rows,
                            const uint8_t* qg, const float* cg, const uint8_t* qu,
                            const float* cu, uint16_t* h);
void oracle_down_rows_fp8(int n, int H, int I, const uint16_t* h, const uint8_t* qd,
                          const float* cd, uint16_t* y);

/* oracle_layer_forward with FP8 expert weights: routed qg, qu [E,I,H] (scales cg, cu [E,I]) and
 * qd [E,H,I] (scales cd [E,H]); shared sqg, squ [I,H] (scales scg, scu [I]) and sqd [H,I]
 * (scales scd [H]), NULL = no shared expert. Everything else as oracle_layer_forward. */
void oracle_layer_forward_fp8(int T, int H, int E, int K, int I, int norm_topk, double scale,
                              double limit, int capacity, const uint16_t* x, const uint16_t* wr,
                              const float* bias, const uint8_t* qg, const float* cg,
                              const uint8_t* qu, const float* cu, const uint8_t* qd,
                              const float* cd, const uint8_t* sqg, const float* scg,
                              const uint8_t* squ, const float* scu, const uint8_t* sqd,
                              const float* scd, int use_logits, float* logits,
                              int32_t* topk_idx, float* topk_w, int32_t* counts,
                              int32_t* offsets, int32_t* row_to_slot, int32_t* slot_to_row,
                              uint16_t* h_routed, uint16_t* y_routed, uint16_t* h_shared,
                              uint16_t* y_shared, uint16_t* out);

/* oracle_layer_dense with FP8 expert weights (same weight arguments as above). */
void oracle_layer_dense_fp8(int T, int H, int E, int K, int I, double limit, const uint16_t* x,
                            const uint8_t* qg, const float* cg, const uint8_t* qu,
                            const float* cu, const uint8_t* qd, const float* cd,
                            const uint8_t* sqg, const float* scg, const uint8_t* squ,
                            const float* scu, const uint8_t* sqd, const float* scd,
                            const int32_t* topk_idx, const float* topk_w,
                            const int32_t* slot_to_row, uint16_t* out);

// ---- FP8 weights and FP8 activations (W8A8), moe_oracle_w8a8.cpp. Per-row dynamic E4M3
// quantisation of the activations entering each expert projection; see that file's header.
uint8_t oracle_e4m3_from_float(float q);
void oracle_e4m3_from_float_array(long n, const float* q, uint8_t* codes);
void oracle_quant_rows_e4m3(int rows, int cols, const uint16_t* v, uint8_t* codes, float* scales);
void oracle_gateup_rows_w8a8(int n, int H, int I, double limit, const uint8_t* xq,
                             const float* sx, const uint8_t* qg, const float* cg,
                             const uint8_t* qu, const float* cu, uint16_t* h);
void oracle_down_rows_w8a8(int n, int H, int I, const uint8_t* hq, const float* sh,
                           const uint8_t* qd, const float* cd, uint16_t* y);
void oracle_layer_forward_w8a8(int T, int H, int E, int K, int I, int norm_topk, double scale,
                               double limit, int capacity, const uint16_t* x,
                               const uint16_t* wr, const float* bias, const uint8_t* qg,
                               const float* cg, const uint8_t* qu, const float* cu,
                               const uint8_t* qd, const float* cd, const uint8_t* sqg,
                               const float* scg, const uint8_t* squ, const float* scu,
                               const uint8_t* sqd, const float* scd, int use_logits,
                               float* logits, int32_t* topk_idx, float* topk_w,
                               int32_t* counts, int32_t* offsets, int32_t* row_to_slot,
                               int32_t* slot_to_row, uint8_t* xq, float* sx,
                               uint16_t* h_routed, uint16_t* y_routed, uint16_t* h_shared,
                               uint16_t* y_shared, uint16_t* out);

// ---- MX block-scaled FP8 weights and activations (MXFP8), moe_oracle_mx.cpp. One E8M0 scale
// byte s (value 2^(s - 127)) per 32 consecutive elements along the reduction dimension, OCP E4M3
// elements; activations quantised per block by the OCP Microscaling conversion rule (shared
// exponent floor(log2(amax)) - 8, clamped to [-127, 127]; elements nearest-even, saturating).
uint8_t oracle_mx_scale_of_amax(double amax);
void oracle_mx_quant_rows(int rows, int cols, const uint16_t* v, uint8_t* codes, uint8_t* scales);
void oracle_mx_dequant(int rows, int cols, const uint8_t* codes, const uint8_t* scales, double* out);
void oracle_gateup_rows_mx(int n, int H, int I, double limit, const uint8_t* xq, const uint8_t* xs,
                           const uint8_t* qg, const uint8_t* sg, const uint8_t* qu, const uint8_t* su,
                           uint16_t* h);
void oracle_down_rows_mx(int n, int H, int I, const uint8_t* hq, const uint8_t* hs, const uint8_t* qd,
                         const uint8_t* sd, uint16_t* y);
void oracle_layer_forward_mx(int T, int H, int E, int K, int I, int norm_topk, double scale,
                             double limit, int capacity, const uint16_t* x, const uint16_t* wr,
                             const float* bias, const uint8_t* qg, const uint8_t* sg,
                             const uint8_t* qu, const uint8_t* su, const uint8_t* qd,
                             const uint8_t* sd, const uint8_t* sqg, const uint8_t* ssg,
                             const uint8_t* squ, const uint8_t* ssu, const uint8_t* sqd,
                             const uint8_t* ssd, int use_logits, float* logits, int32_t* topk_idx,
                             float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* row_to_slot, int32_t* slot_to_row, uint8_t* xq, uint8_t* xs,
                             uint16_t* h_routed, uint16_t* y_routed, uint16_t* h_shared,
                             uint16_t* y_shared, uint16_t* out);

/* Training-side router statistics (Hy3 deep-dive, SparseMoERouter training branch and its
 * load-balancing loss): from fp32 logits [T,E] (bias and noise already added) and the top-k
 * indices [T,K]:
 *   prob_mean[e] = (1/T) sum_t softmax(logits[t])[e]
 *   load_frac[e] = #{(t,j): topk_idx[t,j] = e} / (T*K)        (before any capacity limit)
 *   aux          = E * sum_e prob_mean[e] * load_frac[e]
 *   ema_counts[e] = decay*ema_counts[e] + (1-decay)*count[e]  (in/out, may be NULL)
 *   ema_tokens    = decay*ema_tokens + (1-decay)*T            (in/out, may be NULL)       */
void oracle_router_train_stats(int T, int E, int K, const float* logits, const int32_t* topk_idx,
                               double decay, double* prob_mean, double* load_frac, double* aux,
                               double* ema_counts, double* ema_tokens);

/* ---- backward pass (moe_oracle_bwd.cpp). Intermediate tensors are double arrays; with
 * round_bf16 set, values the GPU stores in bf16 are rounded to bf16 at the same points.
 * Row arrays are in the forward's dispatch order (rows grouped by expert).                  */
/* dy[row(t,j)] = w_j * dout[t]; d_topk_w[t,j] = <dout[t], y[row(t,j)]> (0 for dropped slots) */
void oracle_combine_bwd(int T, int K, int H, int round_bf16, const float* topk_w,
                        const int32_t* slot_to_row, const double* y_rows, const uint16_t* dout,
                        double* dy_rows, double* d_topk_w);
/* dh[r,i] = sum_c dy[r,c] Wd[c,i]   (Wd [H,I] bf16)                                          */
void oracle_down_bwd_rows(int n, int H, int I, int round_bf16, const double* dy,
                          const uint16_t* wd, double* dh);
/* recompute g = x Wg^T, u = x Wu^T; dg = dh * clamp(u) * silu'(clamp(g)) * [|g| <= L],
 * du = dh * silu(clamp(g)) * [|u| <= L]  (no masks when L <= 0)                             */
void oracle_swiglu_bwd_rows(int n, int H, int I, double limit, int round_bf16,
                            const uint16_t* x_rows, const uint16_t* wg, const uint16_t* wu,
                            const double* dh, double* dg, double* du);
/* dx[r,c] = sum_i dg[r,i] Wg[i,c] + du[r,i] Wu[i,c]                                          */
void oracle_gateup_dgrad_rows(int n, int H, int I, int round_bf16, const double* dg,
                              const double* du, const uint16_t* wg, const uint16_t* wu,
                              double* dx);
/* out[m,c] = sum_r A[r,m] B[r,c]   (weight gradients)                                        */
void oracle_wgrad(int n, int M, int N, const double* A, const double* B, double* out);
/* routing-weight gradients (+ d_aux times the load-balancing loss) to logit gradients         */
void oracle_router_bwd(int T, int E, int K, int norm_topk, double scale, const float* logits,
                       const int32_t* topk_idx, const double* d_topk_w, double d_aux,
                       double* d_logits);
/* The whole backward from the forward's routing (logits, top-k, dispatch) and dout [T,H] bf16.
 * Outputs (double): d_topk_w [T,K], d_logits [T,E], dx [T,H], d_wr [E,H], d_wg/d_wu [E,I,H],
 * d_wd [E,H,I], d_sg/d_su [I,H], d_sd [H,I] (shared; unused when sg is NULL); optional row
 * intermediates dh/dg/du [R,I], dx_rows [R,H] and dx_router [T,H] (NULL to skip).            */
void oracle_layer_backward(int T, int H, int E, int K, int I, int norm_topk, double scale,
                           double limit, int round_bf16, const uint16_t* x, const uint16_t* wr,
                           const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                           const uint16_t* sg, const uint16_t* su, const uint16_t* sd,
                           const float* logits, const int32_t* topk_idx, const float* topk_w,
                           const int32_t* counts, const int32_t* offsets,
                           const int32_t* row_to_slot, const int32_t* slot_to_row,
                           const uint16_t* dout, double d_aux, double* d_topk_w,
                           double* d_logits, double* dx, double* d_wr, double* d_wg,
                           double* d_wu, double* d_wd, double* d_sg, double* d_su, double* d_sd,
                           double* dh_rows, double* dg_rows, double* du_rows, double* dx_rows,
                           double* dx_router);

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_num_threads(void);
/* Threads of the following oracle calls (OpenMP; results do not depend on it). */
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
