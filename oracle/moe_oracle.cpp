// moe_oracle.cpp -- plain CPU reference of the sparse MoE FFN layer forward.
//
// TEST INFRASTRUCTURE: loaded only by the tests, the smoke check and the CPU-baseline leg of
// the benchmark. Written from the pages' statement of the layer (see moe_oracle.h for the
// source list); it shares nothing with the HIP library. Every dot product is a sequential
// double-precision sum. The layer's projections produce fp32 values (the pages' checkpoint is
// bf16 and its matrix products accumulate in fp32): the router logits, the gate and up
// pre-activations g, u and the down projection are each the fp32 rounding of their double sum,
// and the router bias is an fp32 add to the fp32 logit. bf16 rounding happens only where the
// layer stores bf16 tensors (h, y, y_shared, out), with this file's own round-to-nearest-even;
// the SwiGLU of the fp32 g, u and the combine are evaluated in double.
//
// Parity pins live in tests/test_oracle_*.py (bf16 bit patterns, softmax closed forms, tie
// order, counting-sort vs a library stable sort, dense-vs-sparse, E=1/k=1 vs a float64 SwiGLU
// FFN, the clamp closed form, capacity hand cases).

#include "moe_oracle.h"

#include <cmath>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

inline double bf(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

// silu(g) * u with the swiglu_limit clamp on both pre-activations ([Hy4-config], section
// "MoE routed experts": swiglu_limit 10 clips SwiGLU activations to +-10; hidden_act silu).
inline double clamped_swiglu(double g, double u, double limit) {
  if (limit > 0.0) {
    g = g < -limit ? -limit : (g > limit ? limit : g);
    u = u < -limit ? -limit : (u > limit ? limit : u);
  }
  return g / (1.0 + std::exp(-g)) * u;
}

// OCP 8-bit floating point, E4M3 encoding: sign bit, 4 exponent bits (bias 7), 3 mantissa
// bits; exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN and there are no
// infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.
inline double e4m3(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return std::nan("");
  const double v = e == 0 ? std::ldexp(static_cast<double>(m), -9)
                          : std::ldexp(static_cast<double>(8 + m), e - 10);  // (1 + m/8) 2^(e-7)
  return (c & 0x80) ? -v : v;
}

// Weight matrices [rows][cols] row-major: bf16 bits, or FP8 E4M3 codes with one fp32 scale per
// row (weight value = scale[row] * e4m3(code)).
struct Bf16W {
  const uint16_t* p;
  int cols;
  double operator()(size_t r, size_t c) const { return bf(p[r * cols + c]); }
};
struct Fp8W {
  const uint8_t* q;
  const float* scale;
  int cols;
  double operator()(size_t r, size_t c) const {
    return static_cast<double>(scale[r]) * e4m3(q[r * cols + c]);
  }
};

// Expert weights of a layer: routed gate/up [E][I][H], down [E][H][I], shared [I][H], [H][I].
struct Bf16Experts {
  const uint16_t *wg, *wu, *wd, *sg, *su, *sd;
  int H, I;
  bool shared() const { return sg != nullptr; }
  Bf16W gate(int e) const { return {wg + static_cast<size_t>(e) * I * H, H}; }
  Bf16W up(int e) const { return {wu + static_cast<size_t>(e) * I * H, H}; }
  Bf16W down(int e) const { return {wd + static_cast<size_t>(e) * H * I, I}; }
  Bf16W sgate() const { return {sg, H}; }
  Bf16W sup() const { return {su, H}; }
  Bf16W sdown() const { return {sd, I}; }
};
struct Fp8Experts {
  const uint8_t *qg, *qu, *qd, *sqg, *squ, *sqd;      // codes
  const float *cg, *cu, *cd, *scg, *scu, *scd;        // per-row scales
  int H, I;
  bool shared() const { return sqg != nullptr; }
  Fp8W gate(int e) const { return {qg + static_cast<size_t>(e) * I * H, cg + static_cast<size_t>(e) * I, H}; }
  Fp8W up(int e) const { return {qu + static_cast<size_t>(e) * I * H, cu + static_cast<size_t>(e) * I, H}; }
  Fp8W down(int e) const { return {qd + static_cast<size_t>(e) * H * I, cd + static_cast<size_t>(e) * H, I}; }
  Fp8W sgate() const { return {sqg, scg, H}; }
  Fp8W sup() const { return {squ, scu, H}; }
  Fp8W sdown() const { return {sqd, scd, I}; }
};

// SwiGLU gate/up half of one expert on n gathered rows (see the header).
template <class W>
static void gateup_impl(int n, int H, int I, double limit, const uint16_t* x_rows, W wg, W wu,
                        uint16_t* h) {
#pragma omp parallel for schedule(static)
  for (long ri = 0; ri < static_cast<long>(n) * I; ++ri) {
    const long r = ri / I, i = ri % I;
    const uint16_t* xr = x_rows + static_cast<size_t>(r) * H;
    double g = 0.0, u = 0.0;
    for (int k = 0; k < H; ++k) {
      const double xv = bf(xr[k]);
      g += xv * wg(i, k);
      u += xv * wu(i, k);
    }
    // g and u are fp32 values: the fp32 rounding of the exact projections
    const double g32 = static_cast<float>(g), u32 = static_cast<float>(u);
    h[static_cast<size_t>(r) * I + i] = oracle_bf16_from_double(clamped_swiglu(g32, u32, limit));
  }
}

// Down projection of one expert (see the header).
template <class W>
static void down_impl(int n, int H, int I, const uint16_t* h, W wd, uint16_t* y) {
#pragma omp parallel for schedule(static)
  for (long rc = 0; rc < static_cast<long>(n) * H; ++rc) {
    const long r = rc / H, c = rc % H;
    const uint16_t* hr = h + static_cast<size_t>(r) * I;
    double s = 0.0;
    for (int i = 0; i < I; ++i) s += bf(hr[i]) * wd(c, i);
    // the fp32 projection, stored as bf16
    y[static_cast<size_t>(r) * H + c] = oracle_bf16_from_double(static_cast<float>(s));
  }
}

// One expert's FFN over n gathered rows (gate/up then down).
template <class W>
static void expert_rows(int n, int H, int I, double limit, const uint16_t* x_rows, W wg, W wu,
                        W wd, uint16_t* h_out, uint16_t* y_out) {
  if (n == 0) return;
  std::vector<uint16_t> hbuf;
  uint16_t* h = h_out;
  if (!h) {
    hbuf.resize(static_cast<size_t>(n) * I);
    h = hbuf.data();
  }
  gateup_impl(n, H, I, limit, x_rows, wg, wu, h);
  down_impl(n, H, I, h, wd, y_out);
}

template <class X>
static void layer_impl(int T, int H, int E, int K, int I, int norm_topk, double scale,
                       double limit, int capacity, const uint16_t* x, const uint16_t* wr,
                       const float* bias, const X& w, int use_logits, float* logits,
                       int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                       int32_t* row_to_slot, int32_t* slot_to_row, uint16_t* h_routed,
                       uint16_t* y_routed, uint16_t* h_shared, uint16_t* y_shared,
                       uint16_t* out) {
  // 1. router projection (skipped when the caller supplies the fp32 logits)
  if (!use_logits) oracle_router_logits(T, H, E, x, wr, bias, nullptr, 0, logits);
  // 2-4. softmax, top-k, renormalisation, routed scaling
  oracle_route_from_logits(T, E, K, norm_topk, scale, logits, topk_idx, topk_w, nullptr);
  // 5. dispatch
  oracle_dispatch(T, K, E, capacity, topk_idx, counts, offsets, row_to_slot, slot_to_row);
  // 6. routed experts, expert-major ([Hy3-explainer] 2.1: each expert runs on its gathered rows)
  for (int e = 0; e < E; ++e) {
    const int n = counts[e];
    if (n == 0) continue;
    std::vector<uint16_t> xg(static_cast<size_t>(n) * H);
    for (int i = 0; i < n; ++i) {
      const int t = row_to_slot[offsets[e] + i] / K;
      std::memcpy(&xg[static_cast<size_t>(i) * H], x + static_cast<size_t>(t) * H,
                  sizeof(uint16_t) * H);
    }
    expert_rows(n, H, I, limit, xg.data(), w.gate(e), w.up(e), w.down(e),
                h_routed ? h_routed + static_cast<size_t>(offsets[e]) * I : nullptr,
                y_routed + static_cast<size_t>(offsets[e]) * H);
  }
  // 7. shared expert on every token, weight 1 ([Hy4-deep-dive]: always active)
  std::vector<uint16_t> ysbuf;
  uint16_t* ys = y_shared;
  if (w.shared()) {
    if (!ys) {
      ysbuf.resize(static_cast<size_t>(T) * H);
      ys = ysbuf.data();
    }
    expert_rows(T, H, I, limit, x, w.sgate(), w.sup(), w.sdown(), h_shared, ys);
  } else {
    ys = nullptr;
  }
  // 8. combine
  oracle_combine(T, K, H, topk_w, slot_to_row, y_routed, ys, out);
}

template <class X>
static void dense_impl(int T, int H, int E, int K, int I, double limit, const uint16_t* x,
                       const X& w, const int32_t* topk_idx, const float* topk_w,
                       const int32_t* slot_to_row, uint16_t* out) {
  // Every expert on every token: y_all[e][t][:]
  std::vector<uint16_t> y_all(static_cast<size_t>(E) * T * H);
  for (int e = 0; e < E; ++e)
    expert_rows(T, H, I, limit, x, w.gate(e), w.up(e), w.down(e), nullptr,
                &y_all[static_cast<size_t>(e) * T * H]);
  std::vector<uint16_t> ys;
  if (w.shared()) {
    ys.resize(static_cast<size_t>(T) * H);
    expert_rows(T, H, I, limit, x, w.sgate(), w.sup(), w.sdown(), nullptr, ys.data());
  }
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int j = 0; j < K; ++j) {
        const size_t s = static_cast<size_t>(t) * K + j;
        const double mask = slot_to_row[s] >= 0 ? 1.0 : 0.0;
        const int e = topk_idx[s];
        acc += mask * static_cast<double>(topk_w[s]) *
               bf(y_all[(static_cast<size_t>(e) * T + t) * H + c]);
      }
      if (w.shared()) acc += bf(ys[static_cast<size_t>(t) * H + c]);
      out[static_cast<size_t>(t) * H + c] = oracle_bf16_from_double(acc);
    }
  }
}

}  // namespace

extern "C" {

uint16_t oracle_bf16_from_double(double v) {
  if (std::isnan(v)) return 0x7FC0;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0x0000;
  const double a = std::fabs(v);
  if (a == 0.0) return sign;
  if (std::isinf(a)) return sign | 0x7F80;
  // a lies in [2^E, 2^(E+1)); bf16 keeps 8 significant bits there, so neighbouring values are
  // 2^(E-7) apart. Below the smallest normal (2^-126) the spacing is fixed at 2^-133.
  int ex = 0;
  std::frexp(a, &ex);
  const int E = ex - 1;
  const int qexp = (E < -126) ? -133 : E - 7;
  const double q = std::ldexp(a, -qexp);  // exact: scaling by a power of two
  const double r = std::nearbyint(q);     // default rounding mode: nearest, ties to even
  const double res = std::ldexp(r, qexp);
  if (res >= std::ldexp(1.0, 128)) return sign | 0x7F80;  // rounds past the largest finite
  const float f = static_cast<float>(res);                 // exact: res is a bf16 value
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return static_cast<uint16_t>(sign | (u >> 16));
}

double oracle_double_from_bf16(uint16_t b) { return bf(b); }

// Training-side router statistics, following the training branch of the Hy3 deep-dive's
// SparseMoERouter: P is the token mean of the softmax probabilities, f the share of the T*K
// selections that went to each expert (counted from the top-k indices, before any capacity
// limit), the load-balancing loss is E * sum_e P[e] f[e], and the expert-count and token-count
// buffers move as exponential moving averages with the given decay (0.9 on the page).
void oracle_router_train_stats(int T, int E, int K, const float* logits, const int32_t* topk_idx,
                               double decay, double* prob_mean, double* load_frac, double* aux,
                               double* ema_counts, double* ema_tokens) {
  std::vector<double> p(static_cast<size_t>(T) * E);
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const float* l = logits + static_cast<size_t>(t) * E;
    double m = l[0];
    for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
    double z = 0.0;
    double* pt = p.data() + static_cast<size_t>(t) * E;
    for (int e = 0; e < E; ++e) {
      pt[e] = std::exp(static_cast<double>(l[e]) - m);
      z += pt[e];
    }
    for (int e = 0; e < E; ++e) pt[e] /= z;
  }
  std::vector<double> counts(E, 0.0);
  for (size_t i = 0; i < static_cast<size_t>(T) * K; ++i) counts[topk_idx[i]] += 1.0;
  double sum = 0.0;
  for (int e = 0; e < E; ++e) {
    double pe = 0.0;
    for (int t = 0; t < T; ++t) pe += p[static_cast<size_t>(t) * E + e];
    prob_mean[e] = pe / T;
    load_frac[e] = counts[e] / (static_cast<double>(T) * K);
    sum += prob_mean[e] * load_frac[e];
  }
  *aux = sum * E;
  if (ema_counts)
    for (int e = 0; e < E; ++e) ema_counts[e] = ema_counts[e] * decay + counts[e] * (1.0 - decay);
  if (ema_tokens) *ema_tokens = *ema_tokens * decay + static_cast<double>(T) * (1.0 - decay);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

void oracle_router_logits(int T, int H, int E, const uint16_t* x, const uint16_t* wr,
                          const float* bias, const int32_t* tokens, int n_tok, float* logits) {
  const int n = tokens ? n_tok : T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n; ++i) {
    const int t = tokens ? tokens[i] : i;
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int h = 0; h < H; ++h)
        s += bf(x[static_cast<size_t>(t) * H + h]) * bf(wr[static_cast<size_t>(e) * H + h]);
      // the fp32 logit, then the bias as an fp32 add
      float l = static_cast<float>(s);
      if (bias) l = l + bias[e];
      logits[static_cast<size_t>(t) * E + e] = l;
    }
  }
}

void oracle_route_from_logits(int T, int E, int K, int norm_topk, double scale,
                              const float* logits, int32_t* topk_idx, float* topk_w,
                              double* probs) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const float* l = logits + static_cast<size_t>(t) * E;
    // Softmax with the maximum subtracted first ([Hy3-deep-dive] Go computeConfidence).
    double m = l[0];
    for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
    std::vector<double> p(E);
    double z = 0.0;
    for (int e = 0; e < E; ++e) {
      p[e] = std::exp(static_cast<double>(l[e]) - m);
      z += p[e];
    }
    for (int e = 0; e < E; ++e) p[e] /= z;
    if (probs)
      for (int e = 0; e < E; ++e) probs[static_cast<size_t>(t) * E + e] = p[e];
    // k rounds of "largest remaining": a strict > keeps the lower index among equal values.
    std::vector<char> taken(E, 0);
    int32_t* idx = topk_idx + static_cast<size_t>(t) * K;
    for (int j = 0; j < K; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      idx[j] = best;
    }
    double denom = 1.0;
    if (norm_topk) {
      denom = 0.0;
      for (int j = 0; j < K; ++j) denom += p[idx[j]];
    }
    for (int j = 0; j < K; ++j)
      topk_w[static_cast<size_t>(t) * K + j] = static_cast<float>(scale * p[idx[j]] / denom);
  }
}

void oracle_dispatch(int T, int K, int E, int capacity, const int32_t* topk_idx,
                     int32_t* counts, int32_t* offsets, int32_t* row_to_slot,
                     int32_t* slot_to_row) {
  const int S = T * K;
  std::vector<std::vector<int32_t>> lists(E);
  for (int s = 0; s < S; ++s) lists[topk_idx[s]].push_back(s);  // ascending slot order
  for (int s = 0; s < S; ++s) slot_to_row[s] = -1;
  for (int r = 0; r < S; ++r) row_to_slot[r] = -1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) {
    if (capacity > 0 && static_cast<int>(lists[e].size()) > capacity) lists[e].resize(capacity);
    counts[e] = static_cast<int32_t>(lists[e].size());
    offsets[e + 1] = offsets[e] + counts[e];
  }
  for (int e = 0; e < E; ++e) {
    for (size_t i = 0; i < lists[e].size(); ++i) {
      const int32_t row = offsets[e] + static_cast<int32_t>(i);
      row_to_slot[row] = lists[e][i];
      slot_to_row[lists[e][i]] = row;
    }
  }
}


void oracle_gateup_rows(int n, int H, int I, double limit, const uint16_t* x_rows,
                        const uint16_t* wg, const uint16_t* wu, uint16_t* h) {
  gateup_impl(n, H, I, limit, x_rows, Bf16W{wg, H}, Bf16W{wu, H}, h);
}

void oracle_down_rows(int n, int H, int I, const uint16_t* h, const uint16_t* wd, uint16_t* y) {
  down_impl(n, H, I, h, Bf16W{wd, I}, y);
}

double oracle_double_from_e4m3(uint8_t code) { return e4m3(code); }

void oracle_gateup_rows_fp8(int n, int H, int I, double limit, const uint16_t* x_rows,
                            const uint8_t* qg, const float* cg, const uint8_t* qu,
                            const float* cu, uint16_t* h) {
  gateup_impl(n, H, I, limit, x_rows, Fp8W{qg, cg, H}, Fp8W{qu, cu, H}, h);
}

void oracle_down_rows_fp8(int n, int H, int I, const uint16_t* h, const uint8_t* qd,
                          const float* cd, uint16_t* y) {
  down_impl(n, H, I, h, Fp8W{qd, cd, I}, y);
}

void oracle_combine(int T, int K, int H, const float* topk_w, const int32_t* slot_to_row,
                    const uint16_t* y_routed, const uint16_t* y_shared, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int j = 0; j < K; ++j) {
        const int32_t row = slot_to_row[static_cast<size_t>(t) * K + j];
        if (row < 0) continue;  // dropped by capacity: contributes nothing
        acc += static_cast<double>(topk_w[static_cast<size_t>(t) * K + j]) *
               bf(y_routed[static_cast<size_t>(row) * H + c]);
      }
      if (y_shared) acc += bf(y_shared[static_cast<size_t>(t) * H + c]);
      out[static_cast<size_t>(t) * H + c] = oracle_bf16_from_double(acc);
    }
  }
}

void oracle_layer_forward(int T, int H, int E, int K, int I, int norm_topk, double scale,
                          double limit, int capacity, const uint16_t* x, const uint16_t* wr,
                          const float* bias, const uint16_t* wg, const uint16_t* wu,
                          const uint16_t* wd, const uint16_t* sg, const uint16_t* su,
                          const uint16_t* sd, int use_logits, float* logits, int32_t* topk_idx,
                          float* topk_w, int32_t* counts, int32_t* offsets,
                          int32_t* row_to_slot, int32_t* slot_to_row, uint16_t* h_routed,
                          uint16_t* y_routed, uint16_t* h_shared, uint16_t* y_shared,
                          uint16_t* out) {
  layer_impl(T, H, E, K, I, norm_topk, scale, limit, capacity, x, wr, bias,
             Bf16Experts{wg, wu, wd, sg, su, sd, H, I}, use_logits, logits, topk_idx, topk_w,
             counts, offsets, row_to_slot, slot_to_row, h_routed, y_routed, h_shared, y_shared,
             out);
}

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
                              uint16_t* y_shared, uint16_t* out) {
  layer_impl(T, H, E, K, I, norm_topk, scale, limit, capacity, x, wr, bias,
             Fp8Experts{qg, qu, qd, sqg, squ, sqd, cg, cu, cd, scg, scu, scd, H, I}, use_logits,
             logits, topk_idx, topk_w, counts, offsets, row_to_slot, slot_to_row, h_routed,
             y_routed, h_shared, y_shared, out);
}

void oracle_layer_dense(int T, int H, int E, int K, int I, double limit, const uint16_t* x,
                        const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                        const uint16_t* sg, const uint16_t* su, const uint16_t* sd,
                        const int32_t* topk_idx, const float* topk_w,
                        const int32_t* slot_to_row, uint16_t* out) {
  dense_impl(T, H, E, K, I, limit, x, Bf16Experts{wg, wu, wd, sg, su, sd, H, I}, topk_idx,
             topk_w, slot_to_row, out);
}

void oracle_layer_dense_fp8(int T, int H, int E, int K, int I, double limit, const uint16_t* x,
                            const uint8_t* qg, const float* cg, const uint8_t* qu,
                            const float* cu, const uint8_t* qd, const float* cd,
                            const uint8_t* sqg, const float* scg, const uint8_t* squ,
                            const float* scu, const uint8_t* sqd, const float* scd,
                            const int32_t* topk_idx, const float* topk_w,
                            const int32_t* slot_to_row, uint16_t* out) {
  dense_impl(T, H, E, K, I, limit, x,
             Fp8Experts{qg, qu, qd, sqg, squ, sqd, cg, cu, cd, scg, scu, scd, H, I}, topk_idx,
             topk_w, slot_to_row, out);
}

}  // extern "C"
