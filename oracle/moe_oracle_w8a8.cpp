// moe_oracle_w8a8.cpp -- plain CPU reference of the FP8 (W8A8) form of the expert FFN: expert
// weights as OCP FP8 E4M3 codes with one fp32 scale per weight row, and the activations that
// enter each expert projection (x for gate/up, h for down) quantised per row to E4M3 with one
// fp32 scale per row.
//
// TEST INFRASTRUCTURE: loaded only by the tests, the smoke check and the CPU-baseline leg of
// the benchmark; shares nothing with the HIP library.
//
// The pages deploy the model from an FP8 checkpoint (Tencent Hunyuan Hy4 Preview deep technical
// analysis, deployment commands; Hy4 config walkthrough, dtype notes) without defining a format.
// This file takes the plain per-row dynamic form:
//   amax  = max_c |v[c]|                      (v: the row's bf16 values, as fp32)
//   scale = amax / 448, inv = 448 / amax      (fp32, each one correctly rounded division)
//   code  = E4M3_RNE(clamp(v[c] * inv, -448, 448))   (fp32 product, then nearest-even E4M3)
//   a row whose 448 / amax overflows fp32 (amax > 0 below 448 / FLT_MAX, about 1.3e-36) and an
//   all-zero row are quantised unscaled: scale 1, code = E4M3_RNE(v[c]) (all zero codes there)
// and computes each projection as (sum_k e4m3(a_code[k]) * e4m3(w_code[k])) * w_scale * a_scale
// with the code products summed sequentially in fp64 (each product of two E4M3 values is
// exact), rounded to an fp32 value, then rounded where the bf16 path rounds (h, y).

#include "moe_oracle.h"

#include <cmath>
#include <cstring>
#include <vector>

namespace {

inline float bf32(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

// value of an E4M3 code (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
// holds the subnormals m * 2^-9; 0x7F / 0xFF are NaN and never produced here)
inline double e4m3_value(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  const double v = e == 0 ? std::ldexp(static_cast<double>(m), -9)
                          : std::ldexp(static_cast<double>(8 + m), e - 10);
  return (c & 0x80) ? -v : v;
}

inline double clamped_swiglu(double g, double u, double limit) {
  if (limit > 0.0) {
    g = g < -limit ? -limit : (g > limit ? limit : g);
    u = u < -limit ? -limit : (u > limit ? limit : u);
  }
  return g / (1.0 + std::exp(-g)) * u;
}

}  // namespace

extern "C" {

// Nearest-even E4M3 code of q, saturating at +-448. Within a binade [2^e, 2^(e+1)), e >= -6,
// the codes are 8 apart per binade and consecutive in magnitude, so the code of |q| is
// 8e + 48 + round(|q| * 2^(3-e)) (a mantissa that rounds up to 16 lands on the next binade's
// first code); below 2^-6 the subnormal code is round(|q| * 2^9). The scalings by powers of two
// are exact, so the only rounding is the one to an integer, nearest-even (rint in the default
// rounding mode). The sign bit is copied, so -0 encodes as 0x80.
uint8_t oracle_e4m3_from_float(float q) {
  const bool neg = std::signbit(q);
  double a = std::fabs(static_cast<double>(q));
  if (a > 448.0) a = 448.0;
  int code;
  if (a < std::ldexp(1.0, -6)) {
    code = static_cast<int>(std::rint(std::ldexp(a, 9)));
  } else {
    int e;
    (void)std::frexp(a, &e);  // a = f * 2^e, f in [0.5, 1): binade exponent e - 1
    e -= 1;
    code = 8 * e + 48 + static_cast<int>(std::rint(std::ldexp(a, 3 - e)));
  }
  return static_cast<uint8_t>(code | (neg ? 0x80 : 0));
}

void oracle_e4m3_from_float_array(long n, const float* q, uint8_t* codes) {
  for (long i = 0; i < n; ++i) codes[i] = oracle_e4m3_from_float(q[i]);
}

void oracle_quant_rows_e4m3(int rows, int cols, const uint16_t* v, uint8_t* codes,
                            float* scales) {
  for (int r = 0; r < rows; ++r) {
    const uint16_t* vr = v + static_cast<size_t>(r) * cols;
    float amax = 0.f;
    for (int c = 0; c < cols; ++c) {
      const float a = std::fabs(bf32(vr[c]));
      if (a > amax) amax = a;
    }
    float inv = 1.f, scale = 1.f;
    if (amax > 0.f) {
      const float q = 448.0f / amax;
      if (std::isfinite(q)) {  // else the row is below what a scaled E4M3 code can reach
        inv = q;
        scale = amax / 448.0f;
      }
    }
    scales[r] = scale;
    uint8_t* cr = codes + static_cast<size_t>(r) * cols;
    for (int c = 0; c < cols; ++c) {
      float q = bf32(vr[c]) * inv;
      q = q < -448.f ? -448.f : (q > 448.f ? 448.f : q);
      cr[c] = oracle_e4m3_from_float(q);
    }
  }
}

// gate/up of one expert on n rows of quantised activations (codes [n][H], scales [n]);
// qg, qu [I][H] codes with scales cg, cu [I]; h [n][I] bf16.
void oracle_gateup_rows_w8a8(int n, int H, int I, double limit, const uint8_t* xq,
                             const float* sx, const uint8_t* qg, const float* cg,
                             const uint8_t* qu, const float* cu, uint16_t* h) {
#pragma omp parallel for schedule(static)
  for (long ri = 0; ri < static_cast<long>(n) * I; ++ri) {
    const long r = ri / I, i = ri % I;
    const uint8_t* a = xq + static_cast<size_t>(r) * H;
    const uint8_t* wg = qg + static_cast<size_t>(i) * H;
    const uint8_t* wu = qu + static_cast<size_t>(i) * H;
    double g = 0.0, u = 0.0;
    for (int k = 0; k < H; ++k) {
      const double av = e4m3_value(a[k]);
      g += av * e4m3_value(wg[k]);
      u += av * e4m3_value(wu[k]);
    }
    // the scaled projections as fp32 values, as in the bf16 form
    const double g32 = static_cast<float>(g * static_cast<double>(cg[i]) * static_cast<double>(sx[r]));
    const double u32 = static_cast<float>(u * static_cast<double>(cu[i]) * static_cast<double>(sx[r]));
    h[static_cast<size_t>(r) * I + i] = oracle_bf16_from_double(clamped_swiglu(g32, u32, limit));
  }
}

// down of one expert on n rows of quantised h (codes [n][I], scales [n]); qd [H][I] codes with
// scales cd [H]; y [n][H] bf16.
void oracle_down_rows_w8a8(int n, int H, int I, const uint8_t* hq, const float* sh,
                           const uint8_t* qd, const float* cd, uint16_t* y) {
#pragma omp parallel for schedule(static)
  for (long rc = 0; rc < static_cast<long>(n) * H; ++rc) {
    const long r = rc / H, c = rc % H;
    const uint8_t* a = hq + static_cast<size_t>(r) * I;
    const uint8_t* w = qd + static_cast<size_t>(c) * I;
    double s = 0.0;
    for (int i = 0; i < I; ++i) s += e4m3_value(a[i]) * e4m3_value(w[i]);
    s = s * static_cast<double>(cd[c]) * static_cast<double>(sh[r]);
    y[static_cast<size_t>(r) * H + c] = oracle_bf16_from_double(static_cast<float>(s));
  }
}

// One expert's FFN on n rows of quantised x: gate/up -> h (bf16) -> per-row quantisation of
// h -> down -> y. h may be NULL.
static void expert_rows_w8a8(int n, int H, int I, double limit, const uint8_t* xq,
                             const float* sx, const uint8_t* qg, const float* cg,
                             const uint8_t* qu, const float* cu, const uint8_t* qd,
                             const float* cd, uint16_t* h_out, uint16_t* y) {
  std::vector<uint16_t> h(static_cast<size_t>(n) * I);
  oracle_gateup_rows_w8a8(n, H, I, limit, xq, sx, qg, cg, qu, cu, h.data());
  std::vector<uint8_t> hq(h.size());
  std::vector<float> sh(n);
  oracle_quant_rows_e4m3(n, I, h.data(), hq.data(), sh.data());
  oracle_down_rows_w8a8(n, H, I, hq.data(), sh.data(), qd, cd, y);
  if (h_out) std::memcpy(h_out, h.data(), sizeof(uint16_t) * h.size());
}

// The layer with FP8 expert weights and per-row FP8 activations. Arguments as
// oracle_layer_forward_fp8; xq [T][H] and sx [T] receive the quantised input.
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
                               uint16_t* y_shared, uint16_t* out) {
  // 1-5: routing and dispatch exactly as in the bf16 layer (the router stays bf16)
  if (!use_logits) oracle_router_logits(T, H, E, x, wr, bias, nullptr, 0, logits);
  oracle_route_from_logits(T, E, K, norm_topk, scale, logits, topk_idx, topk_w, nullptr);
  oracle_dispatch(T, K, E, capacity, topk_idx, counts, offsets, row_to_slot, slot_to_row);
  // the activations of every token, quantised once per row
  oracle_quant_rows_e4m3(T, H, x, xq, sx);
  // 6. routed experts on their gathered rows
  const size_t wi = static_cast<size_t>(I) * H;
  for (int e = 0; e < E; ++e) {
    const int n = counts[e];
    if (n == 0) continue;
    std::vector<uint8_t> xg(static_cast<size_t>(n) * H);
    std::vector<float> sg(n);
    for (int i = 0; i < n; ++i) {
      const int t = row_to_slot[offsets[e] + i] / K;
      std::memcpy(&xg[static_cast<size_t>(i) * H], xq + static_cast<size_t>(t) * H, H);
      sg[i] = sx[t];
    }
    expert_rows_w8a8(n, H, I, limit, xg.data(), sg.data(), qg + e * wi,
                     cg + static_cast<size_t>(e) * I, qu + e * wi, cu + static_cast<size_t>(e) * I,
                     qd + e * wi, cd + static_cast<size_t>(e) * H,
                     h_routed ? h_routed + static_cast<size_t>(offsets[e]) * I : nullptr,
                     y_routed + static_cast<size_t>(offsets[e]) * H);
  }
  // 7. shared expert on every token
  std::vector<uint16_t> ysbuf;
  uint16_t* ys = nullptr;
  if (sqg) {
    ys = y_shared;
    if (!ys) {
      ysbuf.resize(static_cast<size_t>(T) * H);
      ys = ysbuf.data();
    }
    expert_rows_w8a8(T, H, I, limit, xq, sx, sqg, scg, squ, scu, sqd, scd, h_shared, ys);
  }
  // 8. combine
  oracle_combine(T, K, H, topk_w, slot_to_row, y_routed, ys, out);
}

}  // extern "C"
