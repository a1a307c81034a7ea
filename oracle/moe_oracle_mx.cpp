// moe_oracle_mx.cpp -- plain CPU reference of the block-scaled FP8 (MXFP8) form of the expert
// FFN: every 32 consecutive elements along the reduction dimension share one power-of-two scale
// (OCP Microscaling MX v1.0: E8M0 scale byte s, value 2^(s - 127); elements OCP E4M3).
//
// TEST INFRASTRUCTURE: loaded only by the tests, the smoke check and the CPU-baseline leg of
// the benchmark; shares nothing with the HIP library.
//
// The pages deploy the model from an FP8 checkpoint (Tencent Hunyuan Hy4 Preview deep technical
// analysis, deployment commands; Hy4 config walkthrough, dtype notes) without defining its scale
// format. This file takes the MX block format for both operands of each expert projection:
//   weights: codes [N][K] with scales [N][K/32] (given);
//   activations (x for gate/up, h for down): quantised here, per row and per 32-element block,
//   by the MX conversion rule:
//     amax   = max |v| over the block (v: the bf16 values)
//     shared = floor(log2(amax)) - 8, clamped to [-127, 127]  (8: exponent of E4M3's largest
//              normal, 448 = 1.75 * 2^8); an all-zero block takes -127
//     scale byte s = shared + 127,  code = E4M3_RNE(clamp(v / 2^shared, -448, 448))
//   so v / 2^shared lies in [-512, 512) and only magnitudes in (448, 512) saturate.
// Each projection is the sum over k of e4m3(a_code) 2^(sa-127) * e4m3(w_code) 2^(sw-127), every
// term exact in double, summed sequentially in double, rounded to an fp32 value, then rounded
// where the bf16 path rounds (h after the clamped SwiGLU, y).

#include "moe_oracle.h"

#include <cmath>
#include <cstring>
#include <vector>

namespace {

constexpr int kBlock = 32;  // elements per scale block

inline double bf64(uint16_t b) { return oracle_double_from_bf16(b); }

// value of an E4M3 code (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
// holds the subnormals m * 2^-9; 0x7F / 0xFF are NaN and never produced here)
inline double e4m3_value(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  const double v = e == 0 ? std::ldexp(static_cast<double>(m), -9)
                          : std::ldexp(static_cast<double>(8 + m), e - 10);
  return (c & 0x80) ? -v : v;
}

// nearest-even E4M3 code of a double, saturating at +-448 (the same construction as the per-row
// quantiser's: a code per binade step, the only rounding an integer rint)
inline uint8_t e4m3_code(double q) {
  const bool neg = std::signbit(q);
  double a = std::fabs(q);
  if (a > 448.0) a = 448.0;
  int code;
  if (a < std::ldexp(1.0, -6)) {
    code = static_cast<int>(std::rint(std::ldexp(a, 9)));
  } else {
    int e;
    (void)std::frexp(a, &e);
    e -= 1;
    code = 8 * e + 48 + static_cast<int>(std::rint(std::ldexp(a, 3 - e)));
  }
  return static_cast<uint8_t>(code | (neg ? 0x80 : 0));
}

inline double mx_value(uint8_t code, uint8_t s) { return std::ldexp(e4m3_value(code), s - 127); }

inline double clamped_swiglu(double g, double u, double limit) {
  if (limit > 0.0) {
    g = g < -limit ? -limit : (g > limit ? limit : g);
    u = u < -limit ? -limit : (u > limit ? limit : u);
  }
  return g / (1.0 + std::exp(-g)) * u;
}

}  // namespace

extern "C" {

// The MX scale byte of a block with absolute maximum amax (a bf16 value): floor(log2(amax)) - 8
// clamped to [-127, 127], plus the bias 127; 0 for amax == 0.
uint8_t oracle_mx_scale_of_amax(double amax) {
  if (!(amax > 0.0)) return 0;
  int e;
  (void)std::frexp(amax, &e);  // amax = f * 2^e, f in [0.5, 1): floor(log2(amax)) = e - 1
  int shared = (e - 1) - 8;
  if (shared < -127) shared = -127;
  if (shared > 127) shared = 127;
  return static_cast<uint8_t>(shared + 127);
}

// MX quantisation of bf16 rows [rows][cols] (cols a multiple of 32): codes [rows][cols] and
// scale bytes [rows][cols / 32].
void oracle_mx_quant_rows(int rows, int cols, const uint16_t* v, uint8_t* codes, uint8_t* scales) {
  const int nb = cols / kBlock;
  for (int r = 0; r < rows; ++r) {
    const uint16_t* vr = v + static_cast<size_t>(r) * cols;
    for (int b = 0; b < nb; ++b) {
      double amax = 0.0;
      for (int c = 0; c < kBlock; ++c) {
        const double a = std::fabs(bf64(vr[b * kBlock + c]));
        if (a > amax) amax = a;
      }
      const uint8_t s = oracle_mx_scale_of_amax(amax);
      scales[static_cast<size_t>(r) * nb + b] = s;
      for (int c = 0; c < kBlock; ++c) {
        const size_t i = static_cast<size_t>(r) * cols + b * kBlock + c;
        codes[i] = e4m3_code(std::ldexp(bf64(vr[b * kBlock + c]), 127 - s));
      }
    }
  }
}

// Value of MX-encoded data: out[i] = e4m3(codes[i]) * 2^(scales[i / 32] - 127) for one row-major
// matrix [rows][cols].
void oracle_mx_dequant(int rows, int cols, const uint8_t* codes, const uint8_t* scales, double* out) {
  const int nb = cols / kBlock;
  for (long i = 0; i < static_cast<long>(rows) * cols; ++i) {
    const long r = i / cols, c = i % cols;
    out[i] = mx_value(codes[i], scales[r * nb + c / kBlock]);
  }
}

// sum_k of the MX products of row a (codes, scales) and row w over K elements
static double mx_dot(int K, const uint8_t* a, const uint8_t* sa, const uint8_t* w, const uint8_t* sw) {
  double s = 0.0;
  for (int k = 0; k < K; ++k) s += mx_value(a[k], sa[k / kBlock]) * mx_value(w[k], sw[k / kBlock]);
  return s;
}

// gate/up of one expert on n rows of MX activations (codes [n][H], scales [n][H/32]); weights
// qg, qu [I][H] with scales sg, su [I][H/32]; h [n][I] bf16.
void oracle_gateup_rows_mx(int n, int H, int I, double limit, const uint8_t* xq, const uint8_t* xs,
                           const uint8_t* qg, const uint8_t* sg, const uint8_t* qu, const uint8_t* su,
                           uint16_t* h) {
  const int nb = H / kBlock;
#pragma omp parallel for schedule(static)
  for (long ri = 0; ri < static_cast<long>(n) * I; ++ri) {
    const long r = ri / I, i = ri % I;
    const uint8_t* a = xq + static_cast<size_t>(r) * H;
    const uint8_t* as = xs + static_cast<size_t>(r) * nb;
    const double g = static_cast<float>(mx_dot(H, a, as, qg + static_cast<size_t>(i) * H, sg + static_cast<size_t>(i) * nb));
    const double u = static_cast<float>(mx_dot(H, a, as, qu + static_cast<size_t>(i) * H, su + static_cast<size_t>(i) * nb));
    h[static_cast<size_t>(r) * I + i] = oracle_bf16_from_double(clamped_swiglu(g, u, limit));
  }
}

// down of one expert on n rows of MX h (codes [n][I], scales [n][I/32]); qd [H][I] with scales
// sd [H][I/32]; y [n][H] bf16.
void oracle_down_rows_mx(int n, int H, int I, const uint8_t* hq, const uint8_t* hs, const uint8_t* qd,
                         const uint8_t* sd, uint16_t* y) {
  const int nb = I / kBlock;
#pragma omp parallel for schedule(static)
  for (long rc = 0; rc < static_cast<long>(n) * H; ++rc) {
    const long r = rc / H, c = rc % H;
    const double s = mx_dot(I, hq + static_cast<size_t>(r) * I, hs + static_cast<size_t>(r) * nb,
                            qd + static_cast<size_t>(c) * I, sd + static_cast<size_t>(c) * nb);
    y[static_cast<size_t>(r) * H + c] = oracle_bf16_from_double(static_cast<float>(s));
  }
}

// One expert's FFN on n rows of MX x: gate/up -> h (bf16) -> MX quantisation of h -> down -> y.
// h_out may be NULL.
static void expert_rows_mx(int n, int H, int I, double limit, const uint8_t* xq, const uint8_t* xs,
                           const uint8_t* qg, const uint8_t* sg, const uint8_t* qu, const uint8_t* su,
                           const uint8_t* qd, const uint8_t* sd, uint16_t* h_out, uint16_t* y) {
  std::vector<uint16_t> h(static_cast<size_t>(n) * I);
  oracle_gateup_rows_mx(n, H, I, limit, xq, xs, qg, sg, qu, su, h.data());
  std::vector<uint8_t> hq(h.size()), hs(static_cast<size_t>(n) * (I / kBlock));
  oracle_mx_quant_rows(n, I, h.data(), hq.data(), hs.data());
  oracle_down_rows_mx(n, H, I, hq.data(), hs.data(), qd, sd, y);
  if (h_out) std::memcpy(h_out, h.data(), sizeof(uint16_t) * h.size());
}

// The layer with MX expert weights and MX activations. Weight scales are [E][N][K/32] per routed
// matrix stack and [N][K/32] for the shared expert's; everything else as
// oracle_layer_forward_w8a8, with xq [T][H] and xs [T][H/32] receiving the quantised input.
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
                             uint16_t* y_shared, uint16_t* out) {
  // 1-5: routing and dispatch exactly as in the bf16 layer (the router stays bf16)
  if (!use_logits) oracle_router_logits(T, H, E, x, wr, bias, nullptr, 0, logits);
  oracle_route_from_logits(T, E, K, norm_topk, scale, logits, topk_idx, topk_w, nullptr);
  oracle_dispatch(T, K, E, capacity, topk_idx, counts, offsets, row_to_slot, slot_to_row);
  // the activations of every token, quantised once
  const int hb = H / kBlock, ib = I / kBlock;
  oracle_mx_quant_rows(T, H, x, xq, xs);
  // 6. routed experts on their gathered rows
  const size_t wi = static_cast<size_t>(I) * H;
  const size_t si = static_cast<size_t>(I) * hb;  // scale bytes of one [I][H] or [H][I] matrix
  for (int e = 0; e < E; ++e) {
    const int n = counts[e];
    if (n == 0) continue;
    std::vector<uint8_t> xg(static_cast<size_t>(n) * H), xsg(static_cast<size_t>(n) * hb);
    for (int i = 0; i < n; ++i) {
      const int t = row_to_slot[offsets[e] + i] / K;
      std::memcpy(&xg[static_cast<size_t>(i) * H], xq + static_cast<size_t>(t) * H, H);
      std::memcpy(&xsg[static_cast<size_t>(i) * hb], xs + static_cast<size_t>(t) * hb, hb);
    }
    expert_rows_mx(n, H, I, limit, xg.data(), xsg.data(), qg + e * wi, sg + e * si, qu + e * wi,
                   su + e * si, qd + e * wi, sd + static_cast<size_t>(e) * H * ib,
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
    expert_rows_mx(T, H, I, limit, xq, xs, sqg, ssg, squ, ssu, sqd, ssd, h_shared, ys);
  }
  // 8. combine
  oracle_combine(T, K, H, topk_w, slot_to_row, y_routed, ys, out);
}

}  // extern "C"
