// moe_oracle_bwd.cpp -- plain CPU reference of the backward pass of the sparse MoE FFN layer.
//
// TEST INFRASTRUCTURE, like moe_oracle.cpp (same rules: tests, smoke check and CPU baseline
// only; nothing shared with the HIP library). The pages train the router (Hy3 deep-dive
// `SparseMoERouter` training branch with its load-balancing loss; Hy4 deep-dive `MoERouter`
// scores noise) but print no backward pass; this file differentiates the forward that
// moe_oracle.cpp computes, step by step in reverse:
//   combine      out = sum_j w_j y_j + y_shared
//   down         y = h Wd^T
//   SwiGLU       h = silu(clamp(g)) * clamp(u), g = x Wg^T, u = x Wu^T (clamp to [-L, L];
//                 the clamp passes the gradient where -L <= v <= L, as torch.clamp does)
//   routing      w_j = s p_j / sum_S p (or s p_j), p = softmax(logits); the top-k choice is
//                 piecewise constant and carries no gradient
//   router       logits = x Wr^T (+ bias, + noise)
//   loss term    d_aux * E * sum_e P_e f_e with f fixed (a selection frequency)
// Every sum is a sequential double sum. With round_bf16 set, the tensors the GPU stores in bf16
// are rounded to bf16 at the same points (dy, dh, dg, du, the per-row dx, the final dx, and the
// recomputed forward h and y), and the recomputed g, u and y sums are fp32 values first, as in
// the forward; with it clear everything stays exact double, which is what the pins against
// automatic differentiation use.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "moe_oracle.h"

namespace {

inline double bf(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

inline double rnd(double v, int round) {
  return round ? bf(oracle_bf16_from_double(v)) : v;
}

// the fp32 value of a projection (g, u, y), as the forward forms it, when rounding
inline double f32r(double v, int round) { return round ? static_cast<double>(static_cast<float>(v)) : v; }

inline double clampv(double v, double limit) {
  if (limit <= 0.0) return v;
  return v < -limit ? -limit : (v > limit ? limit : v);
}

inline double passes(double v, double limit) {
  return (limit <= 0.0 || (v >= -limit && v <= limit)) ? 1.0 : 0.0;
}

inline double sigmoid(double v) { return 1.0 / (1.0 + std::exp(-v)); }

}  // namespace

extern "C" {

void oracle_combine_bwd(int T, int K, int H, int round, const float* topk_w,
                        const int32_t* slot_to_row, const double* y_rows, const uint16_t* dout,
                        double* dy_rows, double* d_topk_w) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < K; ++j) {
      const size_t s = static_cast<size_t>(t) * K + j;
      const int r = slot_to_row[s];
      if (r < 0) {
        d_topk_w[s] = 0.0;
        continue;
      }
      double d = 0.0;
      for (int c = 0; c < H; ++c) {
        const double go = bf(dout[static_cast<size_t>(t) * H + c]);
        d += go * y_rows[static_cast<size_t>(r) * H + c];
        dy_rows[static_cast<size_t>(r) * H + c] = rnd(static_cast<double>(topk_w[s]) * go, round);
      }
      d_topk_w[s] = d;
    }
  }
}

void oracle_down_bwd_rows(int n, int H, int I, int round, const double* dy, const uint16_t* wd,
                          double* dh) {
#pragma omp parallel for schedule(static)
  for (long ri = 0; ri < static_cast<long>(n) * I; ++ri) {
    const long r = ri / I, i = ri % I;
    double s = 0.0;
    for (int c = 0; c < H; ++c) s += dy[static_cast<size_t>(r) * H + c] * bf(wd[static_cast<size_t>(c) * I + i]);
    dh[ri] = rnd(s, round);
  }
}

void oracle_swiglu_bwd_rows(int n, int H, int I, double limit, int round, const uint16_t* x_rows,
                            const uint16_t* wg, const uint16_t* wu, const double* dh, double* dg,
                            double* du) {
#pragma omp parallel for schedule(static)
  for (long ri = 0; ri < static_cast<long>(n) * I; ++ri) {
    const long r = ri / I, i = ri % I;
    double g = 0.0, u = 0.0;
    for (int k = 0; k < H; ++k) {
      const double xv = bf(x_rows[static_cast<size_t>(r) * H + k]);
      g += xv * bf(wg[static_cast<size_t>(i) * H + k]);
      u += xv * bf(wu[static_cast<size_t>(i) * H + k]);
    }
    g = f32r(g, round);
    u = f32r(u, round);
    const double gc = clampv(g, limit), uc = clampv(u, limit);
    const double sg = sigmoid(gc);
    const double silu = gc * sg;
    const double dsilu = sg * (1.0 + gc * (1.0 - sg));
    dg[ri] = rnd(dh[ri] * uc * dsilu * passes(g, limit), round);
    du[ri] = rnd(dh[ri] * silu * passes(u, limit), round);
  }
}

void oracle_gateup_dgrad_rows(int n, int H, int I, int round, const double* dg, const double* du,
                              const uint16_t* wg, const uint16_t* wu, double* dx) {
#pragma omp parallel for schedule(static)
  for (long rc = 0; rc < static_cast<long>(n) * H; ++rc) {
    const long r = rc / H, c = rc % H;
    double s = 0.0;
    for (int i = 0; i < I; ++i)
      s += dg[static_cast<size_t>(r) * I + i] * bf(wg[static_cast<size_t>(i) * H + c]) +
           du[static_cast<size_t>(r) * I + i] * bf(wu[static_cast<size_t>(i) * H + c]);
    dx[rc] = rnd(s, round);
  }
}

void oracle_wgrad(int n, int M, int N, const double* A, const double* B, double* out) {
#pragma omp parallel for schedule(static)
  for (long mn = 0; mn < static_cast<long>(M) * N; ++mn) {
    const long m = mn / N, c = mn % N;
    double s = 0.0;
    for (int r = 0; r < n; ++r) s += A[static_cast<size_t>(r) * M + m] * B[static_cast<size_t>(r) * N + c];
    out[mn] = s;
  }
}

void oracle_router_bwd(int T, int E, int K, int norm_topk, double scale, const float* logits,
                       const int32_t* topk_idx, const double* d_topk_w, double d_aux,
                       double* d_logits) {
  // load fractions f_e from the selections (the loss term's f, held fixed)
  std::vector<double> f(E, 0.0);
  for (size_t i = 0; i < static_cast<size_t>(T) * K; ++i) f[topk_idx[i]] += 1.0;
  for (int e = 0; e < E; ++e) f[e] /= static_cast<double>(T) * K;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const float* l = logits + static_cast<size_t>(t) * E;
    double m = l[0];
    for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
    std::vector<double> p(E), dp(E, 0.0);
    double z = 0.0;
    for (int e = 0; e < E; ++e) {
      p[e] = std::exp(static_cast<double>(l[e]) - m);
      z += p[e];
    }
    for (int e = 0; e < E; ++e) p[e] /= z;
    const int32_t* idx = topk_idx + static_cast<size_t>(t) * K;
    const double* dw = d_topk_w + static_cast<size_t>(t) * K;
    if (norm_topk) {
      // w_j = s p_j / Z, Z = sum_S p: dp_k = (s / Z) dw_k - (s / Z^2) sum_j dw_j p_j
      double Z = 0.0, wsum = 0.0;
      for (int j = 0; j < K; ++j) Z += p[idx[j]];
      for (int j = 0; j < K; ++j) wsum += dw[j] * p[idx[j]];
      for (int j = 0; j < K; ++j) dp[idx[j]] += scale / Z * dw[j] - scale / (Z * Z) * wsum;
    } else {
      for (int j = 0; j < K; ++j) dp[idx[j]] += scale * dw[j];
    }
    // loss term: d/dp[t,e] of d_aux * E * sum_e (1/T) p[t,e] f_e
    for (int e = 0; e < E; ++e) dp[e] += d_aux * E * f[e] / T;
    // softmax: dl_e = p_e (dp_e - sum_k p_k dp_k)
    double dot = 0.0;
    for (int e = 0; e < E; ++e) dot += p[e] * dp[e];
    for (int e = 0; e < E; ++e) d_logits[static_cast<size_t>(t) * E + e] = p[e] * (dp[e] - dot);
  }
}

void oracle_layer_backward(int T, int H, int E, int K, int I, int norm_topk, double scale,
                           double limit, int round, const uint16_t* x, const uint16_t* wr,
                           const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                           const uint16_t* sg, const uint16_t* su, const uint16_t* sd,
                           const float* logits, const int32_t* topk_idx, const float* topk_w,
                           const int32_t* counts, const int32_t* offsets,
                           const int32_t* row_to_slot, const int32_t* slot_to_row,
                           const uint16_t* dout, double d_aux, double* d_topk_w,
                           double* d_logits, double* dx, double* d_wr, double* d_wg,
                           double* d_wu, double* d_wd, double* d_sg, double* d_su, double* d_sd,
                           double* dh_rows, double* dg_rows, double* du_rows, double* dx_rows,
                           double* dx_router) {
  const size_t R = static_cast<size_t>(offsets[E]);
  const bool shared = sg != nullptr;
  // forward recompute of every kept row's h and y (rounded as the forward stores them)
  std::vector<uint16_t> xg(R * H);
  for (size_t r = 0; r < R; ++r)
    std::memcpy(&xg[r * H], x + static_cast<size_t>(row_to_slot[r] / K) * H, sizeof(uint16_t) * H);
  std::vector<double> h(R * I), y(R * H);
  auto fwd_rows = [&](int n, const uint16_t* xr, const uint16_t* g, const uint16_t* u,
                      const uint16_t* d, double* hh, double* yy) {
#pragma omp parallel for schedule(static)
    for (long ri = 0; ri < static_cast<long>(n) * I; ++ri) {
      const long r = ri / I, i = ri % I;
      double gv = 0.0, uv = 0.0;
      for (int k = 0; k < H; ++k) {
        const double xv = bf(xr[static_cast<size_t>(r) * H + k]);
        gv += xv * bf(g[static_cast<size_t>(i) * H + k]);
        uv += xv * bf(u[static_cast<size_t>(i) * H + k]);
      }
      gv = f32r(gv, round);
      uv = f32r(uv, round);
      const double gc = clampv(gv, limit), uc = clampv(uv, limit);
      hh[ri] = rnd(gc * sigmoid(gc) * uc, round);
    }
#pragma omp parallel for schedule(static)
    for (long rc = 0; rc < static_cast<long>(n) * H; ++rc) {
      const long r = rc / H, c = rc % H;
      double s = 0.0;
      for (int i = 0; i < I; ++i) s += hh[static_cast<size_t>(r) * I + i] * bf(d[static_cast<size_t>(c) * I + i]);
      yy[rc] = rnd(f32r(s, round), round);
    }
  };
  const size_t IH = static_cast<size_t>(I) * H;
  for (int e = 0; e < E; ++e) {
    const int n = counts[e];
    if (n == 0) continue;
    const size_t o = static_cast<size_t>(offsets[e]);
    fwd_rows(n, &xg[o * H], wg + e * IH, wu + e * IH, wd + e * IH, &h[o * I], &y[o * H]);
  }
  // combine backward: routed rows and routing-weight gradients
  std::vector<double> dy(R * H);
  oracle_combine_bwd(T, K, H, round, topk_w, slot_to_row, y.data(), dout, dy.data(), d_topk_w);
  // routed experts, expert-major: dh, dg/du, per-row dx and the weight gradients
  std::vector<double> dh(R * I), dgv(R * I), duv(R * I), dxr(R * H), xgd(R * H);
  for (size_t i = 0; i < R * H; ++i) xgd[i] = bf(xg[i]);
  for (int e = 0; e < E; ++e) {
    const size_t o = static_cast<size_t>(offsets[e]);
    const int n = counts[e];
    double* gwd = d_wd + e * IH;
    double* gwg = d_wg + e * IH;
    double* gwu = d_wu + e * IH;
    if (n == 0) {
      std::fill(gwd, gwd + IH, 0.0);
      std::fill(gwg, gwg + IH, 0.0);
      std::fill(gwu, gwu + IH, 0.0);
      continue;
    }
    oracle_down_bwd_rows(n, H, I, round, &dy[o * H], wd + e * IH, &dh[o * I]);
    oracle_swiglu_bwd_rows(n, H, I, limit, round, &xg[o * H], wg + e * IH, wu + e * IH, &dh[o * I],
                           &dgv[o * I], &duv[o * I]);
    oracle_gateup_dgrad_rows(n, H, I, round, &dgv[o * I], &duv[o * I], wg + e * IH, wu + e * IH,
                             &dxr[o * H]);
    oracle_wgrad(n, H, I, &dy[o * H], &h[o * I], gwd);
    oracle_wgrad(n, I, H, &dgv[o * I], &xgd[o * H], gwg);
    oracle_wgrad(n, I, H, &duv[o * I], &xgd[o * H], gwu);
  }
  if (dh_rows) std::memcpy(dh_rows, dh.data(), sizeof(double) * R * I);
  if (dg_rows) std::memcpy(dg_rows, dgv.data(), sizeof(double) * R * I);
  if (du_rows) std::memcpy(du_rows, duv.data(), sizeof(double) * R * I);
  if (dx_rows) std::memcpy(dx_rows, dxr.data(), sizeof(double) * R * H);
  // shared expert: weight 1, identity rows, output gradient as its dy
  std::vector<double> dxs;
  if (shared) {
    std::vector<double> hs(static_cast<size_t>(T) * I), ys(static_cast<size_t>(T) * H);
    fwd_rows(T, x, sg, su, sd, hs.data(), ys.data());
    std::vector<double> dys(static_cast<size_t>(T) * H), xd(static_cast<size_t>(T) * H);
    for (size_t i = 0; i < static_cast<size_t>(T) * H; ++i) {
      dys[i] = bf(dout[i]);
      xd[i] = bf(x[i]);
    }
    std::vector<double> dhs(static_cast<size_t>(T) * I), dgs(dhs.size()), dus(dhs.size());
    dxs.resize(static_cast<size_t>(T) * H);
    oracle_down_bwd_rows(T, H, I, round, dys.data(), sd, dhs.data());
    oracle_swiglu_bwd_rows(T, H, I, limit, round, x, sg, su, dhs.data(), dgs.data(), dus.data());
    oracle_gateup_dgrad_rows(T, H, I, round, dgs.data(), dus.data(), sg, su, dxs.data());
    oracle_wgrad(T, H, I, dys.data(), hs.data(), d_sd);
    oracle_wgrad(T, I, H, dgs.data(), xd.data(), d_sg);
    oracle_wgrad(T, I, H, dus.data(), xd.data(), d_su);
  }
  // router: routing-weight gradients (and the loss term) to logits, then to Wr and x
  oracle_router_bwd(T, E, K, norm_topk, scale, logits, topk_idx, d_topk_w, d_aux, d_logits);
  std::vector<double> xd(static_cast<size_t>(T) * H);
  for (size_t i = 0; i < xd.size(); ++i) xd[i] = bf(x[i]);
  oracle_wgrad(T, E, H, d_logits, xd.data(), d_wr);
  std::vector<double> dxrt(static_cast<size_t>(T) * H);
#pragma omp parallel for schedule(static)
  for (long tc = 0; tc < static_cast<long>(T) * H; ++tc) {
    const long t = tc / H, c = tc % H;
    double s = 0.0;
    for (int e = 0; e < E; ++e) s += d_logits[static_cast<size_t>(t) * E + e] * bf(wr[static_cast<size_t>(e) * H + c]);
    dxrt[tc] = s;
  }
  if (dx_router) std::memcpy(dx_router, dxrt.data(), sizeof(double) * T * H);
  // dx: the token's routed rows in slot order, then the shared row, then the router term
#pragma omp parallel for schedule(static)
  for (long tc = 0; tc < static_cast<long>(T) * H; ++tc) {
    const long t = tc / H, c = tc % H;
    double s = 0.0;
    for (int j = 0; j < K; ++j) {
      const int r = slot_to_row[static_cast<size_t>(t) * K + j];
      if (r >= 0) s += dxr[static_cast<size_t>(r) * H + c];
    }
    if (shared) s += dxs[tc];
    s += dxrt[tc];
    dx[tc] = rnd(s, round);
  }
}

}  // extern "C"
