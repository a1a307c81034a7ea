// oracle_driver.cpp -- runs every entry point of the CPU oracle on small random inputs, for a build
// under AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers_cpu.py). Checks
// only cheap invariants (counts, bijection, sparse == dense brute force); the numerics are
// pinned elsewhere. Exits non-zero on a failed invariant; the sanitizers abort on a report.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "moe_oracle.h"

namespace {

std::mt19937_64 rng(12345);

std::vector<uint16_t> bf16s(size_t n, double sd) {
  std::normal_distribution<double> nd(0.0, sd);
  std::vector<uint16_t> v(n);
  for (auto& b : v) b = oracle_bf16_from_double(nd(rng));
  return v;
}

std::vector<uint8_t> codes(size_t n) {
  std::uniform_int_distribution<int> ud(0, 255);
  std::vector<uint8_t> v(n);
  for (auto& c : v) {
    c = static_cast<uint8_t>(ud(rng));
    if ((c & 0x7F) == 0x7F) c &= 0xFE;  // no NaN codes
  }
  return v;
}

std::vector<float> scales(size_t n) {
  std::uniform_real_distribution<float> ud(1e-3f, 2e-3f);
  std::vector<float> v(n);
  for (auto& s : v) s = ud(rng);
  return v;
}

int failures = 0;
void check(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

struct Routing {
  std::vector<float> logits, topk_w;
  std::vector<int32_t> idx, counts, offsets, r2s, s2r;
};

void run_layer(int T, int H, int E, int K, int I, int capacity, bool shared) {
  auto x = bf16s(size_t(T) * H, 1.0), wr = bf16s(size_t(E) * H, 0.05);
  auto wg = bf16s(size_t(E) * I * H, 0.05), wu = bf16s(size_t(E) * I * H, 0.05),
       wd = bf16s(size_t(E) * H * I, 0.05);
  auto sg = bf16s(size_t(I) * H, 0.05), su = bf16s(size_t(I) * H, 0.05), sd = bf16s(size_t(H) * I, 0.05);
  std::vector<float> bias(E);
  for (int e = 0; e < E; ++e) bias[e] = static_cast<float>(0.3 * std::log(1.0 / (e + 1)));
  const size_t TK = size_t(T) * K;
  Routing r;
  r.logits.resize(size_t(T) * E);
  r.topk_w.resize(TK);
  r.idx.resize(TK);
  r.counts.resize(E);
  r.offsets.resize(E + 1);
  r.r2s.resize(TK);
  r.s2r.resize(TK);
  std::vector<uint16_t> hr(TK * I), yr(TK * H), hs(size_t(T) * I), ys(size_t(T) * H), out(size_t(T) * H);
  oracle_layer_forward(T, H, E, K, I, 1, 2.827, 10.0, capacity, x.data(), wr.data(), bias.data(),
                       wg.data(), wu.data(), wd.data(), shared ? sg.data() : nullptr,
                       shared ? su.data() : nullptr, shared ? sd.data() : nullptr, 0,
                       r.logits.data(), r.idx.data(), r.topk_w.data(), r.counts.data(),
                       r.offsets.data(), r.r2s.data(), r.s2r.data(), hr.data(), yr.data(),
                       shared ? hs.data() : nullptr, shared ? ys.data() : nullptr, out.data());
  int kept = 0;
  for (int e = 0; e < E; ++e) kept += r.counts[e];
  check(r.offsets[E] == kept, "offsets[E] == sum counts");
  for (int rr = 0; rr < kept; ++rr) check(r.s2r[r.r2s[rr]] == rr, "slot_to_row o row_to_slot == id");
  // sparse == dense brute force
  std::vector<uint16_t> dense(size_t(T) * H);
  oracle_layer_dense(T, H, E, K, I, 10.0, x.data(), wg.data(), wu.data(), wd.data(),
                     shared ? sg.data() : nullptr, shared ? su.data() : nullptr,
                     shared ? sd.data() : nullptr, r.idx.data(), r.topk_w.data(), r.s2r.data(),
                     dense.data());
  check(std::memcmp(dense.data(), out.data(), dense.size() * 2) == 0, "sparse == dense");
  // the router's token-subset mode and the training statistics
  std::vector<int32_t> toks = {0, T - 1};
  std::vector<float> lg2(size_t(T) * E, 0.f);
  oracle_router_logits(T, H, E, x.data(), wr.data(), bias.data(), toks.data(), 2, lg2.data());
  std::vector<double> pm(E), lf(E), ema(E, 1.0), aux(1), emt(1, 10.0), probs(size_t(T) * E);
  oracle_router_train_stats(T, E, K, r.logits.data(), r.idx.data(), 0.9, pm.data(), lf.data(),
                            aux.data(), ema.data(), emt.data());
  oracle_route_from_logits(T, E, K, 0, 1.0, r.logits.data(), r.idx.data(), r.topk_w.data(), probs.data());

  // FP8 weights (codes + row scales) and the W8A8 form
  auto qg = codes(size_t(E) * I * H), qu = codes(size_t(E) * I * H), qd = codes(size_t(E) * H * I);
  auto cg = scales(size_t(E) * I), cu = scales(size_t(E) * I), cd = scales(size_t(E) * H);
  auto sqg = codes(size_t(I) * H), squ = codes(size_t(I) * H), sqd = codes(size_t(H) * I);
  auto scg = scales(I), scu = scales(I), scd = scales(H);
  std::vector<uint16_t> out8(size_t(T) * H), dense8(size_t(T) * H);
  Routing r8 = r;
  oracle_layer_forward_fp8(T, H, E, K, I, 1, 2.827, 10.0, capacity, x.data(), wr.data(), bias.data(),
                           qg.data(), cg.data(), qu.data(), cu.data(), qd.data(), cd.data(),
                           shared ? sqg.data() : nullptr, scg.data(), shared ? squ.data() : nullptr,
                           scu.data(), shared ? sqd.data() : nullptr, scd.data(), 1,
                           r.logits.data(), r8.idx.data(), r8.topk_w.data(), r8.counts.data(),
                           r8.offsets.data(), r8.r2s.data(), r8.s2r.data(), hr.data(), yr.data(),
                           shared ? hs.data() : nullptr, shared ? ys.data() : nullptr, out8.data());
  oracle_layer_dense_fp8(T, H, E, K, I, 10.0, x.data(), qg.data(), cg.data(), qu.data(), cu.data(),
                         qd.data(), cd.data(), shared ? sqg.data() : nullptr, scg.data(),
                         shared ? squ.data() : nullptr, scu.data(), shared ? sqd.data() : nullptr,
                         scd.data(), r8.idx.data(), r8.topk_w.data(), r8.s2r.data(), dense8.data());
  check(std::memcmp(dense8.data(), out8.data(), out8.size() * 2) == 0, "FP8 sparse == dense");
  std::vector<uint8_t> xq(size_t(T) * H);
  std::vector<float> sx(T);
  oracle_layer_forward_w8a8(T, H, E, K, I, 1, 2.827, 10.0, capacity, x.data(), wr.data(), bias.data(),
                            qg.data(), cg.data(), qu.data(), cu.data(), qd.data(), cd.data(),
                            shared ? sqg.data() : nullptr, scg.data(), shared ? squ.data() : nullptr,
                            scu.data(), shared ? sqd.data() : nullptr, scd.data(), 1,
                            r.logits.data(), r8.idx.data(), r8.topk_w.data(), r8.counts.data(),
                            r8.offsets.data(), r8.r2s.data(), r8.s2r.data(), xq.data(), sx.data(),
                            hr.data(), yr.data(), shared ? hs.data() : nullptr,
                            shared ? ys.data() : nullptr, out8.data());

  // MX block-scaled FP8 weights and activations (scales one byte per 32 elements)
  auto mxs = [&](size_t n) {
    std::uniform_int_distribution<int> ud(112, 132);
    std::vector<uint8_t> v(n);
    for (auto& c : v) c = static_cast<uint8_t>(ud(rng));
    return v;
  };
  if (H % 32 == 0 && I % 32 == 0) {
    auto mg = mxs(size_t(E) * I * H / 32), mu = mxs(size_t(E) * I * H / 32), md = mxs(size_t(E) * H * I / 32);
    auto smg = mxs(size_t(I) * H / 32), smu = mxs(size_t(I) * H / 32), smd = mxs(size_t(H) * I / 32);
    std::vector<uint8_t> xs(size_t(T) * H / 32);
    Routing rm = r;
    oracle_layer_forward_mx(T, H, E, K, I, 1, 2.827, 10.0, capacity, x.data(), wr.data(), bias.data(),
                            qg.data(), mg.data(), qu.data(), mu.data(), qd.data(), md.data(),
                            shared ? sqg.data() : nullptr, smg.data(), shared ? squ.data() : nullptr,
                            smu.data(), shared ? sqd.data() : nullptr, smd.data(), 1, r.logits.data(),
                            rm.idx.data(), rm.topk_w.data(), rm.counts.data(), rm.offsets.data(),
                            rm.r2s.data(), rm.s2r.data(), xq.data(), xs.data(), hr.data(), yr.data(),
                            shared ? hs.data() : nullptr, shared ? ys.data() : nullptr, out8.data());
    std::vector<double> deq(size_t(T) * H);
    oracle_mx_dequant(T, H, xq.data(), xs.data(), deq.data());
    for (double d : deq) check(std::isfinite(d), "finite MX value");
  }

  // backward, rounded and exact
  auto dout = bf16s(size_t(T) * H, 1.0);
  const size_t R = size_t(r.offsets[E]);
  std::vector<double> dtw(TK), dlg(size_t(T) * E), dx(size_t(T) * H), dwr(size_t(E) * H),
      dwg(size_t(E) * I * H), dwu(size_t(E) * I * H), dwd(size_t(E) * H * I), dsg(size_t(I) * H),
      dsu(size_t(I) * H), dsd(size_t(H) * I), dh(R * I + 1), dg(R * I + 1), du(R * I + 1),
      dxr(R * H + 1), dxrt(size_t(T) * H);
  for (int round = 0; round < 2; ++round)
    oracle_layer_backward(T, H, E, K, I, 1, 2.827, 10.0, round, x.data(), wr.data(), wg.data(),
                          wu.data(), wd.data(), shared ? sg.data() : nullptr,
                          shared ? su.data() : nullptr, shared ? sd.data() : nullptr,
                          r.logits.data(), r.idx.data(), r.topk_w.data(), r.counts.data(),
                          r.offsets.data(), r.r2s.data(), r.s2r.data(), dout.data(), 0.3,
                          dtw.data(), dlg.data(), dx.data(), dwr.data(), dwg.data(), dwu.data(),
                          dwd.data(), dsg.data(), dsu.data(), dsd.data(), dh.data(), dg.data(),
                          du.data(), dxr.data(), dxrt.data());
}

void run_quantiser() {
  const int rows = 6, cols = 40;
  std::vector<uint16_t> v(size_t(rows) * cols);
  const double mags[rows] = {1.0, 0.0, 1e-37, 1.4e-36, 300.0, 2.0e-40};
  std::normal_distribution<double> nd(0.0, 1.0);
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) v[size_t(r) * cols + c] = oracle_bf16_from_double(mags[r] * nd(rng));
  std::vector<uint8_t> q(v.size());
  std::vector<float> s(rows);
  oracle_quant_rows_e4m3(rows, cols, v.data(), q.data(), s.data());
  for (int r = 0; r < rows; ++r) check(std::isfinite(s[r]) && s[r] > 0.f, "finite positive scale");
  for (uint8_t c : q) check((c & 0x7F) != 0x7F, "no NaN code");
  const float edge[] = {0.f, -0.f, 448.f, -448.f, 1e30f, -1e30f, 1e-30f, 0.0009765625f, 240.5f};
  for (float f : edge) (void)oracle_e4m3_from_float(f);
  for (int c = 0; c < 256; ++c) (void)oracle_double_from_e4m3(static_cast<uint8_t>(c));
  const double bfe[] = {0.0, -0.0, 1e-45, 3.4e38, -3.4e38, 1e300, 1.0000000001, -2.5e-39};
  for (double d : bfe) (void)oracle_double_from_bf16(oracle_bf16_from_double(d));
}

}  // namespace

int main() {
  oracle_set_num_threads(3);
  run_layer(13, 64, 8, 2, 32, 0, true);
  run_layer(9, 32, 6, 3, 64, 2, false);  // capacity drops, no shared expert
  run_layer(1, 32, 4, 4, 32, 0, true);   // K = E
  run_quantiser();
  std::printf("oracle driver: %d failure(s)\n", failures);
  return failures ? 1 : 0;
}
