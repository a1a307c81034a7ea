// abi_driver.cpp -- exercises the host side of the C ABI (include/moe.h) without a GPU, for a
// build under AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers_cpu.py):
// every workspace-size and layout helper on valid, edge and invalid shapes, and every entry
// point on arguments its host checks reject before anything is launched. The pointers passed are
// never dereferenced (a rejected call touches no device memory). Exits non-zero when a call
// returns a code other than the one its checks promise.
#include <climits>
#include <cstdio>
#include <cstdint>

#include "moe.h"

namespace {

int failures = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAILED: %s returned %d, expected %d\n", what, got, want);
    ++failures;
  }
}

moe_shape hy4(int T) {
  moe_shape s{};
  s.T = T;
  s.H = 6144;
  s.E = 256;
  s.K = 8;
  s.I = 2048;
  s.n_shared = 1;
  s.norm_topk_prob = 1;
  s.routed_scaling = 2.827f;
  s.swiglu_limit = 10.f;
  return s;
}

// stand-in device addresses: 256-byte aligned and never dereferenced
uint16_t* const P16 = reinterpret_cast<uint16_t*>(uintptr_t(1) << 20);
float* const PF = reinterpret_cast<float*>(uintptr_t(1) << 20);
int32_t* const PI = reinterpret_cast<int32_t*>(uintptr_t(1) << 20);
uint8_t* const P8 = reinterpret_cast<uint8_t*>(uintptr_t(1) << 20);
void* const PW = reinterpret_cast<void*>(uintptr_t(1) << 20);

}  // namespace

int main() {
  for (int code = -6; code <= 1; ++code)
    if (!moe_strerror(code)) ++failures;

  // sizes and layouts over a range of shapes, including the extremes the checks accept
  const int Ts[] = {1, 3, 64, 1000, 8192, 65536, 1864135, 1864136, 238609293};
  for (int T : Ts) {
    moe_shape s = hy4(T);
    const size_t lw = moe_layer_workspace_size(&s);
    moe_layer_ws_layout lay{};
    const int rc = moe_layer_workspace_layout(&s, &lay);
    if ((rc == MOE_OK) != (lw > 0) || (rc == MOE_OK && lay.total != lw)) {
      std::fprintf(stderr, "FAILED: layout of T=%d\n", T);
      ++failures;
    }
    (void)moe_route_workspace_size(&s);
    (void)moe_route_train_workspace_size(&s);
    (void)moe_permute_workspace_size(&s);
    (void)moe_expert_ffn_workspace_size(&s, 257, T);
    (void)moe_layer_w8a8_workspace_size(&s);
    moe_layer_a8_ws_layout l8{};
    (void)moe_layer_w8a8_workspace_layout(&s, &l8);
    (void)moe_layer_backward_workspace_size(&s);
    moe_layer_mx_ws_layout lm{};
    if ((moe_layer_mx_workspace_layout(&s, &lm) == MOE_OK) != (moe_layer_mx_workspace_size(&s) > 0) ||
        (lm.total && lm.total != moe_layer_mx_workspace_size(&s))) {
      std::fprintf(stderr, "FAILED: MX layout of T=%d\n", T);
      ++failures;
    }
    moe_bwd_ws_layout lb{};
    (void)moe_layer_backward_workspace_layout(&s, &lb);
  }
  expect(moe_layer_workspace_size(nullptr) == 0 ? MOE_OK : -99, MOE_OK, "size of NULL shape");

  // shape errors (each entry point checks before any launch)
  moe_shape bad[8];
  for (auto& b : bad) b = hy4(64);
  bad[0].T = 0;
  bad[1].K = 300;
  bad[2].E = 257;
  bad[3].H = 6100;
  bad[4].n_shared = 2;
  bad[5].routed_scaling = 1.f / 0.f;
  bad[6].T = INT_MAX;
  bad[7].T = 1864136;  // h past 64 GiB at the Hy4 shape
  const int want[8] = {MOE_ERR_INVALID_ARG, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED,
                       MOE_ERR_UNSUPPORTED, MOE_ERR_INVALID_ARG, MOE_ERR_INVALID_ARG,
                       MOE_ERR_UNSUPPORTED, MOE_ERR_UNSUPPORTED};
  for (int i = 0; i < 8; ++i) {
    expect(moe_route(&bad[i], P16, P16, nullptr, nullptr, PF, PI, PW, 1 << 30, nullptr), want[i],
           "moe_route bad shape");
    expect(moe_permute(&bad[i], PI, PI, PI, PI, PI, PW, 1 << 30, nullptr), want[i],
           "moe_permute bad shape");
    expect(moe_layer_forward(&bad[i], P16, P16, nullptr, P16, P16, P16, P16, P16, P16, P16, PW,
                             size_t(1) << 40, nullptr),
           want[i], "moe_layer_forward bad shape");
    expect(moe_layer_forward_noalloc(&bad[i], P16, P16, nullptr, P16, P16, P16, P16, P16, P16,
                                     P16, nullptr),
           want[i], "moe_layer_forward_noalloc bad shape");
    expect(moe_combine(&bad[i], P16, PF, PI, nullptr, P16, nullptr), want[i], "moe_combine bad shape");
    expect(moe_layer_forward_mx(&bad[i], P16, P16, nullptr, P8, P8, P8, P8, P8, P8, P8, P8, P8, P8, P8,
                                P8, P16, PW, size_t(1) << 40, nullptr, nullptr),
           want[i], "moe_layer_forward_mx bad shape");
  }

  // argument errors on a valid shape
  moe_shape s = hy4(64);
  expect(moe_route(&s, nullptr, P16, nullptr, nullptr, PF, PI, PW, 1 << 30, nullptr),
         MOE_ERR_INVALID_ARG, "route NULL x");
  expect(moe_route(&s, P16, P16, nullptr, nullptr, PF, PI, PW, 16, nullptr), MOE_ERR_WORKSPACE,
         "route small ws");
  expect(moe_route(&s, P16, P16, nullptr, nullptr, PF, PI, reinterpret_cast<void*>(uintptr_t(1) << 20 | 8),
                   1 << 30, nullptr),
         MOE_ERR_WORKSPACE, "route misaligned ws");
  expect(moe_route_train(&s, P16, P16, nullptr, nullptr, nullptr, PF, PI, PF, PF, PF, nullptr,
                         nullptr, 1.5f, PW, 1 << 30, nullptr),
         MOE_ERR_INVALID_ARG, "route_train decay");
  expect(moe_expert_ffn(&s, 0, 64, P16, nullptr, nullptr, P16, P16, P16, nullptr, P16, PW, 1 << 30,
                        nullptr),
         MOE_ERR_INVALID_ARG, "ffn groups");
  expect(moe_expert_ffn(&s, 1, 65, P16, nullptr, nullptr, P16, P16, P16, nullptr, P16, PW, 1 << 30,
                        nullptr),
         MOE_ERR_INVALID_ARG, "ffn identity rows past T");
  expect(moe_expert_ffn_fp8(&s, 1, 64, P16, nullptr, nullptr, P8, nullptr, P8, PF, P8, PF, nullptr,
                            P16, PW, 1 << 30, nullptr),
         MOE_ERR_INVALID_ARG, "ffn_fp8 missing scale");
  expect(moe_combine(&s, P16 + 1, PF, PI, nullptr, P16, nullptr), MOE_ERR_INVALID_ARG,
         "combine unaligned");
  expect(moe_layer_forward(&s, P16, P16, nullptr, P16, P16, P16, nullptr, nullptr, nullptr, P16, PW,
                           size_t(1) << 40, nullptr),
         MOE_ERR_INVALID_ARG, "layer missing shared weights");
  expect(moe_layer_forward(&s, P16, P16, nullptr, P16, P16, P16, P16, P16, P16, P16, PW, 1024,
                           nullptr),
         MOE_ERR_WORKSPACE, "layer small ws");
  expect(moe_layer_forward_train(&s, P16, P16, nullptr, P16, P16, P16, P16, P16, P16, P16, nullptr,
                                 PW, size_t(1) << 40, nullptr),
         MOE_ERR_INVALID_ARG, "train forward NULL gu");
  expect(moe_layer_forward_fp8(&s, P16, P16, nullptr, P8, PF, P8, PF, P8, nullptr, P8, PF, P8, PF,
                               P8, PF, P16, PW, size_t(1) << 40, nullptr, nullptr),
         MOE_ERR_INVALID_ARG, "fp8 layer missing scale");
  expect(moe_layer_forward_w8a8(&s, P16, P16, nullptr, P8, PF, P8, PF, P8, PF, P8, PF, P8, PF, P8,
                                PF, P16, PW, 1024, nullptr, nullptr),
         MOE_ERR_WORKSPACE, "w8a8 small ws");
  expect(moe_quantize_rows_e4m3(P16, 4, 60, P8, PF, nullptr), MOE_ERR_INVALID_ARG, "quant cols");
  expect(moe_quantize_rows_mx(P16, 4, 192, P8, P8, nullptr), MOE_ERR_INVALID_ARG, "mx quant cols");
  expect(moe_quantize_rows_mx(P16, 4, 256, P8, P8 + 1, nullptr), MOE_ERR_INVALID_ARG, "mx quant scales align");
  expect(moe_layer_forward_mx(&s, P16, P16, nullptr, P8, P8, P8, nullptr, P8, P8, P8, P8, P8, P8, P8, P8,
                              P16, PW, size_t(1) << 40, nullptr, nullptr),
         MOE_ERR_INVALID_ARG, "mx layer missing scale");
  expect(moe_layer_forward_mx(&s, P16, P16, nullptr, P8, P8, P8, P8, P8, P8, P8, P8, P8, P8, P8, P8, P16,
                              PW, 1024, nullptr, nullptr),
         MOE_ERR_WORKSPACE, "mx layer small ws");
  expect(moe_layer_backward(&s, P16, P16, P16, P16, P16, P16, P16, P16, PW, size_t(1) << 40, nullptr,
                            P16, 0.f, P16, PF, PF, PF, PF, PF, PF, nullptr, nullptr, nullptr, PW,
                            size_t(1) << 40, nullptr),
         MOE_ERR_INVALID_ARG, "backward shared gradients");
  expect(moe_layer_backward(&s, P16, P16, P16, P16, P16, P16, P16, P16, PW, size_t(1) << 40, nullptr,
                            P16, 1.f / 0.f, P16, PF, PF, PF, PF, PF, PF, PF, nullptr, nullptr, PW,
                            size_t(1) << 40, nullptr),
         MOE_ERR_INVALID_ARG, "backward d_aux");
  moe_shape big = hy4(619549);
  expect(moe_layer_backward(&big, P16, P16, P16, P16, P16, P16, P16, P16, PW, size_t(1) << 60,
                            nullptr, P16, 0.f, P16, PF, PF, PF, PF, PF, PF, PF, nullptr, nullptr, PW,
                            size_t(1) << 60, nullptr),
         MOE_ERR_UNSUPPORTED, "backward operands past 64 GiB");
  for (int T : {417, 8192}) {  // 416 tokens is the largest Hy4 batch the 64 MiB scratch holds
    moe_shape pre = hy4(T);
    expect(moe_layer_forward_noalloc(&pre, P16, P16, nullptr, P16, P16, P16, P16, P16, P16, P16,
                                     nullptr),
           MOE_ERR_SCRATCH, "noalloc past its scratch");
  }
  std::printf("abi driver: %d failure(s)\n", failures);
  return failures ? 1 : 0;
}
