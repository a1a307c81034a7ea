// api.hip -- the C ABI (include/moe.h): argument checks, workspace layout, launch order.
//
// Every check runs on the host before anything is enqueued, so a rejected call leaves the
// stream untouched. The library allocates nothing and never synchronises.
#include <cmath>
#include <climits>
#include <mutex>

#include "moe.h"
#include "ffn_kernels.h"
#include "moe_internal.h"

using moe::align_up;

namespace {

// The tiled MFMA kernel addresses each operand row in 16-byte units with a 32-bit offset from the
// operand's base: no activation or weight operand it reads may exceed 64 GiB.
constexpr unsigned long long kMaxOperandBytes = 1ull << 36;

// Bytes of a [rows, cols] bf16 operand fit the tiled kernel's addressing.
bool operand_fits(long long rows, long long cols) {
  return static_cast<unsigned long long>(rows) * static_cast<unsigned long long>(cols) * 2ull <=
         kMaxOperandBytes;
}

// The forward's operands: x [T, H] (rows gathered by token), h [rows, I] with rows layer rows,
// and one expert's weight matrix [I, H] or [H, I].
bool forward_operands_fit(const moe_shape& s, long long rows) {
  return operand_fits(s.T, s.H) && operand_fits(rows, s.I) && operand_fits(s.I, s.H);
}

int check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->T < 1 || s->H < 1 || s->E < 1 || s->K < 1 || s->I < 1) return MOE_ERR_INVALID_ARG;
  if (s->K > s->E) return MOE_ERR_INVALID_ARG;
  if (s->n_shared != 0 && s->n_shared != 1) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(s->routed_scaling) || std::isnan(s->swiglu_limit)) return MOE_ERR_INVALID_ARG;
  if (s->K > 16 || s->E > 256) return MOE_ERR_UNSUPPORTED;
  if (s->H % 256 != 0 || s->I % 256 != 0) return MOE_ERR_UNSUPPORTED;
  // row indices are int32 and rows_max = T + T*K must fit
  const long long rows = static_cast<long long>(s->T) * (s->K + 1);
  if (rows >= INT_MAX) return MOE_ERR_UNSUPPORTED;
  if (!forward_operands_fit(*s, rows)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// ----- workspace layouts (offsets in bytes, every buffer 256-byte aligned)
struct RouteWs {
  size_t partials, total;
  int S;
};
RouteWs route_ws(const moe_shape& s) {
  RouteWs w{};
  w.S = moe::route_splits(s.T, s.H, s.E);
  w.partials = 0;
  w.total = align_up(sizeof(float) * static_cast<size_t>(w.S) * s.T * s.E);
  return w;
}

struct PermuteWs {
  size_t block_counts, block_base, total;
};
PermuteWs permute_ws(const moe_shape& s) {
  PermuteWs w{};
  const size_t nb = static_cast<size_t>(moe::permute_blocks(s.T * s.K)) * s.E * sizeof(int32_t);
  w.block_counts = 0;
  w.block_base = align_up(nb);
  w.total = w.block_base + align_up(nb);
  return w;
}

struct FfnWs {
  size_t offsets, tiles, h, total;
};
FfnWs ffn_ws(const moe_shape& s, int n_groups, int rows_max, bool need_h) {
  FfnWs w{};
  w.offsets = 0;
  w.tiles = align_up(2 * sizeof(int32_t));
  // the tile table is sized for the smallest row tile any FFN kernel uses (16 rows)
  w.h = w.tiles + align_up(moe::tile_table_bytes(moe::max_tiles_for(rows_max, n_groups, 16)));
  w.total = w.h + (need_h ? align_up(sizeof(uint16_t) * static_cast<size_t>(rows_max) * s.I) : 0);
  return w;
}

struct LayerWs {
  moe_layer_ws_layout pub;
  size_t route, permute, ext_offsets, tiles;
};
LayerWs layer_ws(const moe_shape& s) {
  LayerWs w{};
  const size_t TK = static_cast<size_t>(s.T) * s.K;
  const size_t rows = TK + static_cast<size_t>(s.n_shared ? s.T : 0);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  w.pub.logits = take(sizeof(float) * s.T * s.E);
  w.pub.topk_w = take(sizeof(float) * TK);
  w.pub.topk_idx = take(sizeof(int32_t) * TK);
  w.pub.counts = take(sizeof(int32_t) * s.E);
  w.pub.offsets = take(sizeof(int32_t) * (s.E + 1));
  w.pub.row_to_slot = take(sizeof(int32_t) * TK);
  w.pub.slot_to_row = take(sizeof(int32_t) * TK);
  w.pub.h = take(sizeof(uint16_t) * rows * s.I);
  w.pub.y = take(sizeof(uint16_t) * rows * s.H);
  w.route = take(route_ws(s).total);
  w.permute = take(permute_ws(s).total);
  w.ext_offsets = take(sizeof(int32_t) * (s.E + 2));
  w.tiles = take(moe::tile_table_bytes(moe::max_tiles_for(static_cast<int>(rows), s.E + s.n_shared, 16)));
  w.pub.total = o;
  return w;
}

inline bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// One set of expert weights (gate, up, down): bf16, or FP8 E4M3 codes with per-row scales, or
// E4M3 codes with MX block scales (E8M0 bytes, [K/128][N][4] per matrix).
struct Weights {
  bool w8, mx;
  const uint16_t *gate, *up, *down;
  const uint8_t *qgate, *qup, *qdown;
  const float *sgate, *sup, *sdown;
  const uint8_t *xgate, *xup, *xdown;
  static Weights bf16(const uint16_t* g, const uint16_t* u, const uint16_t* d) {
    Weights w{};
    w.gate = g;
    w.up = u;
    w.down = d;
    return w;
  }
  static Weights fp8(const uint8_t* g, const float* gs, const uint8_t* u, const float* us,
                     const uint8_t* d, const float* ds) {
    Weights w{};
    w.w8 = true;
    w.qgate = g;
    w.sgate = gs;
    w.qup = u;
    w.sup = us;
    w.qdown = d;
    w.sdown = ds;
    return w;
  }
  static Weights mxfp8(const uint8_t* g, const uint8_t* gs, const uint8_t* u, const uint8_t* us,
                       const uint8_t* d, const uint8_t* ds) {
    Weights w{};
    w.w8 = w.mx = true;
    w.qgate = g;
    w.xgate = gs;
    w.qup = u;
    w.xup = us;
    w.qdown = d;
    w.xdown = ds;
    return w;
  }
  // every pointer of the set given
  bool complete() const {
    if (mx) return qgate && xgate && qup && xup && qdown && xdown;
    return w8 ? (qgate && sgate && qup && sup && qdown && sdown) : (gate && up && down);
  }
  // no pointer of the set given
  bool empty() const {
    return !gate && !up && !down && !qgate && !sgate && !qup && !sup && !qdown && !sdown && !xgate &&
           !xup && !xdown;
  }
};

// the *_a (groups < g_split) or *_b weights of an FFN problem
void set_weights(moe::FfnProblem& p, const Weights& w, bool a) {
  p.w8 = w.w8;
  (a ? p.gate_a : p.gate_b) = w.gate;
  (a ? p.up_a : p.up_b) = w.up;
  (a ? p.down_a : p.down_b) = w.down;
  (a ? p.qgate_a : p.qgate_b) = w.qgate;
  (a ? p.qup_a : p.qup_b) = w.qup;
  (a ? p.qdown_a : p.qdown_b) = w.qdown;
  (a ? p.sgate_a : p.sgate_b) = w.sgate;
  (a ? p.sup_a : p.sup_b) = w.sup;
  (a ? p.sdown_a : p.sdown_b) = w.sdown;
  (a ? p.xgate_a : p.xgate_b) = w.xgate;
  (a ? p.xup_a : p.xup_b) = w.xup;
  (a ? p.xdown_a : p.xdown_b) = w.xdown;
}

int expert_ffn_impl(const moe_shape* s, int32_t n_groups, int32_t rows_max, const uint16_t* x,
                    const int32_t* row_to_slot, const int32_t* group_offsets, const Weights& wt,
                    uint16_t* h, uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!x || !wt.complete() || !y || !ws) return MOE_ERR_INVALID_ARG;
  if (n_groups < 1 || n_groups > 1024 || rows_max < 1) return MOE_ERR_INVALID_ARG;
  if (!row_to_slot && rows_max > s->T) return MOE_ERR_INVALID_ARG;
  if (!group_offsets && n_groups != 1) return MOE_ERR_INVALID_ARG;
  if (!forward_operands_fit(*s, rows_max)) return MOE_ERR_UNSUPPORTED;
  const FfnWs w = ffn_ws(*s, n_groups, rows_max, h == nullptr);
  if (ws_bytes < w.total || !aligned(ws)) return MOE_ERR_WORKSPACE;
  const int32_t* offs = group_offsets;
  if (!offs) {
    int32_t* o = reinterpret_cast<int32_t*>(at(ws, w.offsets));
    rc = hip_status(moe::launch_single_group_offsets(o, rows_max, stream));
    if (rc != MOE_OK) return rc;
    offs = o;
  }
  moe::FfnProblem p{};
  p.x = x;
  p.T = s->T;
  p.gather = row_to_slot;
  p.n_ident = row_to_slot ? 0 : INT_MAX;
  p.topk = s->K;
  p.offsets = offs;
  p.n_groups = n_groups;
  p.rows_max = rows_max;
  p.g_split = 0;
  set_weights(p, wt, false);
  p.H = s->H;
  p.I = s->I;
  p.limit = s->swiglu_limit;
  p.h = h ? h : reinterpret_cast<uint16_t*>(at(ws, w.h));
  p.y = y;
  p.tiles = reinterpret_cast<int32_t*>(at(ws, w.tiles));
  return hip_status(moe::launch_ffn(p, stream));
}

// The W8A8 workspace: the layer's own layout, then the quantised activations.
struct A8Ws {
  moe_layer_a8_ws_layout pub;
};
A8Ws a8_ws(const moe_shape& s) {
  A8Ws w{};
  const size_t rows = static_cast<size_t>(s.T) * s.K + (s.n_shared ? s.T : 0);
  size_t o = layer_ws(s).pub.total;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  w.pub.xq = take(static_cast<size_t>(s.T) * s.H);
  w.pub.x_scale = take(sizeof(float) * s.T);
  w.pub.hq = take(rows * s.I);
  w.pub.h_scale = take(sizeof(float) * rows);
  w.pub.total = o;
  return w;
}

// The MX workspace: the layer's own layout, then the block-quantised activations with their
// scale planes (one dword of 4 E8M0 bytes per GEMM row and 128-element K-tile; kTiledRows spare
// rows so that a row tile's scale load never leaves the plane).
struct MxWs {
  moe_layer_mx_ws_layout pub;
};
MxWs mx_ws(const moe_shape& s) {
  MxWs w{};
  const size_t rows = static_cast<size_t>(s.T) * s.K + (s.n_shared ? s.T : 0);
  size_t o = layer_ws(s).pub.total;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  w.pub.scale_rows = rows + moe::kTiledRows;
  w.pub.xq = take(static_cast<size_t>(s.T) * s.H);
  w.pub.x_scale = take(static_cast<size_t>(s.H / 128) * w.pub.scale_rows * 4);
  w.pub.hq = take(rows * s.I);
  w.pub.h_scale = take(static_cast<size_t>(s.I / 128) * w.pub.scale_rows * 4);
  w.pub.total = o;
  return w;
}

int layer_impl(const moe_shape* s, const uint16_t* x, const uint16_t* w_router, const float* bias,
               const Weights& routed, const Weights& shared_w, uint16_t* out, void* ws,
               size_t ws_bytes, hipStream_t stream, hipEvent_t const* ev, bool a8 = false,
               float* gu = nullptr) {
  auto mark = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord(ev[i], stream);
  };
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!x || !w_router || !routed.complete() || !out || !ws) return MOE_ERR_INVALID_ARG;
  const bool shared = s->n_shared == 1;
  if (shared != shared_w.complete()) return MOE_ERR_INVALID_ARG;
  if (!shared && !shared_w.empty()) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(out) & 15u) return MOE_ERR_INVALID_ARG;
  const LayerWs w = layer_ws(*s);
  const A8Ws wa = a8_ws(*s);
  const MxWs wm = mx_ws(*s);
  const bool mx = routed.mx;
  if (mx != shared_w.mx && shared) return MOE_ERR_INVALID_ARG;
  const size_t need = mx ? wm.pub.total : a8 ? wa.pub.total : w.pub.total;
  if (ws_bytes < need || !aligned(ws)) return MOE_ERR_WORKSPACE;

  float* logits = reinterpret_cast<float*>(at(ws, w.pub.logits));
  float* topk_w = reinterpret_cast<float*>(at(ws, w.pub.topk_w));
  int32_t* topk_idx = reinterpret_cast<int32_t*>(at(ws, w.pub.topk_idx));
  int32_t* counts = reinterpret_cast<int32_t*>(at(ws, w.pub.counts));
  int32_t* offsets = reinterpret_cast<int32_t*>(at(ws, w.pub.offsets));
  int32_t* r2s = reinterpret_cast<int32_t*>(at(ws, w.pub.row_to_slot));
  int32_t* s2r = reinterpret_cast<int32_t*>(at(ws, w.pub.slot_to_row));
  uint16_t* h = reinterpret_cast<uint16_t*>(at(ws, w.pub.h));
  uint16_t* y = reinterpret_cast<uint16_t*>(at(ws, w.pub.y));
  int32_t* ext = reinterpret_cast<int32_t*>(at(ws, w.ext_offsets));

  mark(0);
  const RouteWs rw = route_ws(*s);
  rc = hip_status(moe::launch_route(*s, x, w_router, bias, nullptr, logits, topk_w, topk_idx,
                                    reinterpret_cast<float*>(at(ws, w.route + rw.partials)), rw.S,
                                    stream));
  if (rc != MOE_OK) return rc;
  mark(1);

  const PermuteWs pw = permute_ws(*s);
  const int n_ident = shared ? s->T : 0;
  rc = hip_status(moe::launch_permute(
      *s, topk_idx, counts, offsets, r2s, s2r,
      reinterpret_cast<int32_t*>(at(ws, w.permute + pw.block_counts)),
      reinterpret_cast<int32_t*>(at(ws, w.permute + pw.block_base)), shared ? ext : nullptr,
      n_ident, stream));
  if (rc != MOE_OK) return rc;
  mark(2);

  // routed experts and the shared expert in one grouped launch per projection:
  // group 0 = shared expert over rows [0, T) (identity), groups 1..E = routed experts
  moe::FfnProblem p{};
  p.x = x;
  p.T = s->T;
  p.gather = r2s;
  p.n_ident = n_ident;
  p.topk = s->K;
  p.offsets = shared ? ext : offsets;
  p.n_groups = s->E + (shared ? 1 : 0);
  p.rows_max = n_ident + s->T * s->K;
  p.g_split = shared ? 1 : 0;
  if (shared) set_weights(p, shared_w, true);
  set_weights(p, routed, false);
  p.H = s->H;
  p.I = s->I;
  p.limit = s->swiglu_limit;
  p.h = h;
  p.y = y;
  p.tiles = reinterpret_cast<int32_t*>(at(ws, w.tiles));
  p.gu = gu;
  if (mx) {
    p.a8 = p.mx = true;
    p.xq = reinterpret_cast<uint8_t*>(at(ws, wm.pub.xq));
    p.xs = reinterpret_cast<uint8_t*>(at(ws, wm.pub.x_scale));
    p.hq = reinterpret_cast<uint8_t*>(at(ws, wm.pub.hq));
    p.hs = reinterpret_cast<uint8_t*>(at(ws, wm.pub.h_scale));
    p.mx_rows = static_cast<int32_t>(wm.pub.scale_rows);
    p.s2r = s2r;
  } else if (a8) {
    p.a8 = true;
    p.xq = reinterpret_cast<uint8_t*>(at(ws, wa.pub.xq));
    p.sx = reinterpret_cast<float*>(at(ws, wa.pub.x_scale));
    p.hq = reinterpret_cast<uint8_t*>(at(ws, wa.pub.hq));
    p.sh = reinterpret_cast<float*>(at(ws, wa.pub.h_scale));
  }
  rc = hip_status(moe::launch_ffn(p, stream, ev ? ev + 3 : nullptr));
  if (rc != MOE_OK) return rc;

  const uint16_t* y_routed = y + static_cast<size_t>(n_ident) * s->H;
  rc = hip_status(moe::launch_combine(*s, y_routed, topk_w, s2r, shared ? y : nullptr, out,
                                      stream));
  mark(6);
  return rc;
}

// ----- the no-allocation entry point's scratch: one static device array per GPU, holding the
// layer's workspace. Host code reaches it only through the address hipGetSymbolAddress returns
// for the current device (the array's name is a host-side stand-in, not a device address).
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device, set once under g_scratch_mu

// The scratch address on the current device, looked up on the first call there.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH: return "shape needs more than the library's static scratch";
    default: return "unknown error";
  }
}

size_t moe_route_workspace_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return route_ws(*s).total;
}

int moe_route(const moe_shape* s, const uint16_t* x, const uint16_t* w_router, const float* bias,
              float* logits, float* topk_w, int32_t* topk_idx, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!x || !w_router || !topk_w || !topk_idx || !ws) return MOE_ERR_INVALID_ARG;
  const RouteWs w = route_ws(*s);
  if (ws_bytes < w.total || !aligned(ws)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_route(*s, x, w_router, bias, nullptr, logits, topk_w, topk_idx,
                                      reinterpret_cast<float*>(at(ws, w.partials)), w.S, stream));
}

namespace {
struct RouteTrainWs {
  RouteWs route;
  size_t base_route, logits, part_p, part_c, total;
};
RouteTrainWs route_train_ws(const moe_shape& s) {
  RouteTrainWs w{};
  w.route = route_ws(s);
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o += align_up(n);
    return at;
  };
  const size_t nb = static_cast<size_t>(moe::router_stats_blocks(s.T));
  w.base_route = take(w.route.total);
  w.logits = take(sizeof(float) * static_cast<size_t>(s.T) * s.E);
  w.part_p = take(sizeof(float) * nb * s.E);
  w.part_c = take(sizeof(int32_t) * nb * s.E);
  w.total = o;
  return w;
}
}  // namespace

size_t moe_route_train_workspace_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return route_train_ws(*s).total;
}

int moe_route_train(const moe_shape* s, const uint16_t* x, const uint16_t* w_router,
                    const float* bias, const float* noise, float* logits, float* topk_w,
                    int32_t* topk_idx, float* prob_mean, float* load_frac, float* aux_loss,
                    float* ema_counts, float* ema_tokens, float ema_decay, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!x || !w_router || !topk_w || !topk_idx || !prob_mean || !load_frac || !aux_loss || !ws)
    return MOE_ERR_INVALID_ARG;
  if (!(ema_decay >= 0.f && ema_decay <= 1.f)) return MOE_ERR_INVALID_ARG;  // also rejects NaN
  const RouteTrainWs w = route_train_ws(*s);
  if (ws_bytes < w.total || !aligned(ws)) return MOE_ERR_WORKSPACE;
  float* lg = logits ? logits : reinterpret_cast<float*>(at(ws, w.logits));
  rc = hip_status(moe::launch_route(
      *s, x, w_router, bias, noise, lg, topk_w, topk_idx,
      reinterpret_cast<float*>(at(ws, w.base_route + w.route.partials)), w.route.S, stream));
  if (rc != MOE_OK) return rc;
  return hip_status(moe::launch_router_stats(
      *s, lg, topk_idx, reinterpret_cast<float*>(at(ws, w.part_p)),
      reinterpret_cast<int32_t*>(at(ws, w.part_c)), ema_decay, prob_mean, load_frac, aux_loss,
      ema_counts, ema_tokens, stream));
}

size_t moe_permute_workspace_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return permute_ws(*s).total;
}

int moe_permute(const moe_shape* s, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                int32_t* row_to_slot, int32_t* slot_to_row, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!topk_idx || !counts || !offsets || !row_to_slot || !slot_to_row || !ws)
    return MOE_ERR_INVALID_ARG;
  const PermuteWs w = permute_ws(*s);
  if (ws_bytes < w.total || !aligned(ws)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_permute(
      *s, topk_idx, counts, offsets, row_to_slot, slot_to_row,
      reinterpret_cast<int32_t*>(at(ws, w.block_counts)),
      reinterpret_cast<int32_t*>(at(ws, w.block_base)), nullptr, 0, stream));
}

size_t moe_expert_ffn_workspace_size(const moe_shape* s, int32_t n_groups, int32_t rows_max) {
  if (check_shape(s) != MOE_OK || n_groups < 1 || n_groups > 1024 || rows_max < 1) return 0;
  return ffn_ws(*s, n_groups, rows_max, true).total;
}

int moe_expert_ffn(const moe_shape* s, int32_t n_groups, int32_t rows_max, const uint16_t* x,
                   const int32_t* row_to_slot, const int32_t* group_offsets,
                   const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                   uint16_t* h, uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  return expert_ffn_impl(s, n_groups, rows_max, x, row_to_slot, group_offsets,
                         Weights::bf16(w_gate, w_up, w_down), h, y, ws, ws_bytes, stream);
}

int moe_expert_ffn_fp8(const moe_shape* s, int32_t n_groups, int32_t rows_max,
                       const uint16_t* x, const int32_t* row_to_slot,
                       const int32_t* group_offsets, const uint8_t* w_gate,
                       const float* w_gate_scale, const uint8_t* w_up, const float* w_up_scale,
                       const uint8_t* w_down, const float* w_down_scale, uint16_t* h,
                       uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  return expert_ffn_impl(s, n_groups, rows_max, x, row_to_slot, group_offsets,
                         Weights::fp8(w_gate, w_gate_scale, w_up, w_up_scale, w_down, w_down_scale),
                         h, y, ws, ws_bytes, stream);
}

int moe_combine(const moe_shape* s, const uint16_t* y_routed, const float* topk_w,
                const int32_t* slot_to_row, const uint16_t* y_shared, uint16_t* out,
                hipStream_t stream) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!y_routed || !topk_w || !slot_to_row || !out) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(y_routed) | reinterpret_cast<uintptr_t>(out) |
       reinterpret_cast<uintptr_t>(y_shared)) & 15u)
    return MOE_ERR_INVALID_ARG;  // 16-byte vector accesses
  return hip_status(moe::launch_combine(*s, y_routed, topk_w, slot_to_row, y_shared, out, stream));
}

size_t moe_layer_workspace_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return layer_ws(*s).pub.total;
}

int moe_layer_workspace_layout(const moe_shape* s, moe_layer_ws_layout* layout) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!layout) return MOE_ERR_INVALID_ARG;
  *layout = layer_ws(*s).pub;
  return MOE_OK;
}

int moe_layer_forward(const moe_shape* s, const uint16_t* x, const uint16_t* w_router,
                      const float* bias, const uint16_t* w_gate, const uint16_t* w_up,
                      const uint16_t* w_down, const uint16_t* s_gate, const uint16_t* s_up,
                      const uint16_t* s_down, uint16_t* out, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  return moe_layer_forward_profiled(s, x, w_router, bias, w_gate, w_up, w_down, s_gate, s_up,
                                    s_down, out, ws, ws_bytes, stream, nullptr);
}

size_t moe_layer_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moe_layer_forward_noalloc(const moe_shape* s, const uint16_t* x, const uint16_t* w_router,
                              const float* bias, const uint16_t* w_gate, const uint16_t* w_up,
                              const uint16_t* w_down, const uint16_t* s_gate,
                              const uint16_t* s_up, const uint16_t* s_down, uint16_t* out,
                              hipStream_t stream) {
  const int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (layer_ws(*s).pub.total > kScratchBytes) return MOE_ERR_SCRATCH;
  if (stream) {  // the scratch is the current device's: the stream must run there
    int cur = -1;
    hipDevice_t sd = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sd) != hipSuccess)
      return MOE_ERR_HIP;
    if (sd != cur) return MOE_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  const int rs = current_scratch(&ws);
  if (rs != MOE_OK) return rs;
  return layer_impl(s, x, w_router, bias, Weights::bf16(w_gate, w_up, w_down),
                    Weights::bf16(s_gate, s_up, s_down), out, ws, kScratchBytes, stream, nullptr);
}

int moe_layer_forward_train(const moe_shape* s, const uint16_t* x, const uint16_t* w_router,
                            const float* bias, const uint16_t* w_gate, const uint16_t* w_up,
                            const uint16_t* w_down, const uint16_t* s_gate, const uint16_t* s_up,
                            const uint16_t* s_down, uint16_t* out, float* gu, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  if (!gu || (reinterpret_cast<uintptr_t>(gu) & 15u)) return MOE_ERR_INVALID_ARG;
  return layer_impl(s, x, w_router, bias, Weights::bf16(w_gate, w_up, w_down),
                    Weights::bf16(s_gate, s_up, s_down), out, ws, ws_bytes, stream, nullptr, false,
                    gu);
}

int moe_layer_forward_profiled(const moe_shape* s, const uint16_t* x, const uint16_t* w_router,
                               const float* bias, const uint16_t* w_gate, const uint16_t* w_up,
                               const uint16_t* w_down, const uint16_t* s_gate,
                               const uint16_t* s_up, const uint16_t* s_down, uint16_t* out,
                               void* ws, size_t ws_bytes, hipStream_t stream,
                               hipEvent_t const* ev) {
  return layer_impl(s, x, w_router, bias, Weights::bf16(w_gate, w_up, w_down),
                    Weights::bf16(s_gate, s_up, s_down), out, ws, ws_bytes, stream, ev);
}

int moe_layer_forward_fp8(const moe_shape* s, const uint16_t* x, const uint16_t* w_router,
                          const float* bias, const uint8_t* w_gate, const float* w_gate_scale,
                          const uint8_t* w_up, const float* w_up_scale, const uint8_t* w_down,
                          const float* w_down_scale, const uint8_t* s_gate,
                          const float* s_gate_scale, const uint8_t* s_up,
                          const float* s_up_scale, const uint8_t* s_down,
                          const float* s_down_scale, uint16_t* out, void* ws, size_t ws_bytes,
                          hipStream_t stream, hipEvent_t const* ev) {
  return layer_impl(s, x, w_router, bias,
                    Weights::fp8(w_gate, w_gate_scale, w_up, w_up_scale, w_down, w_down_scale),
                    Weights::fp8(s_gate, s_gate_scale, s_up, s_up_scale, s_down, s_down_scale),
                    out, ws, ws_bytes, stream, ev);
}

int moe_quantize_rows_e4m3(const uint16_t* x, int32_t rows, int32_t cols, uint8_t* codes,
                           float* scales, hipStream_t stream) {
  if (!x || !codes || !scales || rows < 1 || cols < 8 || cols % 8) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(x) & 15u) || (reinterpret_cast<uintptr_t>(codes) & 7u))
    return MOE_ERR_INVALID_ARG;  // 16-byte loads, 8-byte stores
  return hip_status(moe::launch_quant_rows(x, rows, cols, nullptr, codes, scales, stream));
}

size_t moe_layer_w8a8_workspace_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return a8_ws(*s).pub.total;
}

int moe_layer_w8a8_workspace_layout(const moe_shape* s, moe_layer_a8_ws_layout* layout) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!layout) return MOE_ERR_INVALID_ARG;
  *layout = a8_ws(*s).pub;
  return MOE_OK;
}

int moe_layer_forward_w8a8(const moe_shape* s, const uint16_t* x, const uint16_t* w_router,
                           const float* bias, const uint8_t* w_gate, const float* w_gate_scale,
                           const uint8_t* w_up, const float* w_up_scale, const uint8_t* w_down,
                           const float* w_down_scale, const uint8_t* s_gate,
                           const float* s_gate_scale, const uint8_t* s_up,
                           const float* s_up_scale, const uint8_t* s_down,
                           const float* s_down_scale, uint16_t* out, void* ws, size_t ws_bytes,
                           hipStream_t stream, hipEvent_t const* ev) {
  return layer_impl(s, x, w_router, bias,
                    Weights::fp8(w_gate, w_gate_scale, w_up, w_up_scale, w_down, w_down_scale),
                    Weights::fp8(s_gate, s_gate_scale, s_up, s_up_scale, s_down, s_down_scale),
                    out, ws, ws_bytes, stream, ev, true);
}

size_t moe_layer_mx_workspace_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return mx_ws(*s).pub.total;
}

int moe_layer_mx_workspace_layout(const moe_shape* s, moe_layer_mx_ws_layout* layout) {
  const int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!layout) return MOE_ERR_INVALID_ARG;
  *layout = mx_ws(*s).pub;
  return MOE_OK;
}

int moe_layer_forward_mx(const moe_shape* s, const uint16_t* x, const uint16_t* w_router,
                         const float* bias, const uint8_t* w_gate, const uint8_t* w_gate_scale,
                         const uint8_t* w_up, const uint8_t* w_up_scale, const uint8_t* w_down,
                         const uint8_t* w_down_scale, const uint8_t* s_gate,
                         const uint8_t* s_gate_scale, const uint8_t* s_up,
                         const uint8_t* s_up_scale, const uint8_t* s_down,
                         const uint8_t* s_down_scale, uint16_t* out, void* ws, size_t ws_bytes,
                         hipStream_t stream, hipEvent_t const* ev) {
  return layer_impl(s, x, w_router, bias,
                    Weights::mxfp8(w_gate, w_gate_scale, w_up, w_up_scale, w_down, w_down_scale),
                    Weights::mxfp8(s_gate, s_gate_scale, s_up, s_up_scale, s_down, s_down_scale),
                    out, ws, ws_bytes, stream, ev, true);
}

int moe_quantize_rows_mx(const uint16_t* x, int32_t rows, int32_t cols, uint8_t* codes,
                         uint8_t* scales, hipStream_t stream) {
  if (!x || !codes || !scales || rows < 1 || cols < 1 || cols % 128 != 0) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(x) & 15u) || (reinterpret_cast<uintptr_t>(codes) & 7u) ||
      (reinterpret_cast<uintptr_t>(scales) & 3u))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_quant_mx(x, rows, cols, nullptr, codes, scales, rows, nullptr, 0, 0,
                                         stream));
}

namespace {
struct BwdWs {
  size_t dy, dh, dgu, dx_rows, dx_router, cnt, tiles_tiled, d_topk_w, d_logits;
  size_t dyT, hT, dguT, xgT, ktiles, kt, router_part;
  size_t total;
};
BwdWs bwd_ws(const moe_shape& s) {
  BwdWs w{};
  const size_t rows = static_cast<size_t>(s.T) * s.K + (s.n_shared ? s.T : 0);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  w.dy = take(sizeof(uint16_t) * rows * s.H);
  w.dh = take(sizeof(uint16_t) * rows * s.I);
  w.dgu = take(sizeof(uint16_t) * rows * 2 * s.I);
  w.dx_rows = take(sizeof(uint16_t) * rows * s.H);
  w.dx_router = take(sizeof(float) * static_cast<size_t>(s.T) * s.H);
  w.cnt = take(sizeof(int32_t) * s.E);
  w.tiles_tiled = take(moe::tile_table_bytes(
      moe::max_tiles_for(static_cast<int>(rows), s.E + s.n_shared, moe::kTiledRows)));
  w.d_topk_w = take(sizeof(float) * static_cast<size_t>(s.T) * s.K);
  w.d_logits = take(sizeof(float) * static_cast<size_t>(s.T) * s.E);
  const int mtk = moe::backward_ktiles(static_cast<int>(rows), s.E + s.n_shared);
  const size_t ldk = static_cast<size_t>(mtk) * 64;
  w.dyT = take(sizeof(uint16_t) * s.H * ldk);
  w.hT = take(sizeof(uint16_t) * s.I * ldk);
  w.dguT = take(sizeof(uint16_t) * 2 * s.I * ldk);
  w.xgT = take(sizeof(uint16_t) * s.H * ldk);
  w.ktiles = take(moe::tile_table_bytes(mtk));
  w.kt = take(sizeof(int32_t) * 2 * (s.E + s.n_shared));
  const int rs = moe::router_splits(s.T);
  w.router_part = take(rs > 1 ? sizeof(float) * rs * static_cast<size_t>(s.E) * s.H : 0);
  w.total = o;
  return w;
}
// The backward's tiled-kernel operands: dy [rows, H] and [dg | du] [rows, 2I] (data gradients),
// and the row-contiguous copies [H][ld], [I][ld], [2I][ld] of the weight gradients, whose
// reduction dimension ld is about the layer row count.
bool backward_operands_fit(const moe_shape& s) {
  const long long rows = static_cast<long long>(s.T) * s.K + (s.n_shared ? s.T : 0);
  const long long ld = static_cast<long long>(
                           moe::backward_ktiles(static_cast<int>(rows), s.E + s.n_shared)) * 64;
  return operand_fits(rows, s.H) && operand_fits(rows, 2LL * s.I) && operand_fits(s.H, ld) &&
         operand_fits(2LL * s.I, ld);
}
}  // namespace

size_t moe_layer_backward_workspace_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK || !backward_operands_fit(*s)) return 0;
  return bwd_ws(*s).total;
}

int moe_layer_backward_workspace_layout(const moe_shape* s, moe_bwd_ws_layout* layout) {
  const int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (!backward_operands_fit(*s)) return MOE_ERR_UNSUPPORTED;
  if (!layout) return MOE_ERR_INVALID_ARG;
  const BwdWs w = bwd_ws(*s);
  layout->dy = w.dy;
  layout->dh = w.dh;
  layout->dgu = w.dgu;
  layout->dx_rows = w.dx_rows;
  layout->dx_router = w.dx_router;
  layout->d_topk_w = w.d_topk_w;
  layout->d_logits = w.d_logits;
  layout->total = w.total;
  return MOE_OK;
}

int moe_layer_backward(const moe_shape* s, const uint16_t* x, const uint16_t* w_router,
                       const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                       const uint16_t* s_gate, const uint16_t* s_up, const uint16_t* s_down,
                       const void* fwd_ws, size_t fwd_ws_bytes, const float* gu,
                       const uint16_t* d_out, float d_aux, uint16_t* d_x, float* d_w_router,
                       float* d_w_gate, float* d_w_up, float* d_w_down, float* d_s_gate,
                       float* d_s_up, float* d_s_down, float* d_topk_w, float* d_logits, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  const bool shared = s->n_shared == 1;
  if (!x || !w_router || !w_gate || !w_up || !w_down || !fwd_ws || !d_out || !d_x ||
      !d_w_router || !d_w_gate || !d_w_up || !d_w_down || !ws)
    return MOE_ERR_INVALID_ARG;
  const bool sw = s_gate && s_up && s_down, sg = d_s_gate && d_s_up && d_s_down;
  if (shared != sw || shared != sg) return MOE_ERR_INVALID_ARG;
  if (!shared && (s_gate || s_up || s_down || d_s_gate || d_s_up || d_s_down))
    return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(d_aux)) return MOE_ERR_INVALID_ARG;
  if (!backward_operands_fit(*s)) return MOE_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(d_out) | reinterpret_cast<uintptr_t>(d_x) |
       reinterpret_cast<uintptr_t>(gu)) & 15u)
    return MOE_ERR_INVALID_ARG;  // 16-byte vector accesses
  const LayerWs fw = layer_ws(*s);
  if (fwd_ws_bytes < fw.pub.total || !aligned(fwd_ws)) return MOE_ERR_WORKSPACE;
  const BwdWs w = bwd_ws(*s);
  if (ws_bytes < w.total || !aligned(ws)) return MOE_ERR_WORKSPACE;
  void* fws = const_cast<void*>(fwd_ws);
  moe::BwdProblem b{};
  b.s = *s;
  b.shared = shared;
  b.x = x;
  b.w_router = w_router;
  b.w_gate = w_gate;
  b.w_up = w_up;
  b.w_down = w_down;
  b.s_gate = s_gate;
  b.s_up = s_up;
  b.s_down = s_down;
  b.logits = reinterpret_cast<const float*>(at(fws, fw.pub.logits));
  b.topk_w = reinterpret_cast<const float*>(at(fws, fw.pub.topk_w));
  b.topk_idx = reinterpret_cast<const int32_t*>(at(fws, fw.pub.topk_idx));
  b.row_to_slot = reinterpret_cast<const int32_t*>(at(fws, fw.pub.row_to_slot));
  b.slot_to_row = reinterpret_cast<const int32_t*>(at(fws, fw.pub.slot_to_row));
  b.grp_offsets = reinterpret_cast<const int32_t*>(at(fws, shared ? fw.ext_offsets : fw.pub.offsets));
  b.h = reinterpret_cast<const uint16_t*>(at(fws, fw.pub.h));
  b.y = reinterpret_cast<const uint16_t*>(at(fws, fw.pub.y));
  b.dout = d_out;
  b.d_aux = d_aux;
  b.dy = reinterpret_cast<uint16_t*>(at(ws, w.dy));
  b.dh = reinterpret_cast<uint16_t*>(at(ws, w.dh));
  b.dgu = reinterpret_cast<uint16_t*>(at(ws, w.dgu));
  b.dx_rows = reinterpret_cast<uint16_t*>(at(ws, w.dx_rows));
  b.dx_router = reinterpret_cast<float*>(at(ws, w.dx_router));
  b.cnt = reinterpret_cast<int32_t*>(at(ws, w.cnt));
  b.tiles_tiled = reinterpret_cast<int32_t*>(at(ws, w.tiles_tiled));
  b.dyT = reinterpret_cast<uint16_t*>(at(ws, w.dyT));
  b.hT = reinterpret_cast<uint16_t*>(at(ws, w.hT));
  b.dguT = reinterpret_cast<uint16_t*>(at(ws, w.dguT));
  b.xgT = reinterpret_cast<uint16_t*>(at(ws, w.xgT));
  b.ktiles = reinterpret_cast<int32_t*>(at(ws, w.ktiles));
  b.kt = reinterpret_cast<int32_t*>(at(ws, w.kt));
  b.router_part = reinterpret_cast<float*>(at(ws, w.router_part));
  b.gu = gu;
  b.d_topk_w = d_topk_w ? d_topk_w : reinterpret_cast<float*>(at(ws, w.d_topk_w));
  b.d_logits = d_logits ? d_logits : reinterpret_cast<float*>(at(ws, w.d_logits));
  b.d_x = d_x;
  b.d_w_router = d_w_router;
  b.d_w_gate = d_w_gate;
  b.d_w_up = d_w_up;
  b.d_w_down = d_w_down;
  b.d_s_gate = d_s_gate;
  b.d_s_up = d_s_up;
  b.d_s_down = d_s_down;
  return hip_status(moe::launch_layer_backward(b, stream));
}

}  // extern "C"
