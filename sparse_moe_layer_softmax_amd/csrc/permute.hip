// permute.hip -- deterministic token-to-expert dispatch.
//
// Hy3 explainer (tqpw.cn) section 2.1: each expert runs on the rows routed to it, gathered
// with a per-expert mask. Here the gather order is fixed: rows are grouped by expert and, inside
// an expert, ordered by slot id s = t*K + j (a stable counting sort). A per-expert capacity C
// keeps the first C slots of each expert (the capacity rule of the top-2 / capacity_factor 1.25
// variant declared by the Hy3 deep-dive's `SparseMoERouter`).
//
// Up to kSmallSlots slots (decode), one single-wavefront launch does all of it. Otherwise three
// launches over fixed contiguous chunks of slots:
//  1. histogram: per-chunk expert counts with LDS integer atomics (order-free, so exact);
//  2. scan (one workgroup): per-chunk bases (prefix over chunks), kept counts, expert offsets;
//  3. scatter (one wavefront per chunk): walks its chunk 64 slots at a time; the rank of a slot
//     among earlier slots of the same expert in the same step comes from a ballot-built match
//     mask, so the final row of every slot is a pure function of topk_idx.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxE = 256;

__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ topk_idx,
                                                           int32_t* __restrict__ block_counts,
                                                           int TK, int E, int chunk) {
  __shared__ int cnt[kMaxE];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int beg = blockIdx.x * chunk;
  const int end = min(beg + chunk, TK);
  for (int s = beg + threadIdx.x; s < end; s += blockDim.x) {
    const int e = topk_idx[s];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    block_counts[static_cast<size_t>(blockIdx.x) * E + e] = cnt[e];
}

__global__ __launch_bounds__(256) void permute_scan_kernel(
    const int32_t* __restrict__ block_counts, int32_t* __restrict__ block_base,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_to_slot, int32_t* __restrict__ ext_offsets, int n_ident, int nblk,
    int E, int TK, int capacity) {
  __shared__ int sk[kMaxE + 1];
  __shared__ int wsum[kMaxE / 64];
  const int e = threadIdx.x;  // one expert per thread (blockDim = kMaxE >= E)
  int kept = 0;
  if (e < E) {
    int run = 0;
    // block_counts reads are independent of the running sum: unrolled, eight are in flight
#pragma unroll 8
    for (int b = 0; b < nblk; ++b) {
      const int c = block_counts[static_cast<size_t>(b) * E + e];
      block_base[static_cast<size_t>(b) * E + e] = run;
      run += c;
    }
    kept = (capacity > 0 && run > capacity) ? capacity : run;
  }
  // exclusive scan of the kept counts over the experts: lanes by shuffles, wavefronts through LDS
  // (integer sums, so the result does not depend on the order)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = kept;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int excl = inc - kept;
  for (int j = 0; j < w; ++j) excl += wsum[j];
  if (e < E) sk[e] = excl;
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int j = 0; j < kMaxE / 64; ++j) acc += wsum[j];
    sk[E] = acc;
  }
  __syncthreads();
  if (e < E) {
    counts[e] = kept;
    offsets[e] = sk[e];
    if (ext_offsets) ext_offsets[e + 1] = n_ident + sk[e];
  }
  if (threadIdx.x == 0) {
    offsets[E] = sk[E];
    if (ext_offsets) {
      ext_offsets[0] = 0;
      ext_offsets[E + 1] = n_ident + sk[E];
    }
  }
  // rows past the kept total carry no slot
  for (int r = sk[E] + threadIdx.x; r < TK; r += blockDim.x) row_to_slot[r] = -1;
}

__global__ __launch_bounds__(64) void permute_scatter_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ block_base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ row_to_slot,
    int32_t* __restrict__ slot_to_row, int TK, int E, int chunk, int capacity) {
  __shared__ int run[kMaxE];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) run[e] = block_base[static_cast<size_t>(blockIdx.x) * E + e];
  __syncthreads();
  const int beg = blockIdx.x * chunk;
  const int end = min(beg + chunk, TK);
  for (int base = beg; base < end; base += 64) {
    const int s = base + lane;
    const bool in = s < end;
    int e = in ? topk_idx[s] : -1;
    const bool ok = in && static_cast<unsigned>(e) < static_cast<unsigned>(E);
    if (!ok) e = 0;
    // lanes holding the same expert id: AND of per-bit agreement masks (E <= 256: 8 bits)
    uint64_t match = __ballot(ok);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t b = __ballot((e >> bit) & 1);
      match &= ((e >> bit) & 1) ? b : ~b;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(match & below);
    const int prior = ok ? run[e] : 0;
    __syncthreads();  // every lane has read run[] before the group leaders update it
    const bool leader = ok && (match >> lane) == 1ull;  // highest lane of its group
    if (leader) run[e] = prior + __popcll(match);
    __syncthreads();
    if (in) {
      const int pos = prior + rank;
      if (ok && (capacity <= 0 || pos < capacity)) {
        const int row = offsets[e] + pos;
        row_to_slot[row] = s;
        slot_to_row[s] = row;
      } else {
        slot_to_row[s] = -1;
      }
    }
  }
}

// All three steps in one wavefront, for at most kSmallSlots slots (decode): the histogram with
// LDS integer atomics, the kept counts and their exclusive scan across the lanes (four
// consecutive experts per lane), then the same ballot-ranked walk over the slots as the scatter
// kernel, 64 slots per step. Same results as the three-launch form, in one launch.
constexpr int kSmallSlots = 1024;

__global__ __launch_bounds__(64) void permute_small_kernel(
    const int32_t* __restrict__ topk_idx, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_to_slot,
    int32_t* __restrict__ slot_to_row, int32_t* __restrict__ ext_offsets, int n_ident, int TK,
    int E, int capacity) {
  __shared__ int run[kMaxE];
  __shared__ int off[kMaxE];
  const int lane = threadIdx.x;
  for (int e = lane; e < kMaxE; e += 64) run[e] = 0;
  __syncthreads();
  for (int s = lane; s < TK; s += 64) {
    const int e = topk_idx[s];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&run[e], 1);
  }
  __syncthreads();
  int kept[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    const int c = e < E ? run[e] : 0;
    kept[i] = (capacity > 0 && c > capacity) ? capacity : c;
    sum += kept[i];
  }
  int inc = sum;  // inclusive scan of the lane sums
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  const int total = __shfl(inc, 63);
  int base = inc - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    if (e < E) {
      off[e] = base;
      counts[e] = kept[i];
      offsets[e] = base;
      if (ext_offsets) ext_offsets[e + 1] = n_ident + base;
    }
    base += kept[i];
  }
  if (lane == 0) {
    offsets[E] = total;
    if (ext_offsets) {
      ext_offsets[0] = 0;
      ext_offsets[E + 1] = n_ident + total;
    }
  }
  for (int r = total + lane; r < TK; r += 64) row_to_slot[r] = -1;
  __syncthreads();
  for (int e = lane; e < kMaxE; e += 64) run[e] = 0;
  __syncthreads();
  for (int b0 = 0; b0 < TK; b0 += 64) {
    const int s = b0 + lane;
    const bool in = s < TK;
    int e = in ? topk_idx[s] : -1;
    const bool ok = in && static_cast<unsigned>(e) < static_cast<unsigned>(E);
    if (!ok) e = 0;
    uint64_t match = __ballot(ok);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t bb = __ballot((e >> bit) & 1);
      match &= ((e >> bit) & 1) ? bb : ~bb;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(match & below);
    const int prior = ok ? run[e] : 0;
    __syncthreads();
    const bool leader = ok && (match >> lane) == 1ull;
    if (leader) run[e] = prior + __popcll(match);
    __syncthreads();
    if (in) {
      const int pos = prior + rank;
      if (ok && (capacity <= 0 || pos < capacity)) {
        const int row = off[e] + pos;
        row_to_slot[row] = s;
        slot_to_row[s] = row;
      } else {
        slot_to_row[s] = -1;
      }
    }
  }
}

}  // namespace

int permute_chunk(int TK) {
  if (TK <= 256 * 1024) return 1024;
  const int per = (TK + 255) / 256;
  return (per + 63) / 64 * 64;
}

int permute_blocks(int TK) {
  const int c = permute_chunk(TK);
  return (TK + c - 1) / c;
}

hipError_t launch_permute(const moe_shape& s, const int32_t* topk_idx, int32_t* counts,
                          int32_t* offsets, int32_t* row_to_slot, int32_t* slot_to_row,
                          int32_t* block_counts, int32_t* block_base, int32_t* ext_offsets,
                          int n_ident, hipStream_t stream) {
  const int TK = s.T * s.K;
  if (TK <= kSmallSlots && s.E <= kMaxE) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(64), 0, stream, topk_idx, counts,
                       offsets, row_to_slot, slot_to_row, ext_offsets, n_ident, TK, s.E,
                       s.capacity);
    return hipGetLastError();
  }
  const int chunk = permute_chunk(TK);
  const int nblk = permute_blocks(TK);
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nblk), dim3(256), 0, stream, topk_idx,
                     block_counts, TK, s.E, chunk);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kMaxE), 0, stream, block_counts, block_base,
                     counts, offsets, row_to_slot, ext_offsets, n_ident, nblk, s.E, TK,
                     s.capacity);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(64), 0, stream, topk_idx,
                     block_base, offsets, row_to_slot, slot_to_row, TK, s.E, chunk, s.capacity);
  return hipGetLastError();
}

}  // namespace moe
