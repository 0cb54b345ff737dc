// Index products for expert-parallel layouts, computed locally on one GPU.
//
// Source: "Expert Coupling in MoE Pretraining: Reducing All-to-All Overhead
// with Correlated Placement and Token Shuffling" -- Table III (co-selection
// count W[e,e']), Fig. 2 (co-selection within a layer), Abstract (a dispatcher
// that sends each token to each GPU once), Table I (same-GPU share, distinct
// destinations per token, rows removed as duplicates).
//
// Dispatch plan: each token's distinct destination groups form a 64-bit mask;
// rows are ordered by (group, token) with the same histogram / scan / bitmap
// rank machinery as the expert permutation, keyed by group instead of expert.
// All counters are integers, so the results are exact and reproducible.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxG = 64;
constexpr int kWords = kPermBlock / 64;

__global__ __launch_bounds__(kThreads) void plan_mask_kernel(
    const int32_t* __restrict__ idx, int64_t T, int32_t k, int32_t E, int32_t G,
    PlacementArg pl, int32_t* __restrict__ n_dest, uint64_t* __restrict__ mask_out,
    int32_t* __restrict__ hist, int32_t* __restrict__ stat) {
  __shared__ int32_t h[kMaxG];
  __shared__ int32_t st[3][kThreads];
  const int tid = threadIdx.x;
  if (tid < G) h[tid] = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kPermBlock + tid;
  int32_t rows = 0, single = 0, off_home = 0;
  if (t < T) {
    uint64_t m = 0;
    for (int j = 0; j < k; ++j) {
      const int32_t e = idx[t * k + j];
      if (e >= 0 && e < E) m |= 1ull << pl.group_of[e];
    }
    rows = __popcll(m);
    single = (rows == 1) ? 1 : 0;
    const int64_t home = t / (T / G);
    off_home = __popcll(m & ~(1ull << home));
    n_dest[t] = rows;
    mask_out[t] = m;
    for (uint64_t mm = m; mm; mm &= mm - 1) atomicAdd(&h[__ffsll(static_cast<long long>(mm)) - 1], 1);
  }
  st[0][tid] = rows;
  st[1][tid] = single;
  st[2][tid] = off_home;
  __syncthreads();
  for (int w = kThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) {
      st[0][tid] += st[0][tid + w];
      st[1][tid] += st[1][tid + w];
      st[2][tid] += st[2][tid + w];
    }
    __syncthreads();
  }
  if (tid < G) hist[static_cast<int64_t>(blockIdx.x) * G + tid] = h[tid];
  if (tid < 3) stat[static_cast<int64_t>(blockIdx.x) * 3 + tid] = st[tid][0];
}

__global__ __launch_bounds__(kThreads) void plan_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int32_t k, int32_t E, int32_t G,
    PlacementArg pl, const uint64_t* __restrict__ mask_in, const int32_t* __restrict__ base,
    int32_t* __restrict__ row_token, int32_t* __restrict__ assign_row) {
  __shared__ unsigned long long bits[kMaxG][kWords];
  const int tid = threadIdx.x;
  for (int i = tid; i < G * kWords; i += kThreads) bits[i / kWords][i % kWords] = 0ull;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kPermBlock + tid;
  const int w = tid >> 6, lane = tid & 63;
  const uint64_t m = (t < T) ? mask_in[t] : 0ull;
  for (uint64_t mm = m; mm; mm &= mm - 1)
    atomicOr(&bits[__ffsll(static_cast<long long>(mm)) - 1][w], 1ull << lane);
  __syncthreads();
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int32_t* bb = base + static_cast<int64_t>(blockIdx.x) * G;
  for (uint64_t mm = m; mm; mm &= mm - 1) {
    const int g = __ffsll(static_cast<long long>(mm)) - 1;
    int32_t rank = __popcll(bits[g][w] & below);
    for (int ww = 0; ww < w; ++ww) rank += __popcll(bits[g][ww]);
    row_token[bb[g] + rank] = static_cast<int32_t>(t);
  }
  for (int j = 0; j < k; ++j) {
    const int32_t e = idx[t * k + j];
    if (e < 0 || e >= E) {
      assign_row[t * k + j] = -1;
      continue;
    }
    const int g = pl.group_of[e];
    int32_t rank = __popcll(bits[g][w] & below);
    for (int ww = 0; ww < w; ++ww) rank += __popcll(bits[g][ww]);
    assign_row[t * k + j] = bb[g] + rank;
  }
}

__global__ __launch_bounds__(kThreads) void plan_stats_kernel(const int32_t* __restrict__ stat,
                                                              int32_t nb, int64_t T, int32_t k,
                                                              int32_t* __restrict__ stats) {
  if (threadIdx.x != 0) return;
  int64_t rows = 0, single = 0, off = 0;
  for (int b = 0; b < nb; ++b) {
    rows += stat[b * 3 + 0];
    single += stat[b * 3 + 1];
    off += stat[b * 3 + 2];
  }
  stats[0] = static_cast<int32_t>(rows);
  stats[1] = static_cast<int32_t>(T * k - rows);
  stats[2] = static_cast<int32_t>(single);
  stats[3] = static_cast<int32_t>(off);
}

__global__ __launch_bounds__(kThreads) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n,
                                                            int32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(kThreads) void coselect_kernel(const int32_t* __restrict__ idx,
                                                            int64_t T, int32_t k, int32_t E,
                                                            int32_t* __restrict__ W) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= T) return;
  for (int i = 0; i < k; ++i) {
    const int32_t a = idx[t * k + i];
    if (a < 0 || a >= E) continue;
    for (int j = 0; j < k; ++j) {
      const int32_t b = idx[t * k + j];
      if (j == i || b < 0 || b >= E) continue;
      atomicAdd(&W[static_cast<int64_t>(a) * E + b], 1);
    }
  }
}

}  // namespace

hipError_t launch_coselect(int64_t T, int32_t k, int32_t E, const int32_t* idx, int32_t* W,
                           hipStream_t s) {
  const int64_t n = static_cast<int64_t>(E) * E;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                     W, n, 0);
  if (T > 0)
    hipLaunchKernelGGL(coselect_kernel, dim3((T + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       s, idx, T, k, E, W);
  return hipGetLastError();
}

hipError_t launch_dispatch_plan(int64_t T, int32_t k, int32_t E, int32_t G,
                                const int32_t* idx, const PlacementArg& pl, int32_t* n_dest,
                                int32_t* group_rows, int32_t* group_offsets, int32_t* row_token,
                                int32_t* assign_row, int32_t* stats, uint64_t* ws_mask,
                                int32_t* ws_hist, int32_t* ws_base, int32_t* ws_stat,
                                hipStream_t s) {
  const int64_t nb = (T + kPermBlock - 1) / kPermBlock;
  if (nb > 0)
    hipLaunchKernelGGL(plan_mask_kernel, dim3(nb), dim3(kThreads), 0, s, idx, T, k, E, G, pl,
                       n_dest, ws_mask, ws_hist, ws_stat);
  hipLaunchKernelGGL(key_scan_kernel, dim3(1), dim3(256), 0, s, ws_hist,
                     static_cast<int32_t>(nb), G, ws_base, group_rows, group_offsets);
  if (nb > 0)
    hipLaunchKernelGGL(plan_scatter_kernel, dim3(nb), dim3(kThreads), 0, s, idx, T, k, E, G, pl,
                       ws_mask, ws_base, row_token, assign_row);
  hipLaunchKernelGGL(plan_stats_kernel, dim3(1), dim3(kThreads), 0, s, ws_stat,
                     static_cast<int32_t>(nb), T, k, stats);
  return hipGetLastError();
}

}  // namespace moe
