// Token-shuffle planning on one GPU: cross-layer co-selection counts and the
// owner prediction that the shuffled reduce-scatter would follow.
//
// Source: "Expert Coupling in MoE Pretraining: Reducing All-to-All Overhead
// with Correlated Placement and Token Shuffling" -- Abstract (the experts a
// token picks at one layer predict its picks at the next), Fig. 2(b)
// (cross-layer conditional counts), Fig. 5 step 1 and Fig. 6 (the planner
// predicts each token's owner from its previous-layer routes), Table I
// (local next-layer experts when a token is moved to the predicted GPU versus
// when it stays on its home GPU).
//
// Integer counts only, so every result is exact.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxG = 64;

__global__ __launch_bounds__(kThreads) void zero_i32_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) p[i] = 0;
}

// W[a][b] += 1 for every a in S_cur(t), b in S_next(t): one thread per token,
// integer atomics (exact, order-free).
__global__ __launch_bounds__(kThreads) void coselect_cross_kernel(
    const int32_t* __restrict__ cur, const int32_t* __restrict__ nxt, int64_t T, int32_t k,
    int32_t E, int32_t* __restrict__ W) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= T) return;
  for (int i = 0; i < k; ++i) {
    const int32_t a = cur[t * k + i];
    if (a < 0 || a >= E) continue;
    for (int j = 0; j < k; ++j) {
      const int32_t b = nxt[t * k + j];
      if (b < 0 || b >= E) continue;
      atomicAdd(&W[static_cast<int64_t>(a) * E + b], 1);
    }
  }
}

// M[e1][g] = sum over e2 placed on g of W[e1][e2]: workgroup e1, thread e2
// reads its count (one coalesced row) and adds it to its group's LDS counter
// (integer atomics: exact); workgroup 0 also clears the outputs that the
// planner accumulates into.
__global__ __launch_bounds__(kThreads) void shuffle_mass_kernel(
    const int32_t* __restrict__ W, int32_t E, int32_t G, PlacementArg pl, int32_t* __restrict__ M,
    int32_t* __restrict__ group_tokens, int32_t* __restrict__ stats) {
  __shared__ int32_t m[kMaxG];
  const int e1 = blockIdx.x, tid = threadIdx.x;
  if (tid < G) m[tid] = 0;
  __syncthreads();
  for (int e2 = tid; e2 < E; e2 += kThreads)
    atomicAdd(&m[pl.group_of[e2]], W[static_cast<int64_t>(e1) * E + e2]);
  __syncthreads();
  if (tid < G) M[e1 * G + tid] = m[tid];
  if (e1 == 0) {
    if (tid < G) group_tokens[tid] = 0;
    if (tid < 2) stats[tid] = 0;
  }
}

// One thread per token, 64 tokens per workgroup (many workgroups for one
// batch): score(g) = sum_j M[S_j][g] (64-bit), owner = the first g with the
// largest score; per-workgroup counts of owners and of local next-layer
// assignments, then one integer atomic each.
constexpr int kPlanThreads = 64;
__global__ __launch_bounds__(kPlanThreads) void shuffle_plan_kernel(
    const int32_t* __restrict__ cur, const int32_t* __restrict__ nxt,
    const int32_t* __restrict__ M, int64_t T, int32_t k, int32_t E, int32_t G, PlacementArg pl,
    int32_t* __restrict__ owner, int32_t* __restrict__ group_tokens,
    int32_t* __restrict__ stats) {
  extern __shared__ int32_t sM[];   // [E][G]
  __shared__ int32_t cnt[kMaxG];
  __shared__ int32_t loc[2];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * G; i += kPlanThreads) sM[i] = M[i];
  if (tid < G) cnt[tid] = 0;
  if (tid < 2) loc[tid] = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kPlanThreads + tid;
  if (t < T) {
    int32_t ids[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int32_t e = (j < k) ? cur[t * k + j] : -1;
      ids[j] = (e >= 0 && e < E) ? e : -1;
    }
    int64_t best = -1;
    int best_g = 0;
    for (int g = 0; g < G; ++g) {
      int64_t s = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (ids[j] >= 0) s += sM[ids[j] * G + g];
      if (s > best) {
        best = s;
        best_g = g;
      }
    }
    owner[t] = best_g;
    atomicAdd(&cnt[best_g], 1);
    if (nxt) {
      const int64_t home = t / (T / G);
      int32_t moved = 0, stays = 0;
      for (int j = 0; j < k; ++j) {
        const int32_t e = nxt[t * k + j];
        if (e < 0 || e >= E) continue;
        const int g = pl.group_of[e];
        moved += (g == best_g);
        stays += (g == home);
      }
      if (moved) atomicAdd(&loc[0], moved);
      if (stays) atomicAdd(&loc[1], stays);
    }
  }
  __syncthreads();
  if (tid < G && cnt[tid]) atomicAdd(&group_tokens[tid], cnt[tid]);
  if (tid < 2 && loc[tid]) atomicAdd(&stats[tid], loc[tid]);
}

}  // namespace

hipError_t launch_coselect_cross(int64_t T, int32_t k, int32_t E, const int32_t* cur,
                                 const int32_t* nxt, int32_t* W, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(E) * E;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                     W, n);
  if (T > 0)
    hipLaunchKernelGGL(coselect_cross_kernel, dim3((T + kThreads - 1) / kThreads), dim3(kThreads),
                       0, s, cur, nxt, T, k, E, W);
  return hipGetLastError();
}

hipError_t launch_shuffle_plan(int64_t T, int32_t k, int32_t E, int32_t G, const int32_t* cur,
                               const int32_t* W, const PlacementArg& pl, const int32_t* nxt,
                               int32_t* owner, int32_t* group_tokens, int32_t* stats,
                               int32_t* ws_mass, hipStream_t s) {
  hipLaunchKernelGGL(shuffle_mass_kernel, dim3(E), dim3(kThreads), 0, s, W, E, G, pl, ws_mass,
                     group_tokens, stats);
  if (T > 0) {
    const size_t lds = static_cast<size_t>(E) * G * sizeof(int32_t);
    hipLaunchKernelGGL(shuffle_plan_kernel, dim3((T + kPlanThreads - 1) / kPlanThreads),
                       dim3(kPlanThreads), lds, s, cur, nxt, ws_mass, T, k, E, G, pl, owner,
                       group_tokens, stats);
  }
  return hipGetLastError();
}

}  // namespace moe
