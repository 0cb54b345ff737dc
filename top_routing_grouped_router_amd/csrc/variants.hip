// Definitional variants of the routing rules: per-block expert capacity with
// dropping, and the value of the router z-loss.
//
// Method sources: "Revisiting MoE and Dense Speed-Accuracy Comparisons for LLM
// Training" (Sec. 2.1: Top-K routing with an expert capacity; GShard's
// placement puts second choices after every first choice; ST-MoE's router
// z-loss; Sec. 4: a lower capacity for training than for evaluation);
// "MoE Pretraining: Parallelism Layout Changes the Model, Not Quality" (Two
// Kinds of Layout Effects: capacity and balancing rules evaluated per machine,
// here per contiguous block of T/G tokens).
#include "common.h"

namespace moe {
namespace {

// One workgroup per block r of n tokens.  The block's T/G * k assignments
// queue slot-major (q = j n + token): slot 0 of every token in token order,
// then slot 1, ...  A chunk of 1024 consecutive queue entries is placed at
// once: inside a wavefront, the lanes holding the same expert are found with
// nine ballots over the bits of the expert id, a lane's rank is the number of
// such lanes below it, and each wavefront's per-expert count goes to LDS; the
// place of an entry is then base[e] (entries of earlier chunks) + the counts
// of earlier wavefronts + its rank.  Integer only, so exact.
constexpr int kCapThreads = 1024;
constexpr int kCapWaves = kCapThreads / 64;

__global__ __launch_bounds__(kCapThreads) void capacity_kernel(
    const int32_t* __restrict__ idx, int32_t n, int32_t k, int32_t E, int32_t C,
    int32_t* __restrict__ kept, int32_t* __restrict__ dropped) {
  __shared__ int32_t base[256];
  __shared__ int32_t wcnt[kCapWaves][256];
  __shared__ int32_t wdrop[kCapWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t r = blockIdx.x;
  for (int e = tid; e < 256; e += kCapThreads) base[e] = 0;
  for (int i = tid; i < kCapWaves * 256; i += kCapThreads) wcnt[i / 256][i % 256] = 0;
  __syncthreads();
  const int64_t Q = static_cast<int64_t>(n) * k;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t drops = 0;
  for (int64_t q0 = 0; q0 < Q; q0 += kCapThreads) {
    const int64_t q = q0 + tid;
    const bool live = q < Q;
    const int32_t j = live ? static_cast<int32_t>(q / n) : 0;
    const int64_t t = r * n + (live ? q - static_cast<int64_t>(j) * n : 0);
    const int32_t e = live ? idx[t * k + j] : -1;
    const bool valid = e >= 0 && e < E;
    const int32_t key = valid ? e : 256;   // 9 bits; 256 = no expert
    unsigned long long peers = ~0ull;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
      const bool bit = (key >> b) & 1;
      const unsigned long long m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int32_t rank = __popcll(peers & below);
    if (valid && rank == 0) wcnt[w][e] = __popcll(peers);
    __syncthreads();
    bool drop = false;
    if (live) {
      int32_t out = -1;
      if (valid) {
        int32_t place = base[e] + rank;
        for (int ww = 0; ww < w; ++ww) place += wcnt[ww][e];
        if (place < C) out = e;
        else drop = true;
      }
      kept[t * k + j] = out;
    }
    drops += __popcll(__ballot(drop));
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += kCapThreads) {
      int32_t s = 0;
      for (int ww = 0; ww < kCapWaves; ++ww) {
        s += wcnt[ww][e2];
        wcnt[ww][e2] = 0;
      }
      base[e2] += s;
    }
    __syncthreads();
  }
  if (lane == 0) wdrop[w] = drops;
  __syncthreads();
  if (tid == 0) {
    int32_t s = 0;
    for (int ww = 0; ww < kCapWaves; ++ww) s += wdrop[ww];
    dropped[r] = s;
  }
}

// group_z[r] = mean over block r of lse_t^2, lse_t = log sum_e exp l[t,e].
// One workgroup per block: thread i takes tokens i, i + 256, ... in order,
// then a fixed-shape tree adds the 256 partial sums.
__global__ __launch_bounds__(256) void router_z_kernel(const float* __restrict__ logits,
                                                       int32_t n, int32_t E,
                                                       float* __restrict__ group_z) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  float acc = 0.f;
  for (int32_t tl = tid; tl < n; tl += 256) {
    const float* row = logits + (r * n + tl) * E;
    float m = -INFINITY;
    for (int e = 0; e < E; ++e) m = fmaxf(m, row[e]);
    float s = 0.f;
    for (int e = 0; e < E; ++e) s += __expf(row[e] - m);
    const float lse = m + __logf(s);
    acc = fmaf(lse, lse, acc);
  }
  red[tid] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) red[tid] += red[tid + h];
    __syncthreads();
  }
  if (tid == 0) group_z[r] = (n > 0) ? red[0] / static_cast<float>(n) : 0.f;
}

}  // namespace

hipError_t launch_capacity(int64_t T, int32_t k, int32_t E, int32_t G, int32_t C,
                           const int32_t* idx, int32_t* kept, int32_t* dropped, hipStream_t s) {
  if (G <= 0) return hipSuccess;
  hipLaunchKernelGGL(capacity_kernel, dim3(G), dim3(kCapThreads), 0, s, idx,
                     static_cast<int32_t>(T / G), k, E, C, kept, dropped);
  return hipGetLastError();
}

hipError_t launch_router_z(int64_t T, int32_t E, int32_t G, const float* logits, float* group_z,
                           hipStream_t s) {
  if (G <= 0) return hipSuccess;
  hipLaunchKernelGGL(router_z_kernel, dim3(G), dim3(256), 0, s, logits,
                     static_cast<int32_t>(T / G), E, group_z);
  return hipGetLastError();
}

}  // namespace moe
