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
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

// Capacity in two kernels over (chunk of 256 tokens, block r) workgroups.
// The queue of block r is slot-major (slot 0 of every token in token order,
// then slot 1, ...), so the place of assignment (t, j) with expert e is
//   sum_{j' < j} load_r(j', e)  +  #{t' < t in block r : idx[t', j] = e}.
// cap_hist_kernel counts, per chunk and slot, the assignments of each expert
// (LDS integer atomics: exact).  cap_keep_kernel rebuilds from those counts
// the chunk's base place per (slot, expert), ranks the chunk's tokens of
// each slot stably with an LDS bitmap (popcount of the lower bits), and
// keeps an assignment when its place is below C.  Integer only, so exact.
constexpr int kCapTok = 256;
constexpr int kCapWords = kCapTok / 64;

__global__ __launch_bounds__(kCapTok) void cap_hist_kernel(const int32_t* __restrict__ idx,
                                                           int32_t n, int32_t k, int32_t E,
                                                           int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ dropped) {
  __shared__ int32_t h[16][256];
  const int tid = threadIdx.x;
  const int c = blockIdx.x, r = blockIdx.y, nch = gridDim.x;
  for (int i = tid; i < k * 256; i += kCapTok) h[i / 256][i % 256] = 0;
  if (c == 0 && tid == 0) dropped[r] = 0;
  __syncthreads();
  const int32_t tl = c * kCapTok + tid;
  if (tl < n) {
    const int64_t t = static_cast<int64_t>(r) * n + tl;
    for (int j = 0; j < k; ++j) {
      const int32_t e = idx[t * k + j];
      if (e >= 0 && e < E) atomicAdd(&h[j][e], 1);
    }
  }
  __syncthreads();
  int32_t* out = hist + (static_cast<int64_t>(r) * nch + c) * k * E;
  for (int i = tid; i < k * E; i += kCapTok) out[i] = h[i / E][i % E];
}

__global__ __launch_bounds__(kCapTok) void cap_keep_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ hist, int32_t n, int32_t k,
    int32_t E, int32_t C, int32_t* __restrict__ kept, int32_t* __restrict__ dropped) {
  __shared__ int32_t base[16][256];
  __shared__ unsigned long long bits[256][kCapWords];
  __shared__ int32_t wdrop[kCapWords];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = blockIdx.x, r = blockIdx.y, nch = gridDim.x;
  const int32_t* hr = hist + static_cast<int64_t>(r) * nch * k * E;
  // base[j][e] = sum_{j' < j} (all chunks) + sum_{chunks c' < c} of slot j:
  // per (slot, expert) pair the chunk counts are read 16 at a time (loads
  // issued together), then a prefix over the slots
  __shared__ int32_t tot[16][256];
  for (int i = tid; i < k * E; i += kCapTok) {
    const int j = i / E, e = i - j * E;
    int32_t all = 0, pre = 0;
    for (int c0 = 0; c0 < nch; c0 += 16) {
      int32_t v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        v[u] = hr[(static_cast<int64_t>(min(c0 + u, nch - 1)) * k + j) * E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int32_t x = (c0 + u < nch) ? v[u] : 0;
        all += x;
        pre += (c0 + u < c) ? x : 0;
      }
    }
    tot[j][e] = all;
    base[j][e] = pre;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kCapTok) {
    int32_t run = 0;
    for (int j = 0; j < k; ++j) {
      base[j][e] += run;
      run += tot[j][e];
    }
  }
  const int32_t tl = c * kCapTok + tid;
  const bool live = tl < n;
  const int64_t t = static_cast<int64_t>(r) * n + (live ? tl : 0);
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t drops = 0;
  for (int j = 0; j < k; ++j) {
    for (int i = tid; i < E * kCapWords; i += kCapTok) bits[i / kCapWords][i % kCapWords] = 0ull;
    __syncthreads();   // also orders the base[] writes above before their first use
    const int32_t e = live ? idx[t * k + j] : -1;
    const bool valid = e >= 0 && e < E;
    if (valid) atomicOr(&bits[e][w], 1ull << lane);
    __syncthreads();
    if (live) {
      int32_t out = -1;
      if (valid) {
        int32_t place = base[j][e] + __popcll(bits[e][w] & below);
        for (int ww = 0; ww < w; ++ww) place += __popcll(bits[e][ww]);
        if (place < C) out = e;
        else ++drops;
      }
      kept[t * k + j] = out;
    }
    __syncthreads();
  }
  // wavefront sums, then one integer atomic per workgroup (order-free, exact)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) drops += __shfl_xor(drops, off, 64);
  if (lane == 0) wdrop[w] = drops;
  __syncthreads();
  if (tid == 0) {
    const int32_t s = wdrop[0] + wdrop[1] + wdrop[2] + wdrop[3];
    if (s) atomicAdd(&dropped[r], s);
  }
}

// Router z-loss values in two kernels.  router_z_partial_kernel: workgroup
// (chunk of kZTok tokens, block r); L lanes per token (the smallest power of two
// >= E, at least 4 and at most 64; each lane holds experts l, l + L, ...), so a token's logits are
// read as one contiguous row; the maximum and the sum of exponentials are
// butterflies inside the L-lane segment; all of a wavefront's loads are
// issued before any is used.  The chunk's lse^2 values are added in token
// order.  router_z_fold_kernel adds a block's chunk sums in chunk order.
constexpr int kZTok = 64;   // tokens per workgroup (16 per wavefront)

template <int L, int EPL>
__global__ __launch_bounds__(256) void router_z_partial_kernel(const float* __restrict__ logits,
                                                               int32_t n, int32_t E,
                                                               float* __restrict__ partial) {
  constexpr int TPW = 64 / L;          // tokens per wavefront pass
  constexpr int NP = 16 / TPW;         // passes per wavefront
  static_assert(NP >= 1 && 16 % TPW == 0, "a wavefront covers 16 tokens in whole passes");
  __shared__ float zs[kZTok];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = blockIdx.x, r = blockIdx.y;
  const int seg = lane / L, sl = lane % L;
  float v[NP][EPL];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int32_t tl = c * kZTok + w * 16 + p * TPW + seg;
    const int64_t row = static_cast<int64_t>(r) * n + min(tl, n - 1);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = sl + L * i;
      const float val = logits[row * E + min(e, E - 1)];
      v[p][i] = (tl < n && e < E) ? val : -INFINITY;
    }
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float m = v[p][0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) m = fmaxf(m, v[p][i]);
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) s += (v[p][i] == -INFINITY) ? 0.f : __expf(v[p][i] - m);
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    const int32_t tl = c * kZTok + w * 16 + p * TPW + seg;
    if (sl == 0) {
      const float lse = m + __logf(s);
      zs[w * 16 + p * TPW + seg] = (tl < n) ? lse * lse : 0.f;
    }
  }
  __syncthreads();
  if (tid == 0) {
    float acc = 0.f;
    for (int i = 0; i < kZTok; ++i) acc += zs[i];
    partial[static_cast<int64_t>(r) * gridDim.x + c] = acc;
  }
}

__global__ __launch_bounds__(256) void router_z_fold_kernel(const float* __restrict__ partial,
                                                            int32_t nch, int32_t n, int32_t G,
                                                            float* __restrict__ group_z) {
  for (int r = blockIdx.x * 256 + threadIdx.x; r < G; r += gridDim.x * 256) {
    float acc = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 16) {   // 16 loads in flight, added in chunk order
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        v[u] = partial[static_cast<int64_t>(r) * nch + min(c0 + u, nch - 1)];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (c0 + u < nch) acc += v[u];
    }
    group_z[r] = (n > 0) ? acc / static_cast<float>(n) : 0.f;
  }
}

// Routing flips between two runs ("MoE Pretraining: Parallelism Layout
// Changes the Model, Not Quality", Finding 3): flips[t] = 1 when token t's
// chosen expert sets differ (slot order ignored): each set becomes a 256-bit
// mask.  The count is a workgroup sum plus one integer atomic (exact).
__global__ __launch_bounds__(256) void route_flips_kernel(const int32_t* __restrict__ a,
                                                          const int32_t* __restrict__ b,
                                                          int64_t T, int32_t k, int32_t E,
                                                          int32_t* __restrict__ flips,
                                                          int32_t* __restrict__ n_flips) {
  __shared__ int32_t wsum[4];
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  int32_t f = 0;
  if (t < T) {
    unsigned long long ma[4] = {0ull, 0ull, 0ull, 0ull}, mb[4] = {0ull, 0ull, 0ull, 0ull};
    for (int j = 0; j < k; ++j) {
      const int32_t ea = a[t * k + j], eb = b[t * k + j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (ea >= 0 && ea < E && (ea >> 6) == q) ma[q] |= 1ull << (ea & 63);
        if (eb >= 0 && eb < E && (eb >> 6) == q) mb[q] |= 1ull << (eb & 63);
      }
    }
    f = ((ma[0] ^ mb[0]) | (ma[1] ^ mb[1]) | (ma[2] ^ mb[2]) | (ma[3] ^ mb[3])) ? 1 : 0;
    flips[t] = f;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int32_t c = __popcll(__ballot(f != 0));
  if (lane == 0) wsum[w] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t s = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (s) atomicAdd(n_flips, s);
  }
}

__global__ void zero_one_kernel(int32_t* p) { *p = 0; }

}  // namespace

hipError_t launch_route_flips(int64_t T, int32_t k, int32_t E, const int32_t* a, const int32_t* b,
                              int32_t* flips, int32_t* n_flips, hipStream_t s) {
  hipLaunchKernelGGL(zero_one_kernel, dim3(1), dim3(1), 0, s, n_flips);
  if (T > 0)
    hipLaunchKernelGGL(route_flips_kernel, dim3((T + 255) / 256), dim3(256), 0, s, a, b, T, k, E,
                       flips, n_flips);
  return hipGetLastError();
}

int capacity_chunks(int64_t T, int32_t G) {
  const int64_t n = G > 0 ? T / G : 0;
  return static_cast<int>(std::max<int64_t>((n + kCapTok - 1) / kCapTok, 1));
}

hipError_t launch_capacity(int64_t T, int32_t k, int32_t E, int32_t G, int32_t C,
                           const int32_t* idx, int32_t* kept, int32_t* dropped, int32_t* ws_hist,
                           hipStream_t s) {
  if (G <= 0) return hipSuccess;
  const int32_t n = static_cast<int32_t>(T / G);
  const dim3 grid(capacity_chunks(T, G), G);
  hipLaunchKernelGGL(cap_hist_kernel, grid, dim3(kCapTok), 0, s, idx, n, k, E, ws_hist, dropped);
  hipLaunchKernelGGL(cap_keep_kernel, grid, dim3(kCapTok), 0, s, idx, ws_hist, n, k, E, C, kept,
                     dropped);
  return hipGetLastError();
}

int zloss_chunks(int64_t T, int32_t G) {
  const int64_t n = G > 0 ? T / G : 0;
  return static_cast<int>(std::max<int64_t>((n + kZTok - 1) / kZTok, 1));
}

hipError_t launch_router_z(int64_t T, int32_t E, int32_t G, const float* logits, float* group_z,
                           float* ws_partial, hipStream_t s) {
  if (G <= 0) return hipSuccess;
  const int32_t n = static_cast<int32_t>(T / G);
  const int nch = zloss_chunks(T, G);
  if (n > 0) {
    const dim3 grid(nch, G);
#define MOE_Z(L, EPL) \
  hipLaunchKernelGGL((router_z_partial_kernel<L, EPL>), grid, dim3(256), 0, s, logits, n, E, ws_partial)
    if (E <= 4) MOE_Z(4, 1);
    else if (E <= 8) MOE_Z(8, 1);
    else if (E <= 16) MOE_Z(16, 1);
    else if (E <= 32) MOE_Z(32, 1);
    else if (E <= 64) MOE_Z(64, 1);
    else if (E <= 128) MOE_Z(64, 2);
    else MOE_Z(64, 4);
#undef MOE_Z
  }
  const int fold_blocks = (G + 255) / 256;
  hipLaunchKernelGGL(router_z_fold_kernel, dim3(fold_blocks), dim3(256), 0, s, ws_partial,
                     n > 0 ? nch : 0, n, G, group_z);
  return hipGetLastError();
}

}  // namespace moe
