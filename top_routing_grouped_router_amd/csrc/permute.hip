// Permutation of the T*k (token, slot) assignments into expert-contiguous rows.
//
// Method sources: "Expert Coupling in MoE Pretraining" (Abstract and Fig. 5
// step 3: dispatch of tokens to their experts); "Revisiting MoE and Dense
// Speed-Accuracy Comparisons" (Sec. 2.2: GShard dispatch, where a token's slot
// inside an expert is the running count of earlier tokens that chose it).
//
// A stable counting sort in three small kernels plus one row mover (with at
// most 128 blocks, for rows of at most 1 KB or the plan alone, steps 2-4 run
// as one kernel, perm_scatter_gather_kernel, which with at most 8192
// assignments also does step 1 itself):
//   1. hist:    block b (256 tokens) counts its assignments per expert (LDS
//               integer atomics, exact);
//   2. scan:    one workgroup turns the [blocks, E] counts into expert counts,
//               expert offsets and each block's base row per expert;
//   3. scatter: block b marks, per expert, which of its tokens chose it in an
//               LDS bitmap (one bit per token); the rank of token t inside
//               expert e is the popcount of the bits below t, so rows of one
//               expert come out in ascending token id;
//   4. gather:  each 16-byte piece of X is read once and written to the k
//               rows of its token (coalesced row moves).
// A token whose row lists one expert twice is outside the routing contract
// (a top-k never repeats an expert).  It is still sorted by the definition:
// each of its slots gets a row, in slot order.  A block that holds such a
// token ranks its assignments serially (one thread per expert walks the
// block's tokens and slots in order) instead of by bitmap popcounts, which
// count a token once per expert.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxKeys = 256;
constexpr int kWords = kPermBlock / 64;

__global__ __launch_bounds__(kThreads) void perm_hist_kernel(const int32_t* __restrict__ idx,
                                                             int64_t T, int32_t k, int32_t E,
                                                             int32_t* __restrict__ hist) {
  __shared__ int32_t h[kMaxKeys];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kThreads) h[e] = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kPermBlock + tid;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int32_t e = idx[t * k + j];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) hist[static_cast<int64_t>(blockIdx.x) * E + e] = h[e];
}

}  // namespace

// Shared with the dispatch plan: nb blocks of per-key counts -> key counts,
// exclusive key offsets (offsets[nkeys] = total) and per-block base rows.
// Thread e walks its key's column in chunks of 16 independent loads.
__global__ __launch_bounds__(256) void key_scan_kernel(const int32_t* __restrict__ hist,
                                                       int32_t nb, int32_t nkeys,
                                                       int32_t* __restrict__ base,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets) {
  constexpr int kChunk = 16;
  __shared__ int32_t excl[kMaxKeys + 1];
  const int e = threadIdx.x;
  int32_t total = 0;
  if (e < nkeys) {
    for (int b0 = 0; b0 < nb; b0 += kChunk) {
      int32_t v[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        v[i] = (b0 + i < nb) ? hist[static_cast<int64_t>(b0 + i) * nkeys + e] : 0;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) total += v[i];
    }
    if (counts) counts[e] = total;
  }
  excl[e] = (e < nkeys) ? total : 0;
  __syncthreads();
  if (e == 0) {
    int32_t s = 0;
    for (int i = 0; i < nkeys; ++i) {
      const int32_t c = excl[i];
      excl[i] = s;
      s += c;
    }
    excl[nkeys] = s;
  }
  __syncthreads();
  if (e < nkeys) {
    offsets[e] = excl[e];
    int32_t run = excl[e];
    for (int b0 = 0; b0 < nb; b0 += kChunk) {
      int32_t v[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        v[i] = (b0 + i < nb) ? hist[static_cast<int64_t>(b0 + i) * nkeys + e] : 0;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        if (b0 + i < nb) base[static_cast<int64_t>(b0 + i) * nkeys + e] = run;
        run += v[i];
      }
    }
  }
  if (e == 0) offsets[nkeys] = excl[nkeys];
}

namespace {

constexpr int kMaxK = 16;

// the ids of token t (-1 past T and past slot k), all loads issued together
__device__ __forceinline__ void load_row(const int32_t* __restrict__ idx, int64_t t, int64_t T,
                                         int32_t k, int32_t (&row)[kMaxK]) {
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) row[j] = (t < T && j < k) ? idx[t * k + j] : -1;
}
// the token's bit in the LDS bitmap of each expert it chose; dup = 1 when a
// slot repeats the expert of an earlier slot
__device__ __forceinline__ void mark_row(const int32_t (&row)[kMaxK], int32_t k, int32_t E, int w,
                                         int lane, unsigned long long (*bits)[kWords], int* dup) {
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    const int32_t e = row[j];
    if (j >= k || e < 0 || e >= E) continue;
    atomicOr(&bits[e][w], 1ull << lane);
#pragma unroll
    for (int i = 0; i < j; ++i)
      if (row[i] == e) *dup = 1;
  }
}

// Ranks of every assignment of the block starting at token tb inside its
// expert, by definition: thread e walks the block's tokens in order and each
// token's slots in order (srank[local token * k + slot]).  Ends with a
// workgroup barrier.
__device__ void rank_serially(const int32_t* __restrict__ idx, int64_t T, int32_t k, int32_t E,
                              int64_t tb, int32_t* srank) {
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int32_t r = 0;
    for (int tl = 0; tl < kPermBlock && tb + tl < T; ++tl) {
      int32_t row[kMaxK];   // the token's slots, loaded together
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) row[j] = (j < k) ? idx[(tb + tl) * k + j] : -1;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < k && row[j] == e) srank[tl * k + j] = r++;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void perm_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int32_t k, int32_t E,
    const int32_t* __restrict__ base, int32_t* __restrict__ pos, int32_t* __restrict__ src,
    const float* __restrict__ gate, float* __restrict__ gate_perm) {
  __shared__ unsigned long long bits[kMaxKeys][kWords];
  __shared__ int32_t srank[kPermBlock * kMaxK];
  __shared__ int dup;
  const int tid = threadIdx.x;
  for (int i = tid; i < E * kWords; i += kThreads) bits[i / kWords][i % kWords] = 0ull;
  if (tid == 0) dup = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kPermBlock + tid;
  const int w = tid >> 6, lane = tid & 63;
  int32_t row[kMaxK];   // the token's ids, loaded once
  load_row(idx, t, T, k, row);
  mark_row(row, k, E, w, lane, bits, &dup);
  __syncthreads();
  if (dup) rank_serially(idx, T, k, E, static_cast<int64_t>(blockIdx.x) * kPermBlock, srank);
  if (t < T) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) break;
      const int32_t e = row[j];
      if (e < 0 || e >= E) {
        pos[t * k + j] = -1;
        continue;
      }
      int32_t rank;
      if (dup) {
        rank = srank[tid * k + j];
      } else {
        rank = __popcll(bits[e][w] & below);
        for (int ww = 0; ww < w; ++ww) rank += __popcll(bits[e][ww]);
      }
      const int32_t p = base[static_cast<int64_t>(blockIdx.x) * E + e] + rank;
      pos[t * k + j] = p;
      src[p] = static_cast<int32_t>(t);
      if (gate_perm) gate_perm[p] = gate[t * k + j];
    }
  }
}

// Scan, scatter and gather in one kernel (rows of at most 1 KB, or the plan
// alone).  Workgroup (b, q) (256 threads; q < kSgSplit) rebuilds, from the
// [nb, E] block counts (or, hist == NULL, from the ids themselves), the expert
// totals and block b's prefix (LDS integer atomics: exact, order-free), scans the totals into expert offsets
// (workgroup (0, 0) publishes counts and offsets), ranks the 256 tokens of
// block b with the LDS bitmap like perm_scatter_kernel, writes pos/src for its
// quarter of them and copies their rows once from X to each token's k rows of
// x_perm.  The redundant scan and ranking are cheap; the split spreads the
// copy over 4 nb workgroups.
constexpr int kSgSplit = 4;
constexpr int kSgTok = kPermBlock / kSgSplit;
constexpr int kSgMaxBlocks = 128;
constexpr int64_t kSgNoHist = 8192;   // assignments up to which no histogram kernel runs
__global__ __launch_bounds__(kThreads) void perm_scatter_gather_kernel(
    const int32_t* __restrict__ idx, int64_t T, int32_t k, int32_t E,
    const int32_t* __restrict__ hist, int32_t nb, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pos, int32_t* __restrict__ src,
    const uint4* __restrict__ x, uint4* __restrict__ xp, int32_t vpr,
    const float* __restrict__ gate, float* __restrict__ gate_perm) {
  __shared__ unsigned long long bits[kMaxKeys][kWords];
  __shared__ int32_t tot[kMaxKeys], pre[kMaxKeys], base[kMaxKeys + 1];
  __shared__ int32_t spos[kSgTok * kMaxK];
  __shared__ int32_t srank[kPermBlock * kMaxK];
  __shared__ int dup;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / kSgSplit, q = blockIdx.x % kSgSplit;
  for (int i = tid; i < E * kWords; i += kThreads) bits[i / kWords][i % kWords] = 0ull;
  for (int e = tid; e < E; e += kThreads) {
    tot[e] = 0;
    pre[e] = 0;
  }
  if (tid == 0) dup = 0;
  __syncthreads();
  if (!hist) {
    // few assignments, no block counts: the totals and block b's prefix
    // straight from the ids
    const int64_t n = T * k, nb_pre = static_cast<int64_t>(b) * kPermBlock * k;
    constexpr int kU = 8;
    for (int64_t i0 = tid; i0 < n; i0 += kThreads * kU) {
      int32_t v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = i0 + u * kThreads;
        v[u] = (i < n) ? idx[i] : -1;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (v[u] < 0 || v[u] >= E) continue;
        atomicAdd(&tot[v[u]], 1);
        if (i0 + u * kThreads < nb_pre) atomicAdd(&pre[v[u]], 1);
      }
    }
  } else {
    const int64_t n = static_cast<int64_t>(nb) * E;
    constexpr int kU = 8;
    for (int64_t i0 = tid; i0 < n; i0 += kThreads * kU) {
      int32_t v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = i0 + u * kThreads;
        v[u] = (i < n) ? hist[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = i0 + u * kThreads;
        if (i >= n || v[u] == 0) continue;
        const int e = static_cast<int>(i % E);
        atomicAdd(&tot[e], v[u]);
        if (i / E < b) atomicAdd(&pre[e], v[u]);
      }
    }
  }
  __syncthreads();
  if (tid < 64) {   // exclusive scan of the totals by wavefront 0, 64 experts at a time
    int32_t carry = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + tid;
      const int32_t v = (e < E) ? tot[e] : 0;
      int32_t incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int32_t o = __shfl_up(incl, off, 64);
        if (tid >= off) incl += o;
      }
      if (e < E) base[e] = carry + incl - v;
      carry += __shfl(incl, 63, 64);
    }
    if (tid == 0) base[E] = carry;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += kThreads) {
      offsets[e] = base[e];
      if (e < E && counts) counts[e] = tot[e];
    }
  }
  const int64_t t = static_cast<int64_t>(b) * kPermBlock + tid;
  const int w = tid >> 6, lane = tid & 63;
  const bool live = t < T;
  int32_t row[kMaxK];   // the token's ids, loaded once
  load_row(idx, t, T, k, row);
  mark_row(row, k, E, w, lane, bits, &dup);
  __syncthreads();
  if (dup) rank_serially(idx, T, k, E, static_cast<int64_t>(b) * kPermBlock, srank);
  if (live && w == q) {   // this workgroup's quarter: tokens 64 q ... 64 q + 63 of block b
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) break;
      const int32_t e = row[j];
      int32_t p = -1;
      if (e >= 0 && e < E) {
        int32_t rank;
        if (dup) {
          rank = srank[tid * k + j];
        } else {
          rank = __popcll(bits[e][w] & below);
          for (int ww = 0; ww < w; ++ww) rank += __popcll(bits[e][ww]);
        }
        p = base[e] + pre[e] + rank;
        src[p] = static_cast<int32_t>(t);
        if (gate_perm) gate_perm[p] = gate[t * k + j];
      }
      pos[t * k + j] = p;
      spos[lane * k + j] = p;
    }
  }
  __syncthreads();
  if (!x || !xp) return;
  const int64_t t0 = static_cast<int64_t>(b) * kPermBlock + q * kSgTok;
  const int ntok = static_cast<int>(max<int64_t>(0, min<int64_t>(kSgTok, T - t0)));
  const int total = ntok * vpr;
  for (int i = tid; i < total; i += kThreads) {
    const int tl = i / vpr, c = i - tl * vpr;
    const uint4 val = x[(t0 + tl) * vpr + c];
    for (int j = 0; j < k; ++j) {
      const int32_t p = spos[tl * k + j];
      if (p >= 0) xp[static_cast<int64_t>(p) * vpr + c] = val;
    }
  }
}

// x_perm[pos[t, j]] = x[t], moved as 16-byte pieces
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(const uint4* __restrict__ x,
                                                               const int32_t* __restrict__ pos,
                                                               uint4* __restrict__ xp,
                                                               int64_t T, int32_t vec_per_row,
                                                               int32_t k) {
  const int64_t total = T * vec_per_row;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; v < total;
       v += stride) {
    const int64_t t = v / vec_per_row;
    const int32_t c = static_cast<int32_t>(v - t * vec_per_row);
    const uint4 val = ld_nt16(x + v);
    for (int j = 0; j < k; ++j) {
      const int64_t p = pos[t * k + j];
      if (p >= 0) xp[p * vec_per_row + c] = val;
    }
  }
}

}  // namespace

hipError_t launch_permute(const moe_dims& dm, const int32_t* idx, int32_t* counts,
                          int32_t* offsets, int32_t* pos, int32_t* src, const void* x,
                          void* x_perm, int32_t* ws_hist, int32_t* ws_base, hipStream_t s,
                          const float* gate, float* gate_perm) {
  const int64_t nb = (dm.T + kPermBlock - 1) / kPermBlock;
  const int elem = (dm.act == MOE_BF16) ? 2 : 4;
  const int32_t vpr = dm.d * elem / 16;
  // few blocks, and short rows or no rows to move (the plan only): scan,
  // scatter and gather fused (every one of the 4 nb workgroups reads the
  // whole [nb, E] block histogram, so the fused form is kept to nb <= 128,
  // T <= 32768); with at most kSgNoHist assignments each of them counts the
  // ids itself and the histogram kernel is skipped
  const bool rows = x && x_perm;
  const bool fused = nb > 0 && nb <= kSgMaxBlocks && (!rows || dm.d * elem <= 1024) &&
                     dm.k <= kMaxK;
  const bool no_hist = fused && dm.T * dm.k <= kSgNoHist;
  if (nb > 0 && !no_hist) {
    hipLaunchKernelGGL(perm_hist_kernel, dim3(nb), dim3(kThreads), 0, s, idx, dm.T, dm.k, dm.E,
                       ws_hist);
  }
  if (fused) {
    hipLaunchKernelGGL(perm_scatter_gather_kernel, dim3(nb * kSgSplit), dim3(kThreads), 0, s, idx, dm.T,
                       dm.k, dm.E, no_hist ? nullptr : ws_hist, static_cast<int32_t>(nb), counts,
                       offsets, pos, src,
                       static_cast<const uint4*>(x), static_cast<uint4*>(x_perm), vpr, gate,
                       gate_perm);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(key_scan_kernel, dim3(1), dim3(256), 0, s, ws_hist,
                     static_cast<int32_t>(nb), dm.E, ws_base, counts, offsets);
  if (nb > 0) {
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(nb), dim3(kThreads), 0, s, idx, dm.T, dm.k,
                       dm.E, ws_base, pos, src, gate, gate_perm);
  }
  if (rows && dm.T > 0) {
    const int64_t total = dm.T * vpr;
    const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 1 << 16);
    hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(x), pos, static_cast<uint4*>(x_perm), dm.T,
                       vpr, dm.k);
  }
  return hipGetLastError();
}

}  // namespace moe
