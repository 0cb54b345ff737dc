// Router: logits, wavefront top-k, renormalised gates, margins, near-ties and
// per-block load-balancing statistics.
//
// Method sources: "Expert Coupling in MoE Pretraining" (Abstract: each token
// is routed to k of E experts); "Revisiting MoE and Dense Speed-Accuracy
// Comparisons" (Sec. 2.1 Top-K routing and the GShard balancing loss, Sec. 3.6
// the second expert is the second best, Sec. 2.2 outer batches); "MoE
// Pretraining: Parallelism Layout Changes the Model" (Finding 3: the margin
// between the k-th and (k+1)-th scores; balancing statistics per machine).
//
// The main kernel gives each workgroup a tile of consecutive tokens (a tile
// never straddles two balancing blocks): logits (on the matrix cores, bf16 or
// fp32, for 64-token tiles; on the vector ALUs for the smaller tiles that
// balancing blocks of other sizes need), then one 16-lane group (or one
// wavefront) per token for top-k, gates, margin and the full softmax, and
// per-tile partial sums of the balancing statistics, which a second kernel
// folds per block in a fixed order (no floating-point atomics).
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kDChunk = 32;
constexpr int kMaxE = 256;
constexpr int kOutPerThread = kRouteTileMax * kMaxE / kThreads;  // 32

struct RouteArgs {
  const void* x;
  const float* wr;
  float* logits;
  int32_t* idx;
  float* gate;
  float* margin;
  float* psum;            // [tiles, E] partial sums of the full softmax
  int32_t* pcnt;          // [tiles, E] partial expert counts
  int32_t* ptie;          // [tiles] partial near-tie counts
  int32_t* gcount;        // [G, E] or NULL
  float* gprob;           // [G, E] or NULL
  float* gaux;            // [G] or NULL
  int32_t* tie_count;     // [1]
  int64_t T;
  int32_t d, E, k, tile, G, n_tiles;
  float eps;
};

__device__ __forceinline__ int ep4(int E) { return (E + 3) & ~3; }

struct Key {
  float v;
  int32_t i;
};

// (v, i) beats (w, j) when v > w, or v == w and i < j
__device__ __forceinline__ bool better(float v, int32_t i, float w, int32_t j) {
  return v > w || (v == w && i < j);
}

__device__ __forceinline__ Key wave_argmax(Key k) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float v = __shfl_xor(k.v, off, 64);
    int32_t i = __shfl_xor(k.i, off, 64);
    if (better(v, i, k.v, k.i)) { k.v = v; k.i = i; }
  }
  return k;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <typename TX>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
  __shared__ float xs[kRouteTileMax][kDChunk + 1];
  __shared__ float wsh[kMaxE][kDChunk + 1];
  __shared__ float ls[kRouteTileMax][kMaxE + 1];
  __shared__ float psum_w[4][kMaxE];
  __shared__ int32_t pcnt_w[4][kMaxE];
  __shared__ int32_t tie_w[4];

  const int tid = threadIdx.x;
  const int E = a.E, d = a.d, k = a.k, tile = a.tile;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tile;
  const int ntok = static_cast<int>(min<int64_t>(tile, a.T - t0));
  const int nout = ntok * E;
  const TX* x = static_cast<const TX*>(a.x);

  // ---------------- phase 1: logits of the tile
  float acc[kOutPerThread];
#pragma unroll
  for (int i = 0; i < kOutPerThread; ++i) acc[i] = 0.f;

  // chunk c0 + kDChunk is loaded into registers while chunk c0 is summed,
  // so a chunk costs one memory latency in total, not one each
  constexpr int kXPer = kRouteTileMax * kDChunk / kThreads;   // 4
  constexpr int kWPer = kMaxE * kDChunk / kThreads;           // 32
  float xr[kXPer], wv[kWPer];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {
      const int v = tid + u * kThreads, t = v / kDChunk, c = v % kDChunk;
      xr[u] = (t < ntok && c0 < d) ? Act<TX>::load(x + (t0 + t) * d + c0 + c) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kWPer; ++u) {
      const int v = tid + u * kThreads, e = v / kDChunk, c = v % kDChunk;
      wv[u] = (e < E && c0 < d) ? a.wr[static_cast<int64_t>(e) * d + c0 + c] : 0.f;
    }
  };
  load_chunk(0);
  for (int c0 = 0; c0 < d; c0 += kDChunk) {
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {
      const int v = tid + u * kThreads;
      if (v < tile * kDChunk) xs[v / kDChunk][v % kDChunk] = xr[u];
    }
#pragma unroll
    for (int u = 0; u < kWPer; ++u) {
      const int v = tid + u * kThreads;
      if (v < E * kDChunk) wsh[v / kDChunk][v % kDChunk] = wv[u];
    }
    __syncthreads();
    load_chunk(c0 + kDChunk);
#pragma unroll
    for (int i = 0; i < kOutPerThread; ++i) {
      const int o = tid + i * kThreads;
      if (o < nout) {
        const int t = o / E, e = o % E;
        float s = acc[i];
#pragma unroll 8
        for (int c = 0; c < kDChunk; ++c) s = fmaf(xs[t][c], wsh[e][c], s);
        acc[i] = s;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < kOutPerThread; ++i) {
    const int o = tid + i * kThreads;
    if (o < nout) {
      const int t = o / E, e = o % E;
      ls[t][e] = acc[i];
      a.logits[(t0 + t) * E + e] = acc[i];
    }
  }
  __syncthreads();

  // ---------------- phase 2: one wavefront per token
  const int wave = tid >> 6, lane = tid & 63;
  float my_psum[kMaxE / 64];
  int32_t my_cnt[kMaxE / 64];
#pragma unroll
  for (int s = 0; s < kMaxE / 64; ++s) { my_psum[s] = 0.f; my_cnt[s] = 0; }
  int32_t ties = 0;

  for (int t = wave; t < ntok; t += 4) {
    float v[kMaxE / 64];
    uint32_t taken = 0;
#pragma unroll
    for (int s = 0; s < kMaxE / 64; ++s) {
      const int e = lane + 64 * s;
      v[s] = (e < E) ? ls[t][e] : -INFINITY;
    }
    // round r's winner is known to every lane; lane r keeps it
    float my_v = -INFINITY, v_top = -INFINITY, v_km1 = 0.f, v_k = 0.f;
    int32_t my_i = 0;
    const int rounds = (k < E) ? k + 1 : k;
    for (int r = 0; r < rounds; ++r) {
      Key best{-INFINITY, 0x7fffffff};
#pragma unroll
      for (int s = 0; s < kMaxE / 64; ++s) {
        const int e = lane + 64 * s;
        if (e < E && !(taken & (1u << s)) && better(v[s], e, best.v, best.i)) {
          best.v = v[s];
          best.i = e;
        }
      }
      best = wave_argmax(best);
      if (r == 0) v_top = best.v;
      if (r == k - 1) v_km1 = best.v;
      if (r == k) v_k = best.v;
      if (lane == r) { my_v = best.v; my_i = best.i; }
      // the (k+1)-th round only reads the runner-up: it is not chosen
      if (r < k && (best.i & 63) == lane) taken |= 1u << (best.i >> 6);
    }
    // full softmax for the balancing statistics
    float ex[kMaxE / 64];
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxE / 64; ++s) {
      const int e = lane + 64 * s;
      ex[s] = (e < E) ? __expf(v[s] - v_top) : 0.f;
      part += ex[s];
    }
    const float inv = 1.0f / wave_sum(part);
#pragma unroll
    for (int s = 0; s < kMaxE / 64; ++s) {
      my_psum[s] += ex[s] * inv;
      if (taken & (1u << s)) my_cnt[s] += 1;
    }
    // gates: softmax over the k chosen logits (lane j holds choice j)
    const float my_e = (lane < k) ? __expf(my_v - v_top) : 0.f;
    const float z = wave_sum(my_e);
    const int64_t tg = t0 + t;
    if (lane < k) {
      a.idx[tg * k + lane] = my_i;
      a.gate[tg * k + lane] = my_e / z;
    }
    const float m = (k < E) ? v_km1 - v_k : INFINITY;
    if (lane == 0) {
      a.margin[tg] = m;
      ties += (m < a.eps) ? 1 : 0;
    }
  }
#pragma unroll
  for (int s = 0; s < kMaxE / 64; ++s) {
    const int e = lane + 64 * s;
    if (e < E) {
      psum_w[wave][e] = my_psum[s];
      pcnt_w[wave][e] = my_cnt[s];
    }
  }
  if (lane == 0) tie_w[wave] = ties;
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    float s = psum_w[0][e];
    int32_t c = pcnt_w[0][e];
    for (int w = 1; w < 4; ++w) {
      s += psum_w[w][e];
      c += pcnt_w[w][e];
    }
    a.psum[static_cast<int64_t>(blockIdx.x) * ep4(E) + e] = s;
    a.pcnt[static_cast<int64_t>(blockIdx.x) * ep4(E) + e] = c;
  }
  if (tid == 0) a.ptie[blockIdx.x] = tie_w[0] + tie_w[1] + tie_w[2] + tie_w[3];
}

// ---------------------------------------------------------------------------
// Matrix-core router for bf16 hidden states (tiles of 64 tokens).
//
// fp32 router weights are split exactly into three bf16 terms, w = hi + mid +
// lo (hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid); each
// remainder is exact in fp32).  A bf16 x times a bf16 term is exact in fp32,
// so three v_mfma_f32_16x16x32_bf16 passes into one fp32 accumulator give an
// fp32-accumulated dot product with the fp32 weights.  The split happens while
// a 32-wide chunk of Wr is staged into LDS, shared by the 4 wavefronts; each
// wavefront owns 16 tokens and reads its x fragments straight from HBM, two
// chunks ahead.  The accumulators leave lane l holding tokens 4(l/16)+q and
// experts 16j + l%16, so every token's E logits sit in one 16-lane group:
// top-k, gates, margin and the full softmax run there with 16-lane shuffles.
// ---------------------------------------------------------------------------
constexpr int kMTile = 64;       // tokens per workgroup
constexpr int kMBK = 64;         // k chunk (two 32-wide MFMA sub-steps)
constexpr int kMLd = kMBK + 8;   // LDS row stride (elements)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Reductions over the 16 lanes of a DPP row: rotations by 8, 4, 2 and 1
// lanes within the row (row_ror, a VALU operand modifier rather than an LDS
// round trip).  At each level a lane combines the same two partial results as
// its partner does, so all 16 lanes end bitwise identical.
template <int CTRL>
__device__ __forceinline__ int row_rot(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);   // every lane has a source
}
template <int CTRL>
__device__ __forceinline__ float row_rot(float v) {
  return __int_as_float(row_rot<CTRL>(__float_as_int(v)));
}
constexpr int kRowRor8 = 0x128, kRowRor4 = 0x124, kRowRor2 = 0x122, kRowRor1 = 0x121;

template <int CTRL>
__device__ __forceinline__ void argmax_level(Key& k) {
  const float v = row_rot<CTRL>(k.v);
  const int32_t i = row_rot<CTRL>(k.i);
  if (better(v, i, k.v, k.i)) {
    k.v = v;
    k.i = i;
  }
}

__device__ __forceinline__ Key group16_argmax(Key k) {
  argmax_level<kRowRor8>(k);
  argmax_level<kRowRor4>(k);
  argmax_level<kRowRor2>(k);
  argmax_level<kRowRor1>(k);
  return k;
}

__device__ __forceinline__ float group16_sum(float v) {
  v += row_rot<kRowRor8>(v);
  v += row_rot<kRowRor4>(v);
  v += row_rot<kRowRor2>(v);
  v += row_rot<kRowRor1>(v);
  return v;
}

// Selection keys: one unsigned 64-bit integer per (logit, expert) whose
// order is the selection order, larger logit first and, on equal logits, the
// smaller expert id (the high word is the logit's bits made monotone: sign
// bit set for non-negative values, all bits inverted for negative ones; the
// low word is the inverted expert id).  -0 is folded into +0 first so that
// equal logits give equal high words.  Key 0 lies below every real key and
// marks experts already taken or absent.
__device__ __forceinline__ uint64_t sel_key(float v, int32_t e) {
  uint32_t u = __float_as_uint(v + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(~e);
}
__device__ __forceinline__ float sel_key_value(uint64_t k) {
  uint32_t u = static_cast<uint32_t>(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}
__device__ __forceinline__ int32_t sel_key_expert(uint64_t k) {
  return static_cast<int32_t>(~static_cast<uint32_t>(k));
}
template <int CTRL>
__device__ __forceinline__ uint64_t key_max_level(uint64_t k) {
  const uint32_t lo = static_cast<uint32_t>(row_rot<CTRL>(static_cast<int>(static_cast<uint32_t>(k))));
  const uint32_t hi = static_cast<uint32_t>(row_rot<CTRL>(static_cast<int>(static_cast<uint32_t>(k >> 32))));
  const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
  return o > k ? o : k;
}

// Per-token epilogue shared by the matrix-core router kernels (NW wavefronts
// per workgroup): lane (g, c) of wavefront `wave` holds the logits of tokens
// t0 + 16 wave + 4 g + q (q < 4) for experts 16 j + c in acc[j][q].  Writes
// logits, top-k ids and gates, margins, and the workgroup's LB partial sums
// (fixed-order folds).
template <int NT, int NW = 4>
__device__ __forceinline__ void route_tile_epilogue(const RouteArgs& a, const f32x4_t (&acc)[NT],
                                                    int64_t t0) {
  __shared__ float psum_w[NW][16 * NT];
  __shared__ int32_t pcnt_w[NW][16 * NT];
  __shared__ int32_t tie_w[NW];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int E = a.E, k = a.k;
  float my_psum[NT];
  int32_t my_cnt[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) { my_psum[j] = 0.f; my_cnt[j] = 0; }
  int32_t ties = 0;
  // the lane's 4 tokens go through every step together, so the 4 dependency
  // chains of each cross-lane reduction interleave
  float v[4][NT];
  bool live[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t tg = t0 + wave * 16 + g * 4 + q;
    live[q] = tg < a.T;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int e = 16 * j + c;
      v[q][j] = (e < E) ? acc[j][q] : -INFINITY;
      if (live[q] && e < E) a.logits[tg * E + e] = acc[j][q];
    }
  }
  uint64_t key[4][NT];
  uint64_t my_key[4], k_top[4], k_km1[4], k_k[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int j = 0; j < NT; ++j) key[q][j] = (16 * j + c < E) ? sel_key(v[q][j], 16 * j + c) : 0ull;
    my_key[q] = k_top[q] = k_km1[q] = k_k[q] = 0ull;
  }
  // round r finds the r-th best key of each token (a max over the lane's own
  // keys, then over the 16 lanes); rounds before k retire it
  const int rounds = (k < E) ? k + 1 : k;
  for (int r = 0; r < rounds; ++r) {
    uint64_t best[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      best[q] = key[q][0];
#pragma unroll
      for (int j = 1; j < NT; ++j) best[q] = key[q][j] > best[q] ? key[q][j] : best[q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) best[q] = key_max_level<kRowRor8>(best[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q) best[q] = key_max_level<kRowRor4>(best[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q) best[q] = key_max_level<kRowRor2>(best[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q) best[q] = key_max_level<kRowRor1>(best[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (r == 0) k_top[q] = best[q];
      if (r == k - 1) k_km1[q] = best[q];
      if (r == k) k_k[q] = best[q];
      if (c == r) my_key[q] = best[q];
      if (r < k) {
#pragma unroll
        for (int j = 0; j < NT; ++j) key[q][j] = (key[q][j] == best[q]) ? 0ull : key[q][j];
      }
    }
  }
  // taken experts: the real keys retired by the first k rounds
  uint32_t taken[4];
  float my_v[4], v_top[4], v_km1[4], v_k[4];
  int32_t my_i[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v_top[q] = sel_key_value(k_top[q]);
    v_km1[q] = sel_key_value(k_km1[q]);
    v_k[q] = sel_key_value(k_k[q]);
    taken[q] = 0u;
#pragma unroll
    for (int j = 0; j < NT; ++j)
      if (16 * j + c < E && key[q][j] == 0ull) taken[q] |= 1u << j;
    my_v[q] = (c < k) ? sel_key_value(my_key[q]) : -INFINITY;
    my_i[q] = (c < k) ? sel_key_expert(my_key[q]) : 0;
  }
  float ex[4][NT], part[4], my_e[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    part[q] = 0.f;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int e = 16 * j + c;
      ex[q][j] = (e < E) ? __expf(v[q][j] - v_top[q]) : 0.f;
      part[q] += ex[q][j];
    }
    my_e[q] = (c < k) ? __expf(my_v[q] - v_top[q]) : 0.f;
  }
  float z[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) z[q] = my_e[q];
#pragma unroll
  for (int q = 0; q < 4; ++q) { part[q] += row_rot<kRowRor8>(part[q]); z[q] += row_rot<kRowRor8>(z[q]); }
#pragma unroll
  for (int q = 0; q < 4; ++q) { part[q] += row_rot<kRowRor4>(part[q]); z[q] += row_rot<kRowRor4>(z[q]); }
#pragma unroll
  for (int q = 0; q < 4; ++q) { part[q] += row_rot<kRowRor2>(part[q]); z[q] += row_rot<kRowRor2>(z[q]); }
#pragma unroll
  for (int q = 0; q < 4; ++q) { part[q] += row_rot<kRowRor1>(part[q]); z[q] += row_rot<kRowRor1>(z[q]); }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t tg = t0 + wave * 16 + g * 4 + q;
    const float inv = 1.0f / part[q];
    if (live[q]) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        my_psum[j] += ex[q][j] * inv;
        if (taken[q] & (1u << j)) my_cnt[j] += 1;
      }
      if (c < k) {
        a.idx[tg * k + c] = my_i[q];
        a.gate[tg * k + c] = my_e[q] / z[q];
      }
      const float m = (k < E) ? v_km1[q] - v_k[q] : INFINITY;
      if (c == 0) {
        a.margin[tg] = m;
        ties += (m < a.eps) ? 1 : 0;
      }
    }
  }
  // fold the 4 lane groups (fixed xor order), then the 4 waves (fixed order)
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    float s = my_psum[j];
    int32_t n = my_cnt[j];
    s += __shfl_xor(s, 16, 64);
    n += __shfl_xor(n, 16, 64);
    s += __shfl_xor(s, 32, 64);
    n += __shfl_xor(n, 32, 64);
    if (g == 0) {
      psum_w[wave][16 * j + c] = s;
      pcnt_w[wave][16 * j + c] = n;
    }
  }
  ties += __shfl_xor(ties, 16, 64);
  ties += __shfl_xor(ties, 32, 64);
  if (lane == 0) tie_w[wave] = ties;
  __syncthreads();
  for (int e = tid; e < E; e += 64 * NW) {
    float s = psum_w[0][e];
    int32_t n = pcnt_w[0][e];
#pragma unroll
    for (int w = 1; w < NW; ++w) {   // wavefront order
      s += psum_w[w][e];
      n += pcnt_w[w][e];
    }
    const int64_t o = static_cast<int64_t>(blockIdx.x) * ep4(E) + e;
    a.psum[o] = s;
    a.pcnt[o] = n;
  }
  int32_t tt = tie_w[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) tt += tie_w[w];
  if (tid == 0) a.ptie[blockIdx.x] = tt;
}

template <int NT>   // 16-expert tiles: E <= 16 NT
__global__ __launch_bounds__(kThreads) void route_mfma_kernel(RouteArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t wsh[3][16 * NT][kMLd];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int E = a.E, d = a.d, k = a.k;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kMTile;
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const int nk = d / kMBK;

  // A fragment source: token row t0 + 16 wave + c, k offset 8 g
  const int64_t my_row = t0 + wave * 16 + c;
  const bool row_ok = my_row < a.T;
  const bf16_t* xrow = x + (row_ok ? my_row : 0) * d + g * 8;

  // Wr staging: NT*16 rows x kMBK k fp32 (NT*16*kMBK/4 float4), split into 3 bf16 terms
  constexpr int kWVec = NT * 16 * (kMBK / 4);
  constexpr int kWPer = (kWVec + kThreads - 1) / kThreads;
  float4 wv[kWPer];
  auto wload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int v = tid + i * kThreads;
      const int e = v / (kMBK / 4), q = v % (kMBK / 4);
      wv[i] = (v < kWVec && e < E)
                  ? *reinterpret_cast<const float4*>(a.wr + static_cast<int64_t>(e) * d +
                                                     kt * kMBK + q * 4)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto wstore = [&]() {
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int v = tid + i * kThreads;
      if (v >= kWVec) continue;
      const int e = v / (kMBK / 4), q = v % (kMBK / 4);
      const float w[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
      uint32_t hi[2], mi[2], lo[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        bf16_t h2[2], m2[2], l2[2];
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const float f0 = w[2 * p + z];
          const bf16_t h = f32_to_bf16(f0);
          const float r1 = f0 - bf16_to_f32(h);
          const bf16_t m = f32_to_bf16(r1);
          const float r2 = r1 - bf16_to_f32(m);
          h2[z] = h;
          m2[z] = m;
          l2[z] = f32_to_bf16(r2);
        }
        hi[p] = h2[0] | (static_cast<uint32_t>(h2[1]) << 16);
        mi[p] = m2[0] | (static_cast<uint32_t>(m2[1]) << 16);
        lo[p] = l2[0] | (static_cast<uint32_t>(l2[1]) << 16);
      }
      *reinterpret_cast<uint2*>(&wsh[0][e][q * 4]) = make_uint2(hi[0], hi[1]);
      *reinterpret_cast<uint2*>(&wsh[1][e][q * 4]) = make_uint2(mi[0], mi[1]);
      *reinterpret_cast<uint2*>(&wsh[2][e][q * 4]) = make_uint2(lo[0], lo[1]);
    }
  };

  f32x4_t acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // X fragments two chunks ahead: lane (g, c) holds 8 k values of sub-step s
  // of its token row
  constexpr int kAhead = 2;
  uint4 xa[kAhead][2];
#pragma unroll
  for (int i = 0; i < kAhead; ++i)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      xa[i][s2] = (row_ok && i < nk)
                      ? *reinterpret_cast<const uint4*>(xrow + i * kMBK + s2 * 32)
                      : make_uint4(0u, 0u, 0u, 0u);
  wload(0);
  for (int kt = 0; kt < nk; ++kt) {
    wstore();
    __syncthreads();
    if (kt + 1 < nk) wload(kt + 1);
    const uint4 cur0 = xa[0][0], cur1 = xa[0][1];
#pragma unroll
    for (int i = 0; i + 1 < kAhead; ++i) {
      xa[i][0] = xa[i + 1][0];
      xa[i][1] = xa[i + 1][1];
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      xa[kAhead - 1][s2] = (row_ok && kt + kAhead < nk)
                               ? *reinterpret_cast<const uint4*>(xrow + (kt + kAhead) * kMBK +
                                                                 s2 * 32)
                               : make_uint4(0u, 0u, 0u, 0u);
    // sub-steps in k order, and per expert block hi, mid, lo: the fp32 sum
    // runs in the same order as with 32-wide chunks
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(s2 == 0 ? &cur0 : &cur1);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) {
          const bf16x8_t bfr =
              *reinterpret_cast<const bf16x8_t*>(&wsh[sp][16 * j + c][s2 * 32 + g * 8]);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, acc[j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  route_tile_epilogue<NT>(a, acc, t0);
}

// Matrix-core router for small E d (the split weight fits in LDS whole):
// the workgroup splits fp32 Wr exactly into bf16 hi + mid + lo parts straight
// into LDS (rounding to nearest even at each stage, so hi + mid + lo is the
// fp32 weight and bf16 x bf16 products accumulated in fp32 give the fp32
// logits), with one barrier; each wavefront holds its 16 tokens' X fragments
// for the whole of K in registers (all loads issued at once) and runs the
// MFMAs with B fragments from LDS.
template <int NT, int NKC>   // NKC: K chunks of 32 (d = 32 NKC)
__global__ __launch_bounds__(kThreads) void route_lds_kernel(RouteArgs a) {
  constexpr int kLd = 32 * NKC + 8;
  __shared__ __attribute__((aligned(16))) bf16_t wsh_dyn[3 * 16 * NT * kLd];   // [3][16 NT][kLd]
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int E = a.E, d = a.d;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kMTile;
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const int64_t my_row = t0 + wave * 16 + c;
  const bool row_ok = my_row < a.T;
  const bf16_t* xrow = x + (row_ok ? my_row : 0) * d + g * 8;
  uint4 xa[NKC];
#pragma unroll
  for (int kt = 0; kt < NKC; ++kt) {
    xa[kt] = *reinterpret_cast<const uint4*>(xrow + kt * 32);
    if (!row_ok) xa[kt] = make_uint4(0u, 0u, 0u, 0u);
  }
  // split Wr (E x d fp32; rows >= E are zero) into LDS, 4 weights per
  // vector; the vectors of a thread are loaded in batches of 8 before any is
  // split, so their latencies overlap
  constexpr int kRowsP = 16 * NT;
  constexpr int kDv = 8 * NKC;                        // float4 vectors per row (d / 4)
  constexpr int kPer = kRowsP * kDv / kThreads;       // vectors per thread
  static_assert(kRowsP * kDv % kThreads == 0, "whole vectors per thread");
  constexpr int kBatch = kPer < 8 ? kPer : 8;
#pragma unroll
  for (int b0 = 0; b0 < kPer; b0 += kBatch) {
    float4 wb[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int v = tid + (b0 + u) * kThreads;
      const int e = v / kDv, q = v % kDv;
      wb[u] = (e < E) ? *reinterpret_cast<const float4*>(a.wr + static_cast<int64_t>(e) * d + q * 4)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int v = tid + (b0 + u) * kThreads;
      const int e = v / kDv, q = v % kDv;
      const float4 w4 = wb[u];
      const float w[4] = {w4.x, w4.y, w4.z, w4.w};
      uint32_t hi[2], mi[2], lo[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        bf16_t h2[2], m2[2], l2[2];
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const float f0 = w[2 * p + z];
          const bf16_t h = f32_to_bf16(f0);
          const float r1 = f0 - bf16_to_f32(h);
          const bf16_t m = f32_to_bf16(r1);
          const float r2 = r1 - bf16_to_f32(m);
          h2[z] = h;
          m2[z] = m;
          l2[z] = f32_to_bf16(r2);
        }
        hi[p] = h2[0] | (static_cast<uint32_t>(h2[1]) << 16);
        mi[p] = m2[0] | (static_cast<uint32_t>(m2[1]) << 16);
        lo[p] = l2[0] | (static_cast<uint32_t>(l2[1]) << 16);
      }
      bf16_t* row = wsh_dyn + e * kLd + q * 4;
      *reinterpret_cast<uint2*>(row) = make_uint2(hi[0], hi[1]);
      *reinterpret_cast<uint2*>(row + kRowsP * kLd) = make_uint2(mi[0], mi[1]);
      *reinterpret_cast<uint2*>(row + 2 * kRowsP * kLd) = make_uint2(lo[0], lo[1]);
    }
  }
  __syncthreads();
  f32x4_t acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < NKC; ++kt) {
    const bf16x8_t af = __builtin_bit_cast(bf16x8_t, xa[kt]);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) {
        const bf16x8_t bfr = *reinterpret_cast<const bf16x8_t*>(
            wsh_dyn + (sp * kRowsP + 16 * j + c) * kLd + kt * 32 + g * 8);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, acc[j], 0, 0, 0);
      }
  }
  route_tile_epilogue<NT>(a, acc, t0);
}

// fp32 hidden states on the fp32 matrix cores (v_mfma_f32_16x16x4_f32), one
// wavefront of 16 tokens per workgroup (small fp32 batches then still spread
// over every CU), with the C layout and epilogue of the bf16 routers.  For one
// 16-wide k block lane (g, c) loads k = 4 g ... 4 g + 3 of its token row c and
// of expert row 16 j + c as one float4 each, and MFMA step s takes element s
// of both: A and B use the same k assignment, so the 4 steps cover the block.
// Every wavefront reads X and Wr straight from global memory into registers,
// KB blocks per batch (10 to 18 float4 per lane for both operands; blocks
// past d read zeros), the next batch in flight while the current one runs.
template <int NT>   // 16-expert tiles: E <= 16 NT
__global__ __launch_bounds__(64) void route_f32_kernel(RouteArgs a) {
  constexpr int KB = NT == 1 ? 8 : NT == 2 ? 4 : NT <= 8 ? 2 : 1;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int E = a.E, d = a.d;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouteF32Tile;
  const int64_t my_row = t0 + wave * 16 + c;
  const bool row_ok = my_row < a.T;
  const float* xrow = static_cast<const float*>(a.x) + (row_ok ? my_row : 0) * d + 4 * g;
  const float* wrow[NT];
  bool w_ok[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int e = 16 * j + c;
    w_ok[j] = e < E;
    wrow[j] = a.wr + static_cast<int64_t>(w_ok[j] ? e : 0) * d + 4 * g;
  }
  const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 xc[KB], wc[KB][NT], xn[KB], wn[KB][NT];
  auto load = [&](int bt, float4 (&xo)[KB], float4 (&wo)[KB][NT]) {
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const int k0 = (bt * KB + b) * 16;
      const bool k_ok = k0 < d;
      xo[b] = (row_ok && k_ok) ? *reinterpret_cast<const float4*>(xrow + k0) : zero4;
#pragma unroll
      for (int j = 0; j < NT; ++j)
        wo[b][j] = (w_ok[j] && k_ok) ? *reinterpret_cast<const float4*>(wrow[j] + k0) : zero4;
    }
  };
  f32x4_t acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nb = (d + 16 * KB - 1) / (16 * KB);
  load(0, xc, wc);
  for (int bt = 0; bt < nb; ++bt) {
    if (bt + 1 < nb) load(bt + 1, xn, wn);
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const float xs[4] = {xc[b].x, xc[b].y, xc[b].z, xc[b].w};
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const float ws[4] = {wc[b][j].x, wc[b][j].y, wc[b][j].z, wc[b][j].w};
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[st], ws[st], acc[j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      xc[b] = xn[b];
#pragma unroll
      for (int j = 0; j < NT; ++j) wc[b][j] = wn[b][j];
    }
  }
  route_tile_epilogue<NT, 1>(a, acc, t0);
}

// Second launch of the two-kernel paths (every path but the streaming one):
// one workgroup (1024 threads) per balancing block r (grid G), all experts in
// one pass: thread (slice, e) with slice < SL = 1024 / E_p (E_p: E rounded up
// to a power of two, at least 16) adds tiles slice, slice + SL, ... of block r
// in tile order (16 loads in flight); the slice sums are folded in a fixed
// order, first across the slices inside a wavefront (lane xor 16, then 32),
// then across wavefronts through LDS in wavefront order.  The expert products
// f_e P_e and (block 0) the near-tie counts are reduced by wavefront 0 alone,
// again in a fixed order.
constexpr int kFinThreads = 1024;
constexpr int kFinWaves = kFinThreads / 64;
__global__ __launch_bounds__(kFinThreads) void route_finalize_kernel(
    const float* psum, const int32_t* pcnt, const int32_t* ptie, int32_t n_tiles,
    int32_t tiles_per_group, int64_t T, int32_t E, int32_t k, int32_t* gcount, float* gprob,
    float* gaux, int32_t* tie_count) {
  __shared__ float sp[kFinThreads];
  __shared__ int32_t sc[kFinThreads];
  __shared__ float fp[kMaxE];
  __shared__ int32_t st[kFinWaves];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Ep = E <= 16 ? 16 : E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256;
  const int SL = kFinThreads / Ep;
  const int slice = tid / Ep, e = tid % Ep;
  const int64_t G = gridDim.x;
  const double per_group = static_cast<double>(T) / static_cast<double>(G);
  for (int i = tid; i < kMaxE; i += kFinThreads) fp[i] = 0.f;
  float s = 0.f;
  int32_t c = 0;
  if (e < E) {
    for (int i0 = slice; i0 < tiles_per_group; i0 += SL * 16) {
      float ps[16];
      int32_t pc[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = min(i0 + SL * u, tiles_per_group - 1);
        const int64_t tile = static_cast<int64_t>(r) * tiles_per_group + i;
        ps[u] = psum[tile * ep4(E) + e];
        pc[u] = pcnt[tile * ep4(E) + e];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (i0 + SL * u >= tiles_per_group) break;
        s += ps[u];
        c += pc[u];
      }
    }
  }
  // slices inside one wavefront (E_p < 64): lanes e, e + E_p, ... of a wavefront
  if (Ep <= 16) {
    s += __shfl_xor(s, 16, 64);
    c += __shfl_xor(c, 16, 64);
  }
  if (Ep <= 32) {
    s += __shfl_xor(s, 32, 64);
    c += __shfl_xor(c, 32, 64);
  }
  sp[tid] = s;
  sc[tid] = c;
  __syncthreads();
  if (tid < E) {
    // one partial per wavefront for E_p <= 64, else one per slice
    const int step = Ep < 64 ? 64 : Ep;
    const int n_part = kFinThreads / step;
    float S = 0.f;
    int32_t C = 0;
    for (int q = 0; q < n_part; ++q) {
      S += sp[q * step + tid];
      C += sc[q * step + tid];
    }
    const float P = (per_group > 0) ? static_cast<float>(S / per_group) : 0.f;
    const float fr = (per_group > 0) ? static_cast<float>(C / (per_group * k)) : 0.f;
    if (gcount) gcount[static_cast<int64_t>(r) * E + tid] = C;
    if (gprob) gprob[static_cast<int64_t>(r) * E + tid] = P;
    fp[tid] = fr * P;
  }
  int32_t t = 0;
  if (r == 0 && tie_count) {
    for (int i = tid; i < n_tiles; i += kFinThreads) t += ptie[i];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) t += __shfl_xor(t, m, 64);
    if (lane == 0) st[wave] = t;
  }
  __syncthreads();
  if (wave == 0) {
    // fixed order over the (zero-padded) 256 products: 4 per lane, then a
    // lane xor tree
    float v = ((fp[lane] + fp[lane + 64]) + fp[lane + 128]) + fp[lane + 192];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if (lane == 0 && gaux) gaux[r] = static_cast<float>(E) * v;
    if (r == 0 && tie_count) {
      int32_t tt = lane < kFinWaves ? st[lane] : 0;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) tt += __shfl_xor(tt, m, 64);
      if (lane == 0) *tie_count = tt;
    }
  }
}

// ---------------------------------------------------------------------------
// Router for bf16 hidden states, E <= 64 and d > 256: the weight streamed.
//
// The fp32 router weight is split exactly into three bf16 terms on the fly
// (hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid), each remainder
// exact in fp32, so hi + mid + lo = w); a bf16 x times a bf16 term is exact in
// fp32, so three v_mfma_f32_16x16x32_bf16 passes into one fp32 accumulator give
// an fp32-accumulated dot product with the fp32 weights.
//
// 64 tokens per workgroup, 4 wavefronts; wavefront w computes expert block
// w % NT for the token blocks w / NT + (4 / NT) i.  The k loop runs in 64-wide
// chunks, S - 1 chunks ahead: each wavefront moves its own 16 tokens' X chunk
// into an LDS ring with direct-to-LDS loads, laid out as two A fragments, and
// the fp32 weights of its own expert block in the B-fragment layout (lane
// 16 g + c: expert 16 j + c, k = 8 g ... 8 g + 7 of each 32-wide half), which
// it reads back and splits in registers.  Only direct-to-LDS loads fill the
// ring: register-destination loads carried around the loop would make the
// compiler drain the memory counter at the loop head.  Fragment reads from LDS are
// inline-asm ds_read_b128 that wait for themselves, and each chunk waits for
// its own loads with an explicit vmcnt plus a barrier (the compiler would
// drain every direct-to-LDS load in flight before its own LDS reads).  The
// logits then pass through LDS so that each wavefront holds its 16 tokens' E
// logits in the epilogue's layout.
// ---------------------------------------------------------------------------
namespace rdma {
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nbytes, 0x00020000);
}
// The per-lane offset (voff) stays in one loop-invariant register; the
// per-chunk offset goes in the scalar soff.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, bf16_t* lds, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, static_cast<int>(voff),
                                           static_cast<int>(soff), 0, 0);
}
__device__ __forceinline__ float4 ldf4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                        r, static_cast<int>(voff), static_cast<int>(soff), 0));
}
// s_waitcnt with vmcnt = N (bits 3-0 and 15-14), expcnt and lgkmcnt left free
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
}  // namespace rdma

// hi, mid, lo bf16 terms of 8 fp32 weights, packed as three B fragments
__device__ __forceinline__ void split8(const float4& w0, const float4& w1, bf16x8_t& hi,
                                       bf16x8_t& mid, bf16x8_t& lo) {
  const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    h[p] = bf16x2_rne(w[2 * p], w[2 * p + 1]);
    const float r0 = w[2 * p] - __uint_as_float(h[p] << 16);
    const float r1 = w[2 * p + 1] - __uint_as_float(h[p] & 0xFFFF0000u);
    m[p] = bf16x2_rne(r0, r1);
    l[p] = bf16x2_rne(r0 - __uint_as_float(m[p] << 16), r1 - __uint_as_float(m[p] & 0xFFFF0000u));
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  mid = __builtin_bit_cast(bf16x8_t, make_uint4(m[0], m[1], m[2], m[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

// A fragments of one chunk from LDS: the wavefront's token blocks i and both
// 32-wide halves, frag[i][h] at byte offset (2 (4 / NT) i + h) 1 KB from addr;
// one wait for all of them, inside the same asm block.
template <int NT>
__device__ __forceinline__ void read_a(bf16x8_t (&f)[NT][2], uint32_t addr);
template <>
__device__ __forceinline__ void read_a<1>(bf16x8_t (&f)[1][2], uint32_t addr) {
  asm volatile(
      "ds_read_b128 %0, %2 offset:0\n\t"
      "ds_read_b128 %1, %2 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0][0]), "=&v"(f[0][1])
      : "v"(addr)
      : "memory");
}
template <>
__device__ __forceinline__ void read_a<2>(bf16x8_t (&f)[2][2], uint32_t addr) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:0\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:4096\n\t"
      "ds_read_b128 %3, %4 offset:5120\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0][0]), "=&v"(f[0][1]), "=&v"(f[1][0]), "=&v"(f[1][1])
      : "v"(addr)
      : "memory");
}
template <>
__device__ __forceinline__ void read_a<4>(bf16x8_t (&f)[4][2], uint32_t addr) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:0\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\t"
      "ds_read_b128 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0][0]), "=&v"(f[0][1]), "=&v"(f[1][0]), "=&v"(f[1][1]), "=&v"(f[2][0]),
        "=&v"(f[2][1]), "=&v"(f[3][0]), "=&v"(f[3][1])
      : "v"(addr)
      : "memory");
}

// fp32 weights of one chunk from LDS: 4 x 16 bytes at (q) 1 KB from addr
__device__ __forceinline__ void read_w4(float4 (&f)[4], uint32_t addr) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:0\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "ds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
      : "v"(addr)
      : "memory");
}

template <int NT, int S>   // NT: 16-expert blocks (E <= 16 NT); S: ring stages
__global__ __launch_bounds__(kThreads, 1) void route_stream_kernel(RouteArgs a) {
  // a stage: 8 A fragments (4 token blocks x 2 halves) of 1 KB, then per
  // wavefront 4 KB of fp32 weights (lane-major: 1 KB per 16-byte quarter)
  constexpr int kFrag = 512;                    // bf16 elements per KB
  constexpr int kStage = (8 + 4 * 4) * kFrag;
  constexpr int BSTEP = 4 / NT;                 // token-block stride of one wavefront
  constexpr int kLdL = 68;                      // logit exchange row stride (floats)
  static_assert(S >= 2 && 64 * kLdL * 4 <= S * kStage * 2, "exchange fits the ring");
  __shared__ __attribute__((aligned(16))) bf16_t xs[S * kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int d = a.d;
  const int nk = d / 64;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kMTile;
  const int jw = wave % NT;
  const int bw0 = wave / NT;

  const int rows = static_cast<int>(min<int64_t>(kMTile, a.T - t0));
  const bf16_t* xbase = static_cast<const bf16_t*>(a.x) + t0 * d;
  const auto rx = rdma::rsrc(xbase, static_cast<uint32_t>(rows) * d * 2);
  const auto rxz = rdma::rsrc(xbase, 0);
  const auto rw = rdma::rsrc(a.wr, static_cast<uint32_t>(a.E) * d * 4);
  const auto rwz = rdma::rsrc(a.wr, 0);
  // per-lane offsets, loop invariant: X row 16 wave + c at k 8 g (bf16); the
  // weights of expert 16 jw + c at k 8 g (fp32; rows past E read 0)
  const uint32_t xvoff = static_cast<uint32_t>(((16 * wave + c) * d + 8 * g) * 2);
  const uint32_t wvoff = static_cast<uint32_t>(((16 * jw + c) * d + 8 * g) * 4);

  auto issue = [&](int kt, int slot) {
    const bool on = kt < nk;
    bf16_t* st = xs + slot * kStage;
    const uint32_t sx = static_cast<uint32_t>(kt) * 128, sw = static_cast<uint32_t>(kt) * 256;
    rdma::dma16(on ? rx : rxz, st + (2 * wave) * kFrag, xvoff, sx);
    rdma::dma16(on ? rx : rxz, st + (2 * wave + 1) * kFrag, xvoff, sx + 64);
#pragma unroll
    for (int q = 0; q < 4; ++q)   // half h = q / 2 at k + 32 h, + 4 weights for odd q
      rdma::dma16(on ? rw : rwz, st + (8 + 4 * wave + q) * kFrag, wvoff,
                  sw + (q >> 1) * 128 + (q & 1) * 16);
  };

  f32x4_t acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint32_t lds_x = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) bf16_t*)xs));
  const uint32_t a_addr = lds_x + bw0 * 2048 + lane * 16;
  const uint32_t w_addr = lds_x + (8 + 4 * wave) * 1024 + lane * 16;

#pragma unroll
  for (int u = 0; u < S - 1; ++u) issue(u, u);
  for (int kt0 = 0; kt0 < nk; kt0 += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int kt = kt0 + u;
      if (kt < nk) {
        // this chunk's 6 loads done (the 6 of each of the S - 2 later chunks
        // may still be in flight), and every wavefront past the previous
        // chunk's reads, whose stage the next issue overwrites
        rdma::wait_vm<6 * (S - 2)>();
        __builtin_amdgcn_s_barrier();
        issue(kt + S - 1, (u + S - 1) % S);
        float4 wv[4];
        read_w4(wv, w_addr + u * kStage * 2);
        bf16x8_t af[NT][2];
        read_a<NT>(af, a_addr + u * kStage * 2);
        bf16x8_t bf[2][3];
        split8(wv[0], wv[1], bf[0][0], bf[0][1], bf[0][2]);
        split8(wv[2], wv[3], bf[1][0], bf[1][1], bf[1][2]);
        // per token block: k order, then the hi, mid, lo terms
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int sp = 0; sp < 3; ++sp)
              acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i][h], bf[h][sp], acc[i], 0, 0, 0);
      }
    }
  }
  rdma::wait_vm<0>();
  __syncthreads();
  // logits through LDS: wavefront w then holds tokens 16 w + 4 g + q, experts
  // 16 j + c in acc_e[j][q]
  float* L = reinterpret_cast<float*>(xs);
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int b = bw0 + BSTEP * i;
#pragma unroll
    for (int q = 0; q < 4; ++q) L[(16 * b + 4 * g + q) * kLdL + 16 * jw + c] = acc[i][q];
  }
  __syncthreads();
  f32x4_t acc_e[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc_e[j][q] = L[(16 * wave + 4 * g + q) * kLdL + 16 * j + c];
  route_tile_epilogue<NT>(a, acc_e, t0);
}

}  // namespace

// bf16 hidden states with E <= 64: for d <= 256 the split weight sits in LDS
// whole (route_lds_kernel); beyond, it is streamed (route_split_kernel).
bool route_in_lds(const moe_dims& dm) {
  return dm.act == MOE_BF16 && dm.E <= 64 && dm.d <= 256 && dm.d % 64 == 0;
}
bool route_split_ok(const moe_dims& dm) {
  return dm.act == MOE_BF16 && dm.E <= 64 && dm.d > 256 && dm.d % 64 == 0;
}
int route_split_nt(const moe_dims& dm) {
  const int nt = (dm.E + 15) / 16;
  return nt <= 1 ? 1 : nt <= 2 ? 2 : 4;
}

hipError_t launch_route(const moe_dims& dm, const void* x, const float* wr, float* logits,
                        int32_t* idx, float* gate, float* margin, float eps, int32_t* tie_count,
                        int32_t G, int32_t* gcount, float* gprob, float* gaux, int tile,
                        float* ws_psum, int32_t* ws_pcnt, int32_t* ws_ptie,
                        hipStream_t s) {
  const int64_t n_tiles = (dm.T + tile - 1) / tile;
  RouteArgs a{x, wr, logits, idx, gate, margin, ws_psum, ws_pcnt, ws_ptie,
              gcount, gprob, gaux, tie_count, dm.T, dm.d, dm.E, dm.k, tile, G,
              static_cast<int32_t>(n_tiles), eps};
  if (n_tiles > 0) {
    if (tile == kRouteMfmaTile && route_split_ok(dm)) {
      // streaming path
      switch (route_split_nt(dm)) {
        case 1: hipLaunchKernelGGL((route_stream_kernel<1, 5>), dim3(n_tiles), dim3(kThreads), 0, s, a); break;
        case 2: hipLaunchKernelGGL((route_stream_kernel<2, 5>), dim3(n_tiles), dim3(kThreads), 0, s, a); break;
        default: hipLaunchKernelGGL((route_stream_kernel<4, 5>), dim3(n_tiles), dim3(kThreads), 0, s, a); break;
      }
    } else if (tile == kRouteMfmaTile && route_in_lds(dm)) {
      const int nt = (dm.E + 15) / 16;
      const int nt_p = nt <= 1 ? 1 : nt <= 2 ? 2 : 4;
#define MOE_RL(N, K)                                                                          \
  hipLaunchKernelGGL((route_lds_kernel<N, K>), dim3(n_tiles), dim3(kThreads), 0, s, a)
#define MOE_RL_D(N)                              \
  switch (dm.d / 32) {                           \
    case 2: MOE_RL(N, 2); break;                 \
    case 4: MOE_RL(N, 4); break;                 \
    case 6: MOE_RL(N, 6); break;                 \
    default: MOE_RL(N, 8); break;                \
  }
      if (nt_p == 1) { MOE_RL_D(1) } else if (nt_p == 2) { MOE_RL_D(2) } else { MOE_RL_D(4) }
#undef MOE_RL_D
#undef MOE_RL
    } else if (tile == kRouteF32Tile && dm.act == MOE_F32) {
      const int ntf = (dm.E + 15) / 16;
#define MOE_RF(N)                                                                      \
  case N:                                                                              \
    hipLaunchKernelGGL(route_f32_kernel<N>, dim3(n_tiles), dim3(64), 0, s, a);         \
    break;
      switch (ntf <= 1 ? 1 : ntf <= 2 ? 2 : ntf <= 4 ? 4 : ntf <= 8 ? 8 : 16) {
        MOE_RF(1)
        MOE_RF(2)
        MOE_RF(4)
        MOE_RF(8)
        default: MOE_RF(16)
      }
#undef MOE_RF
    } else if (tile == kRouteMfmaTile) {
      const int ntm = (dm.E + 15) / 16;
#define MOE_RM(N)                                                                        \
  case N:                                                                                \
    hipLaunchKernelGGL(route_mfma_kernel<N>, dim3(n_tiles), dim3(kThreads), 0, s, a);    \
    break;
      switch (ntm <= 1 ? 1 : ntm <= 2 ? 2 : ntm <= 4 ? 4 : ntm <= 8 ? 8 : 16) {
        MOE_RM(1)
        MOE_RM(2)
        MOE_RM(4)
        MOE_RM(8)
        default: MOE_RM(16)
      }
#undef MOE_RM
    } else if (dm.act == MOE_BF16) {
      hipLaunchKernelGGL(route_kernel<bf16_t>, dim3(n_tiles), dim3(kThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL(route_kernel<float>, dim3(n_tiles), dim3(kThreads), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int32_t tiles_per_group = static_cast<int32_t>(n_tiles / G);
  hipLaunchKernelGGL(route_finalize_kernel, dim3(G), dim3(kFinThreads), 0, s, ws_psum, ws_pcnt,
                     ws_ptie, static_cast<int32_t>(n_tiles), tiles_per_group, dm.T, dm.E, dm.k,
                     gcount, gprob, gaux, tie_count);
  return hipGetLastError();
}

}  // namespace moe
