// Router backward, fused with the unpermute-and-sum of the expert input grads.
//
// The router's forward is logits -> top-k -> softmax over the k chosen logits
// ("Revisiting MoE and Dense Speed-Accuracy Comparisons", Sec. 2.1 Top-K
// routing; "Expert Coupling in MoE Pretraining", Abstract).  Its adjoint is
//   dl[t, S_j] = g_j (dg_j - sum_i g_i dg_i)   (zero for unchosen experts),
//   dX[t]     += sum_j dl[t, S_j] Wr[S_j],
//   dWr[e]     = sum_t dl[t, e] X[t].
// Three kernels: the dX rows (k expert-gradient rows plus k router rows,
// summed in fp32 in slot order and rounded once; dl computed per token on the
// way and scattered into permuted row order), dWr partial sums over contiguous
// parts of each expert's rows (the permutation lists them in ascending token
// order), and a fixed-order reduction of the parts.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// One thread per 16-byte chunk of a dX row (grid-stride):
//   dl[t,j] = g_j (dg_j - sum_i g_i dg_i)          (the fp32 sum in slot order)
//   dX[t]   = sum_j dx_perm[pos[t,j]] + sum_j dl[t,j] wr[idx[t,j]]
// summed in fp32 in slot order and rounded once.  The thread holding chunk 0
// of a row also scatters dl into permuted row order for the dWr kernel.  K is
// the compile-time k (0: runtime k <= 16); every load of a token is issued
// before any is used (indices clamped, invalid slots masked), so a row costs
// one memory latency rather than one per slot.
template <typename TA, int K>
__global__ __launch_bounds__(kThreads) void router_dx_kernel(
    const uint4* __restrict__ dxp, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const float* __restrict__ dgate, const float* __restrict__ wr, uint4* __restrict__ dx,
    float* __restrict__ dl_perm, int64_t T, int32_t vpr, int32_t d, int32_t k, int32_t E) {
  constexpr int kPer = Act<TA>::kPer16B;
  constexpr int KM = K > 0 ? K : 16;
  const int kk = K > 0 ? K : k;
  const int64_t total = T * vpr;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; v < total;
       v += stride) {
    const int64_t t = v / vpr;
    const int32_t c = static_cast<int32_t>(v - t * vpr);
    float g[KM], dg[KM];
    int32_t p[KM], e[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int64_t q = t * kk + min(j, kk - 1);
      g[j] = gate[q];
      dg[j] = dgate[q];
      p[j] = pos[q];
      e[j] = idx[q];
    }
    uint4 rows[KM];
    float w[KM][kPer];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      rows[j] = dxp ? dxp[static_cast<int64_t>(max(p[j], 0)) * vpr + c] : make_uint4(0u, 0u, 0u, 0u);
      const float* wp = wr + static_cast<int64_t>(min(max(e[j], 0), E - 1)) * d +
                        static_cast<int64_t>(c) * kPer;
#pragma unroll
      for (int i = 0; i < kPer; ++i) w[j][i] = wp[i];
    }
    float inner = 0.f;
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < kk) inner = fmaf(g[j], dg[j], inner);
    float dl[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) dl[j] = g[j] * (dg[j] - inner);
    if (c == 0) {
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j < kk && p[j] >= 0) dl_perm[p[j]] = dl[j];
    }
    float acc[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j >= kk || !dxp || p[j] < 0) continue;
      float r[kPer];
      unpack16(rows[j], r, TA{});
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] += r[i];
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j >= kk || e[j] < 0 || e[j] >= E) continue;
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] = fmaf(dl[j], w[j][i], acc[i]);
    }
    dx[v] = pack16(acc, TA{});
  }
}

// dWr[e] = sum over rows p of expert e (ascending token order) of
// dl_perm[p] * x[src[p]].  The expert's rows are cut into `splits` contiguous
// parts; workgroup (col block, split, e) sums its part: wavefront w takes the
// runs of kRows rows w, w + 4, ... of it in order (a run's row ids and dl are
// one vector load, then all kRows x rows are in flight), and the four
// wavefronts are combined in order.  A second kernel adds the parts in split
// order.  Each lane owns 4 columns.  (A last-workgroup-reduces variant needs a
// device-scope release per workgroup, which on this multi-L2 part writes back
// the XCD's L2 each time: measured 2.5x slower than the second launch, with
// the release alone, and worse with a full fence.)

__device__ __forceinline__ void load4(const float* p, float* v) {
  const float4 q = *reinterpret_cast<const float4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void load4(const bf16_t* p, float* v) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xFFFF0000u);
  v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xFFFF0000u);
}

constexpr int kRows = 8;   // rows per wavefront in flight

template <typename TA>
__global__ __launch_bounds__(kThreads) void router_dwr_partial_kernel(
    const TA* __restrict__ x, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ src, const float* __restrict__ dl_perm,
    float* __restrict__ partial, int32_t d, int32_t splits) {
  __shared__ float red[4][256];
  const int e = blockIdx.z, sp = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int col0 = blockIdx.x * 256 + lane * 4;
  const int32_t p0 = offsets[e], n = offsets[e + 1] - p0;
  const int32_t lo = p0 + static_cast<int32_t>((static_cast<int64_t>(n) * sp) / splits);
  const int32_t hi = p0 + static_cast<int32_t>((static_cast<int64_t>(n) * (sp + 1)) / splits);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (col0 < d) {   // lanes 0 .. kRows - 1 always pass (d % 64 == 0)
    for (int32_t p = lo + wave * kRows; p < hi; p += 4 * kRows) {
      // rows p .. p + kRows - 1: lanes 0 .. kRows - 1 load their ids and
      // weights (one vector load each, clamped in bounds), then broadcast
      const int32_t my_q = min(p + (lane & (kRows - 1)), hi - 1);
      const int32_t my_s = src[my_q];
      const float my_g = dl_perm[my_q];
      int32_t s[kRows];
      float g[kRows];
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        s[u] = __builtin_amdgcn_readlane(my_s, u);
        g[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g), u));
      }
      float v[kRows][4];
#pragma unroll
      for (int u = 0; u < kRows; ++u) load4(x + static_cast<int64_t>(s[u]) * d + col0, v[u]);
      // branch-free: a branch here would let the compiler sink each load into
      // its own block and serialise them; rows past hi weigh 0
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        const float w = (p + u < hi) ? g[u] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, v[u][i], acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][lane * 4 + i] = acc[i];
  __syncthreads();
  if (wave == 0 && col0 < d) {
    float* out = partial + (static_cast<int64_t>(e) * splits + sp) * d + col0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[i] = ((red[0][lane * 4 + i] + red[1][lane * 4 + i]) + red[2][lane * 4 + i]) +
               red[3][lane * 4 + i];
  }
}

// Adds the per-split partial sums of dWr.  Workgroup (column block of 64,
// expert): thread (split lane sl = t / 16, column group cg = t % 16) adds
// splits sl, sl + 16, ... in order (all loads issued first), then thread
// group sl = 0 adds the 16 lane sums in order: a fixed summation order, so
// the result is reproducible, and one memory latency per thread.
__global__ __launch_bounds__(kThreads) void router_dwr_reduce_kernel(
    const float* __restrict__ partial, float* __restrict__ dwr, int32_t E, int32_t d,
    int32_t splits) {
  __shared__ float4 red[16][16];
  const int e = blockIdx.y;
  const int sl = threadIdx.x >> 4, cg = threadIdx.x & 15;
  const int col = blockIdx.x * 64 + cg * 4;
  const bool ok = col < d;   // d is a multiple of 64; kept for safety
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (ok) {
    constexpr int kMaxPer = 4;   // splits <= 64
    float4 v[kMaxPer];
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
      const int sp = min(sl + 16 * u, splits - 1);
      v[u] = *reinterpret_cast<const float4*>(partial + (static_cast<int64_t>(e) * splits + sp) * d + col);
    }
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
      if (sl + 16 * u >= splits) break;
      s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
    }
  }
  red[sl][cg] = s;
  __syncthreads();
  if (sl == 0 && ok) {
    float4 r = red[0][cg];
    for (int q = 1; q < 16; ++q) {
      const float4 o = red[q][cg];
      r.x += o.x; r.y += o.y; r.z += o.z; r.w += o.w;
    }
    *reinterpret_cast<float4*>(dwr + static_cast<int64_t>(e) * d + col) = r;
  }
}

}  // namespace

// row splits per expert for the router weight gradient: about 2048 workgroups
int route_bwd_splits(const moe_dims& dm) {
  const int64_t base = static_cast<int64_t>(dm.E) * ((dm.d + 255) / 256);
  const int64_t s = (2048 + base - 1) / base;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(s, 64)));
}

hipError_t launch_route_bwd(const moe_dims& dm, const void* x, const float* wr,
                            const int32_t* idx, const float* gate, const float* dgate,
                            const int32_t* offsets, const int32_t* pos, const int32_t* src,
                            const void* dx_perm, void* dx, float* dwr, float* ws_dl_perm,
                            float* ws_dl_sel, float* ws_partial, hipStream_t s) {
  if (dm.T > 0) {
    const int elem = (dm.act == MOE_BF16) ? 2 : 4;
    const int32_t vpr = dm.d * elem / 16;
    const int64_t total = dm.T * vpr;
    const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 1 << 16);
    const uint4* dxp = static_cast<const uint4*>(dx_perm);
    uint4* dxo = static_cast<uint4*>(dx);
#define MOE_DX(TA, KC)                                                                        \
  hipLaunchKernelGGL((router_dx_kernel<TA, KC>), dim3(blocks), dim3(kThreads), 0, s, dxp, pos, \
                     idx, gate, dgate, wr, dxo, ws_dl_perm, dm.T, vpr, dm.d, dm.k, dm.E)
    if (dm.act == MOE_BF16) {
      switch (dm.k) {
        case 1: MOE_DX(bf16_t, 1); break;
        case 2: MOE_DX(bf16_t, 2); break;
        case 4: MOE_DX(bf16_t, 4); break;
        case 6: MOE_DX(bf16_t, 6); break;
        case 8: MOE_DX(bf16_t, 8); break;
        default: MOE_DX(bf16_t, 0); break;
      }
    } else {
      switch (dm.k) {
        case 1: MOE_DX(float, 1); break;
        case 2: MOE_DX(float, 2); break;
        case 4: MOE_DX(float, 4); break;
        case 6: MOE_DX(float, 6); break;
        case 8: MOE_DX(float, 8); break;
        default: MOE_DX(float, 0); break;
      }
    }
#undef MOE_DX
  }
  const int splits = route_bwd_splits(dm);
  const dim3 grid((dm.d + 255) / 256, splits, dm.E);
  if (dm.act == MOE_BF16)
    hipLaunchKernelGGL(router_dwr_partial_kernel<bf16_t>, grid, dim3(kThreads), 0, s,
                       static_cast<const bf16_t*>(x), offsets, src, ws_dl_perm, ws_partial, dm.d,
                       splits);
  else
    hipLaunchKernelGGL(router_dwr_partial_kernel<float>, grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(x), offsets, src, ws_dl_perm, ws_partial, dm.d,
                       splits);
  hipLaunchKernelGGL(router_dwr_reduce_kernel, dim3((dm.d + 63) / 64, dm.E), dim3(kThreads), 0,
                     s, ws_partial, dwr, dm.E, dm.d, splits);
  return hipGetLastError();
}

}  // namespace moe
