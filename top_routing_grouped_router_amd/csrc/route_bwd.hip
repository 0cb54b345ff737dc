// Router backward, fused with the unpermute-and-sum of the expert input grads.
//
// The router's forward is logits -> top-k -> softmax over the k chosen logits
// ("Revisiting MoE and Dense Speed-Accuracy Comparisons", Sec. 2.1 Top-K
// routing; "Expert Coupling in MoE Pretraining", Abstract).  Its adjoint is
//   dl[t, S_j] = g_j (dg_j - sum_i g_i dg_i)   (zero for unchosen experts),
//   dX[t]     += sum_j dl[t, S_j] Wr[S_j],
//   dWr[e]     = sum_t dl[t, e] X[t].
// Three kernels: per-token dl (also scattered into permuted row order), the
// dX rows (k expert-gradient rows plus k router rows, summed in fp32 in slot
// order and rounded once), and dWr as an ordered sum over each expert's rows
// (the permutation already lists them in ascending token order).
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void router_dl_kernel(const float* __restrict__ gate,
                                                             const float* __restrict__ dgate,
                                                             const int32_t* __restrict__ pos,
                                                             float* __restrict__ dl_sel,
                                                             float* __restrict__ dl_perm,
                                                             int64_t T, int32_t k) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= T) return;
  float inner = 0.f;
  for (int j = 0; j < k; ++j) inner = fmaf(gate[t * k + j], dgate[t * k + j], inner);
  for (int j = 0; j < k; ++j) {
    const float dl = gate[t * k + j] * (dgate[t * k + j] - inner);
    dl_sel[t * k + j] = dl;
    const int32_t p = pos[t * k + j];
    if (p >= 0) dl_perm[p] = dl;
  }
}

// dX[t] = sum_j dx_perm[pos[t,j]] + sum_j dl[t,j] * wr[idx[t,j]]
template <typename TA>
__global__ __launch_bounds__(kThreads) void router_dx_kernel(
    const uint4* __restrict__ dxp, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ idx, const float* __restrict__ dl_sel,
    const float* __restrict__ wr, uint4* __restrict__ dx, int64_t T, int32_t vpr, int32_t d,
    int32_t k, int32_t E) {
  constexpr int kPer = Act<TA>::kPer16B;
  const int64_t total = T * vpr;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; v < total;
       v += stride) {
    const int64_t t = v / vpr;
    const int32_t c = static_cast<int32_t>(v - t * vpr);
    float acc[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
    if (dxp) {
      for (int j = 0; j < k; ++j) {
        const int64_t p = pos[t * k + j];
        if (p < 0) continue;
        float r[kPer];
        unpack16(dxp[p * vpr + c], r, TA{});
#pragma unroll
        for (int i = 0; i < kPer; ++i) acc[i] += r[i];
      }
    }
    for (int j = 0; j < k; ++j) {
      const int32_t e = idx[t * k + j];
      if (e < 0 || e >= E) continue;
      const float g = dl_sel[t * k + j];
      const float* w = wr + static_cast<int64_t>(e) * d + static_cast<int64_t>(c) * kPer;
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] = fmaf(g, w[i], acc[i]);
    }
    dx[v] = pack16(acc, TA{});
  }
}

// dWr[e] = sum over rows p of expert e (ascending token order) of
// dl_perm[p] * x[src[p]].  The expert's rows are cut into `splits` contiguous
// parts; workgroup (col block, split, e) sums its part (wave w takes rows
// w, w+4, ..., four rows in flight; the four waves are combined in order), and
// a second kernel adds the parts in split order.  Each lane owns 4 columns.

__device__ __forceinline__ void load4(const float* p, float* v) {
  const float4 q = *reinterpret_cast<const float4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void load4(const bf16_t* p, float* v) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xFFFF0000u);
  v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xFFFF0000u);
}

template <typename TA>
__global__ __launch_bounds__(kThreads) void router_dwr_partial_kernel(
    const TA* __restrict__ x, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ src, const float* __restrict__ dl_perm,
    float* __restrict__ partial, int32_t d, int32_t splits) {
  __shared__ float red[4][256];
  const int e = blockIdx.z, sp = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col0 = blockIdx.x * 256 + lane * 4;
  const int32_t p0 = offsets[e], n = offsets[e + 1] - p0;
  const int32_t lo = p0 + static_cast<int32_t>((static_cast<int64_t>(n) * sp) / splits);
  const int32_t hi = p0 + static_cast<int32_t>((static_cast<int64_t>(n) * (sp + 1)) / splits);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (col0 < d) {
    int32_t p = lo + wave;
    for (; p + 12 < hi; p += 16) {
      float g[4], v[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        g[u] = dl_perm[p + 4 * u];
        load4(x + static_cast<int64_t>(src[p + 4 * u]) * d + col0, v[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(g[u], v[u][i], acc[i]);
    }
    for (; p < hi; p += 4) {
      const float g = dl_perm[p];
      float v[4];
      load4(x + static_cast<int64_t>(src[p]) * d + col0, v);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(g, v[i], acc[i]);
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

__global__ __launch_bounds__(kThreads) void router_dwr_reduce_kernel(
    const float* __restrict__ partial, float* __restrict__ dwr, int32_t E, int32_t d,
    int32_t splits) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= static_cast<int64_t>(E) * d) return;
  const int64_t e = i / d, col = i - e * d;
  const float* p = partial + e * splits * d + col;
  float s = p[0];
  for (int k = 1; k < splits; ++k) s += p[static_cast<int64_t>(k) * d];
  dwr[i] = s;
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
    hipLaunchKernelGGL(router_dl_kernel, dim3((dm.T + kThreads - 1) / kThreads), dim3(kThreads),
                       0, s, gate, dgate, pos, ws_dl_sel, ws_dl_perm, dm.T, dm.k);
    const int elem = (dm.act == MOE_BF16) ? 2 : 4;
    const int32_t vpr = dm.d * elem / 16;
    const int64_t total = dm.T * vpr;
    const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 1 << 16);
    if (dm.act == MOE_BF16)
      hipLaunchKernelGGL(router_dx_kernel<bf16_t>, dim3(blocks), dim3(kThreads), 0, s,
                         static_cast<const uint4*>(dx_perm), pos, idx, ws_dl_sel, wr,
                         static_cast<uint4*>(dx), dm.T, vpr, dm.d, dm.k, dm.E);
    else
      hipLaunchKernelGGL(router_dx_kernel<float>, dim3(blocks), dim3(kThreads), 0, s,
                         static_cast<const uint4*>(dx_perm), pos, idx, ws_dl_sel, wr,
                         static_cast<uint4*>(dx), dm.T, vpr, dm.d, dm.k, dm.E);
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
  const int64_t n = static_cast<int64_t>(dm.E) * dm.d;
  hipLaunchKernelGGL(router_dwr_reduce_kernel, dim3((n + kThreads - 1) / kThreads),
                     dim3(kThreads), 0, s, ws_partial, dwr, dm.E, dm.d, splits);
  return hipGetLastError();
}

}  // namespace moe
