// Gate-weighted combine of each token's k expert rows, and its adjoint.
//
// Method sources: "Expert Coupling in MoE Pretraining" (Abstract and Fig. 5
// step 5: combine the expert results; the backward pass routes the gradients
// the same way); "Revisiting MoE and Dense Speed-Accuracy Comparisons"
// (Sec. 2.2: GShard combine).
//
// Both kernels are gathers keyed by the token, so no two threads ever write
// the same output and no atomics are needed: the sum over the k slots runs in
// slot order in fp32, which makes the result bitwise reproducible.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// out[t] = sum_j gate[t,j] * rows[pos[t,j]]; one thread per 16-byte piece.
// K is the compile-time k (0: runtime k <= 16); every load of a piece (its k
// positions and gates, then its k rows, clamped in bounds) is issued before
// any is used, so a piece costs one memory latency rather than one per slot.
template <typename TA, int K>
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint4* __restrict__ rows,
                                                           const int32_t* __restrict__ pos,
                                                           const float* __restrict__ gate,
                                                           uint4* __restrict__ out, int64_t T,
                                                           int32_t vpr, int32_t k) {
  constexpr int kPer = Act<TA>::kPer16B;
  constexpr int KM = K > 0 ? K : 16;
  const int kk = K > 0 ? K : k;
  const int64_t total = T * vpr;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; v < total;
       v += stride) {
    const int64_t t = v / vpr;
    const int32_t c = static_cast<int32_t>(v - t * vpr);
    int32_t p[KM];
    float g[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int64_t q = t * kk + min(j, kk - 1);
      p[j] = (j < kk) ? pos[q] : -1;
      g[j] = gate ? gate[q] : 1.0f;
    }
    uint4 rv[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) rv[j] = ld_nt16(rows + static_cast<int64_t>(max(p[j], 0)) * vpr + c);
    float acc[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (p[j] < 0) continue;
      float r[kPer];
      unpack16(rv[j], r, TA{});
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] = fmaf(g[j], r[i], acc[i]);
    }
    st_nt16(out + v, pack16(acc, TA{}));
  }
}

// dy_perm[pos[t,j]] = gate[t,j] * dy[t];  dgate[t,j] = <dy[t], y_perm[pos[t,j]]>
// A group of L lanes (a power of two <= 64) owns one token; the dot product is
// reduced across the group with xor shuffles in a fixed pattern.
template <typename TA, int L>
__global__ __launch_bounds__(kThreads) void combine_bwd_kernel(
    const uint4* __restrict__ dy, const uint4* __restrict__ yp, const int32_t* __restrict__ pos,
    const float* __restrict__ gate, uint4* __restrict__ dyp, float* __restrict__ dgate,
    int64_t T, int32_t vpr, int32_t k) {
  constexpr int kPer = Act<TA>::kPer16B;
  const int lane_in = threadIdx.x % L;
  const int64_t groups_per_block = kThreads / L;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * groups_per_block + threadIdx.x / L;
  const bool live = t < T;
  for (int j = 0; j < k; ++j) {
    const int64_t p = live ? pos[t * k + j] : -1;
    const float g = live ? gate[t * k + j] : 0.f;
    float dot = 0.f;
    if (p >= 0) {
      for (int c = lane_in; c < vpr; c += L) {
        float a[kPer], b[kPer];
        unpack16(ld_nt16(dy + t * vpr + c), a, TA{});
        unpack16(ld_nt16(yp + p * vpr + c), b, TA{});
        float s[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          dot = fmaf(a[i], b[i], dot);
          s[i] = g * a[i];
        }
        dyp[p * vpr + c] = pack16(s, TA{});
      }
    }
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (live && lane_in == 0) dgate[t * k + j] = (p >= 0) ? dot : 0.f;
  }
}

template <typename TA>
hipError_t combine_bwd_dispatch(int L, dim3 grid, hipStream_t s, const uint4* dy,
                                const uint4* yp, const int32_t* pos, const float* gate,
                                uint4* dyp, float* dgate, int64_t T, int32_t vpr, int32_t k) {
#define MOE_CB(LL)                                                                         \
  case LL:                                                                                 \
    hipLaunchKernelGGL((combine_bwd_kernel<TA, LL>), grid, dim3(kThreads), 0, s, dy, yp, pos, \
                       gate, dyp, dgate, T, vpr, k);                                       \
    break;
  switch (L) {
    MOE_CB(8)
    MOE_CB(16)
    MOE_CB(32)
    default: MOE_CB(64)
  }
#undef MOE_CB
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const moe_dims& dm, const void* rows, const int32_t* pos,
                          const float* gate, void* out, hipStream_t s) {
  if (dm.T == 0) return hipSuccess;
  const int elem = (dm.act == MOE_BF16) ? 2 : 4;
  const int32_t vpr = dm.d * elem / 16;
  const int64_t total = dm.T * vpr;
  const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 1 << 16);
  const uint4* rv = static_cast<const uint4*>(rows);
  uint4* ov = static_cast<uint4*>(out);
#define MOE_C(TA, KC)                                                                         \
  hipLaunchKernelGGL((combine_kernel<TA, KC>), dim3(blocks), dim3(kThreads), 0, s, rv, pos, gate, \
                     ov, dm.T, vpr, dm.k)
#define MOE_C_K(TA)                  \
  switch (dm.k) {                    \
    case 1: MOE_C(TA, 1); break;     \
    case 2: MOE_C(TA, 2); break;     \
    case 4: MOE_C(TA, 4); break;     \
    case 6: MOE_C(TA, 6); break;     \
    case 8: MOE_C(TA, 8); break;     \
    default: MOE_C(TA, 0); break;    \
  }
  if (dm.act == MOE_BF16) {
    MOE_C_K(bf16_t)
  } else {
    MOE_C_K(float)
  }
#undef MOE_C_K
#undef MOE_C
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const moe_dims& dm, const void* dy, const void* y_perm,
                              const int32_t* pos, const float* gate, void* dy_perm,
                              float* dgate, hipStream_t s) {
  if (dm.T == 0) return hipSuccess;
  const int elem = (dm.act == MOE_BF16) ? 2 : 4;
  const int32_t vpr = dm.d * elem / 16;
  int L = 8;
  while (L < 64 && L < vpr) L <<= 1;
  const int64_t per_block = kThreads / L;
  const dim3 grid((dm.T + per_block - 1) / per_block);
  if (dm.act == MOE_BF16)
    return combine_bwd_dispatch<bf16_t>(L, grid, s, static_cast<const uint4*>(dy),
                                        static_cast<const uint4*>(y_perm), pos, gate,
                                        static_cast<uint4*>(dy_perm), dgate, dm.T, vpr, dm.k);
  return combine_bwd_dispatch<float>(L, grid, s, static_cast<const uint4*>(dy),
                                     static_cast<const uint4*>(y_perm), pos, gate,
                                     static_cast<uint4*>(dy_perm), dgate, dm.T, vpr, dm.k);
}

// Gate-folded backward: dgate[t, j] = the sum of the column-tile parts of
// row pos[t, j] in tile order (0 for a dropped slot), one thread per slot.
namespace {
__global__ __launch_bounds__(kThreads) void dgate_from_parts_kernel(
    const float* __restrict__ part, int32_t nparts, const int32_t* __restrict__ pos,
    float* __restrict__ dgate, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n) return;
  const int32_t p = pos[i];
  float s = 0.f;
  if (p >= 0)
    for (int q = 0; q < nparts; ++q) s += part[static_cast<int64_t>(p) * nparts + q];
  dgate[i] = s;
}
}  // namespace

hipError_t launch_dgate_from_parts(const moe_dims& dm, const float* part, int32_t nparts,
                                   const int32_t* pos, float* dgate, hipStream_t s) {
  const int64_t n = dm.T * dm.k;
  if (n > 0)
    hipLaunchKernelGGL(dgate_from_parts_kernel, dim3((n + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, s, part, nparts, pos, dgate, n);
  return hipGetLastError();
}

}  // namespace moe
