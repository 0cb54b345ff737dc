// Expert-parallel dispatch emulated on one device.
//
// Method source: "Expert Coupling in MoE Pretraining" -- Abstract (the
// dispatcher sends each token to each GPU once) and Fig. 5 (dispatch, then
// each GPU runs its experts on the rows it received).  With the deduplicated
// plan of moe_dispatch_plan, the send buffer holds one row per (group, token)
// in (group, token) order, so group g's slice [group_offsets[g],
// group_offsets[g+1]) is what GPU g would receive; a receiver expands its rows
// into its experts' contiguous segments.  On one device every slice is
// "received" in place and the expansion covers all experts, which must give
// the permutation's x_perm bit for bit.
//
// Both kernels are 16-byte row moves, one thread per piece, grid-stride.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// send[r] = x[row_token[r]] for r < *n_rows (a device value: the plan's total)
__global__ __launch_bounds__(kThreads) void ep_pack_kernel(const uint4* __restrict__ x,
                                                           const int32_t* __restrict__ row_token,
                                                           const int32_t* __restrict__ n_rows,
                                                           uint4* __restrict__ send,
                                                           int64_t cap_rows, int32_t vpr) {
  const int64_t rows = min(static_cast<int64_t>(*n_rows), cap_rows);
  const int64_t total = rows * vpr;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; v < total;
       v += stride) {
    const int64_t r = v / vpr;
    const int32_t c = static_cast<int32_t>(v - r * vpr);
    send[v] = x[static_cast<int64_t>(row_token[r]) * vpr + c];
  }
}

// x_perm[pos[t,j]] = recv[assign_row[t,j]] for every assignment (t, j)
template <int K>   // compile-time k (0: runtime k <= 16)
__global__ __launch_bounds__(kThreads) void ep_expand_kernel(const uint4* __restrict__ recv,
                                                             const int32_t* __restrict__ assign_row,
                                                             const int32_t* __restrict__ pos,
                                                             uint4* __restrict__ xp, int64_t T,
                                                             int32_t k, int32_t vpr) {
  constexpr int KM = K > 0 ? K : 16;
  const int kk = K > 0 ? K : k;
  const int64_t total = T * vpr;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; v < total;
       v += stride) {
    const int64_t t = v / vpr;
    const int32_t c = static_cast<int32_t>(v - t * vpr);
    int32_t r[KM], p[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {   // all loads first (clamped slot index)
      const int64_t q = t * kk + min(j, kk - 1);
      r[j] = assign_row[q];
      p[j] = pos[q];
    }
    uint4 val[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) val[j] = recv[static_cast<int64_t>(r[j]) * vpr + c];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < kk) xp[static_cast<int64_t>(p[j]) * vpr + c] = val[j];
  }
}

}  // namespace

hipError_t launch_ep_pack(const moe_dims& dm, int32_t G, const void* x,
                          const int32_t* group_offsets, const int32_t* row_token, void* send,
                          hipStream_t s) {
  const int elem = (dm.act == MOE_BF16) ? 2 : 4;
  const int32_t vpr = dm.d * elem / 16;
  const int64_t cap = dm.T * dm.k;
  if (cap == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((cap * vpr + kThreads - 1) / kThreads, 1 << 16);
  hipLaunchKernelGGL(ep_pack_kernel, dim3(blocks), dim3(kThreads), 0, s,
                     static_cast<const uint4*>(x), row_token, group_offsets + G,
                     static_cast<uint4*>(send), cap, vpr);
  return hipGetLastError();
}

hipError_t launch_ep_expand(const moe_dims& dm, const void* recv, const int32_t* assign_row,
                            const int32_t* pos, void* x_perm, hipStream_t s) {
  if (dm.T == 0) return hipSuccess;
  const int elem = (dm.act == MOE_BF16) ? 2 : 4;
  const int32_t vpr = dm.d * elem / 16;
  const int64_t total = dm.T * vpr;
  const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 1 << 16);
  const uint4* rv = static_cast<const uint4*>(recv);
  uint4* xp = static_cast<uint4*>(x_perm);
#define MOE_EX(KC)                                                                          \
  hipLaunchKernelGGL((ep_expand_kernel<KC>), dim3(blocks), dim3(kThreads), 0, s, rv, assign_row, \
                     pos, xp, dm.T, dm.k, vpr)
  switch (dm.k) {
    case 1: MOE_EX(1); break;
    case 2: MOE_EX(2); break;
    case 4: MOE_EX(4); break;
    case 6: MOE_EX(6); break;
    case 8: MOE_EX(8); break;
    default: MOE_EX(0); break;
  }
#undef MOE_EX
  return hipGetLastError();
}

}  // namespace moe
