// Shared device helpers and launcher declarations of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------- bf16 helpers

typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// round to nearest, ties to even (finite inputs)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// two values rounded to nearest even and packed (lo in bits 0-15): one
// v_cvt_pk_bf16_f32 on gfx950
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f32x2_hw v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}

template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
  static constexpr int kPer16B = 4;
};
template <> struct Act<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ bf16_t from_f32(float v) { return f32_to_bf16(v); }
  static constexpr int kPer16B = 8;
};

// unpack a 16-byte vector of act values into fp32
__device__ __forceinline__ void unpack16(const uint4& v, float* out, float) {
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack16(const uint4& v, float* out, bf16_t) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ uint4 pack16(const float* in, float) {
  return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]),
                    __float_as_uint(in[2]), __float_as_uint(in[3]));
}
__device__ __forceinline__ uint4 pack16(const float* in, bf16_t) {
  return make_uint4(bf16x2_rne(in[0], in[1]), bf16x2_rne(in[2], in[3]),
                    bf16x2_rne(in[4], in[5]), bf16x2_rne(in[6], in[7]));
}

// 16-byte load with the nontemporal hint (data read once: streamed past the
// caches' normal retention)
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt16(const uint4* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt16(uint4* p, uint4 v) {
  __builtin_nontemporal_store(u32x4_nt{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_nt*>(p));
}

// v_rcp_f32 instead of a full division (about 1 ulp); exp(-z) = inf gives 0
__device__ __forceinline__ float sigmoid_f(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

// ---------------------------------------------------------------- workspace

inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// ---------------------------------------------------------------- launchers
// All launchers enqueue on `stream` and return hipSuccess or the launch error.

// route
constexpr int kRouteTileMax = 32;   // tokens per workgroup of the vector-ALU router
constexpr int kRouteMfmaTile = 64;  // tokens per workgroup of the matrix-core router (bf16 x)
constexpr int kRouteF32Tile = 16;   // tokens per workgroup of the fp32 matrix-core router
hipError_t launch_route(const moe_dims& dm, const void* x, const float* wr, float* logits,
                        int32_t* idx, float* gate, float* margin, float eps, int32_t* tie_count,
                        int32_t G, int32_t* gcount, float* gprob, float* gaux, int tile,
                        float* ws_psum, int32_t* ws_pcnt, int32_t* ws_ptie, hipStream_t s);

// permutation (also used by the dispatch plan with "groups" as keys)
constexpr int kPermBlock = 256;     // tokens per permutation block
hipError_t launch_permute(const moe_dims& dm, const int32_t* idx, int32_t* counts,
                          int32_t* offsets, int32_t* pos, int32_t* src, const void* x,
                          void* x_perm, int32_t* ws_hist, int32_t* ws_base, hipStream_t s,
                          const float* gate = nullptr, float* gate_perm = nullptr);

// shared by the permutation and the dispatch plan
__global__ void key_scan_kernel(const int32_t* hist, int32_t nb, int32_t nkeys, int32_t* base,
                                int32_t* counts, int32_t* offsets);

// grouped GEMMs.  x_rows: NULL, or the gather table of the expert input: row p
// of the expert input is then row x_rows[p] of x_perm (which is X [T,d])
hipError_t launch_swiglu_fwd(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                             const int32_t* offsets, const void* w1, const void* w3,
                             const void* w2, void* a, void* b, void* h, void* y, hipStream_t s);
hipError_t launch_swiglu_bwd(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                             const int32_t* offsets,
                             const void* w1, const void* w3, const void* w2, const void* a,
                             const void* b, const void* h, const void* dy_perm, void* dx_perm,
                             void* dw1, void* dw3, void* dw2, bool wgrad_f32, void* ws_da,
                             void* ws_db, float* ws_partial, hipStream_t s);

// kernel-level phases of the expert GEMMs (dispatch on the activation type)
hipError_t launch_expert_up(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                            const int32_t* offsets, const void* w1, const void* w3, void* a,
                            void* b, void* h, hipStream_t s);
hipError_t launch_expert_down(const moe_dims& dm, const void* h, const int32_t* offsets,
                              const void* w2, void* y, hipStream_t s);
hipError_t launch_expert_dgrad_down(const moe_dims& dm, const void* dy_perm,
                                    const int32_t* offsets, const void* w2, const void* a,
                                    const void* b, void* da, void* db, hipStream_t s);
hipError_t launch_expert_dgrad_up(const moe_dims& dm, const void* da, const void* db,
                                  const int32_t* offsets, const void* w1, const void* w3,
                                  void* dx_perm, hipStream_t s);
hipError_t launch_expert_wgrad(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                               const int32_t* offsets, const void* h, const void* dy_perm,
                               const void* da, const void* db, void* dw1, void* dw3, void* dw2,
                               bool wgrad_f32, float* partial, hipStream_t s);

// bf16 matrix-core implementations (gemm_bf16.hip)
hipError_t launch_up_bf16(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                          const int32_t* offsets, const void* w1, const void* w3, void* a,
                          void* b, void* h, hipStream_t s);
hipError_t launch_down_bf16(const moe_dims& dm, const void* h, const int32_t* offsets,
                            const void* w2, void* y, hipStream_t s);
hipError_t launch_dgrad_down_bf16(const moe_dims& dm, const void* dy_perm, const int32_t* offsets,
                                  const void* w2, const void* a, const void* b, void* da,
                                  void* db, hipStream_t s);
hipError_t launch_dgrad_up_bf16(const moe_dims& dm, const void* da, const void* db,
                                const int32_t* offsets, const void* w1, const void* w3,
                                void* dx_perm, hipStream_t s);
// out_f32: dW1, dW3, dW2 are fp32 (the fp32 accumulators stored unrounded)
hipError_t launch_wgrad_bf16(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                             const int32_t* offsets, const void* h, const void* dy_perm,
                             const void* da, const void* db, void* dw1, void* dw3, void* dw2,
                             bool out_f32, float* partial, hipStream_t s);
// gate folded into the expert rows (gathered expert input): UP
// stores g h; DGRAD_DOWN reads dy through the table, scales dh by g and writes
// per-row dgate parts; WGRAD reads dy through the table for dW2
bool folded_bf16_ok(const moe_dims& dm);
int dgate_parts_bf16(const moe_dims& dm);
hipError_t launch_up_folded_bf16(const moe_dims& dm, const void* x, const int32_t* x_rows,
                                 const int32_t* offsets, const float* gate_rows, const void* w1,
                                 const void* w3, void* a, void* b, void* hg, hipStream_t s);
hipError_t launch_dgrad_down_folded_bf16(const moe_dims& dm, const void* dy,
                                         const int32_t* x_rows, const int32_t* offsets,
                                         const float* gate_rows, const void* w2, const void* a,
                                         const void* b, void* da, void* db, float* dgate_part,
                                         hipStream_t s);
hipError_t launch_wgrad_folded_bf16(const moe_dims& dm, const void* x, const int32_t* x_rows,
                                    const int32_t* offsets, const void* hg, const void* dy,
                                    const void* da, const void* db, void* dw1, void* dw3,
                                    void* dw2, hipStream_t s);
// split-K count of the weight gradients, and the fp32 partial tiles it needs
int wgrad_splits_bf16(const moe_dims& dm, bool out_f32 = false);
size_t wgrad_partial_bytes_bf16(const moe_dims& dm, bool out_f32 = false);

// combine
hipError_t launch_combine(const moe_dims& dm, const void* rows, const int32_t* pos,
                          const float* gate, void* out, hipStream_t s);
hipError_t launch_dgate_from_parts(const moe_dims& dm, const float* part, int32_t nparts,
                                   const int32_t* pos, float* dgate, hipStream_t s);
hipError_t launch_combine_bwd(const moe_dims& dm, const void* dy, const void* y_perm,
                              const int32_t* pos, const float* gate, void* dy_perm,
                              float* dgate, hipStream_t s);

// router backward
hipError_t launch_route_bwd(const moe_dims& dm, const void* x, const float* wr,
                            const int32_t* idx, const float* gate, const float* dgate,
                            const int32_t* offsets, const int32_t* pos, const int32_t* src,
                            const void* dx_perm, void* dx, float* dwr, float* ws_dl_perm,
                            float* ws_dl_sel, float* ws_partial, hipStream_t s,
                            const float* dgate_part = nullptr, int32_t nparts = 0,
                            float* dgate_out = nullptr);
int route_bwd_splits(const moe_dims& dm);   // row splits per expert for the router weight gradient
// the router weight gradient on the matrix cores (dl in token-slot order in
// ws_dl_sel, route_bwd_mfma_splits token splits: partials E x splits x d)
bool route_bwd_mfma_ok(const moe_dims& dm);
int route_bwd_mfma_ld(const moe_dims& dm);
int64_t route_bwd_mfma_len(const moe_dims& dm);
int route_bwd_mfma_splits(const moe_dims& dm);
// dense form: dropped assignments and the auxiliary losses
hipError_t launch_route_bwd_dense(const moe_dims& dm, const void* x, const float* wr,
                                  const float* logits, const int32_t* idx, const float* gate,
                                  const float* dgate, const int32_t* pos, const void* dx_perm,
                                  int32_t G, const int32_t* count, float aux_coef, float z_coef,
                                  void* dx, float* dwr, float* dlogits, float* ws_dl,
                                  float* ws_partial, hipStream_t s);
int route_bwd_dense_splits(const moe_dims& dm);   // token splits of its weight gradient

// per-block capacity with dropping; per-block mean of logsumexp^2
hipError_t launch_capacity(int64_t T, int32_t k, int32_t E, int32_t G, int32_t C,
                           const int32_t* idx, int32_t* kept, int32_t* dropped, int32_t* ws_hist,
                           hipStream_t s);
int capacity_chunks(int64_t T, int32_t G);   // token chunks per block (workspace: G chunks k E ints)
hipError_t launch_router_z(int64_t T, int32_t E, int32_t G, const float* logits, float* group_z,
                           float* ws_partial, hipStream_t s);
int zloss_chunks(int64_t T, int32_t G);      // token chunks per block (workspace: G chunks floats)
hipError_t launch_route_flips(int64_t T, int32_t k, int32_t E, const int32_t* a, const int32_t* b,
                              int32_t* flips, int32_t* n_flips, hipStream_t s);

// index products
hipError_t launch_coselect(int64_t T, int32_t k, int32_t E, const int32_t* idx, int32_t* W,
                           hipStream_t s);

struct PlacementArg {
  int32_t group_of[256];
};
hipError_t launch_dispatch_plan(int64_t T, int32_t k, int32_t E, int32_t G,
                                const int32_t* idx, const PlacementArg& pl, int32_t* n_dest,
                                int32_t* group_rows, int32_t* group_offsets, int32_t* row_token,
                                int32_t* assign_row, int32_t* stats, uint64_t* ws_mask,
                                int32_t* ws_hist, int32_t* ws_base, int32_t* ws_stat,
                                hipStream_t s);

// token-shuffle planning: cross-layer co-selection and the owner prediction
hipError_t launch_coselect_cross(int64_t T, int32_t k, int32_t E, const int32_t* cur,
                                 const int32_t* nxt, int32_t* W, hipStream_t s);
hipError_t launch_shuffle_plan(int64_t T, int32_t k, int32_t E, int32_t G, const int32_t* cur,
                               const int32_t* W, const PlacementArg& pl, const int32_t* nxt,
                               int32_t* owner, int32_t* group_tokens, int32_t* stats,
                               int32_t* ws_mass, hipStream_t s);

// expert-parallel dispatch emulated on one device
hipError_t launch_ep_pack(const moe_dims& dm, int32_t G, const void* x,
                          const int32_t* group_offsets, const int32_t* row_token, void* send,
                          hipStream_t s);
hipError_t launch_ep_expand(const moe_dims& dm, const void* recv, const int32_t* assign_row,
                            const int32_t* pos, void* x_perm, hipStream_t s);

}  // namespace moe
