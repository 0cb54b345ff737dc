// Grouped GEMMs of the SwiGLU experts, forward and backward.
//
// Method sources: "Revisiting MoE and Dense Speed-Accuracy Comparisons for LLM
// Training" (Sec. 2.1: SwiGLU activation, Shazeer 2020, in a LLaMA2-style
// block); "MoE Pretraining: Parallelism Layout Changes the Model" (Methodology:
// SwiGLU experts); "Expert Coupling in MoE Pretraining" (Fig. 5 step 4: the
// expert computation, in the forward and backward passes).
//
// Every product here has the form C[m][n] = sum_k A(m,k) B(n,k) over one
// expert's rows.  Five modes:
//   UP          a|b = x_perm W1|W3^T, epilogue h = silu(a) b     (rows split by expert)
//   DOWN        y_perm = h W2^T                                 (rows split by expert)
//   DGRAD_DOWN  dh = dy_perm W2; epilogue da, db from saved a, b (rows split by expert)
//   DGRAD_UP    dx_perm = da W1 + db W3                         (rows split by expert)
//   WGRAD       dW2 = dy^T h, dW1 = da^T x, dW3 = db^T x        (reduction over rows)
// This file holds the fp32 path (bf16 runs on gemm_bf16.hip's kernels).
// Tiles of A and B are staged through LDS in k-contiguous form whatever their
// layout in HBM (operands stored with m or n contiguous are transposed while
// being written to LDS), so one compute core serves all modes: 16x16x4 fp32
// MFMA, 4 waves x (64x64) per 128x128 tile.
// A workgroup's (expert, row tile) comes from the expert offsets on the device,
// so the host never reads the routing.  Each output element is produced by
// exactly one workgroup with a fixed k order: results are reproducible.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 128;

enum Mode { UP = 0, DOWN = 1, DGRAD_DOWN = 2, DGRAD_UP = 3, WGRAD = 4 };

struct GemmArgs {
  const void* a0;      // first A source
  const void* a1;      // second A source (DGRAD_UP: db; WGRAD z=1,2 selects)
  const void* b0;
  const void* b1;
  const void* aux0;    // DGRAD_DOWN: saved a
  const void* aux1;    // DGRAD_DOWN: saved b
  void* c0;
  void* c1;
  void* c2;
  const int32_t* offsets;
  const int32_t* x_rows;   // NULL, or: row p of the expert input is row x_rows[p] of X
  int32_t E, d, f;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename TA> struct Core;

// ------------------------------------------------------------------ fp32 MFMA core
// v_mfma_f32_16x16x4_f32, 4 waves x (64x64) per 128x128 tile; accumulator
// lane (g, r) of a 16x16 block holds rows 4 g + q, column r.  Within a BK = 32 tile, lane (g, r) of a 16-row block takes k = 8 g
// ... 8 g + 7 of its row (two 16-byte LDS reads) and feeds k = 8 g + s at
// step s; A and B use the same assignment, so each of the 8 steps sums k
// = s, 8 + s, 16 + s, 24 + s and the 8 steps cover the tile.
template <> struct Core<float> {
  static constexpr int BK = 32;
  static constexpr int LD = BK + 4;     // 144-byte rows: 16-byte aligned staging and reads
  typedef float T;
  f32x4 acc[4][4];

  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ void compute(const T* As, const T* Bs) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int r = lane & 15, k0 = (lane >> 4) * 8;
    float a[4][8], b[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 lo = *reinterpret_cast<const float4*>(As + (wm * 64 + i * 16 + r) * LD + k0);
      const float4 hi = *reinterpret_cast<const float4*>(As + (wm * 64 + i * 16 + r) * LD + k0 + 4);
      a[i][0] = lo.x; a[i][1] = lo.y; a[i][2] = lo.z; a[i][3] = lo.w;
      a[i][4] = hi.x; a[i][5] = hi.y; a[i][6] = hi.z; a[i][7] = hi.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 lo = *reinterpret_cast<const float4*>(Bs + (wn * 64 + j * 16 + r) * LD + k0);
      const float4 hi = *reinterpret_cast<const float4*>(Bs + (wn * 64 + j * 16 + r) * LD + k0 + 4);
      b[j][0] = lo.x; b[j][1] = lo.y; b[j][2] = lo.z; b[j][3] = lo.w;
      b[j][4] = hi.x; b[j][5] = hi.y; b[j][6] = hi.z; b[j][7] = hi.w;
    }
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][st], b[j][st], acc[i][j], 0, 0, 0);
  }
  template <typename F>
  __device__ void for_each(F&& fn) const {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          fn(wm * 64 + i * 16 + (lane >> 4) * 4 + q, wn * 64 + j * 16 + (lane & 15), acc[i][j][q]);
  }
  // pairs (a, b) whose B-tile rows are r and r + 32 inside one 64-row block
  template <typename F>
  __device__ void for_each_pair(F&& fn) const {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          fn(wm * 64 + i * 16 + (lane >> 4) * 4 + q, wn * 64 + j * 16 + (lane & 15),
             acc[i][j][q], acc[i][j + 2][q]);
  }
};

// ------------------------------------------------------------------ LDS staging
// K-major source: tile row r (< 128) starts at row_ptr(r) + k0; rows >= valid are zero.
template <typename T, int BK, int LD, typename RowPtr>
__device__ __forceinline__ void stage_kmajor(T* lds, RowPtr row_ptr, int valid, int k0) {
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kPerRow = BK / kVec;
  for (int v = threadIdx.x; v < 128 * kPerRow; v += kThreads) {
    const int r = v / kPerRow, c = (v % kPerRow) * kVec;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < valid) val = *reinterpret_cast<const uint4*>(row_ptr(r) + k0 + c);
    *reinterpret_cast<uint4*>(lds + r * LD + c) = val;
  }
}

// MN-major source: element (k, mn) at base[k * ld + mn] for the tile's k rows
// [0, BK) and mn columns [0, 128); k >= kvalid or mn >= mnvalid read as zero.
// Written transposed so that LDS holds [mn][k].
template <typename T, int BK, int LD>
__device__ __forceinline__ void stage_mnmajor(T* lds, const T* base, int64_t ld, int kvalid,
                                              int mnvalid) {
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kPerRow = 128 / kVec;
  for (int v = threadIdx.x; v < BK * kPerRow; v += kThreads) {
    const int kr = v / kPerRow, c = (v % kPerRow) * kVec;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (kr < kvalid && c < mnvalid) val = *reinterpret_cast<const uint4*>(base + kr * ld + c);
    const T* e = reinterpret_cast<const T*>(&val);
#pragma unroll
    for (int i = 0; i < kVec; ++i) lds[(c + i) * LD + kr] = e[i];
  }
}

// As stage_mnmajor, with k row kr at row_ptr(kr) (mn offset applied by the caller)
template <typename T, int BK, int LD, typename RowPtr>
__device__ __forceinline__ void stage_mnmajor_rows(T* lds, RowPtr row_ptr, int kvalid,
                                                   int mnvalid) {
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kPerRow = 128 / kVec;
  for (int v = threadIdx.x; v < BK * kPerRow; v += kThreads) {
    const int kr = v / kPerRow, c = (v % kPerRow) * kVec;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (kr < kvalid && c < mnvalid) val = *reinterpret_cast<const uint4*>(row_ptr(kr) + c);
    const T* e = reinterpret_cast<const T*>(&val);
#pragma unroll
    for (int i = 0; i < kVec; ++i) lds[(c + i) * LD + kr] = e[i];
  }
}

template <typename TA>
__device__ __forceinline__ void store_act(TA* p, float v) { *p = Act<TA>::from_f32(v); }

// the value v takes when stored as TA
template <typename TA>
__device__ __forceinline__ float round_act(float v) { return Act<TA>::to_f32(Act<TA>::from_f32(v)); }

// ------------------------------------------------------------------ row-tile lookup
// Finds the expert and first row of this workgroup's row tile from the expert
// offsets: tile counts per expert are prefix-summed across wave 0's lanes
// (4 experts per lane).  Returns false when the workgroup has no tile.
__device__ bool find_row_tile(const int32_t* offsets, int E, int tile, int* e_out, int* m0_out,
                              int* mend_out) {
  __shared__ int s_e, s_m0, s_mend;
  if (threadIdx.x == 0) s_e = -1;
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    // five independent clamped loads (offsets[E] repeats past the end, so
    // those experts count zero rows): one memory latency, no branches
    int o[5];
#pragma unroll
    for (int s = 0; s < 5; ++s) o[s] = offsets[min(lane * 4 + s, E)];
    int tiles[4], sum = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      tiles[s] = (o[s + 1] - o[s] + BM - 1) / BM;
      sum += tiles[s];
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const int excl = incl - sum;
    // exactly one lane owns the tile (the lanes' ranges [excl, incl) are disjoint)
    if (tile >= excl && tile < incl) {
      int rem = tile - excl;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (rem >= 0 && rem < tiles[s]) {
          const int e = lane * 4 + s;
          s_e = e;
          s_m0 = o[s] + rem * BM;
          s_mend = o[s + 1];
        }
        rem -= tiles[s];
      }
    }
  }
  __syncthreads();
  *e_out = s_e;
  *m0_out = s_m0;
  *mend_out = s_mend;
  return s_e >= 0;
}

// ------------------------------------------------------------------ the kernel
template <typename TA, int MODE>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs g) {
  typedef Core<TA> C;
  constexpr int BK = C::BK, LD = C::LD;
  __shared__ __attribute__((aligned(16))) TA As[BM * LD];
  __shared__ __attribute__((aligned(16))) TA Bs[BN * LD];

  const int d = g.d, f = g.f;
  C core;
  core.zero();

  if constexpr (MODE == WGRAD) {
    // blockIdx.z: 0 -> dW2[e] [d, f] = dy^T h;  1 -> dW1[e] = da^T x;  2 -> dW3[e] = db^T x
    const int z = blockIdx.z;
    const int e = blockIdx.y;
    const int Mdim = (z == 0) ? d : f;
    const int Ndim = (z == 0) ? f : d;
    const int tiles_n = (Ndim + BN - 1) / BN;
    const int m0 = (blockIdx.x / tiles_n) * BM;
    const int n0 = (blockIdx.x % tiles_n) * BN;
    if (m0 >= Mdim) return;
    const TA* Asrc = static_cast<const TA*>(z == 0 ? g.a0 : (z == 1 ? g.a1 : g.aux0));
    const TA* Bsrc = static_cast<const TA*>(z == 0 ? g.b0 : g.b1);
    const int p0 = g.offsets[e], p1 = g.offsets[e + 1];
    for (int p = p0; p < p1; p += BK) {
      const int kvalid = min(BK, p1 - p);
      stage_mnmajor<TA, BK, LD>(As, Asrc + static_cast<int64_t>(p) * Mdim + m0, Mdim, kvalid,
                                Mdim - m0);
      if (z != 0 && g.x_rows)   // B = X rows gathered by the table
        stage_mnmajor_rows<TA, BK, LD>(
            Bs, [&](int kr) { return Bsrc + static_cast<int64_t>(g.x_rows[p + kr]) * Ndim + n0; },
            kvalid, Ndim - n0);
      else
        stage_mnmajor<TA, BK, LD>(Bs, Bsrc + static_cast<int64_t>(p) * Ndim + n0, Ndim, kvalid,
                                  Ndim - n0);
      __syncthreads();
      core.compute(As, Bs);
      __syncthreads();
    }
    TA* out = static_cast<TA*>(z == 0 ? g.c0 : (z == 1 ? g.c1 : g.c2)) +
              static_cast<int64_t>(e) * d * f;
    core.for_each([&](int r, int c, float v) {
      const int m = m0 + r, n = n0 + c;
      if (m < Mdim && n < Ndim) store_act(out + static_cast<int64_t>(m) * Ndim + n, v);
    });
  } else {
    int e, m0, mend;
    if (!find_row_tile(g.offsets, g.E, blockIdx.x, &e, &m0, &mend)) return;
    const int rows = min(BM, mend - m0);
    const int n0 = blockIdx.y * ((MODE == UP) ? 64 : BN);

    if constexpr (MODE == UP) {
      const TA* x = static_cast<const TA*>(g.a0);
      const TA* w1 = static_cast<const TA*>(g.b0) + static_cast<int64_t>(e) * f * d;
      const TA* w3 = static_cast<const TA*>(g.b1) + static_cast<int64_t>(e) * f * d;
      // input row r of the tile: expert row m0 + r, or the X row the table gives
      auto x_row = [&](int r) {
        const int64_t q = g.x_rows ? g.x_rows[m0 + r] : m0 + r;
        return x + q * d;
      };
      for (int k0 = 0; k0 < d; k0 += BK) {
        stage_kmajor<TA, BK, LD>(As, x_row, rows, k0);
        stage_kmajor<TA, BK, LD>(Bs, [&](int r) {
          const int q = r >> 5;
          const TA* w = (q & 1) ? w3 : w1;
          return w + static_cast<int64_t>(n0 + 32 * (q >> 1) + (r & 31)) * d;
        }, BN, k0);
        __syncthreads();
        core.compute(As, Bs);
        __syncthreads();
      }
      TA* ao = static_cast<TA*>(g.c0);
      TA* bo = static_cast<TA*>(g.c1);
      TA* ho = static_cast<TA*>(g.c2);
      core.for_each_pair([&](int r, int c, float av, float bv) {
        if (r >= rows) return;
        // B-tile row c (< 32 within its 64-row block) is f column n0 + 32 (c / 64) + c % 32
        const int n = n0 + 32 * (c >> 6) + (c & 31);
        const int64_t o = static_cast<int64_t>(m0 + r) * f + n;
        // a and b are stored activations; h is formed from the stored values
        const float as = round_act<TA>(av), bs = round_act<TA>(bv);
        store_act(ao + o, as);
        store_act(bo + o, bs);
        store_act(ho + o, silu_f(as) * bs);
      });
    } else if constexpr (MODE == DOWN) {
      const TA* h = static_cast<const TA*>(g.a0) + static_cast<int64_t>(m0) * f;
      const TA* w2 = static_cast<const TA*>(g.b0) + static_cast<int64_t>(e) * d * f;
      const int nvalid = min(BN, d - n0);
      for (int k0 = 0; k0 < f; k0 += BK) {
        stage_kmajor<TA, BK, LD>(As, [&](int r) { return h + static_cast<int64_t>(r) * f; },
                                 rows, k0);
        stage_kmajor<TA, BK, LD>(Bs, [&](int r) {
          return w2 + static_cast<int64_t>(n0 + min(r, nvalid - 1)) * f;
        }, nvalid, k0);
        __syncthreads();
        core.compute(As, Bs);
        __syncthreads();
      }
      TA* yo = static_cast<TA*>(g.c0);
      core.for_each([&](int r, int c, float v) {
        if (r < rows && c < nvalid) store_act(yo + static_cast<int64_t>(m0 + r) * d + n0 + c, v);
      });
    } else if constexpr (MODE == DGRAD_DOWN) {
      // dh[p][n] = sum_k dy[p][k] W2[e][k][n], n < f
      const TA* dy = static_cast<const TA*>(g.a0) + static_cast<int64_t>(m0) * d;
      const TA* w2 = static_cast<const TA*>(g.b0) + static_cast<int64_t>(e) * d * f;
      const int nvalid = min(BN, f - n0);
      for (int k0 = 0; k0 < d; k0 += BK) {
        stage_kmajor<TA, BK, LD>(As, [&](int r) { return dy + static_cast<int64_t>(r) * d; },
                                 rows, k0);
        stage_mnmajor<TA, BK, LD>(Bs, w2 + static_cast<int64_t>(k0) * f + n0, f, BK, nvalid);
        __syncthreads();
        core.compute(As, Bs);
        __syncthreads();
      }
      const TA* sa = static_cast<const TA*>(g.aux0);
      const TA* sb = static_cast<const TA*>(g.aux1);
      TA* dao = static_cast<TA*>(g.c0);
      TA* dbo = static_cast<TA*>(g.c1);
      core.for_each([&](int r, int c, float dh_acc) {
        if (r >= rows || c >= nvalid) return;
        const float dh = round_act<TA>(dh_acc);   // dh is a stored-precision activation gradient
        const int64_t o = static_cast<int64_t>(m0 + r) * f + n0 + c;
        const float av = Act<TA>::load(sa + o), bv = Act<TA>::load(sb + o);
        const float s = sigmoid_f(av);
        const float act = av * s;
        const float dact = s * (1.0f + av * (1.0f - s));
        store_act(dao + o, dh * bv * dact);
        store_act(dbo + o, dh * act);
      });
    } else {  // DGRAD_UP: dx[p][n] = sum_k da[p][k] W1[e][k][n] + db[p][k] W3[e][k][n]
      const TA* da = static_cast<const TA*>(g.a0) + static_cast<int64_t>(m0) * f;
      const TA* db = static_cast<const TA*>(g.a1) + static_cast<int64_t>(m0) * f;
      const TA* w1 = static_cast<const TA*>(g.b0) + static_cast<int64_t>(e) * f * d;
      const TA* w3 = static_cast<const TA*>(g.b1) + static_cast<int64_t>(e) * f * d;
      const int nvalid = min(BN, d - n0);
      for (int kk = 0; kk < 2 * f; kk += BK) {
        const bool second = kk >= f;
        const int k0 = second ? kk - f : kk;
        const TA* asrc = second ? db : da;
        const TA* bsrc = second ? w3 : w1;
        stage_kmajor<TA, BK, LD>(As, [&](int r) { return asrc + static_cast<int64_t>(r) * f; },
                                 rows, k0);
        stage_mnmajor<TA, BK, LD>(Bs, bsrc + static_cast<int64_t>(k0) * d + n0, d, BK, nvalid);
        __syncthreads();
        core.compute(As, Bs);
        __syncthreads();
      }
      TA* dxo = static_cast<TA*>(g.c0);
      core.for_each([&](int r, int c, float v) {
        if (r < rows && c < nvalid) store_act(dxo + static_cast<int64_t>(m0 + r) * d + n0 + c, v);
      });
    }
  }
}

template <int MODE>
hipError_t launch_f32(dim3 grid, const GemmArgs& g, hipStream_t s) {
  hipLaunchKernelGGL((grouped_gemm_kernel<float, MODE>), grid, dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

GemmArgs base_args(const moe_dims& dm, const int32_t* offsets) {
  GemmArgs g{};
  g.offsets = offsets;
  g.E = dm.E;
  g.d = dm.d;
  g.f = dm.f;
  return g;
}

unsigned row_tiles(const moe_dims& dm) {
  return static_cast<unsigned>((dm.T * dm.k + BM - 1) / BM + dm.E);
}

}  // namespace

// Each phase dispatches on the activation type: bf16 runs on gemm_bf16.hip's
// kernels, fp32 on the kernel above (fp32 matrix cores).

hipError_t launch_expert_up(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                            const int32_t* offsets, const void* w1, const void* w3, void* a,
                            void* b, void* h, hipStream_t s) {
  if (dm.T * dm.k == 0) return hipSuccess;
  if (dm.act == MOE_BF16)
    return launch_up_bf16(dm, x_perm, x_rows, offsets, w1, w3, a, b, h, s);
  GemmArgs g = base_args(dm, offsets);
  g.a0 = x_perm;
  g.x_rows = x_rows;
  g.b0 = w1;
  g.b1 = w3;
  g.c0 = a;
  g.c1 = b;
  g.c2 = h;
  return launch_f32<UP>(dim3(row_tiles(dm), dm.f / 64), g, s);
}

hipError_t launch_expert_down(const moe_dims& dm, const void* h, const int32_t* offsets,
                              const void* w2, void* y, hipStream_t s) {
  if (dm.T * dm.k == 0) return hipSuccess;
  if (dm.act == MOE_BF16) return launch_down_bf16(dm, h, offsets, w2, y, s);
  GemmArgs g = base_args(dm, offsets);
  g.a0 = h;
  g.b0 = w2;
  g.c0 = y;
  return launch_f32<DOWN>(dim3(row_tiles(dm), (dm.d + BN - 1) / BN), g, s);
}

hipError_t launch_expert_dgrad_down(const moe_dims& dm, const void* dy_perm,
                                    const int32_t* offsets, const void* w2, const void* a,
                                    const void* b, void* da, void* db, hipStream_t s) {
  if (dm.T * dm.k == 0) return hipSuccess;
  if (dm.act == MOE_BF16) return launch_dgrad_down_bf16(dm, dy_perm, offsets, w2, a, b, da, db, s);
  GemmArgs g = base_args(dm, offsets);
  g.a0 = dy_perm;
  g.b0 = w2;
  g.aux0 = a;
  g.aux1 = b;
  g.c0 = da;
  g.c1 = db;
  return launch_f32<DGRAD_DOWN>(dim3(row_tiles(dm), (dm.f + BN - 1) / BN), g, s);
}

hipError_t launch_expert_dgrad_up(const moe_dims& dm, const void* da, const void* db,
                                  const int32_t* offsets, const void* w1, const void* w3,
                                  void* dx_perm, hipStream_t s) {
  if (dm.T * dm.k == 0) return hipSuccess;
  if (dm.act == MOE_BF16) return launch_dgrad_up_bf16(dm, da, db, offsets, w1, w3, dx_perm, s);
  GemmArgs g = base_args(dm, offsets);
  g.a0 = da;
  g.a1 = db;
  g.b0 = w1;
  g.b1 = w3;
  g.c0 = dx_perm;
  return launch_f32<DGRAD_UP>(dim3(row_tiles(dm), (dm.d + BN - 1) / BN), g, s);
}

hipError_t launch_expert_wgrad(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                               const int32_t* offsets, const void* h, const void* dy_perm,
                               const void* da, const void* db, void* dw1, void* dw3, void* dw2,
                               bool wgrad_f32, float* partial, hipStream_t s) {
  if (dm.act == MOE_BF16)
    return launch_wgrad_bf16(dm, x_perm, x_rows, offsets, h, dy_perm, da, db, dw1, dw3, dw2,
                             wgrad_f32, partial, s);
  if (!wgrad_f32) return hipErrorNotSupported;   // fp32 layers keep fp32 weight gradients
  // weight gradients (also for experts with no rows: they get zeros)
  GemmArgs g = base_args(dm, offsets);
  g.a0 = dy_perm;   // z = 0: A = dy (m over d), B = h (n over f)
  g.b0 = h;
  g.a1 = da;        // z = 1: A = da (m over f), B = x (n over d)
  g.aux0 = db;      // z = 2: A = db (m over f), B = x (n over d)
  g.b1 = x_perm;
  g.x_rows = x_rows;
  g.c0 = dw2;
  g.c1 = dw1;
  g.c2 = dw3;
  const unsigned tiles = static_cast<unsigned>(((dm.d + BM - 1) / BM) * ((dm.f + BN - 1) / BN));
  return launch_f32<WGRAD>(dim3(tiles, dm.E, 3), g, s);
}

hipError_t launch_swiglu_fwd(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                             const int32_t* offsets, const void* w1, const void* w3,
                             const void* w2, void* a, void* b, void* h, void* y, hipStream_t s) {
  hipError_t e = launch_expert_up(dm, x_perm, x_rows, offsets, w1, w3, a, b, h, s);
  if (e != hipSuccess) return e;
  return launch_expert_down(dm, h, offsets, w2, y, s);
}

hipError_t launch_swiglu_bwd(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                             const int32_t* offsets,
                             const void* w1, const void* w3, const void* w2, const void* a,
                             const void* b, const void* h, const void* dy_perm, void* dx_perm,
                             void* dw1, void* dw3, void* dw2, bool wgrad_f32, void* ws_da,
                             void* ws_db, float* ws_partial, hipStream_t s) {
  hipError_t e = launch_expert_dgrad_down(dm, dy_perm, offsets, w2, a, b, ws_da, ws_db, s);
  if (e != hipSuccess) return e;
  e = launch_expert_dgrad_up(dm, ws_da, ws_db, offsets, w1, w3, dx_perm, s);
  if (e != hipSuccess) return e;
  return launch_expert_wgrad(dm, x_perm, x_rows, offsets, h, dy_perm, ws_da, ws_db, dw1, dw3,
                             dw2, wgrad_f32, ws_partial, s);
}

}  // namespace moe
