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

// ------------------------------------------------------------------ staging
// One operand stage (128 rows or columns x BK k) goes global -> registers ->
// LDS in two calls, so that a step's loads can be issued before the previous
// step's MFMAs and stored after them.  kVec elements per 16-byte vector,
// kPer vectors per thread.
template <typename T, int BK>
struct Regs {
  static constexpr int kVec = 16 / static_cast<int>(sizeof(T));
  static constexpr int kPer = 128 * BK / kVec / kThreads;
  uint4 v[kPer];
};

// K-major source: tile row r (< 128) starts at row_ptr(r); rows >= valid are
// zero.  A thread's vectors sit in fixed rows, so their addresses (less k0)
// are worked out once per tile (NULL for a zero row).
template <typename T, int BK>
struct KRows {
  const T* p[Regs<T, BK>::kPer];
};
template <typename T, int BK, typename RowPtr>
__device__ __forceinline__ KRows<T, BK> k_rows(RowPtr row_ptr, int valid) {
  constexpr int kPerRow = BK / Regs<T, BK>::kVec;
  KRows<T, BK> kr;
#pragma unroll
  for (int i = 0; i < Regs<T, BK>::kPer; ++i) {
    const int v = threadIdx.x + i * kThreads;
    const int r = v / kPerRow, c = (v % kPerRow) * Regs<T, BK>::kVec;
    kr.p[i] = (r < valid) ? row_ptr(r) + c : nullptr;
  }
  return kr;
}
template <typename T, int BK>
__device__ __forceinline__ void load_kmajor(Regs<T, BK>& rg, const KRows<T, BK>& kr, int k0) {
#pragma unroll
  for (int i = 0; i < Regs<T, BK>::kPer; ++i)
    rg.v[i] = kr.p[i] ? *reinterpret_cast<const uint4*>(kr.p[i] + k0) : make_uint4(0, 0, 0, 0);
}
template <typename T, int BK, int LD>
__device__ __forceinline__ void store_kmajor(const Regs<T, BK>& rg, T* lds) {
  constexpr int kPerRow = BK / Regs<T, BK>::kVec;
#pragma unroll
  for (int i = 0; i < Regs<T, BK>::kPer; ++i) {
    const int v = threadIdx.x + i * kThreads;
    const int r = v / kPerRow, c = (v % kPerRow) * Regs<T, BK>::kVec;
    *reinterpret_cast<uint4*>(lds + r * LD + c) = rg.v[i];
  }
}

// MN-major source: element (k, mn) of k row kr at row_ptr(kr)[mn] for the
// tile's k rows [0, BK) and mn columns [0, 128); k >= kvalid or mn >= mnvalid
// read as zero.  Stored transposed, so that LDS holds [mn][k].
template <typename T, int BK, typename RowPtr>
__device__ __forceinline__ void load_mnmajor(Regs<T, BK>& rg, RowPtr row_ptr, int kvalid,
                                             int mnvalid) {
  constexpr int kPerRow = 128 / Regs<T, BK>::kVec;
#pragma unroll
  for (int i = 0; i < Regs<T, BK>::kPer; ++i) {
    const int v = threadIdx.x + i * kThreads;
    const int kr = v / kPerRow, c = (v % kPerRow) * Regs<T, BK>::kVec;
    rg.v[i] = (kr < kvalid && c < mnvalid) ? *reinterpret_cast<const uint4*>(row_ptr(kr) + c)
                                           : make_uint4(0, 0, 0, 0);
  }
}
template <typename T, int BK, int LD>
__device__ __forceinline__ void store_mnmajor(const Regs<T, BK>& rg, T* lds) {
  constexpr int kPerRow = 128 / Regs<T, BK>::kVec;
#pragma unroll
  for (int i = 0; i < Regs<T, BK>::kPer; ++i) {
    const int v = threadIdx.x + i * kThreads;
    const int kr = v / kPerRow, c = (v % kPerRow) * Regs<T, BK>::kVec;
    const T* e = reinterpret_cast<const T*>(&rg.v[i]);
#pragma unroll
    for (int q = 0; q < Regs<T, BK>::kVec; ++q) lds[(c + q) * LD + kr] = e[q];
  }
}

// The K loop: step j's operands are loaded into registers while step j - 1's
// MFMAs run, then stored into LDS buffer j & 1; with two buffers one barrier
// per step suffices (a buffer is rewritten only after every wavefront has
// passed the barrier that follows its last use).  load(j) fills the
// registers, store(As, Bs) writes them.
template <typename C, typename T, int LD, typename Load, typename Store>
__device__ __forceinline__ void run_steps(C& core, T* lds, int n, Load&& load, Store&& store) {
  if (n <= 0) return;
  load(0);
  for (int j = 0; j < n; ++j) {
    // buffer j & 1 by offset arithmetic on the LDS array (the compiler then
    // keeps LDS addressing, not generic loads that would wait on the prefetch)
    T* const A = lds + (j & 1) * ((BM + BN) * LD);
    T* const B = A + BM * LD;
    store(A, B);
    __syncthreads();
    if (j + 1 < n) load(j + 1);
    core.compute(A, B);
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
  __shared__ __attribute__((aligned(16))) TA lds[2 * (BM + BN) * LD];

  const int d = g.d, f = g.f;
  C core;
  core.zero();
  Regs<TA, BK> ra, rb;

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
    const bool gathered = z != 0 && g.x_rows;   // B = X rows gathered by the table
    run_steps<C, TA, LD>(
        core, lds, (p1 - p0 + BK - 1) / BK,
        [&](int j) {
          const int p = p0 + j * BK;
          const int kvalid = min(BK, p1 - p);
          load_mnmajor<TA, BK>(
              ra, [&](int kr) { return Asrc + static_cast<int64_t>(p + kr) * Mdim + m0; },
              kvalid, Mdim - m0);
          if (gathered)
            load_mnmajor<TA, BK>(
                rb, [&](int kr) { return Bsrc + static_cast<int64_t>(g.x_rows[p + kr]) * Ndim + n0; },
                kvalid, Ndim - n0);
          else
            load_mnmajor<TA, BK>(
                rb, [&](int kr) { return Bsrc + static_cast<int64_t>(p + kr) * Ndim + n0; },
                kvalid, Ndim - n0);
        },
        [&](TA* As, TA* Bs) {
          store_mnmajor<TA, BK, LD>(ra, As);
          store_mnmajor<TA, BK, LD>(rb, Bs);
        });
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
    auto store_kk = [&](TA* As, TA* Bs) {   // both operands k-major
      store_kmajor<TA, BK, LD>(ra, As);
      store_kmajor<TA, BK, LD>(rb, Bs);
    };
    auto store_km = [&](TA* As, TA* Bs) {   // A k-major, B mn-major
      store_kmajor<TA, BK, LD>(ra, As);
      store_mnmajor<TA, BK, LD>(rb, Bs);
    };

    if constexpr (MODE == UP) {
      const TA* x = static_cast<const TA*>(g.a0);
      const TA* w1 = static_cast<const TA*>(g.b0) + static_cast<int64_t>(e) * f * d;
      const TA* w3 = static_cast<const TA*>(g.b1) + static_cast<int64_t>(e) * f * d;
      // input row r of the tile: expert row m0 + r, or the X row the table
      // gives (the thread's table entries are loaded together, clamped to a
      // valid row, before any is used)
      int64_t xq[Regs<TA, BK>::kPer];
      constexpr int kPerRowK = BK / Regs<TA, BK>::kVec;
      if (g.x_rows) {
#pragma unroll
        for (int i = 0; i < Regs<TA, BK>::kPer; ++i)
          xq[i] = g.x_rows[m0 + min((static_cast<int>(threadIdx.x) + i * kThreads) / kPerRowK,
                                     rows - 1)];
      } else {
#pragma unroll
        for (int i = 0; i < Regs<TA, BK>::kPer; ++i)
          xq[i] = m0 + (threadIdx.x + i * kThreads) / kPerRowK;
      }
      KRows<TA, BK> xa;
#pragma unroll
      for (int i = 0; i < Regs<TA, BK>::kPer; ++i) {
        const int v = threadIdx.x + i * kThreads;
        xa.p[i] = (v / kPerRowK < rows) ? x + xq[i] * d + (v % kPerRowK) * Regs<TA, BK>::kVec
                                        : nullptr;
      }
      // B-tile row r: f row n0 + 32 (r / 64) + r % 32 of W1 (r % 64 < 32) or W3
      auto w_row = [&](int r) {
        const int q = r >> 5;
        const TA* w = (q & 1) ? w3 : w1;
        return w + static_cast<int64_t>(n0 + 32 * (q >> 1) + (r & 31)) * d;
      };
      const KRows<TA, BK> wb = k_rows<TA, BK>(w_row, BN);
      run_steps<C, TA, LD>(
          core, lds, d / BK,
          [&](int j) {
            load_kmajor<TA, BK>(ra, xa, j * BK);
            load_kmajor<TA, BK>(rb, wb, j * BK);
          },
          store_kk);
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
      const KRows<TA, BK> ha =
          k_rows<TA, BK>([&](int r) { return h + static_cast<int64_t>(r) * f; }, rows);
      const KRows<TA, BK> wb =
          k_rows<TA, BK>([&](int r) { return w2 + static_cast<int64_t>(n0 + r) * f; }, nvalid);
      run_steps<C, TA, LD>(
          core, lds, f / BK,
          [&](int j) {
            load_kmajor<TA, BK>(ra, ha, j * BK);
            load_kmajor<TA, BK>(rb, wb, j * BK);
          },
          store_kk);
      TA* yo = static_cast<TA*>(g.c0);
      core.for_each([&](int r, int c, float v) {
        if (r < rows && c < nvalid) store_act(yo + static_cast<int64_t>(m0 + r) * d + n0 + c, v);
      });
    } else if constexpr (MODE == DGRAD_DOWN) {
      // dh[p][n] = sum_k dy[p][k] W2[e][k][n], n < f
      const TA* dy = static_cast<const TA*>(g.a0) + static_cast<int64_t>(m0) * d;
      const TA* w2 = static_cast<const TA*>(g.b0) + static_cast<int64_t>(e) * d * f;
      const int nvalid = min(BN, f - n0);
      const KRows<TA, BK> dya =
          k_rows<TA, BK>([&](int r) { return dy + static_cast<int64_t>(r) * d; }, rows);
      run_steps<C, TA, LD>(
          core, lds, d / BK,
          [&](int j) {
            const int k0 = j * BK;
            load_kmajor<TA, BK>(ra, dya, k0);
            load_mnmajor<TA, BK>(
                rb, [&](int kr) { return w2 + static_cast<int64_t>(k0 + kr) * f + n0; }, BK,
                nvalid);
          },
          store_km);
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
      // one K loop over 2f: da against W1, then db against W3
      const KRows<TA, BK> daa =
          k_rows<TA, BK>([&](int r) { return da + static_cast<int64_t>(r) * f; }, rows);
      const KRows<TA, BK> dba =
          k_rows<TA, BK>([&](int r) { return db + static_cast<int64_t>(r) * f; }, rows);
      run_steps<C, TA, LD>(
          core, lds, 2 * f / BK,
          [&](int j) {
            const int kk = j * BK;
            const bool second = kk >= f;
            const int k0 = second ? kk - f : kk;
            const TA* bsrc = second ? w3 : w1;
            load_kmajor<TA, BK>(ra, second ? dba : daa, k0);
            load_mnmajor<TA, BK>(
                rb, [&](int kr) { return bsrc + static_cast<int64_t>(k0 + kr) * d + n0; }, BK,
                nvalid);
          },
          store_km);
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
