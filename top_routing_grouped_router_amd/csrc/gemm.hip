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
// MFMA, 4 waves per tile, in two shapes: 128x128 (2 x 2 waves of 64x64) and,
// for grids that would leave CUs idle, 64x64 (4 x 1 waves of 16x64).
// A workgroup's (expert, row tile) comes from the expert offsets on the device,
// so the host never reads the routing.  Each output element is produced by
// exactly one workgroup with a fixed k order: results are reproducible.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 32;        // k per step
constexpr int LD = BK + 4;    // LDS row stride (144 bytes: 16-byte aligned staging and reads)

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

// ------------------------------------------------------------------ tile shapes
// WM x WN wavefronts, each owning RB x CB blocks of 16 x 16.
template <int WM_, int WN_, int RB_, int CB_>
struct Tile {
  static constexpr int WM = WM_, WN = WN_, RB = RB_, CB = CB_;
  static constexpr int BM = WM * RB * 16, BN = WN * CB * 16;
  static_assert(WM * WN * 64 == kThreads, "4 wavefronts");
  static_assert(CB % 2 == 0 && CB * 16 >= 64, "UP pairs columns c and c + 32 of a wave");
};
typedef Tile<2, 2, 4, 4> BigTile;     // 128 x 128
typedef Tile<4, 1, 1, 4> SmallTile;   //  64 x  64

// ------------------------------------------------------------------ fp32 MFMA core
// v_mfma_f32_16x16x4_f32; accumulator lane (g, r) of a 16x16 block holds rows
// 4 g + q, column r.  Within a BK = 32 step, lane (g, r) of a 16-row block
// takes k = 8 g ... 8 g + 7 of its row (two 16-byte LDS reads) and feeds k =
// 8 g + s at MFMA step s; A and B use the same assignment, so each of the 8
// steps sums k = s, 8 + s, 16 + s, 24 + s and the 8 steps cover the step.
template <class TL>
struct Core {
  f32x4 acc[TL::RB][TL::CB];

  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < TL::RB; ++i)
#pragma unroll
      for (int j = 0; j < TL::CB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ void compute(const float* As, const float* Bs) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave / TL::WN, wn = wave % TL::WN;
    const int r = lane & 15, k0 = (lane >> 4) * 8;
    float a[TL::RB][8], b[TL::CB][8];
#pragma unroll
    for (int i = 0; i < TL::RB; ++i) {
      const float* p = As + (wm * TL::RB * 16 + i * 16 + r) * LD + k0;
      const float4 lo = *reinterpret_cast<const float4*>(p);
      const float4 hi = *reinterpret_cast<const float4*>(p + 4);
      a[i][0] = lo.x; a[i][1] = lo.y; a[i][2] = lo.z; a[i][3] = lo.w;
      a[i][4] = hi.x; a[i][5] = hi.y; a[i][6] = hi.z; a[i][7] = hi.w;
    }
#pragma unroll
    for (int j = 0; j < TL::CB; ++j) {
      const float* p = Bs + (wn * TL::CB * 16 + j * 16 + r) * LD + k0;
      const float4 lo = *reinterpret_cast<const float4*>(p);
      const float4 hi = *reinterpret_cast<const float4*>(p + 4);
      b[j][0] = lo.x; b[j][1] = lo.y; b[j][2] = lo.z; b[j][3] = lo.w;
      b[j][4] = hi.x; b[j][5] = hi.y; b[j][6] = hi.z; b[j][7] = hi.w;
    }
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int i = 0; i < TL::RB; ++i)
#pragma unroll
        for (int j = 0; j < TL::CB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][st], b[j][st], acc[i][j], 0, 0, 0);
  }
  // visit every accumulator as (tile row, tile col, value)
  template <typename F>
  __device__ void for_each(F&& fn) const {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave / TL::WN, wn = wave % TL::WN;
#pragma unroll
    for (int i = 0; i < TL::RB; ++i)
#pragma unroll
      for (int j = 0; j < TL::CB; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          fn(wm * TL::RB * 16 + i * 16 + (lane >> 4) * 4 + q,
             wn * TL::CB * 16 + j * 16 + (lane & 15), acc[i][j][q]);
  }
  // SwiGLU pairs: tile columns c and c + 32 inside one 64-column block of a
  // wave (the a and b columns of the same f column in UP)
  template <typename F>
  __device__ void for_each_pair(F&& fn) const {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave / TL::WN, wn = wave % TL::WN;
#pragma unroll
    for (int i = 0; i < TL::RB; ++i)
#pragma unroll
      for (int j0 = 0; j0 < TL::CB; j0 += 4)
#pragma unroll
        for (int j = j0; j < j0 + 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            fn(wm * TL::RB * 16 + i * 16 + (lane >> 4) * 4 + q,
               wn * TL::CB * 16 + j * 16 + (lane & 15), acc[i][j][q], acc[i][j + 2][q]);
  }
};

// ------------------------------------------------------------------ staging
// One operand stage (ROWS rows or columns x BK k) goes global -> registers ->
// LDS in two calls, so that a step's loads can be issued before the previous
// step's MFMAs and stored after them.  4 floats per 16-byte vector, kPer
// vectors per thread.
template <int ROWS>
struct Regs {
  static constexpr int kVec = 4;
  static constexpr int kPer = ROWS * BK / kVec / kThreads;
  static_assert(kPer >= 1 && ROWS * BK / kVec % kThreads == 0, "whole vectors per thread");
  uint4 v[kPer];
};

// K-major source: tile row r (< ROWS) starts at row_ptr(r); rows >= valid are
// zero.  A thread's vectors sit in fixed rows, so their addresses (less k0)
// are worked out once per tile (NULL for a zero row).
template <int ROWS>
struct KRows {
  const float* p[Regs<ROWS>::kPer];
};
template <int ROWS, typename RowPtr>
__device__ __forceinline__ KRows<ROWS> k_rows(RowPtr row_ptr, int valid) {
  constexpr int kPerRow = BK / 4;
  KRows<ROWS> kr;
#pragma unroll
  for (int i = 0; i < Regs<ROWS>::kPer; ++i) {
    const int v = threadIdx.x + i * kThreads;
    const int r = v / kPerRow, c = (v % kPerRow) * 4;
    kr.p[i] = (r < valid) ? row_ptr(r) + c : nullptr;
  }
  return kr;
}
template <int ROWS>
__device__ __forceinline__ void load_kmajor(Regs<ROWS>& rg, const KRows<ROWS>& kr, int k0) {
#pragma unroll
  for (int i = 0; i < Regs<ROWS>::kPer; ++i)
    rg.v[i] = kr.p[i] ? *reinterpret_cast<const uint4*>(kr.p[i] + k0) : make_uint4(0, 0, 0, 0);
}
template <int ROWS>
__device__ __forceinline__ void store_kmajor(const Regs<ROWS>& rg, float* lds) {
  constexpr int kPerRow = BK / 4;
#pragma unroll
  for (int i = 0; i < Regs<ROWS>::kPer; ++i) {
    const int v = threadIdx.x + i * kThreads;
    const int r = v / kPerRow, c = (v % kPerRow) * 4;
    *reinterpret_cast<uint4*>(lds + r * LD + c) = rg.v[i];
  }
}

// MN-major source: element (k, mn) of k row kr at row_ptr(kr)[mn] for the
// tile's k rows [0, BK) and mn columns [0, COLS); k >= kvalid or mn >= mnvalid
// read as zero.  Stored transposed, so that LDS holds [mn][k].
template <int COLS, typename RowPtr>
__device__ __forceinline__ void load_mnmajor(Regs<COLS>& rg, RowPtr row_ptr, int kvalid,
                                             int mnvalid) {
  constexpr int kPerRow = COLS / 4;
#pragma unroll
  for (int i = 0; i < Regs<COLS>::kPer; ++i) {
    const int v = threadIdx.x + i * kThreads;
    const int kr = v / kPerRow, c = (v % kPerRow) * 4;
    rg.v[i] = (kr < kvalid && c < mnvalid) ? *reinterpret_cast<const uint4*>(row_ptr(kr) + c)
                                           : make_uint4(0, 0, 0, 0);
  }
}
template <int COLS>
__device__ __forceinline__ void store_mnmajor(const Regs<COLS>& rg, float* lds) {
  constexpr int kPerRow = COLS / 4;
#pragma unroll
  for (int i = 0; i < Regs<COLS>::kPer; ++i) {
    const int v = threadIdx.x + i * kThreads;
    const int kr = v / kPerRow, c = (v % kPerRow) * 4;
    const float* e = reinterpret_cast<const float*>(&rg.v[i]);
#pragma unroll
    for (int q = 0; q < 4; ++q) lds[(c + q) * LD + kr] = e[q];
  }
}

// The K loop: step j's operands are loaded into registers while step j - 1's
// MFMAs run, then stored into LDS buffer j & 1; with two buffers one barrier
// per step suffices (a buffer is rewritten only after every wavefront has
// passed the barrier that follows its last use).  load(j, ra, rb) fills the
// registers, store(ra, rb, As, Bs) writes them.  (Loading two steps ahead
// measured no faster at C1 and doubles the staging registers.)
template <class TL, typename Load, typename Store>
__device__ __forceinline__ void run_steps(Core<TL>& core, float* lds, int n, Load&& load,
                                          Store&& store) {
  if (n <= 0) return;
  Regs<TL::BM> ra;
  Regs<TL::BN> rb;
  load(0, ra, rb);
  for (int j = 0; j < n; ++j) {
    // buffer j & 1 by offset arithmetic on the LDS array (the compiler then
    // keeps LDS addressing, not generic loads that would wait on the prefetch)
    float* const A = lds + (j & 1) * ((TL::BM + TL::BN) * LD);
    float* const B = A + TL::BM * LD;
    store(ra, rb, A, B);
    __syncthreads();
    if (j + 1 < n) load(j + 1, ra, rb);
    core.compute(A, B);
  }
}

__device__ __forceinline__ void store_act(float* p, float v) { *p = v; }

// ------------------------------------------------------------------ row-tile lookup
// Finds the expert and first row of this workgroup's row tile (tiles of BM
// rows) from the expert offsets: tile counts per expert are prefix-summed
// across wave 0's lanes (4 experts per lane).  Returns false when the
// workgroup has no tile.
template <int BM>
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
template <class TL, int MODE>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs g) {
  constexpr int BM = TL::BM, BN = TL::BN;
  __shared__ __attribute__((aligned(16))) float lds[2 * (BM + BN) * LD];

  const int d = g.d, f = g.f;
  Core<TL> core;
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
    const float* Asrc = static_cast<const float*>(z == 0 ? g.a0 : (z == 1 ? g.a1 : g.aux0));
    const float* Bsrc = static_cast<const float*>(z == 0 ? g.b0 : g.b1);
    const int p0 = g.offsets[e], p1 = g.offsets[e + 1];
    const bool gathered = z != 0 && g.x_rows;   // B = X rows gathered by the table
    run_steps<TL>(
        core, lds, (p1 - p0 + BK - 1) / BK,
        [&](int j, Regs<BM>& ra, Regs<BN>& rb) {
          const int p = p0 + j * BK;
          const int kvalid = min(BK, p1 - p);
          load_mnmajor<BM>(
              ra, [&](int kr) { return Asrc + static_cast<int64_t>(p + kr) * Mdim + m0; },
              kvalid, Mdim - m0);
          if (gathered)
            load_mnmajor<BN>(
                rb, [&](int kr) { return Bsrc + static_cast<int64_t>(g.x_rows[p + kr]) * Ndim + n0; },
                kvalid, Ndim - n0);
          else
            load_mnmajor<BN>(
                rb, [&](int kr) { return Bsrc + static_cast<int64_t>(p + kr) * Ndim + n0; },
                kvalid, Ndim - n0);
        },
        [&](const Regs<BM>& ra, const Regs<BN>& rb, float* As, float* Bs) {
          store_mnmajor<BM>(ra, As);
          store_mnmajor<BN>(rb, Bs);
        });
    float* out = static_cast<float*>(z == 0 ? g.c0 : (z == 1 ? g.c1 : g.c2)) +
                 static_cast<int64_t>(e) * d * f;
    core.for_each([&](int r, int c, float v) {
      const int m = m0 + r, n = n0 + c;
      if (m < Mdim && n < Ndim) store_act(out + static_cast<int64_t>(m) * Ndim + n, v);
    });
  } else {
    int e, m0, mend;
    if (!find_row_tile<BM>(g.offsets, g.E, blockIdx.x, &e, &m0, &mend)) return;
    const int rows = min(BM, mend - m0);
    const int n0 = blockIdx.y * ((MODE == UP) ? BN / 2 : BN);
    // both operands k-major, or A k-major and B mn-major
    auto store_kk = [](const Regs<BM>& ra, const Regs<BN>& rb, float* As, float* Bs) {
      store_kmajor<BM>(ra, As);
      store_kmajor<BN>(rb, Bs);
    };
    auto store_km = [](const Regs<BM>& ra, const Regs<BN>& rb, float* As, float* Bs) {
      store_kmajor<BM>(ra, As);
      store_mnmajor<BN>(rb, Bs);
    };

    if constexpr (MODE == UP) {
      const float* x = static_cast<const float*>(g.a0);
      const float* w1 = static_cast<const float*>(g.b0) + static_cast<int64_t>(e) * f * d;
      const float* w3 = static_cast<const float*>(g.b1) + static_cast<int64_t>(e) * f * d;
      // input row r of the tile: expert row m0 + r, or the X row the table
      // gives (the thread's table entries are loaded together, clamped to a
      // valid row, before any is used)
      constexpr int kPer = Regs<BM>::kPer, kPerRowK = BK / 4;
      int64_t xq[kPer];
      if (g.x_rows) {
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          xq[i] = g.x_rows[m0 + min((static_cast<int>(threadIdx.x) + i * kThreads) / kPerRowK,
                                     rows - 1)];
      } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i) xq[i] = m0 + (threadIdx.x + i * kThreads) / kPerRowK;
      }
      KRows<BM> xa;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int v = threadIdx.x + i * kThreads;
        xa.p[i] = (v / kPerRowK < rows) ? x + xq[i] * d + (v % kPerRowK) * 4 : nullptr;
      }
      // B-tile row r: f row n0 + 32 (r / 64) + r % 32 of W1 (r % 64 < 32) or W3
      auto w_row = [&](int r) {
        const int q = r >> 5;
        const float* w = (q & 1) ? w3 : w1;
        return w + static_cast<int64_t>(n0 + 32 * (q >> 1) + (r & 31)) * d;
      };
      const KRows<BN> wb = k_rows<BN>(w_row, BN);
      run_steps<TL>(
          core, lds, d / BK,
          [&](int j, Regs<BM>& ra, Regs<BN>& rb) {
            load_kmajor<BM>(ra, xa, j * BK);
            load_kmajor<BN>(rb, wb, j * BK);
          },
          store_kk);
      float* ao = static_cast<float*>(g.c0);
      float* bo = static_cast<float*>(g.c1);
      float* ho = static_cast<float*>(g.c2);
      core.for_each_pair([&](int r, int c, float av, float bv) {
        if (r >= rows) return;
        // B-tile row c (< 32 within its 64-row block) is f column n0 + 32 (c / 64) + c % 32
        const int n = n0 + 32 * (c >> 6) + (c & 31);
        const int64_t o = static_cast<int64_t>(m0 + r) * f + n;
        store_act(ao + o, av);
        store_act(bo + o, bv);
        store_act(ho + o, silu_f(av) * bv);
      });
    } else if constexpr (MODE == DOWN) {
      const float* h = static_cast<const float*>(g.a0) + static_cast<int64_t>(m0) * f;
      const float* w2 = static_cast<const float*>(g.b0) + static_cast<int64_t>(e) * d * f;
      const int nvalid = min(BN, d - n0);
      const KRows<BM> ha =
          k_rows<BM>([&](int r) { return h + static_cast<int64_t>(r) * f; }, rows);
      const KRows<BN> wb =
          k_rows<BN>([&](int r) { return w2 + static_cast<int64_t>(n0 + r) * f; }, nvalid);
      run_steps<TL>(
          core, lds, f / BK,
          [&](int j, Regs<BM>& ra, Regs<BN>& rb) {
            load_kmajor<BM>(ra, ha, j * BK);
            load_kmajor<BN>(rb, wb, j * BK);
          },
          store_kk);
      float* yo = static_cast<float*>(g.c0);
      core.for_each([&](int r, int c, float v) {
        if (r < rows && c < nvalid) store_act(yo + static_cast<int64_t>(m0 + r) * d + n0 + c, v);
      });
    } else if constexpr (MODE == DGRAD_DOWN) {
      // dh[p][n] = sum_k dy[p][k] W2[e][k][n], n < f
      const float* dy = static_cast<const float*>(g.a0) + static_cast<int64_t>(m0) * d;
      const float* w2 = static_cast<const float*>(g.b0) + static_cast<int64_t>(e) * d * f;
      const int nvalid = min(BN, f - n0);
      const KRows<BM> dya =
          k_rows<BM>([&](int r) { return dy + static_cast<int64_t>(r) * d; }, rows);
      run_steps<TL>(
          core, lds, d / BK,
          [&](int j, Regs<BM>& ra, Regs<BN>& rb) {
            const int k0 = j * BK;
            load_kmajor<BM>(ra, dya, k0);
            load_mnmajor<BN>(
                rb, [&](int kr) { return w2 + static_cast<int64_t>(k0 + kr) * f + n0; }, BK,
                nvalid);
          },
          store_km);
      const float* sa = static_cast<const float*>(g.aux0);
      const float* sb = static_cast<const float*>(g.aux1);
      float* dao = static_cast<float*>(g.c0);
      float* dbo = static_cast<float*>(g.c1);
      core.for_each([&](int r, int c, float dh) {
        if (r >= rows || c >= nvalid) return;
        const int64_t o = static_cast<int64_t>(m0 + r) * f + n0 + c;
        const float av = sa[o], bv = sb[o];
        const float s = sigmoid_f(av);
        const float act = av * s;
        const float dact = s * (1.0f + av * (1.0f - s));
        store_act(dao + o, dh * bv * dact);
        store_act(dbo + o, dh * act);
      });
    } else {  // DGRAD_UP: dx[p][n] = sum_k da[p][k] W1[e][k][n] + db[p][k] W3[e][k][n]
      const float* da = static_cast<const float*>(g.a0) + static_cast<int64_t>(m0) * f;
      const float* db = static_cast<const float*>(g.a1) + static_cast<int64_t>(m0) * f;
      const float* w1 = static_cast<const float*>(g.b0) + static_cast<int64_t>(e) * f * d;
      const float* w3 = static_cast<const float*>(g.b1) + static_cast<int64_t>(e) * f * d;
      const int nvalid = min(BN, d - n0);
      // one K loop over 2f: da against W1, then db against W3
      const KRows<BM> daa =
          k_rows<BM>([&](int r) { return da + static_cast<int64_t>(r) * f; }, rows);
      const KRows<BM> dba =
          k_rows<BM>([&](int r) { return db + static_cast<int64_t>(r) * f; }, rows);
      run_steps<TL>(
          core, lds, 2 * f / BK,
          [&](int j, Regs<BM>& ra, Regs<BN>& rb) {
            const int kk = j * BK;
            const bool second = kk >= f;
            const int k0 = second ? kk - f : kk;
            const float* bsrc = second ? w3 : w1;
            load_kmajor<BM>(ra, second ? dba : daa, k0);
            load_mnmajor<BN>(
                rb, [&](int kr) { return bsrc + static_cast<int64_t>(k0 + kr) * d + n0; }, BK,
                nvalid);
          },
          store_km);
      float* dxo = static_cast<float*>(g.c0);
      core.for_each([&](int r, int c, float v) {
        if (r < rows && c < nvalid) store_act(dxo + static_cast<int64_t>(m0 + r) * d + n0 + c, v);
      });
    }
  }
}

GemmArgs base_args(const moe_dims& dm, const int32_t* offsets) {
  GemmArgs g{};
  g.offsets = offsets;
  g.E = dm.E;
  g.d = dm.d;
  g.f = dm.f;
  return g;
}

template <class TL, int MODE>
dim3 grid_of(const moe_dims& dm) {
  const unsigned row_tiles = static_cast<unsigned>((dm.T * dm.k + TL::BM - 1) / TL::BM + dm.E);
  switch (MODE) {
    case UP: return dim3(row_tiles, dm.f / (TL::BN / 2));
    case DOWN: case DGRAD_UP: return dim3(row_tiles, (dm.d + TL::BN - 1) / TL::BN);
    case DGRAD_DOWN: return dim3(row_tiles, (dm.f + TL::BN - 1) / TL::BN);
    default:
      return dim3(static_cast<unsigned>(((dm.d + TL::BM - 1) / TL::BM) *
                                        ((dm.f + TL::BN - 1) / TL::BN)),
                  dm.E, 3);
  }
}

// The 128 x 128 tile when its grid gives at least two workgroups per CU,
// otherwise the 64 x 64 tile (four times the workgroups).
template <int MODE>
hipError_t launch_f32(const moe_dims& dm, const GemmArgs& g, hipStream_t s) {
  constexpr int kCUs = 256;   // MI355X
  const dim3 big = grid_of<BigTile, MODE>(dm);
  if (static_cast<int64_t>(big.x) * big.y * big.z >= 2 * kCUs) {
    hipLaunchKernelGGL((grouped_gemm_kernel<BigTile, MODE>), big, dim3(kThreads), 0, s, g);
  } else {
    const dim3 small = grid_of<SmallTile, MODE>(dm);
    hipLaunchKernelGGL((grouped_gemm_kernel<SmallTile, MODE>), small, dim3(kThreads), 0, s, g);
  }
  return hipGetLastError();
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
  return launch_f32<UP>(dm, g, s);
}

hipError_t launch_expert_down(const moe_dims& dm, const void* h, const int32_t* offsets,
                              const void* w2, void* y, hipStream_t s) {
  if (dm.T * dm.k == 0) return hipSuccess;
  if (dm.act == MOE_BF16) return launch_down_bf16(dm, h, offsets, w2, y, s);
  GemmArgs g = base_args(dm, offsets);
  g.a0 = h;
  g.b0 = w2;
  g.c0 = y;
  return launch_f32<DOWN>(dm, g, s);
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
  return launch_f32<DGRAD_DOWN>(dm, g, s);
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
  return launch_f32<DGRAD_UP>(dm, g, s);
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
  return launch_f32<WGRAD>(dm, g, s);
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
