// Grouped GEMMs of the SwiGLU experts in bf16 on CDNA4 matrix cores.
//
// Method sources: "Revisiting MoE and Dense Speed-Accuracy Comparisons for LLM
// Training" (Sec. 2.1: SwiGLU activation in a LLaMA2-style block); "Expert
// Coupling in MoE Pretraining" (Fig. 5 step 4: the expert computation, run in
// the forward and backward passes); "MoE Pretraining: Parallelism Layout
// Changes the Model" (Methodology: SwiGLU experts).
//
// Every product is C[m][n] = sum_k A(m,k) B(n,k) over one expert's rows, in
// one of five modes (see grouped GEMM modes in gemm.hip):
//   UP          [a | b] = x_perm [W1 | W3]^T; epilogue h = silu(a) b
//   DOWN        y_perm = h W2^T
//   DGRAD_DOWN  dh = dy_perm W2; epilogue da = dh b silu'(a), db = dh silu(a)
//   DGRAD_UP    dx_perm = da W1 + db W3   (one K loop over 2f)
//   WGRAD       dW2 = dy^T h, dW1 = da^T x, dW3 = db^T x   (K = the expert's rows)
//
// Kernel structure (K step 64, v_mfma_f32_32x32x16_bf16), in two tile
// configurations:
//   small: 128 x 128 tile, 4 wavefronts of 64 x 64 (shapes with few or short
//          tiles);
//   big:   256 x 256 tile, 8 wavefronts of 128 x 64, one workgroup per CU
//          (large expert GEMMs: twice the matrix-core work per LDS byte).
//  * LDS holds both operand tiles k-contiguous, 16-byte chunks XOR-swizzled by
//    row (see swz), double-buffered: global loads of step k+1 are in flight
//    while step k runs on the matrix cores.
//  * Operands stored m- or n-contiguous in HBM (W in dgrad, both operands of
//    wgrad) are loaded as 4 x 8 blocks (four 16-byte rows per thread) and
//    transposed in registers before the LDS store, so the matrix-core loop is
//    the same in every mode.
//  * The MFMA takes the B fragment as its first source: each lane then owns
//    runs of 4 consecutive output columns of one row, which the epilogue
//    writes to LDS as 8-byte pieces and stores to HBM in coalesced 16-byte
//    chunks (with the mode's elementwise work applied on the way).
//  * Row tiles come from the expert offsets on the device; the flat tile
//    index is remapped so that each XCD (workgroups are dealt round-robin to
//    the 8 XCDs) works through a contiguous run of tiles, n fastest, which
//    keeps a row tile's A panel and the expert's B panel in that XCD's L2.
// Each output element is produced by one workgroup in a fixed k order, so
// results are bitwise reproducible.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;   // small kernels (reduce)
constexpr int BK = 64;
constexpr int kXcd = 8;

enum Mode { UP = 0, DOWN = 1, DGRAD_DOWN = 2, DGRAD_UP = 3, WGRAD = 4 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tile configurations.  Both use v_mfma_f32_32x32x16_bf16 fragments (on gfx950
// this shape sustains about 2.5x the rate of 16x16x32 in a dependency-free
// stream); wavefronts form a WAVES_M x WAVES_N grid, each owning FM x FN
// fragments of 32 x 32.
template <bool BIG> struct Cfg;
template <> struct Cfg<false> {   // 128 x 128, 4 wavefronts of 64 x 64
  static constexpr int THREADS = 256, BM = 128, BN = 128, WAVES_N = 2, FM = 2, FN = 2;
};
template <> struct Cfg<true> {    // 256 x 256, 8 wavefronts of 128 x 64
  static constexpr int BM = 256, BN = 256, WAVES_N = 4, FM = 4, FN = 2;
};

struct Args {
  const bf16_t* a0;
  const bf16_t* a1;
  const bf16_t* b0;
  const bf16_t* b1;
  const bf16_t* aux0;
  const bf16_t* aux1;
  bf16_t* c0;
  bf16_t* c1;
  bf16_t* c2;
  const int32_t* offsets;
  // NULL, or the gather table of the expert input (UP's A, WGRAD's x operand):
  // row p is then row x_rows[p] of X [T, d] (x_bytes = T d 2 < 2^31)
  const int32_t* x_rows;
  int32_t x_bytes;
  int32_t E, d, f;
  int32_t n_tiles_n;     // row modes: tiles along n
  int32_t grid_pad;      // flat grid size (multiple of 8)
  // Gate folded into the expert rows (NULL otherwise): UP stores g h;
  // DGRAD_DOWN reads dy through x_rows, scales dh by g and writes <u, h> per
  // row and column tile to dgate_part [rows][n_tiles_n].  (The folded weight
  // gradients read dy through x_rows: the FOLD_A instances.)
  const float* gate_rows;
  float* dgate_part;
  // weight gradients only: c0, c1, c2 hold fp32 (not bf16) elements
  int32_t out_f32;
};

// LDS address (elements) of 16-byte chunk `chunk` of k-contiguous row r (128
// bytes per row, so rows 2q and 2q + 1 fill the 64 banks).  The chunk is XORed
// with S(r) = ((r >> 1) ^ ((r >> 4) << 2)) & 7, chosen for the access
// patterns of gfx950's 64-bank LDS:
//  * fragment reads (16 lanes per clock, 16 consecutive rows, one logical
//    chunk): S is a bijection on each parity class of an aligned 16-row group,
//    so the 16 lanes hit 16 distinct 16-byte bank groups;
//  * k-contiguous stores (16 lanes = two whole rows): distinct by construction;
//  * transposed 8-byte stores (32 lanes per clock = rows 8 j + 2 c + parity of j
//    for 4 consecutive j, 4 chunks x 2 halves each, see mstore_raw): rows 16
//    apart get S values 4 apart, so their chunk sets are disjoint.
__device__ __forceinline__ int swz(int r, int chunk) {
  return r * BK + ((chunk ^ (((r >> 1) ^ ((r >> 4) << 2)) & 7)) << 3);
}

// ------------------------------------------------------------------ staging
// Loads never branch: an out-of-range row or column reads zeros through the
// buffer resource (below), so all of a step's global loads are in flight
// together (a guarded load would end in a wait for the loads issued before it).

// k-contiguous operand: ROWS rows x 64 k = ROWS x 8 chunks, ROWS x 8 / NT per thread.
template <int ROWS, int NT>
struct KPart {
  uint4 v[ROWS * 8 / NT];
};

// m/n-contiguous operand: element (k, j) at base[k * ld + j]; the 64 k x COLS j
// tile is cut into 16 x (COLS / 8) blocks of 4 k x 8 j, COLS x 2 / NT per
// thread.  Within a wavefront, lane bits 0-2 pick the k quad and bits 3-5 the
// j block, so a load instruction reads 128 contiguous bytes of each of 8 k
// rows, and each group of 16 lanes stores to 16 distinct bank slots after the
// transpose.
template <int COLS, int NT>
struct MPart {
  uint4 v[COLS * 2 / NT][4];
};

template <int NT>
__device__ __forceinline__ void mblock(int i, int* jb, int* kq) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  *kq = (wave & 1) * 8 + (lane & 7);
  *jb = i * (NT / 16) + (wave >> 1) * 8 + (lane >> 3);
}

// Buffer-resource loads (persistent kernel).  A resource covers
// [base, base + nbytes); a lane whose byte offset lies at or past nbytes reads
// zeros, so rows past an expert's end and columns past the matrix edge need no
// clamp or mask.  Bases and sizes are wavefront-uniform (scalar registers);
// the per-lane offsets are fixed per tile and the K step only moves the base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const bf16_t* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base), 0, nbytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), 0, 0));
}
constexpr uint32_t kOutOfRange = 0x80000000u;   // above every resource size (< 2^31)

template <int ROWS, int NT>
__device__ __forceinline__ void kstore_raw(const KPart<ROWS, NT>& p, bf16_t* lds) {
#pragma unroll
  for (int i = 0; i < ROWS * 8 / NT; ++i) {
    const int v = threadIdx.x + NT * i;
    *reinterpret_cast<uint4*>(lds + swz(v >> 3, v & 7)) = p.v[i];
  }
}

template <int COLS, int NT>
__device__ __forceinline__ void mstore_raw(const MPart<COLS, NT>& p, bf16_t* lds) {
#pragma unroll
  for (int i = 0; i < COLS * 2 / NT; ++i) {
    int jb, kq;
    mblock<NT>(i, &jb, &kq);
    const uint32_t in[4][4] = {{p.v[i][0].x, p.v[i][0].y, p.v[i][0].z, p.v[i][0].w},
                               {p.v[i][1].x, p.v[i][1].y, p.v[i][1].z, p.v[i][1].w},
                               {p.v[i][2].x, p.v[i][2].y, p.v[i][2].z, p.v[i][2].w},
                               {p.v[i][3].x, p.v[i][3].y, p.v[i][3].z, p.v[i][3].w}};
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
      const uint32_t A0 = in[0][c2], A1 = in[1][c2], A2 = in[2][c2], A3 = in[3][c2];
      const uint2 even = make_uint2((A0 & 0xFFFFu) | (A1 << 16), (A2 & 0xFFFFu) | (A3 << 16));
      const uint2 odd =
          make_uint2((A0 >> 16) | (A1 & 0xFFFF0000u), (A2 >> 16) | (A3 & 0xFFFF0000u));
      // lanes of odd j blocks write the odd row first, so each store
      // instruction covers both bank halves
      const int p = jb & 1;
      const int row = jb * 8 + 2 * c2;
      *reinterpret_cast<uint2*>(lds + swz(row + p, kq >> 1) + 4 * (kq & 1)) = p ? odd : even;
      *reinterpret_cast<uint2*>(lds + swz(row + 1 - p, kq >> 1) + 4 * (kq & 1)) = p ? even : odd;
    }
  }
}

// ------------------------------------------------------------------ matrix-core step
template <bool BIG>
using AccT = f32x16[Cfg<BIG>::FM][Cfg<BIG>::FN];

// Fragment (i, j) of wavefront (wm, wn) covers tile rows wm 32 FM + 32 i +
// [0, 32) and columns j (BN / FN) + 32 wn + [0, 32), so the FN fragments of a
// lane sit BN / FN columns apart (in UP: a and b of the same f column).
// One K step with the fragments of sub-step ss + 1 read from LDS while the
// MFMAs of sub-step ss run, and `mid` (the LDS store of the next step's
// operands) placed before sub-step 2.  Scheduling groups then interleave, in
// one basic block: the step's global loads (issued by the caller just before)
// with the MFMAs of sub-steps 0-1, and the LDS stores with those of 2-3.
constexpr int kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100, kSgDsWrite = 0x200;

template <bool BIG, int NVMEM, int NDSW, typename Mid>
__device__ __forceinline__ void mma_step_pipe(AccT<BIG>& acc, const bf16_t* As, const bf16_t* Bs,
                                              Mid&& mid) {
  typedef Cfg<BIG> C;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r = lane & 31, g = lane >> 5;
  bf16x8 af[2][C::FM], bfr[2][C::FN];
  auto rd = [&](int b, int kk) {
    const int chunk = kk + g;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
      af[b][i] = *reinterpret_cast<const bf16x8*>(As + swz(wm * 32 * C::FM + i * 32 + r, chunk));
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      bfr[b][j] =
          *reinterpret_cast<const bf16x8*>(Bs + swz(j * (C::BN / C::FN) + wn * 32 + r, chunk));
  };
  rd(0, 0);
#pragma unroll
  for (int ss = 0; ss < BK / 16; ++ss) {
    if (ss + 1 < BK / 16) rd((ss + 1) & 1, 2 * (ss + 1));
    if (ss == 2) mid();
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ss & 1][j], af[ss & 1][i],
                                                            acc[i][j], 0, 0, 0);
  }
  constexpr int MF = C::FM * C::FN, DR = C::FM + C::FN;
  constexpr int VM = (NVMEM + 2 * MF - 1) / (2 * MF), DW = (NDSW + 2 * MF - 1) / (2 * MF);
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, DR, 0);
#pragma unroll
  for (int ss = 0; ss < 2; ++ss) {
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, DR, 0);
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgVmemRead, VM, 0);
    }
  }
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, DR, 0);
#pragma unroll
  for (int ss = 2; ss < 4; ++ss) {
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDsWrite, DW, 0);
    }
  }
}

template <bool BIG>
__device__ __forceinline__ void zero_acc(AccT<BIG>& acc) {
#pragma unroll
  for (int i = 0; i < Cfg<BIG>::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg<BIG>::FN; ++j) acc[i][j] = f32x16{};
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return make_uint2(bf16x2_rne(a, b), bf16x2_rne(c, d));
}

// Visit the accumulators as (row m, first column n of a run of 4, 4 values).
template <bool BIG, typename F>
__device__ __forceinline__ void for_each_quad(const AccT<BIG>& acc, F&& fn) {
  typedef Cfg<BIG> C;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int m = wm * 32 * C::FM + i * 32 + (lane & 31);
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        const int n = j * (C::BN / C::FN) + wn * 32 + vb * 8 + (lane >> 5) * 4;
        fn(m, n, acc[i][j][4 * vb], acc[i][j][4 * vb + 1], acc[i][j][4 * vb + 2],
           acc[i][j][4 * vb + 3]);
      }
    }
}

// ------------------------------------------------------------------ tile lookup
// Sums across lanes through DPP operand modifiers (no LDS round trip).
// row16_sum: rotations by 8, 4, 2 and 1 lanes within each 16-lane row; at
// each level a lane adds the same two partial sums as its partner, so all 16
// lanes end with the same bits.  row32_sum: then rows 1 and 3 add lane 15 of
// rows 0 and 2 (row_bcast:15), so lanes 16-31 and 48-63 hold the sums of
// lanes 0-31 and 32-63.
template <int CTRL>
__device__ __forceinline__ float dpp_rot(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_rot<0x128>(v);   // row_ror:8
  v += dpp_rot<0x124>(v);   // row_ror:4
  v += dpp_rot<0x122>(v);   // row_ror:2
  v += dpp_rot<0x121>(v);   // row_ror:1
  return v;
}
__device__ __forceinline__ float row32_sum(float v) {
  v = row16_sum(v);
  // rows 1 and 3 receive lane 15 of rows 0 and 2; rows 0 and 2 receive 0
  return v + __int_as_float(
                 __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
}

__device__ __forceinline__ int flat_tile() {
  const int per = gridDim.x / kXcd;            // the grid is a multiple of 8
  return (blockIdx.x % kXcd) * per + blockIdx.x / kXcd;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t bf_pack(float lo, float hi) {
  return bf16x2_rne(lo, hi);
}

// Work list of a persistent row-mode workgroup.  Row tiles are BM rows of one
// expert (ceil(M_e / BM) per expert, in expert order); item it is (row tile
// it / n_tiles_n, column tile it % n_tiles_n).  The workgroup with remapped
// index flat takes items flat, flat + G, flat + 2 G, ... (G workgroups), so
// each round of G items is one contiguous run, cut into one contiguous slice
// per XCD: a row tile's column tiles share that XCD's L2.
constexpr int kMaxItems = 64;
constexpr int kRowSets = 3;     // register staging sets of the persistent row kernel
constexpr int kWgradSets = 2;   // the same for the weight-gradient stream
constexpr int kWgradNoSplitItems = 160;

struct RowSched {
  int32_t pref[257];     // row tiles of the experts before e
  int32_t off[257];      // expert row offsets
  int4 desc[kMaxItems];  // expert, first row, end row of the expert, column tile
};

// Builds the prefix of row tiles per expert (wavefront 0: five independent
// clamped loads per lane, then a lane scan) and the workgroup's item table.
// Returns the number of items (the host sizes the grid so that it is at most
// kMaxItems).
template <int BM, int NT>
__device__ int build_row_sched(RowSched& S, const int32_t* offsets, int E, int ntn) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
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
    int run = incl - sum;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = lane * 4 + s;
      if (e <= E) {
        S.pref[e] = run;
        S.off[e] = o[s];
      }
      run += tiles[s];
    }
    if (lane == 63 && E == 256) {
      S.pref[256] = incl;
      S.off[256] = o[4];
    }
  }
  __syncthreads();
  const int G = gridDim.x, flat = flat_tile();
  const int total = S.pref[E] * ntn;
  const int n = flat < total ? min((total - flat + G - 1) / G, kMaxItems) : 0;
  for (int t = threadIdx.x; t < n; t += NT) {
    const int it = flat + t * G;
    const int rt = it / ntn, nt = it - rt * ntn;
    int lo = 0, hi = E - 1;   // first expert e with pref[e + 1] > rt
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (S.pref[mid + 1] > rt) hi = mid; else lo = mid + 1;
    }
    S.desc[t] = make_int4(lo, S.off[lo] + (rt - S.pref[lo]) * BM, S.off[lo + 1], nt);
  }
  __syncthreads();
  return n;
}

template <int V>
using IC = std::integral_constant<int, V>;

// Persistent software pipeline over a workgroup's items, item i taking
// nk_of(i) >= 1 K steps (S steps in all).
// The flattened step sequence runs without a break across items: loads for the
// next item's first steps are in flight while the current item finishes and
// its epilogue runs.  NSETS register staging sets rotate: step j's operands
// are loaded into set j % NSETS while step j - NSETS + 1 computes, stored to
// LDS buffer j & 1 between the two halves of step j - 1, and consumed at step
// j, so each load has NSETS - 1.5 steps of matrix-core work to land.  Loads
// never branch (steps past the end reload the last one), so the wait before a
// store covers only the oldest set.  One barrier per step.
//   load(item, kt, IC<set>); store(IC<set>, As, Bs); epilogue(item, buf) may
//   use the LDS buffer the step just consumed (it ends with a barrier); the
//   accumulators are then cleared.
template <bool BIG, int NSETS, int NVMEM, int NDSW, typename NkOf, typename Prep, typename Load,
          typename Store, typename Epi>
__device__ __forceinline__ void run_stream(AccT<BIG>& acc, bf16_t* lds, int n_items, int S,
                                           NkOf&& nk_of, Prep&& prep, Load&& load,
                                           Store&& store, Epi&& epilogue) {
  constexpr int BM = Cfg<BIG>::BM, BN = Cfg<BIG>::BN;
  bf16_t* const As0 = lds;
  bf16_t* const Bs0 = lds + BM * BK;
  bf16_t* const As1 = lds + (BM + BN) * BK;
  bf16_t* const Bs1 = lds + (2 * BM + BN) * BK;
  int li = 0, lk = 0, lnk = nk_of(0);   // load cursor (lnk: K steps of item li)
  auto advance = [&]() {
    if (++lk == lnk) {
      if (li + 1 < n_items) {
        ++li;
        lk = 0;
        lnk = nk_of(li);
      } else {
        --lk;   // past the end: reload the last step
      }
    }
  };
  auto next_load = [&](auto set) {
    prep(li);
    load(li, lk, set);
    advance();
  };
  int ci = 0, ck = 0, cnk = lnk;   // compute cursor
  int j = 0;                       // step
  auto step = [&](auto set) {
    constexpr int s = decltype(set)::value;
    const bool odd = j & 1;
    bf16_t* const ca = odd ? As1 : As0;
    bf16_t* const cb = odd ? Bs1 : Bs0;
    bf16_t* const na = odd ? As0 : As1;
    bf16_t* const nb = odd ? Bs0 : Bs1;
    prep(li);
    // one basic block from here to the barrier: set s held step j (already
    // in LDS) and now takes step j + NSETS; the store of step j + 1's set
    // past the last step writes the idle buffer and is harmless
    load(li, lk, set);
    mma_step_pipe<BIG, NVMEM, NDSW>(acc, ca, cb,
                                    [&] { store(IC<(s + 1) % NSETS>{}, na, nb); });
    __syncthreads();
    advance();
    if (++ck == cnk) {
      epilogue(ci, ca);
      zero_acc<BIG>(acc);
      ck = 0;
      ++ci;
      if (ci < n_items) cnk = nk_of(ci);
    }
    return ++j < S;
  };
  next_load(IC<0>{});
  if constexpr (NSETS > 1) next_load(IC<1>{});
  if constexpr (NSETS > 2) next_load(IC<2>{});
  if constexpr (NSETS > 3) next_load(IC<3>{});
  static_assert(NSETS >= 2 && NSETS <= 4, "2 to 4 staging sets");
  store(IC<0>{}, As0, Bs0);
  __syncthreads();
  while (true) {
    if (!step(IC<0>{})) break;
    if (!step(IC<1>{})) break;
    if constexpr (NSETS > 2)
      if (!step(IC<2>{})) break;
    if constexpr (NSETS > 3)
      if (!step(IC<3>{})) break;
  }
}

// ------------------------------------------------------------------ kernels
// Row-split modes (UP, DOWN, DGRAD_DOWN, DGRAD_UP), persistent: G workgroups
// (at most what is resident at once) each run their item list.
// GATHER (UP only): the A rows come from X through the gather table x_rows.
template <int MODE, bool BIG, bool GATHER = false, bool FOLD = false>
__global__ __launch_bounds__(Cfg<BIG>::THREADS, 2) void rows_kernel(Args g) {
  typedef Cfg<BIG> C;
  constexpr int BM = C::BM, BN = C::BN, NT = C::THREADS;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * (BM + BN) * BK];
  __shared__ RowSched sched;
  const int n_items = build_row_sched<BM, NT>(sched, g.offsets, g.E, g.n_tiles_n);
  if (n_items == 0) return;
  const int d = g.d, f = g.f;
  // UP covers BN/2 f columns of a and the same BN/2 of b per tile
  constexpr int kUpHalf = BN / 2;
  const int Ndim = (MODE == DOWN || MODE == DGRAD_UP) ? d : f;
  const int K = (MODE == UP || MODE == DGRAD_DOWN) ? d : (MODE == DOWN ? f : 2 * f);
  const int nk = K / BK;
  const int64_t E_fd = static_cast<int64_t>(f) * d;
  const int lda = (MODE == UP || MODE == DGRAD_DOWN) ? d : f;

  AccT<BIG> acc;
  zero_acc<BIG>(acc);

  constexpr int NSETS = (MODE == DGRAD_DOWN || MODE == DGRAD_UP || GATHER) ? 2 : kRowSets;
  constexpr int KA = BM * 8 / NT;   // A chunks per thread
  constexpr int KB = BN * 8 / NT;   // k-contiguous B chunks per thread (UP, DOWN)
  constexpr int MB = BN * 2 / NT;   // n-contiguous B blocks per thread (DGRAD modes)
  static_assert(KB % 2 == 0 && (NT / 8) * (KB / 2) == kUpHalf, "UP: first half of B chunks is W1");
  KPart<BM, NT> pa[NSETS];
  KPart<BN, NT> pb[NSETS];   // k-contiguous B (UP, DOWN)
  MPart<BN, NT> pm[NSETS];   // n-contiguous B (DGRAD_DOWN, DGRAD_UP)
  const int ldb = (MODE == DGRAD_DOWN) ? f : d;   // leading dimension of an n-contiguous B

  // per-item lane offsets (bytes from the item's base) and uniform item data
  uint32_t voff_a[KA], voff_b[KB], voff_m[MB];
  int p_item = -1, p_e = 0, p_m0 = 0, p_mend = 0, p_n0 = 0;
  static_assert(!GATHER || MODE == UP || (MODE == DGRAD_DOWN && FOLD),
                "gathered A rows: UP, and DGRAD_DOWN with the gate folded");
  static_assert(!FOLD || (GATHER && !BIG && (MODE == UP || MODE == DGRAD_DOWN)),
                "gate folded: gathered small-tile UP and DGRAD_DOWN");
  // gather: xs holds the table entries of this lane's A rows for the item of
  // the next load call (fetched one load call ahead, unconditionally, before
  // that call's operand loads, so waiting for them never waits for operands)
  int32_t xs[KA];
  auto fetch_rows = [&](int item) {
    const int4 ds = sched.desc[item];
    const int m0 = __builtin_amdgcn_readfirstlane(ds.y);
    const int mlast = __builtin_amdgcn_readfirstlane(ds.z) - 1;
#pragma unroll
    for (int i = 0; i < KA; ++i)
      xs[i] = g.x_rows[min(m0 + static_cast<int>(threadIdx.x >> 3) + (NT / 8) * i, mlast)];
  };
  auto prep = [&](int item) {
    const int4 ds = sched.desc[item];
    p_e = __builtin_amdgcn_readfirstlane(ds.x);
    p_m0 = __builtin_amdgcn_readfirstlane(ds.y);
    p_mend = __builtin_amdgcn_readfirstlane(ds.z);
    p_n0 = __builtin_amdgcn_readfirstlane(ds.w) * ((MODE == UP) ? kUpHalf : BN);
    const int t = threadIdx.x, c8 = (t & 7) * 8;
    if constexpr (GATHER) {
#pragma unroll
      for (int i = 0; i < KA; ++i) {
        const int r = (t >> 3) + (NT / 8) * i;
        voff_a[i] = (p_m0 + r < p_mend)
                        ? (static_cast<uint32_t>(xs[i]) * lda + c8) * 2
                        : kOutOfRange;
      }
    } else {
#pragma unroll
      for (int i = 0; i < KA; ++i) voff_a[i] = (((t >> 3) + (NT / 8) * i) * lda + c8) * 2;
    }
    if constexpr (MODE == UP || MODE == DOWN) {
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        int r = (t >> 3) + (NT / 8) * i;
        if (MODE == UP && i >= KB / 2) r -= kUpHalf;
        voff_b[i] = (r * ((MODE == UP) ? d : f) + c8) * 2;
      }
    } else {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        int jb, kq;
        mblock<NT>(i, &jb, &kq);
        voff_m[i] = (p_n0 + jb * 8 < Ndim) ? static_cast<uint32_t>((kq * 4 * ldb + jb * 8) * 2)
                                           : kOutOfRange;
      }
    }
  };

  auto load = [&](int item, int kt, auto set_c) {
    constexpr int set = decltype(set_c)::value;
    int k0 = kt * BK;
    int half = 0;
    if (MODE == DGRAD_UP && k0 >= f) {
      half = 1;
      k0 -= f;
    }
    // A rows [m0, mend) of the expert, K from k0: rows past mend read zeros
    // (gathered: X rows through the table, offsets in voff_a)
    if constexpr (GATHER) fetch_rows((kt + 1 < nk) ? item : min(item + 1, n_items - 1));
    const bf16_t* abase = GATHER ? g.a0 + k0
                                 : ((MODE == DGRAD_UP && half) ? g.a1 : g.a0) +
                                       static_cast<int64_t>(p_m0) * lda + k0;
    const auto ra = rsrc_at(abase, GATHER ? g.x_bytes - k0 * 2 : ((p_mend - p_m0) * lda - k0) * 2);
#pragma unroll
    for (int i = 0; i < KA; ++i) pa[set].v[i] = bload(ra, voff_a[i]);
    const int64_t wexp = static_cast<int64_t>(p_e) * E_fd;
    if constexpr (MODE == UP) {
      const int nb = (kUpHalf * d - k0) * 2;
      const auto r1 = rsrc_at(g.b0 + wexp + static_cast<int64_t>(p_n0) * d + k0, nb);
      const auto r3 = rsrc_at(g.b1 + wexp + static_cast<int64_t>(p_n0) * d + k0, nb);
#pragma unroll
      for (int i = 0; i < KB; ++i) pb[set].v[i] = bload(i < KB / 2 ? r1 : r3, voff_b[i]);
    } else if constexpr (MODE == DOWN) {
      // W2[e] rows n0.. (over d), K = f; rows past d read zeros
      const auto rb = rsrc_at(g.b0 + wexp + static_cast<int64_t>(p_n0) * f + k0,
                              ((d - p_n0) * f - k0) * 2);
#pragma unroll
      for (int i = 0; i < KB; ++i) pb[set].v[i] = bload(rb, voff_b[i]);
    } else {
      // DGRAD_DOWN: W2[e] [d][f], element (k, n) at k f + n;
      // DGRAD_UP:   W1/W3[e] [f][d], element (k, n) at k d + n
      const int krows = (MODE == DGRAD_DOWN) ? d : f;
      const bf16_t* wb = ((MODE == DGRAD_UP && half) ? g.b1 : g.b0) + wexp;
      const auto rm = rsrc_at(wb + static_cast<int64_t>(k0) * ldb + p_n0,
                              ((krows - k0) * ldb - p_n0) * 2);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) pm[set].v[i][r] = bload(rm, voff_m[i] + r * ldb * 2);
    }
  };
  auto store = [&](auto set_c, bf16_t* As, bf16_t* Bs) {
    constexpr int set = decltype(set_c)::value;
    kstore_raw<BM, NT>(pa[set], As);
    if constexpr (MODE == UP || MODE == DOWN)
      kstore_raw<BN, NT>(pb[set], Bs);
    else
      mstore_raw<BN, NT>(pm[set], Bs);
  };

  // Epilogue through the LDS buffer the last step consumed (free until the
  // next store into it; the final barrier keeps it so): the accumulators are
  // rounded to bf16 and staged as [BM][BN] with 16-byte chunks XOR-swizzled by
  // row, then read back as whole rows and written in coalesced 16-byte chunks
  // with the mode's elementwise work applied.  DGRAD_DOWN issues all of its
  // saved-a/b loads before staging, so their latency overlaps the staging.
  static_assert((BM + BN) * BK >= BM * BN, "one staging pass");
  constexpr int CH = BN / 8;                 // 16-byte chunks per staged row
  constexpr int kOutIt = BM * CH / NT;       // readback chunks per thread (N modes)
  auto epilogue = [&](int item, bf16_t* buf) {
    const int4 ds = sched.desc[item];
    const int m0 = ds.y, rows = min(BM, ds.z - m0);
    const int n0 = ds.w * ((MODE == UP) ? kUpHalf : BN);
    const int nch = (MODE == UP) ? kUpHalf / 8 : min(BN, Ndim - n0) / 8;
    uint4 aux_a[(MODE == DGRAD_DOWN) ? kOutIt : 1], aux_b[(MODE == DGRAD_DOWN) ? kOutIt : 1];
    // folded gate of each readback row, loaded with the saved a/b (before staging)
    constexpr int kGateIt = !FOLD ? 1 : (MODE == UP) ? BM * (kUpHalf / 8) / NT : kOutIt;
    float gate_r[kGateIt];
    if constexpr (FOLD) {
      constexpr int kRowCh = (MODE == UP) ? kUpHalf / 8 : CH;
#pragma unroll
      for (int it = 0; it < kGateIt; ++it) {
        const int r = min((static_cast<int>(threadIdx.x) + NT * it) / kRowCh, rows - 1);
        gate_r[it] = g.gate_rows[m0 + r];
      }
    }
    if constexpr (MODE == DGRAD_DOWN) {
#pragma unroll
      for (int it = 0; it < kOutIt; ++it) {
        const int v = threadIdx.x + NT * it;
        const int r = min(v / CH, rows - 1), c = min(v % CH, nch - 1);   // clamped: in bounds
        const int64_t o = static_cast<int64_t>(m0 + r) * Ndim + n0 + c * 8;
        aux_a[it] = ld_nt16(reinterpret_cast<const uint4*>(g.aux0 + o));
        aux_b[it] = ld_nt16(reinterpret_cast<const uint4*>(g.aux1 + o));
      }
    }
    // The row swizzle key (r & 15 = lane & 15 for every fragment) goes through
    // an opaque move so that the staging addresses are formed here rather
    // than hoisted out of the step loop into registers held across it.
    int key;
    asm volatile("v_mov_b32 %0, %1" : "=v"(key) : "v"(static_cast<int>(threadIdx.x & 15)));
    for_each_quad<BIG>(acc, [&](int m, int n, float v0, float v1, float v2, float v3) {
      *reinterpret_cast<uint2*>(buf + m * BN + (((n >> 3) ^ key) << 3) + (n & 4)) =
          pack4(v0, v1, v2, v3);
    });
    __syncthreads();
    auto chunk = [&](int r, int c) {
      return *reinterpret_cast<const uint4*>(buf + r * BN + ((c ^ (r & 15)) << 3));
    };
    if constexpr (MODE == UP) {
      // staged columns [0, BN/2) hold a, [BN/2, BN) hold b of f columns n0 + c
      constexpr int kCh = kUpHalf / 8;
#pragma unroll
      for (int it = 0; it < BM * kCh / NT; ++it) {
        const int v = threadIdx.x + NT * it;
        const int r = v / kCh, c = v % kCh;
        if (r >= rows) continue;
        const uint4 av = chunk(r, c), bv = chunk(r, c + kCh);
        const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w};
        uint32_t hw[4];
        if constexpr (FOLD) {   // the row's gate on h
          const float gr = gate_r[it];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            hw[q] = bf_pack(silu_f(bf_lo(aw[q])) * bf_lo(bw[q]) * gr,
                            silu_f(bf_hi(aw[q])) * bf_hi(bw[q]) * gr);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            hw[q] = bf_pack(silu_f(bf_lo(aw[q])) * bf_lo(bw[q]),
                            silu_f(bf_hi(aw[q])) * bf_hi(bw[q]));
        }
        const int64_t o = static_cast<int64_t>(m0 + r) * f + n0 + c * 8;
        *reinterpret_cast<uint4*>(g.c0 + o) = av;
        *reinterpret_cast<uint4*>(g.c1 + o) = bv;
        *reinterpret_cast<uint4*>(g.c2 + o) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      }
    } else if constexpr (MODE == DGRAD_DOWN && FOLD) {
      // gate folded: the staged product is u = dy W2 (rounded); the row's
      // dgate part is <u, silu(a) b> over this column tile (a 16-lane sum in a
      // fixed order), dh = g u, then da = dh b silu'(a), db = dh silu(a)
      static_assert(CH == 16, "one row per 16 lanes");
      // the da/db stores go out first; the parts of a group of iterations wait
      // in registers and their 16-lane sums run together (xor 8, 4, 2, 1)
      constexpr int kGrp = kOutIt < 4 ? kOutIt : 4;
      static_assert(kOutIt % kGrp == 0, "whole groups");
#pragma unroll
      for (int i0 = 0; i0 < kOutIt; i0 += kGrp) {
      float partv[kGrp];
#pragma unroll
      for (int ig = 0; ig < kGrp; ++ig) {
        const int it = i0 + ig;
        const int v = threadIdx.x + NT * it;
        const int r = v / CH, c = v % CH;
        const bool ok = r < rows && c < nch;
        const uint4 uv = chunk(r, c), av = aux_a[it], bv = aux_b[it];
        const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
        const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w};
        const float gr = gate_r[it];
        float part = 0.f;
        uint32_t daw[4], dbw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float da2[2], db2[2];
          const float uu[2] = {bf_lo(uw[q]), bf_hi(uw[q])};
          const float aa[2] = {bf_lo(aw[q]), bf_hi(aw[q])};
          const float bb[2] = {bf_lo(bw[q]), bf_hi(bw[q])};
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float sg = sigmoid_f(aa[u]);
            const float sa = aa[u] * sg;   // silu(a)
            part = fmaf(uu[u], sa * bb[u], part);
            const float dh = gr * uu[u];
            da2[u] = dh * bb[u] * (sg * (1.0f + aa[u] * (1.0f - sg)));
            db2[u] = dh * sa;
          }
          daw[q] = bf_pack(da2[0], da2[1]);
          dbw[q] = bf_pack(db2[0], db2[1]);
        }
        partv[ig] = ok ? part : 0.f;
        if (ok) {
          const int64_t o = static_cast<int64_t>(m0 + r) * Ndim + n0 + c * 8;
          *reinterpret_cast<uint4*>(g.c0 + o) = make_uint4(daw[0], daw[1], daw[2], daw[3]);
          *reinterpret_cast<uint4*>(g.c1 + o) = make_uint4(dbw[0], dbw[1], dbw[2], dbw[3]);
        }
      }
      static_assert(CH == 16, "one row per 16 lanes");
#pragma unroll
      for (int ig = 0; ig < kGrp; ++ig) partv[ig] = row16_sum(partv[ig]);
#pragma unroll
      for (int ig = 0; ig < kGrp; ++ig) {
        const int v = threadIdx.x + NT * (i0 + ig);
        const int r = v / CH, c = v % CH;
        if (c == 0 && r < rows)
          g.dgate_part[static_cast<int64_t>(m0 + r) * g.n_tiles_n + ds.w] = partv[ig];
      }
      }
    } else {
#pragma unroll
      for (int it = 0; it < kOutIt; ++it) {
        const int v = threadIdx.x + NT * it;
        const int r = v / CH, c = v % CH;
        if (r >= rows || c >= nch) continue;
        const uint4 hv = chunk(r, c);
        const int64_t o = static_cast<int64_t>(m0 + r) * Ndim + n0 + c * 8;
        if constexpr (MODE == DGRAD_DOWN) {
          // dh (rounded); da = dh b silu'(a), db = dh silu(a)
          const uint4 av = aux_a[it], bv = aux_b[it];
          const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
          const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w};
          uint32_t daw[4], dbw[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float da2[2], db2[2];
            const float hh[2] = {bf_lo(hw[q]), bf_hi(hw[q])};
            const float aa[2] = {bf_lo(aw[q]), bf_hi(aw[q])};
            const float bb[2] = {bf_lo(bw[q]), bf_hi(bw[q])};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const float sg = sigmoid_f(aa[u]);
              da2[u] = hh[u] * bb[u] * (sg * (1.0f + aa[u] * (1.0f - sg)));
              db2[u] = hh[u] * (aa[u] * sg);
            }
            daw[q] = bf_pack(da2[0], da2[1]);
            dbw[q] = bf_pack(db2[0], db2[1]);
          }
          *reinterpret_cast<uint4*>(g.c0 + o) = make_uint4(daw[0], daw[1], daw[2], daw[3]);
          *reinterpret_cast<uint4*>(g.c1 + o) = make_uint4(dbw[0], dbw[1], dbw[2], dbw[3]);
        } else {
          *reinterpret_cast<uint4*>(g.c0 + o) = hv;
        }
      }
    }
    __syncthreads();
  };
  auto prep_if = [&](int item) {
    if (item != p_item) {
      prep(item);
      p_item = item;
    }
  };
  constexpr int kVmem = KA + ((MODE == UP || MODE == DOWN) ? KB : MB * 4);
  constexpr int kDsw = KA + ((MODE == UP || MODE == DOWN) ? KB : MB * 8);
  if constexpr (GATHER) fetch_rows(0);
  run_stream<BIG, NSETS, kVmem + (GATHER ? KA : 0), kDsw>(
      acc, lds, n_items, n_items * nk, [nk](int) { return nk; }, prep_if, load, store, epilogue);
}

// expert and first row of row tile `tile` (tiles of BM rows; prefix sum of
// per-expert tile counts across wave 0, 4 experts per lane); false when there
// is no such tile
template <int BM>
__device__ bool find_row_tile_at(int* scratch, const int32_t* offsets, int E, int tile, int* e_out,
                                 int* m0_out, int* mend_out) {
  int& s_e = scratch[0];
  int& s_m0 = scratch[1];
  int& s_mend = scratch[2];
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

// the same with its three results in static LDS
template <int BM>
__device__ bool find_row_tile(const int32_t* offsets, int E, int tile, int* e_out, int* m0_out,
                              int* mend_out) {
  __shared__ int s[3];
  return find_row_tile_at<BM>(s, offsets, E, tile, e_out, m0_out, mend_out);
}

// ------------------------------------------------------------------ direct-to-LDS big tile
// Row modes at the big tile, one tile per workgroup: operand tiles go from
// HBM/L2 straight into LDS by buffer loads with the LDS destination (no
// register staging).  Each wavefront instruction fills 1 KB of LDS; the global
// addresses carry the swizzle of the LDS layout (logical chunk = physical ^
// key(row)), so the fragment reads are conflict-free.  The compiler does not
// track these LDS writes, so each step waits on the vector-memory counter
// explicitly and joins the workgroup with a plain s_barrier (a fenced barrier
// would also drain the prefetch).
namespace dma {
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, bf16_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, static_cast<int>(voff), 0, 0, 0);
}
// s_waitcnt with vmcnt = N (N < 64: bits 3-0 and 15-14), expcnt and lgkmcnt left free
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
}  // namespace dma

// The big UP/DOWN tile with 64-wide k steps: each row of a stage is 128 bytes,
// a whole cache line, so every line of A and B is requested from L2 once (with
// 32-wide steps each line is requested twice, half per step: measured 2.3x the
// requests and 6% slower).  A ring of five 32 KB slots, each holding the A or
// the B operand of one step, keeps about a step and a half of fills in flight
// across every barrier (two 64 KB stages drained the fills once per step: UP
// measured 2-3% slower at C5).  The 16-byte chunks of a row are XORed with
// (row >> 1) & 7, so any 16 consecutive rows read at one logical chunk (a
// fragment read) hit distinct banks; the DMA writes carry the same swizzle in
// their global addresses.
namespace dma64 {
constexpr int BM = 256, BN = 256, BKS = 64, NST = 2, NT = 512, WAVES_N = 4, FM = 4, FN = 2;
constexpr int kStage = (BM + BN) * BKS;   // elements per stage (64 KB)
constexpr int kSlot = BM * BKS;           // one operand of a step (32 KB)
constexpr int kSlots = 5;                 // the ring of the UP/DOWN tile (160 KB)
}  // namespace dma64

template <int MODE, bool FOLD = false>
__global__ __launch_bounds__(dma64::NT, 1) void dma_rows_kernel(Args g) {
  using namespace dma64;
  static_assert(MODE == UP || MODE == DOWN, "k-contiguous modes only");
  static_assert(BM == BN, "A and B parts of a step fill equal slots");
  __shared__ __attribute__((aligned(16))) bf16_t lds[kSlots * kSlot];
  const int flat = flat_tile();
  const int row_tile = flat / g.n_tiles_n;
  const int nt = flat - row_tile * g.n_tiles_n;
  int e, m0, mend;
  // the lookup's three results pass through the first bytes of the LDS
  if (!find_row_tile_at<BM>(reinterpret_cast<int*>(lds), g.offsets, g.E, row_tile, &e, &m0,
                            &mend))
    return;
  e = __builtin_amdgcn_readfirstlane(e);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  mend = __builtin_amdgcn_readfirstlane(mend);
  __syncthreads();   // every lane holds them before the first fill lands there
  const int rows = min(BM, mend - m0);
  const int d = g.d, f = g.f;
  constexpr int kUpHalf = BN / 2;
  const int n0 = nt * ((MODE == UP) ? kUpHalf : BN);
  const int K = (MODE == UP) ? d : f;
  const int nk = K / BKS;
  const int lda = (MODE == UP) ? d : f;
  const int64_t E_fd = static_cast<int64_t>(f) * d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // this wavefront's DMA instructions: A rows 32 wave + [0, 32) and B rows
  // 32 wave + [0, 32), 8 rows of 128 bytes per instruction (lane l: row
  // + l / 8, physical chunk l % 8, logical chunk (l % 8) ^ ((row >> 1) & 7))
  const bool gather = (MODE == UP) && g.x_rows != nullptr;
  uint32_t voa[4], vob[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = wave * 32 + u * 8 + (lane >> 3);
    const int logical = (lane & 7) ^ ((row >> 1) & 7);
    if (gather) {
      const uint32_t src = static_cast<uint32_t>(g.x_rows[min(m0 + row, mend - 1)]);
      voa[u] = (m0 + row < mend) ? (src * lda + logical * 8) * 2 : kOutOfRange;
    } else {
      voa[u] = (row * lda + logical * 8) * 2;
    }
    const int brow = (MODE == UP && row >= kUpHalf) ? row - kUpHalf : row;
    vob[u] = (brow * ((MODE == UP) ? d : f) + logical * 8) * 2;
  }
  const bf16_t* abase = gather ? g.a0 : g.a0 + static_cast<int64_t>(m0) * lda;
  const int a_rows_bytes = gather ? g.x_bytes : (mend - m0) * lda * 2;
  const bf16_t* bbase;
  int b_bytes;
  if constexpr (MODE == UP) {
    bbase = (wave < 4 ? g.b0 : g.b1) + e * E_fd + static_cast<int64_t>(n0) * d;
    b_bytes = kUpHalf * d * 2;
  } else {
    bbase = g.b0 + e * E_fd + static_cast<int64_t>(n0) * f;
    b_bytes = (d - n0) * f * 2;
  }
  // half-step h: the A (h even) or B (h odd) operand of step h / 2, four
  // instructions per wavefront, into ring slot `slot` (h mod 5)
  auto issue_half = [&](int h, int slot) {
    bf16_t* dst = lds + slot * kSlot + wave * 32 * BKS;
    const int k0 = (h >> 1) * BKS;
    if ((h & 1) == 0) {
      const auto ra = rsrc_at(abase + k0, a_rows_bytes - k0 * 2);
#pragma unroll
      for (int u = 0; u < 4; ++u) dma::dma16(ra, dst + u * 8 * BKS, voa[u]);
    } else {
      const auto rb = rsrc_at(bbase + k0, b_bytes - k0 * 2);
#pragma unroll
      for (int u = 0; u < 4; ++u) dma::dma16(rb, dst + u * 8 * BKS, vob[u]);
    }
  };

  AccT<true> acc;
  zero_acc<true>(acc);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int r = lane & 31, gq = lane >> 5;
  // byte addresses (within a slot) of this lane's fragment rows for the
  // four 16-wide sub-steps; fragment i / j adds i * 32 / j * 128 rows, which
  // keeps (row >> 1) & 7 and so the swizzle
  uint32_t a_addr[4], b_addr[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int pc = (2 * kk + gq) ^ ((r >> 1) & 7);
    a_addr[kk] = ((wm * 32 * FM + r) * BKS + pc * 8) * 2;
    b_addr[kk] = ((wn * 32 + r) * BKS + pc * 8) * 2;
  }
  const uint32_t lds_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) bf16_t*)lds));
  typedef float f32x16v __attribute__((ext_vector_type(16)));
  f32x16v c00 = acc[0][0], c01 = acc[0][1], c10 = acc[1][0], c11 = acc[1][1];
  f32x16v c20 = acc[2][0], c21 = acc[2][1], c30 = acc[3][0], c31 = acc[3][1];
  bf16x8 p0[6], p1[6];
#define MOE_MF(c, b, a) "v_mfma_f32_32x32x16_bf16 " c ", " b ", " a ", " c "\n\t"
#define MOE_RD(o, addr, off) "ds_read_b128 " o ", " addr " offset:" off "\n\t"
  // reads six fragments at (aaddr, baddr) into `out` while running the eight
  // MFMAs of the fragments `in`, and waits for its reads
  auto half_asm = [&](const bf16x8 (&in)[6], bf16x8 (&out)[6], uint32_t aaddr, uint32_t baddr) {
    asm volatile(
        MOE_RD("%8", "%20", "0")       MOE_MF("%0", "%18", "%14")
        MOE_RD("%9", "%20", "4096")    MOE_MF("%1", "%19", "%14")
        MOE_RD("%10", "%20", "8192")   MOE_MF("%2", "%18", "%15")
        MOE_RD("%11", "%20", "12288")  MOE_MF("%3", "%19", "%15")
        MOE_RD("%12", "%21", "0")      MOE_MF("%4", "%18", "%16")
        MOE_RD("%13", "%21", "16384")  MOE_MF("%5", "%19", "%16")
                                       MOE_MF("%6", "%18", "%17")
                                       MOE_MF("%7", "%19", "%17")
        "s_waitcnt lgkmcnt(0)"
        : "+v"(c00), "+v"(c01), "+v"(c10), "+v"(c11), "+v"(c20), "+v"(c21), "+v"(c30),
          "+v"(c31), "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]),
          "=&v"(out[4]), "=&v"(out[5])
        : "v"(in[0]), "v"(in[1]), "v"(in[2]), "v"(in[3]), "v"(in[4]), "v"(in[5]), "v"(aaddr),
          "v"(baddr)
        : "memory");
  };
#undef MOE_MF
#undef MOE_RD
  auto read_p = [&](bf16x8 (&out)[6], uint32_t aaddr, uint32_t baddr) {
    asm volatile(
        "ds_read_b128 %0, %6 offset:0\n\t"
        "ds_read_b128 %1, %6 offset:4096\n\t"
        "ds_read_b128 %2, %6 offset:8192\n\t"
        "ds_read_b128 %3, %6 offset:12288\n\t"
        "ds_read_b128 %4, %7 offset:0\n\t"
        "ds_read_b128 %5, %7 offset:16384\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), "=&v"(out[4]),
          "=&v"(out[5])
        : "v"(aaddr), "v"(baddr)
        : "memory");
  };
  auto slot_addr = [&](int slot) { return lds_base + slot * kSlot * 2; };
  // A ring of five 32 KB slots, one operand of one step each, so that the
  // fills never drain: half-step h (the A or B operand of step h / 2) sits in
  // slot h mod 5.  Prologue: half-steps 0-4 (steps 0 and 1, the A operand of
  // step 2); the kk = 0 fragments of step 0 once it has landed.
  const int nh = 2 * nk;
#pragma unroll
  for (int h = 0; h < kSlots; ++h)
    if (h < nh) issue_half(h, h);
  if (nk >= 3) dma::wait_vm<12>();
  else if (nk == 2) dma::wait_vm<8>();
  else dma::wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  read_p(p0, slot_addr(0) + a_addr[0], slot_addr(1) + b_addr[0]);
  // step kt (slots sa, sb): sub-steps 0-2 while reading 1-3; then the wait
  // for step kt + 1 (the A operand of step kt + 2, issued last, may stay in
  // flight), the barrier that sees step kt + 1 landed everywhere and step kt
  // read by everyone, half-steps 2 kt + 5 and 2 kt + 6 into the freed slots,
  // and sub-step 3 while reading sub-step 0 of step kt + 1
  int sa = 0, sb = 1;
  for (int kt = 0; kt < nk; ++kt) {
    const uint32_t ca = slot_addr(sa), cb = slot_addr(sb);
    const int na = sa + 2 < kSlots ? sa + 2 : sa + 2 - kSlots;
    const int nb = sb + 2 < kSlots ? sb + 2 : sb + 2 - kSlots;
    half_asm(p0, p1, ca + a_addr[1], cb + b_addr[1]);
    half_asm(p1, p0, ca + a_addr[2], cb + b_addr[2]);
    half_asm(p0, p1, ca + a_addr[3], cb + b_addr[3]);
    if (kt + 2 < nk) dma::wait_vm<4>();
    else dma::wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    if (2 * kt + 5 < nh) issue_half(2 * kt + 5, sa);
    if (2 * kt + 6 < nh) issue_half(2 * kt + 6, sb);
    half_asm(p1, p0, slot_addr(na) + a_addr[0], slot_addr(nb) + b_addr[0]);
    sa = na;
    sb = nb;
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  acc[0][0] = c00; acc[0][1] = c01; acc[1][0] = c10; acc[1][1] = c11;
  acc[2][0] = c20; acc[2][1] = c21; acc[3][0] = c30; acc[3][1] = c31;
  dma::wait_vm<0>();
  __syncthreads();

  // epilogue: the whole 256 x 256 tile staged as bf16 over the two stages
  // (128 KB), 16-byte chunks XOR-swizzled by row, then coalesced stores
  bf16_t* out = lds;
  {
    int skey;
    asm volatile("v_mov_b32 %0, %1" : "=v"(skey) : "v"(static_cast<int>(threadIdx.x & 15)));
    for_each_quad<true>(acc, [&](int m, int n, float v0, float v1, float v2, float v3) {
      *reinterpret_cast<uint2*>(out + m * BN + (((n >> 3) ^ skey) << 3) + (n & 4)) =
          pack4(v0, v1, v2, v3);
    });
  }
  __syncthreads();
  auto chunk_at = [&](int rr, int c) {
    return *reinterpret_cast<const uint4*>(out + rr * BN + ((c ^ (rr & 15)) << 3));
  };
  if constexpr (MODE == UP) {
    constexpr int kCh = kUpHalf / 8;
    constexpr int kIt = BM * kCh / NT;
    static_assert(BM * kCh % NT == 0, "whole iterations");
    // the gates of the thread's rows are loaded first (clamped in bounds), so
    // the epilogue waits for one latency, not one per row
    float grs[kIt];
    if constexpr (FOLD) {
#pragma unroll
      for (int it = 0; it < kIt; ++it)
        grs[it] = g.gate_rows[m0 + min((tid + NT * it) / kCh, rows - 1)];
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int v = tid + NT * it;
      const int rr = v / kCh, c = v % kCh;
      if (rr >= rows) continue;
      const uint4 av = chunk_at(rr, c), bv = chunk_at(rr, c + kCh);
      const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w};
      uint32_t hw[4];
      if constexpr (FOLD) {   // the row's gate on h
        const float gr = grs[it];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          hw[q] = bf_pack(silu_f(bf_lo(aw[q])) * bf_lo(bw[q]) * gr,
                          silu_f(bf_hi(aw[q])) * bf_hi(bw[q]) * gr);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          hw[q] = bf_pack(silu_f(bf_lo(aw[q])) * bf_lo(bw[q]),
                          silu_f(bf_hi(aw[q])) * bf_hi(bw[q]));
      }
      const int64_t o = static_cast<int64_t>(m0 + rr) * f + n0 + c * 8;
      *reinterpret_cast<uint4*>(g.c0 + o) = av;
      *reinterpret_cast<uint4*>(g.c1 + o) = bv;
      *reinterpret_cast<uint4*>(g.c2 + o) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    }
  } else {
    constexpr int kCh = BN / 8;
    const int nch = min(BN, d - n0) / 8;
    for (int v = tid; v < BM * kCh; v += NT) {
      const int rr = v / kCh, c = v % kCh;
      if (rr >= rows || c >= nch) continue;
      *reinterpret_cast<uint4*>(g.c0 + static_cast<int64_t>(m0 + rr) * d + n0 + c * 8) =
          chunk_at(rr, c);
    }
  }
}

// Weight gradients with the big tile on a 4-stage LDS ring of 32-row steps: both
// operands are row-major over the expert's rows p ([p][m] and [p][n]), so a
// stage holds them as they lie in HBM, [32 rows][256 columns] (512-byte rows),
// filled by buffer loads with the LDS destination, and the MFMA fragments
// (8 consecutive p for one column) come from the gfx950 transposing LDS read:
// within each 16-lane group, lane s reads 8 bytes of row s / 4 at column
// 4 (s % 4), and lane j receives column j of the four rows.  The 16-byte
// chunks of a row are XORed with 4 (row & 3), so the four rows a group reads
// fall in distinct banks; the DMA writes carry the same swizzle in their
// global addresses.
namespace dmaw {
constexpr int BM = 256, BN = 256, BKS = 32, NST = 4, NT = 512, WAVES_N = 4, FM = 4, FN = 2;
constexpr int kStage = (BM + BN) * BKS;      // elements
constexpr int kRowBytes = BM * 2;           // 512
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_t;
__device__ __forceinline__ bf16x8 tr_frag(const bf16_t* lds, uint32_t byte_lo, uint32_t byte_hi) {
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4s_t)(reinterpret_cast<const char*>(lds) + byte_lo));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4s_t)(reinterpret_cast<const char*>(lds) + byte_hi));
  typedef short v8s __attribute__((ext_vector_type(8)));
  const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}
__device__ __forceinline__ void mem_fence_compiler() { asm volatile("" ::: "memory"); }
}  // namespace dmaw

// Tile order of the big weight-gradient kernel.  A tile's reduction runs over
// its expert's rows, so its duration follows the expert's row count, which top-k
// routing leaves uneven (at 16384 tokens, 64 experts and k = 6 the synthetic
// routing gives 274 to 4216 rows).  The tiles of one product (dW2, dW1 or dW3)
// of one expert form a group that stays on one XCD, where its tiles share the
// expert's operand panels in L2.  Groups are ranked by their expert's row count,
// largest first (equal counts: lower expert id first; an expert's three products
// in the order dW2, dW1, dW3), and dealt to the 8 XCDs in a snake: round r goes
// over XCDs 0..7 when r is even and 7..0 when it is odd.  Every XCD then gets
// about the same number of rows and runs its largest groups first, where expert
// order left one XCD with 16% more rows than the mean at that shape.  Workgroup
// b runs on XCD b mod 8 as that XCD's (b / 8)-th; its round is (b / 8) / tpe.
// The grid is 8 * ceil(3 E / 8) * tpe; a workgroup past the last group gets
// false (uniform over the workgroup, before any barrier).  p0, p1: the expert's
// row offsets.
__device__ bool wgrad_snake_tile(const int32_t* offsets, int E, int tpe, int* z_out, int* e_out,
                                 int* t_out, int* p0_out, int* p1_out) {
  __shared__ int s_off[257];
  __shared__ int s_rank[256];
  __shared__ int s_e;
  const int xcd = blockIdx.x % kXcd, j = blockIdx.x / kXcd;
  const int r = j / tpe;
  const int i = r * kXcd + ((r & 1) ? kXcd - 1 - xcd : xcd);
  if (i >= 3 * E) return false;
  const int q = i / 3;
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int m = tid; m <= E; m += nt) {
    s_off[m] = offsets[m];
    if (m < E) s_rank[m] = 0;
  }
  __syncthreads();
  // rank of expert u = the experts with more rows, or as many and a lower id;
  // wavefront w counts over m = w, w + nw, ... and adds its count into LDS
  const int lane = tid & 63, w = tid >> 6, nw = nt >> 6;
  for (int u = lane; u < E; u += 64) {
    const int cu = s_off[u + 1] - s_off[u];
    int rk = 0;
    for (int m = w; m < E; m += nw) {
      const int cm = s_off[m + 1] - s_off[m];
      rk += (cm > cu || (cm == cu && m < u)) ? 1 : 0;
    }
    if (rk) atomicAdd(&s_rank[u], rk);
  }
  __syncthreads();
  for (int u = tid; u < E; u += nt)
    if (s_rank[u] == q) s_e = u;   // the ranks are a permutation of 0 .. E - 1
  __syncthreads();
  const int e = s_e;
  *z_out = i - 3 * q;
  *e_out = e;
  *t_out = j - r * tpe;
  *p0_out = s_off[e];
  *p1_out = s_off[e + 1];
  return true;
}

// GATHER: as in the small-tile kernel, the x operand of dW1 and dW3 comes from
// X through the gather table, entries fetched NST - 1 = 3 steps ahead.
template <bool GATHER, bool FOLD_A = false>
__global__ __launch_bounds__(dmaw::NT, 1) void wgrad_dma_kernel(Args g, int32_t tiles_per_expert) {
  using namespace dmaw;
  // four stage arrays (distinct objects: a transposing read of one stage is
  // ordered only after the DMA into that stage)
  __shared__ __attribute__((aligned(16))) bf16_t st0[kStage];
  __shared__ __attribute__((aligned(16))) bf16_t st1[kStage];
  __shared__ __attribute__((aligned(16))) bf16_t st2[kStage];
  __shared__ __attribute__((aligned(16))) bf16_t st3[kStage];

  int z, e, t, p0, p1;
  if (!wgrad_snake_tile(g.offsets, g.E, tiles_per_expert, &z, &e, &t, &p0, &p1)) return;
  z = __builtin_amdgcn_readfirstlane(z);
  e = __builtin_amdgcn_readfirstlane(e);
  t = __builtin_amdgcn_readfirstlane(t);
  p0 = __builtin_amdgcn_readfirstlane(p0);
  p1 = __builtin_amdgcn_readfirstlane(p1);
  const int d = g.d, f = g.f;
  const int Mdim = (z == 0) ? d : f, Ndim = (z == 0) ? f : d;
  const int tiles_n = (Ndim + BN - 1) / BN;
  const int m0 = (t / tiles_n) * BM, n0 = (t % tiles_n) * BN;
  if (m0 >= Mdim) return;
  const bf16_t* Asrc = (z == 0) ? g.a0 : (z == 1 ? g.a1 : g.aux0);
  const bf16_t* Bsrc = (z == 0) ? g.b0 : g.b1;
  bf16_t* dst = ((z == 0) ? g.c0 : (z == 1 ? g.c1 : g.c2)) + static_cast<int64_t>(e) * d * f;
  const int nk = (p1 - p0 + BKS - 1) / BKS;
  const int mvalid = min(BM, Mdim - m0), nvalid = min(BN, Ndim - n0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (nk == 0) {   // the expert has no rows: its weight gradient is zero
    for (int v = tid; v < BM * (BN / 8); v += NT) {
      const int r = v / (BN / 8), c = v % (BN / 8);
      if (r < mvalid && c * 8 < nvalid)
        *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(m0 + r) * Ndim + n0 + c * 8) =
            make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }

  // DMA: wavefront w fills rows 4 w .. 4 w + 3 of the A and the B tile, two
  // rows (1 KB) per instruction; lane l -> row + l / 32, physical chunk l % 32
  uint32_t voa[2], vob[2];
  int acol[2], bcol[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = wave * 4 + u * 2 + (lane >> 5);
    const int logical = (lane & 31) ^ (4 * (row & 3));
    const int col = logical * 8;
    voa[u] = (m0 + col < Mdim) ? static_cast<uint32_t>((row * Mdim + col) * 2) : kOutOfRange;
    vob[u] = (n0 + col < Ndim) ? static_cast<uint32_t>((row * Ndim + col) * 2) : kOutOfRange;
    acol[u] = (m0 + col < Mdim) ? col : -1;
    bcol[u] = (n0 + col < Ndim) ? col : -1;
  }
  const bool gz = GATHER && z != 0;   // B rows gathered from X
  const bool ga = FOLD_A && z == 0;   // A rows (dy) gathered from dY [T, d]
  int32_t xs[NST][2];                 // table entries of the rows of step s in slot s % NST
  auto fetch = [&](int slot, int kt) {
    const int pb = p0 + kt * BKS;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      xs[slot][u] = g.x_rows[min(pb + wave * 4 + u * 2 + (lane >> 5), p1 - 1)];
  };
  // step kt into the stage at As; steps at or past nk read through an empty
  // resource, so their stage is zero and adds nothing
  auto issue = [&](bf16_t* As, int kt, int slot) {
    bf16_t* Bs = As + BKS * BM;
    const bool live = kt < nk;
    const int p = p0 + min(kt, nk - 1) * BKS;
    const auto ra = (FOLD_A && ga) ? rsrc_at(Asrc + m0, live ? g.x_bytes - m0 * 2 : 0)
                                   : rsrc_at(Asrc + static_cast<int64_t>(p) * Mdim + m0,
                                             live ? ((p1 - p) * Mdim - m0) * 2 : 0);
    uint32_t va[2] = {voa[0], voa[1]};
    uint32_t vb[2] = {vob[0], vob[1]};
    __amdgpu_buffer_rsrc_t rb;
    if constexpr (GATHER) {
      if (FOLD_A && ga) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int q = kt * BKS + wave * 4 + u * 2 + (lane >> 5);   // row of the expert
          va[u] = (p0 + q < p1 && acol[u] >= 0)
                      ? (static_cast<uint32_t>(xs[slot][u]) * Mdim + acol[u]) * 2
                      : kOutOfRange;
        }
      }
      rb = gz ? rsrc_at(Bsrc + n0, live ? g.x_bytes - n0 * 2 : 0)
              : rsrc_at(Bsrc + static_cast<int64_t>(p) * Ndim + n0,
                        live ? ((p1 - p) * Ndim - n0) * 2 : 0);
      if (gz) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int q = kt * BKS + wave * 4 + u * 2 + (lane >> 5);   // row of the expert
          vb[u] = (p0 + q < p1 && bcol[u] >= 0)
                      ? (static_cast<uint32_t>(xs[slot][u]) * Ndim + bcol[u]) * 2
                      : kOutOfRange;
        }
      }
    } else {
      rb = rsrc_at(Bsrc + static_cast<int64_t>(p) * Ndim + n0,
                   live ? ((p1 - p) * Ndim - n0) * 2 : 0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) dma::dma16(ra, As + (wave * 4 + u * 2) * BM, va[u]);
#pragma unroll
    for (int u = 0; u < 2; ++u) dma::dma16(rb, Bs + (wave * 4 + u * 2) * BN, vb[u]);
  };

  // transposing-read addresses (bytes within a stage) for sub-step 0, half 0;
  // + 4 rows (2048 B) for half 1, + 16 rows (8192 B) for sub-step 1
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int G = lane >> 4, sl = lane & 15;
  const int row0 = 8 * (G >> 1) + (sl >> 2);
  const int sw = 4 * (row0 & 3);
  uint32_t ta[FM], tb[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int col = wm * 128 + i * 32 + 16 * (G & 1) + 4 * (sl & 3);
    ta[i] = row0 * kRowBytes + (((col >> 3) ^ sw) << 4) + ((col >> 2) & 1) * 8;
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = j * 128 + wn * 32 + 16 * (G & 1) + 4 * (sl & 3);
    tb[j] = BKS * BM * 2 + row0 * kRowBytes + (((col >> 3) ^ sw) << 4) + ((col >> 2) & 1) * 8;
  }
  AccT<true> acc;
  zero_acc<true>(acc);
  bf16x8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto read_sub = [&](bf16x8 (&fa)[FM], bf16x8 (&fb)[FN], const bf16_t* stage, int kk) {
    const uint32_t off = kk * 16 * kRowBytes;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = tr_frag(stage, ta[i] + off, ta[i] + off + 4 * kRowBytes);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = tr_frag(stage, tb[j] + off, tb[j] + off + 4 * kRowBytes);
  };
  auto mma_sub = [&](const bf16x8 (&fa)[FM], const bf16x8 (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };
  // per step a wavefront issues 4 DMA loads (and, gathering, 2 table loads)
  constexpr int kPerStep = GATHER ? 6 : 4;
  auto sync_stage = [&]() {   // the wave's DMA of the next stage landed, then everyone's
    mem_fence_compiler();
    dma::wait_vm<kPerStep>();
    __builtin_amdgcn_s_barrier();
    mem_fence_compiler();
  };
  if constexpr (GATHER) {
    fetch(0, 0);
    fetch(1, 1);
    fetch(2, 2);
    fetch(3, 3);
  }
  issue(st0, 0, 0);
  if constexpr (GATHER) fetch(0, 4);
  issue(st1, 1, 1);
  if constexpr (GATHER) fetch(1, 5);
  issue(st2, 2, 2);
  mem_fence_compiler();
  dma::wait_vm<2 * kPerStep>();
  __builtin_amdgcn_s_barrier();
  mem_fence_compiler();
  read_sub(fa0, fb0, st0, 0);
  // step kt: stage kt % 4 current, (kt + 1) % 4 next, DMA into (kt + 3) % 4;
  // the step count is padded to a multiple of 4 with zero steps
  // (gathering: step s's table entries sit in slot s % 4; issuing step s
  // first fetches those of step s + 3, whose slot step s - 1 has freed)
  auto step = [&](int kt, int q, const bf16_t* cur, const bf16_t* nxt, bf16_t* fill) {
    read_sub(fa1, fb1, cur, 1);
    mma_sub(fa0, fb0);
    sync_stage();                   // stage kt + 1 ready; stage kt - 1 no longer read
    if constexpr (GATHER) fetch((q + 2) & 3, kt + 6);
    issue(fill, kt + 3, (q + 3) & 3);
    read_sub(fa0, fb0, nxt, 0);
    mma_sub(fa1, fb1);
  };
  const int nk4 = (nk + 3) & ~3;
  for (int kt = 0; kt < nk4; kt += 4) {
    step(kt, 0, st0, st1, st3);
    step(kt + 1, 1, st1, st2, st0);
    step(kt + 2, 2, st2, st3, st1);
    step(kt + 3, 3, st3, st0, st2);
  }
  mem_fence_compiler();
  dma::wait_vm<0>();
  __syncthreads();

  // epilogue: bf16 tile staged over the ring (rows [64 q, 64 q + 64) in stage
  // q), chunks XORed by row, then coalesced 16-byte stores of the valid part
  auto row_ptr = [&](int m) -> bf16_t* {
    const int q = m >> 6;
    bf16_t* base = (q == 0) ? st0 : (q == 1) ? st1 : (q == 2) ? st2 : st3;
    return base + (m & 63) * BN;
  };
  {
    int skey;
    asm volatile("v_mov_b32 %0, %1" : "=v"(skey) : "v"(static_cast<int>(threadIdx.x & 15)));
    for_each_quad<true>(acc, [&](int m, int n, float v0, float v1, float v2, float v3) {
      *reinterpret_cast<uint2*>(row_ptr(m) + (((n >> 3) ^ skey) << 3) + (n & 4)) =
          pack4(v0, v1, v2, v3);
    });
  }
  __syncthreads();
  const int nch = nvalid / 8;
  for (int v = tid; v < BM * (BN / 8); v += NT) {
    const int r = v / (BN / 8), c = v % (BN / 8);
    if (r >= mvalid || c >= nch) continue;
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(m0 + r) * Ndim + n0 + c * 8) =
        *reinterpret_cast<const uint4*>(row_ptr(r) + ((c ^ (r & 15)) << 3));
  }
}

// Input gradients with the big tile and 64-wide k steps (whole 128-byte lines
// of the k-contiguous A rows, as in dma_rows_kernel).  Stage = A [256 rows]
// [64 k] (128-byte rows, chunks XORed with (row >> 1) & 7) + B [64 k][256 n]
// (512-byte rows as they lie in W); two distinct stage arrays of 64 KB, the
// step count padded to even with a zero step.
template <int MODE, bool FOLD = false>
__global__ __launch_bounds__(dma64::NT, 1) void dgrad_dma_kernel(Args g) {
  using namespace dma64;
  static_assert(!FOLD || MODE == DGRAD_DOWN, "gate folded: DGRAD_DOWN");
  using dma::dma16;
  using dma::wait_vm;
  static_assert(MODE == DGRAD_DOWN || MODE == DGRAD_UP, "dgrad modes");
  constexpr int kAB = BM * BKS;   // A part of a stage (elements)
  __shared__ __attribute__((aligned(16))) bf16_t st0[kStage];
  __shared__ __attribute__((aligned(16))) bf16_t st1[kStage];

  const int flat = flat_tile();
  const int row_tile = flat / g.n_tiles_n;
  const int nt = flat - row_tile * g.n_tiles_n;
  int e, m0, mend;
  if (!find_row_tile<BM>(g.offsets, g.E, row_tile, &e, &m0, &mend)) return;
  e = __builtin_amdgcn_readfirstlane(e);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  mend = __builtin_amdgcn_readfirstlane(mend);
  const int rows = min(BM, mend - m0);
  const int d = g.d, f = g.f;
  const int n0 = nt * BN;
  const int Ndim = (MODE == DGRAD_DOWN) ? f : d;   // output columns
  const int lda = (MODE == DGRAD_DOWN) ? d : f;    // A row length
  const int ldb = Ndim;                            // B row length (element (k, n) at k ldb + n)
  const int Kh = (MODE == DGRAD_DOWN) ? d : f;     // K per half (DGRAD_UP: da then db)
  const int nk = ((MODE == DGRAD_DOWN) ? d : 2 * f) / BKS;
  const int64_t E_fd = static_cast<int64_t>(f) * d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  uint32_t voa[4], vob[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = wave * 32 + u * 8 + (lane >> 3);    // A: 8 rows of 128 B
    const int logical = (lane & 7) ^ ((row >> 1) & 7);
    if constexpr (FOLD) {   // dy rows through the table (rows past the tile read zeros)
      const uint32_t src = static_cast<uint32_t>(g.x_rows[min(m0 + row, mend - 1)]);
      voa[u] = (m0 + row < mend) ? (src * lda + logical * 8) * 2 : kOutOfRange;
    } else {
      voa[u] = (row * lda + logical * 8) * 2;
    }
    const int brow = wave * 8 + u * 2 + (lane >> 5);    // B: 2 rows of 512 B
    const int blog = (lane & 31) ^ (4 * (brow & 3));
    vob[u] = (n0 + blog * 8 < Ndim) ? static_cast<uint32_t>((brow * ldb + blog * 8) * 2)
                                    : kOutOfRange;
  }
  auto issue = [&](bf16_t* As, int kt) {
    bf16_t* Bs = As + kAB;
    const bool live = kt < nk;
    int k0 = min(kt, nk - 1) * BKS;
    int half = 0;
    if (MODE == DGRAD_UP && k0 >= f) {
      half = 1;
      k0 -= f;
    }
    const bf16_t* abase = FOLD ? g.a0 + k0
                               : ((MODE == DGRAD_UP && half) ? g.a1 : g.a0) +
                                     static_cast<int64_t>(m0) * lda + k0;
    const bf16_t* wbase = ((MODE == DGRAD_UP && half) ? g.b1 : g.b0) + e * E_fd +
                          static_cast<int64_t>(k0) * ldb + n0;
    const auto ra = rsrc_at(abase, !live ? 0 : FOLD ? g.x_bytes - k0 * 2
                                                    : ((mend - m0) * lda - k0) * 2);
    const auto rb = rsrc_at(wbase, live ? ((Kh - k0) * ldb - n0) * 2 : 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) dma16(ra, As + (wave * 32 + u * 8) * BKS, voa[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) dma16(rb, Bs + (wave * 8 + u * 2) * BN, vob[u]);
  };

  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int r = lane & 31, gq = lane >> 5;
  const int key = (r >> 1) & 7;
  uint32_t a_addr[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    a_addr[kk] = ((wm * 32 * FM + r) * BKS + (((2 * kk + gq) ^ key) * 8)) * 2;
  const int G = lane >> 4, sl = lane & 15;
  const int row0 = 8 * (G >> 1) + (sl >> 2);
  const int sw = 4 * (row0 & 3);
  uint32_t tb[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = j * 128 + wn * 32 + 16 * (G & 1) + 4 * (sl & 3);
    tb[j] = kAB * 2 + row0 * (BN * 2) + (((col >> 3) ^ sw) << 4) + ((col >> 2) & 1) * 8;
  }
  auto base_of = [](const bf16_t* st) {
    return static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const bf16_t*)st));
  };
  typedef float f32x16v __attribute__((ext_vector_type(16)));
  f32x16v c00 = {}, c01 = {}, c10 = {}, c11 = {}, c20 = {}, c21 = {}, c30 = {}, c31 = {};
  bf16x8 fa0[FM], fa1[FM], fb0[FN], fb1[FN];
  auto read_b = [&](bf16x8 (&fb)[FN], const bf16_t* st, int kk) {
    const uint32_t off = kk * 16 * (BN * 2);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = dmaw::tr_frag(st, tb[j] + off, tb[j] + off + 4 * (BN * 2));
  };
  auto read_a = [&](bf16x8 (&fa)[FM], uint32_t addr) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:0\n\t"
        "ds_read_b128 %1, %4 offset:4096\n\t"
        "ds_read_b128 %2, %4 offset:8192\n\t"
        "ds_read_b128 %3, %4 offset:12288\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(fa[0]), "=&v"(fa[1]), "=&v"(fa[2]), "=&v"(fa[3])
        : "v"(addr)
        : "memory");
  };
#define MOE_MF(c, b, a) "v_mfma_f32_32x32x16_bf16 " c ", " b ", " a ", " c "\n\t"
#define MOE_RD(o, off) "ds_read_b128 " o ", %18 offset:" off "\n\t"
  // the eight MFMAs of fragments (ain, bin) with four A fragment reads at
  // `addr` into aout interleaved; ends by waiting for the reads
  auto mma_read = [&](const bf16x8 (&ain)[FM], const bf16x8 (&bin)[FN], bf16x8 (&aout)[FM],
                      uint32_t addr) {
    asm volatile(
        MOE_RD("%8", "0")      MOE_MF("%0", "%16", "%12")
        MOE_RD("%9", "4096")   MOE_MF("%1", "%17", "%12")
        MOE_RD("%10", "8192")  MOE_MF("%2", "%16", "%13")
        MOE_RD("%11", "12288") MOE_MF("%3", "%17", "%13")
                              MOE_MF("%4", "%16", "%14")
                              MOE_MF("%5", "%17", "%14")
                              MOE_MF("%6", "%16", "%15")
                              MOE_MF("%7", "%17", "%15")
        "s_waitcnt lgkmcnt(0)"
        : "+v"(c00), "+v"(c01), "+v"(c10), "+v"(c11), "+v"(c20), "+v"(c21), "+v"(c30),
          "+v"(c31), "=&v"(aout[0]), "=&v"(aout[1]), "=&v"(aout[2]), "=&v"(aout[3])
        : "v"(ain[0]), "v"(ain[1]), "v"(ain[2]), "v"(ain[3]), "v"(bin[0]), "v"(bin[1]),
          "v"(addr)
        : "memory");
  };
#undef MOE_MF
#undef MOE_RD
  issue(st0, 0);
  issue(st1, 1);
  dmaw::mem_fence_compiler();
  wait_vm<8>();
  __builtin_amdgcn_s_barrier();
  dmaw::mem_fence_compiler();
  read_b(fb0, st0, 0);
  read_a(fa0, base_of(st0) + a_addr[0]);
  // step kt: sub-steps 0-2 of stage kt while reading 1-3 (each asm block ends
  // by waiting for every LDS read issued before it), the barrier that sees
  // step kt + 1 landed and stage kt read by everyone, the DMA of step kt + 2
  // into stage kt, then sub-step 3 while reading sub-step 0 of step kt + 1
  auto step = [&](int kt, bf16_t* cur, const bf16_t* nxt) {
    read_b(fb1, cur, 1);
    mma_read(fa0, fb0, fa1, base_of(cur) + a_addr[1]);
    read_b(fb0, cur, 2);
    mma_read(fa1, fb1, fa0, base_of(cur) + a_addr[2]);
    read_b(fb1, cur, 3);
    mma_read(fa0, fb0, fa1, base_of(cur) + a_addr[3]);
    dmaw::mem_fence_compiler();
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    dmaw::mem_fence_compiler();
    issue(cur, kt + 2);
    read_b(fb0, nxt, 0);
    mma_read(fa1, fb1, fa0, base_of(nxt) + a_addr[0]);
  };
  const int nk2 = (nk + 1) & ~1;
  for (int kt = 0; kt < nk2; kt += 2) {
    step(kt, st0, st1);
    step(kt + 1, st1, st0);
  }
  dmaw::mem_fence_compiler();
  wait_vm<0>();
  // cover the longest MFMA-to-VALU read-after-write distance
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __syncthreads();
  AccT<true> acc;
  acc[0][0] = c00; acc[0][1] = c01; acc[1][0] = c10; acc[1][1] = c11;
  acc[2][0] = c20; acc[2][1] = c21; acc[3][0] = c30; acc[3][1] = c31;

  // epilogue: bf16 tile (dh or dx) staged over the two stages, rows
  // [128 q, 128 q + 128) in stage q, chunks XORed by row; DGRAD_DOWN then
  // applies da = dh b silu'(a), db = dh silu(a) with the saved a, b
  auto row_ptr = [&](int m) -> bf16_t* { return ((m >> 7) ? st1 : st0) + (m & 127) * BN; };
  {
    int skey;
    asm volatile("v_mov_b32 %0, %1" : "=v"(skey) : "v"(static_cast<int>(threadIdx.x & 15)));
    for_each_quad<true>(acc, [&](int m, int n, float v0, float v1, float v2, float v3) {
      *reinterpret_cast<uint2*>(row_ptr(m) + (((n >> 3) ^ skey) << 3) + (n & 4)) =
          pack4(v0, v1, v2, v3);
    });
  }
  __syncthreads();
  const int nch = min(BN, Ndim - n0) / 8;
  if constexpr (FOLD) {
    // gate folded: the staged product is u = dy W2 (rounded); the row's dgate
    // part is <u, silu(a) b> over this column tile (a 32-lane sum in a fixed
    // order, row32_sum: 32 lanes hold one row), dh = g u, da = dh b silu'(a),
    // db = dh silu(a)
    static_assert(BN / 8 == 32, "one row per 32 lanes");
    // the a, b and gate loads of a group of kGrp iterations are issued before
    // any is used (the accumulators are in LDS by now, so their registers
    // hold them); the da/db stores go out in the loop, and the 32-lane sums
    // of the group's parts run together after it
    constexpr int kIt = BM * (BN / 8) / NT;
    constexpr int kGrp = 8;   // two groups per tile (all 16 at once would spill)
    static_assert(kIt % kGrp == 0, "whole groups");
    for (int i0 = 0; i0 < kIt; i0 += kGrp) {
    uint4 av[kGrp], bv[kGrp];
    float gr[kGrp];
#pragma unroll
    for (int ig = 0; ig < kGrp; ++ig) {
      const int v = tid + NT * (i0 + ig);
      const int rr = v / (BN / 8), c = v % (BN / 8);
      const int rl = min(rr, rows - 1), cl = min(c, nch - 1);   // clamped: in bounds
      const int64_t ol = static_cast<int64_t>(m0 + rl) * Ndim + n0 + cl * 8;
      av[ig] = ld_nt16(reinterpret_cast<const uint4*>(g.aux0 + ol));
      bv[ig] = ld_nt16(reinterpret_cast<const uint4*>(g.aux1 + ol));
      gr[ig] = g.gate_rows[m0 + rl];
    }
    float partv[kGrp];
#pragma unroll
    for (int ig = 0; ig < kGrp; ++ig) {
      const int v = tid + NT * (i0 + ig);
      const int rr = v / (BN / 8), c = v % (BN / 8);
      const bool ok = rr < rows && c < nch;
      const uint4 uv = *reinterpret_cast<const uint4*>(row_ptr(rr) + ((c ^ (rr & 15)) << 3));
      const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
      const uint32_t aw[4] = {av[ig].x, av[ig].y, av[ig].z, av[ig].w};
      const uint32_t bw[4] = {bv[ig].x, bv[ig].y, bv[ig].z, bv[ig].w};
      float part = 0.f;
      uint32_t daw[4], dbw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float da2[2], db2[2];
        const float uu[2] = {bf_lo(uw[q]), bf_hi(uw[q])};
        const float aa[2] = {bf_lo(aw[q]), bf_hi(aw[q])};
        const float bb[2] = {bf_lo(bw[q]), bf_hi(bw[q])};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float sg = sigmoid_f(aa[u]);
          const float sa = aa[u] * sg;   // silu(a)
          part = fmaf(uu[u], sa * bb[u], part);
          const float dh = gr[ig] * uu[u];
          da2[u] = dh * bb[u] * (sg * (1.0f + aa[u] * (1.0f - sg)));
          db2[u] = dh * sa;
        }
        daw[q] = bf_pack(da2[0], da2[1]);
        dbw[q] = bf_pack(db2[0], db2[1]);
      }
      partv[ig] = ok ? part : 0.f;
      if (ok) {
        const int64_t o = static_cast<int64_t>(m0 + rr) * Ndim + n0 + c * 8;
        *reinterpret_cast<uint4*>(g.c0 + o) = make_uint4(daw[0], daw[1], daw[2], daw[3]);
        *reinterpret_cast<uint4*>(g.c1 + o) = make_uint4(dbw[0], dbw[1], dbw[2], dbw[3]);
      }
    }
#pragma unroll
    for (int ig = 0; ig < kGrp; ++ig) partv[ig] = row32_sum(partv[ig]);
#pragma unroll
    for (int ig = 0; ig < kGrp; ++ig) {
      const int v = tid + NT * (i0 + ig);
      const int rr = v / (BN / 8), c = v % (BN / 8);
      if (c == 16 && rr < rows)   // lanes 16-31 of the row's 32 hold its sum
        g.dgate_part[static_cast<int64_t>(m0 + rr) * g.n_tiles_n + nt] = partv[ig];
    }
    }
    return;
  }
  if constexpr (MODE == DGRAD_DOWN) {
    // the saved a and b of a group of kGrp iterations are loaded before any
    // is used (clamped in bounds), as in the gate-folded epilogue above
    constexpr int kIt = BM * (BN / 8) / NT;
    constexpr int kGrp = 8;
    static_assert(kIt % kGrp == 0, "whole groups");
    for (int i0 = 0; i0 < kIt; i0 += kGrp) {
      uint4 av[kGrp], bv[kGrp];
#pragma unroll
      for (int ig = 0; ig < kGrp; ++ig) {
        const int v = tid + NT * (i0 + ig);
        const int rr = v / (BN / 8), c = v % (BN / 8);
        const int rl = min(rr, rows - 1), cl = min(c, nch - 1);   // clamped: in bounds
        const int64_t ol = static_cast<int64_t>(m0 + rl) * Ndim + n0 + cl * 8;
        av[ig] = ld_nt16(reinterpret_cast<const uint4*>(g.aux0 + ol));
        bv[ig] = ld_nt16(reinterpret_cast<const uint4*>(g.aux1 + ol));
      }
#pragma unroll
      for (int ig = 0; ig < kGrp; ++ig) {
        const int v = tid + NT * (i0 + ig);
        const int rr = v / (BN / 8), c = v % (BN / 8);
        if (rr >= rows || c >= nch) continue;
        const uint4 hv = *reinterpret_cast<const uint4*>(row_ptr(rr) + ((c ^ (rr & 15)) << 3));
        const int64_t o = static_cast<int64_t>(m0 + rr) * Ndim + n0 + c * 8;
        const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
        const uint32_t aw[4] = {av[ig].x, av[ig].y, av[ig].z, av[ig].w};
        const uint32_t bw[4] = {bv[ig].x, bv[ig].y, bv[ig].z, bv[ig].w};
        uint32_t daw[4], dbw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float da2[2], db2[2];
          const float hh[2] = {bf_lo(hw[q]), bf_hi(hw[q])};
          const float aa[2] = {bf_lo(aw[q]), bf_hi(aw[q])};
          const float bb[2] = {bf_lo(bw[q]), bf_hi(bw[q])};
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float sg = sigmoid_f(aa[u]);
            da2[u] = hh[u] * bb[u] * (sg * (1.0f + aa[u] * (1.0f - sg)));
            db2[u] = hh[u] * (aa[u] * sg);
          }
          daw[q] = bf_pack(da2[0], da2[1]);
          dbw[q] = bf_pack(db2[0], db2[1]);
        }
        *reinterpret_cast<uint4*>(g.c0 + o) = make_uint4(daw[0], daw[1], daw[2], daw[3]);
        *reinterpret_cast<uint4*>(g.c1 + o) = make_uint4(dbw[0], dbw[1], dbw[2], dbw[3]);
      }
    }
    return;
  }
  for (int v = tid; v < BM * (BN / 8); v += NT) {
    const int rr = v / (BN / 8), c = v % (BN / 8);
    if (rr >= rows || c >= nch) continue;
    const uint4 hv = *reinterpret_cast<const uint4*>(row_ptr(rr) + ((c ^ (rr & 15)) << 3));
    const int64_t o = static_cast<int64_t>(m0 + rr) * Ndim + n0 + c * 8;
    *reinterpret_cast<uint4*>(g.c0 + o) = hv;
  }
}

// Weight gradients with the small tile (128 x 128, 4 wavefronts of 64 x 64) on
// a 4-stage LDS-DMA ring, one tile per workgroup: the same scheme as
// wgrad_dma_kernel at half the width (256-byte rows: a DMA instruction fills
// four rows; the 16 chunks of a row are XORed with 4 (row & 3)).
namespace dmas {
constexpr int BM = 128, BN = 128, BKS = 32, NT = 256, WAVES_N = 2, FM = 2, FN = 2;
constexpr int kHalf = BKS * BM;              // elements of the A (or B) part
constexpr int kStage = 2 * kHalf;            // 16 KB
constexpr int kRowBytes = BM * 2;            // 256
}  // namespace dmas

// NST = 4 (64 KB, two workgroups per CU) or 8 (128 KB, one workgroup per CU,
// for grids that give each CU at most one tile: twice the loads in flight).
// GATHER: the x operand of dW1 and dW3 (B of z = 1, 2) is read from X through
// the gather table; the table entries of a step's rows are loaded NST - 1
// steps before its DMA is issued (a register ring, one slot per stage), so
// waiting for them never waits for DMA still meant to be in flight.
template <int NST, bool GATHER, bool FOLD_A = false>
__global__ __launch_bounds__(dmas::NT, 8 / NST) void wgrad_dma_small_kernel(Args g,
                                                                          int32_t tiles_per_expert) {
  using namespace dmas;
  static_assert(NST == 4 || NST == 8, "4 or 8 stages");
  constexpr int kX = NST == 8 ? kStage : 8;   // stages 4-7 exist only with NST = 8
  __shared__ __attribute__((aligned(16))) bf16_t st0[kStage];
  __shared__ __attribute__((aligned(16))) bf16_t st1[kStage];
  __shared__ __attribute__((aligned(16))) bf16_t st2[kStage];
  __shared__ __attribute__((aligned(16))) bf16_t st3[kStage];
  __shared__ __attribute__((aligned(16))) bf16_t st4[kX];
  __shared__ __attribute__((aligned(16))) bf16_t st5[kX];
  __shared__ __attribute__((aligned(16))) bf16_t st6[kX];
  __shared__ __attribute__((aligned(16))) bf16_t st7[kX];

  // item order: the dW2 tiles, then the dW1 and dW3 tiles of each (e, tile) as
  // adjacent items, so both read the same x rows on one XCD at the same time
  const int flat = flat_tile();
  const int per_z = g.E * tiles_per_expert;
  if (flat >= 3 * per_z) return;
  const int z = flat < per_z ? 0 : 1 + ((flat - per_z) & 1);
  const int rem = flat < per_z ? flat : (flat - per_z) >> 1;
  const int e = rem / tiles_per_expert, t = rem % tiles_per_expert;
  const int d = g.d, f = g.f;
  const int Mdim = (z == 0) ? d : f, Ndim = (z == 0) ? f : d;
  const int tiles_n = (Ndim + BN - 1) / BN;
  const int m0 = (t / tiles_n) * BM, n0 = (t % tiles_n) * BN;
  if (m0 >= Mdim) return;
  const bf16_t* Asrc = (z == 0) ? g.a0 : (z == 1 ? g.a1 : g.aux0);
  const bf16_t* Bsrc = (z == 0) ? g.b0 : g.b1;
  bf16_t* dst = ((z == 0) ? g.c0 : (z == 1 ? g.c1 : g.c2)) + static_cast<int64_t>(e) * d * f;
  const int p0 = g.offsets[e], p1 = g.offsets[e + 1];
  const int nk = (p1 - p0 + BKS - 1) / BKS;
  const int mvalid = min(BM, Mdim - m0), nvalid = min(BN, Ndim - n0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (nk == 0) {
    for (int v = tid; v < BM * (BN / 8); v += NT) {
      const int r = v / (BN / 8), c = v % (BN / 8);
      if (r < mvalid && c * 8 < nvalid)
        *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(m0 + r) * Ndim + n0 + c * 8) =
            make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }
  // DMA: wavefront w fills rows 8 w .. 8 w + 7 of A and of B, four rows per
  // instruction; lane l -> row + l / 16, physical chunk l % 16
  uint32_t voa[2], vob[2];
  int acol[2], bcol[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = wave * 8 + u * 4 + (lane >> 4);
    const int logical = (lane & 15) ^ (4 * (row & 3));
    const int col = logical * 8;
    voa[u] = (m0 + col < Mdim) ? static_cast<uint32_t>((row * Mdim + col) * 2) : kOutOfRange;
    vob[u] = (n0 + col < Ndim) ? static_cast<uint32_t>((row * Ndim + col) * 2) : kOutOfRange;
    acol[u] = (m0 + col < Mdim) ? col : -1;
    bcol[u] = (n0 + col < Ndim) ? col : -1;
  }
  const bool gz = GATHER && z != 0;                 // B rows gathered from X
  const bool ga = FOLD_A && z == 0;   // A rows (dy) gathered from dY [T, d]
  int32_t xs[NST][2];                 // table entries of the rows of step s in slot s % NST
  auto fetch = [&](int slot, int kt) {
    const int pb = p0 + kt * BKS;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      xs[slot][u] = g.x_rows[min(pb + wave * 8 + u * 4 + (lane >> 4), p1 - 1)];
  };
  auto issue = [&](bf16_t* As, int kt, int slot) {
    bf16_t* Bs = As + kHalf;
    const bool live = kt < nk;
    const int p = p0 + min(kt, nk - 1) * BKS;
    const auto ra = (FOLD_A && ga) ? rsrc_at(Asrc + m0, live ? g.x_bytes - m0 * 2 : 0)
                                   : rsrc_at(Asrc + static_cast<int64_t>(p) * Mdim + m0,
                                             live ? ((p1 - p) * Mdim - m0) * 2 : 0);
    uint32_t va[2] = {voa[0], voa[1]};
    uint32_t vb[2] = {vob[0], vob[1]};
    __amdgpu_buffer_rsrc_t rb;
    if constexpr (GATHER) {
      if (FOLD_A && ga) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int q = kt * BKS + wave * 8 + u * 4 + (lane >> 4);   // row of the expert
          va[u] = (p0 + q < p1 && acol[u] >= 0)
                      ? (static_cast<uint32_t>(xs[slot][u]) * Mdim + acol[u]) * 2
                      : kOutOfRange;
        }
      }
      rb = gz ? rsrc_at(Bsrc + n0, live ? g.x_bytes - n0 * 2 : 0)
              : rsrc_at(Bsrc + static_cast<int64_t>(p) * Ndim + n0,
                        live ? ((p1 - p) * Ndim - n0) * 2 : 0);
      if (gz) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int q = kt * BKS + wave * 8 + u * 4 + (lane >> 4);   // row of the expert
          vb[u] = (p0 + q < p1 && bcol[u] >= 0)
                      ? (static_cast<uint32_t>(xs[slot][u]) * Ndim + bcol[u]) * 2
                      : kOutOfRange;
        }
      }
    } else {
      rb = rsrc_at(Bsrc + static_cast<int64_t>(p) * Ndim + n0,
                   live ? ((p1 - p) * Ndim - n0) * 2 : 0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) dma::dma16(ra, As + (wave * 8 + u * 4) * BM, va[u]);
#pragma unroll
    for (int u = 0; u < 2; ++u) dma::dma16(rb, Bs + (wave * 8 + u * 4) * BN, vb[u]);
  };
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int G = lane >> 4, sl = lane & 15;
  const int row0 = 8 * (G >> 1) + (sl >> 2);
  const int sw = 4 * (row0 & 3);
  uint32_t ta[FM], tb[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int col = wm * 64 + i * 32 + 16 * (G & 1) + 4 * (sl & 3);
    ta[i] = row0 * kRowBytes + (((col >> 3) ^ sw) << 4) + ((col >> 2) & 1) * 8;
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = j * 64 + wn * 32 + 16 * (G & 1) + 4 * (sl & 3);
    tb[j] = kHalf * 2 + row0 * kRowBytes + (((col >> 3) ^ sw) << 4) + ((col >> 2) & 1) * 8;
  }
  AccT<false> acc;
  zero_acc<false>(acc);
  bf16x8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto read_sub = [&](bf16x8 (&fa)[FM], bf16x8 (&fb)[FN], const bf16_t* stage, int kk) {
    const uint32_t off = kk * 16 * kRowBytes;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = dmaw::tr_frag(stage, ta[i] + off, ta[i] + off + 4 * kRowBytes);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[j] = dmaw::tr_frag(stage, tb[j] + off, tb[j] + off + 4 * kRowBytes);
  };
  auto mma_sub = [&](const bf16x8 (&fa)[FM], const bf16x8 (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };
  // each wavefront issues 4 loads per step.  At the barrier of step kt the
  // loads of steps kt + 1 .. kt + NST - 2 are outstanding and step kt + 1 must
  // have landed: NST - 3 steps may stay in flight
  auto sync_stage = [&]() {
    dmaw::mem_fence_compiler();
    dma::wait_vm<(4 + (GATHER ? 2 : 0)) * (NST - 3)>();
    __builtin_amdgcn_s_barrier();
    dmaw::mem_fence_compiler();
  };
  bf16_t* const stg[8] = {st0, st1, st2, st3, st4, st5, st6, st7};
  if constexpr (GATHER) {
    // table entries of steps 0 .. NST - 2 now; each issue of step s fetches
    // those of step s + NST - 1 (before its own DMA)
#pragma unroll
    for (int q = 0; q < NST - 1; ++q) fetch(q, q);
  }
#pragma unroll
  for (int q = 0; q < NST - 1; ++q) {
    if constexpr (GATHER) fetch((q + NST - 1) % NST, q + NST - 1);
    issue(stg[q], q, q);
  }
  dmaw::mem_fence_compiler();
  dma::wait_vm<(4 + (GATHER ? 2 : 0)) * (NST - 2)>();   // step 0 has landed
  __builtin_amdgcn_s_barrier();
  dmaw::mem_fence_compiler();
  read_sub(fa0, fb0, st0, 0);
  auto step = [&](int kt, int q, const bf16_t* cur, const bf16_t* nxt, bf16_t* fill) {
    read_sub(fa1, fb1, cur, 1);
    mma_sub(fa0, fb0);
    sync_stage();
    const int t = kt + NST - 1;   // the step whose DMA this issues, slot (q + NST - 1) % NST
    if constexpr (GATHER) fetch((q + NST - 2) % NST, t + NST - 1);
    issue(fill, t, (q + NST - 1) % NST);
    read_sub(fa0, fb0, nxt, 0);
    mma_sub(fa1, fb1);
  };
  const int nkp = (nk + NST - 1) / NST * NST;
  for (int kt = 0; kt < nkp; kt += NST) {
#pragma unroll
    for (int q = 0; q < NST; ++q)
      step(kt + q, q, stg[q], stg[(q + 1) % NST], stg[(q + NST - 1) % NST]);
  }
  dmaw::mem_fence_compiler();
  dma::wait_vm<0>();
  __syncthreads();
  // epilogue: bf16 tile staged over stages 0-1 (rows [64 q, 64 q + 64) in stage
  // q), chunks XORed by row, then coalesced 16-byte stores of the valid part
  auto row_ptr = [&](int m) -> bf16_t* { return ((m >> 6) ? st1 : st0) + (m & 63) * BN; };
  {
    int skey;
    asm volatile("v_mov_b32 %0, %1" : "=v"(skey) : "v"(static_cast<int>(threadIdx.x & 15)));
    for_each_quad<false>(acc, [&](int m, int n, float v0, float v1, float v2, float v3) {
      *reinterpret_cast<uint2*>(row_ptr(m) + (((n >> 3) ^ skey) << 3) + (n & 4)) =
          pack4(v0, v1, v2, v3);
    });
  }
  __syncthreads();
  const int nch = nvalid / 8;
  for (int v = tid; v < BM * (BN / 8); v += NT) {
    const int r = v / (BN / 8), c = v % (BN / 8);
    if (r >= mvalid || c >= nch) continue;
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(m0 + r) * Ndim + n0 + c * 8) =
        *reinterpret_cast<const uint4*>(row_ptr(r) + ((c ^ (r & 15)) << 3));
  }
}

// Weight gradients with the small tile, persistent (same pipeline as the row
// modes).  Items are (z, expert, tile, split), dealt like the row items; item
// K ranges follow the expert's row count.  A workgroup first decodes its
// items: those whose K range is empty write a zero tile (or zero partial)
// straight away, the rest run through the stream.  Both operands are
// m/n-contiguous ([rows p][M] and [rows p][N]) and go through buffer loads
// (rows past the split's end and columns past the matrix edge read zeros) and
// the in-register transpose.  splits == 1: the bf16 tile is staged through
// the consumed LDS buffer and stored in 16-byte chunks; splits > 1: the fp32
// partial tile goes out from the accumulators for wgrad_reduce_kernel.
struct WgSched {
  int4 d0[kMaxItems];   // z, e, m0, n0
  int4 d1[kMaxItems];   // first row, end row, K steps, tile | split << 16
  int n, S;
};

// GATHER: the x operand of dW1 and dW3 (B of z = 1, 2) is read from X through
// the gather table (each step loads the table entries of its rows first;
// this kernel serves only the small tile counts that need split K).
template <bool GATHER>
__global__ __launch_bounds__(Cfg<false>::THREADS, 2) void wgrad_stream_kernel(
    Args g, int32_t tiles_per_expert, int32_t splits, float* partial) {
  constexpr bool BIG = false;
  typedef Cfg<BIG> C;
  constexpr int BM = C::BM, BN = C::BN, NT = C::THREADS;
  constexpr int MA = BM * 2 / NT, MBn = BN * 2 / NT;   // 4 x 8 blocks per thread
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * (BM + BN) * BK];
  __shared__ WgSched sched;
  __shared__ int4 cand0[kMaxItems], cand1[kMaxItems];

  const int d = g.d, f = g.f, E = g.E;
  const int G = gridDim.x, flat = flat_tile();
  const int per_z = E * tiles_per_expert * splits;
  const int total = 3 * per_z;
  const int n_cand = flat < total ? min((total - flat + G - 1) / G, kMaxItems) : 0;
  for (int t = threadIdx.x; t < n_cand; t += NT) {
    const int it = flat + t * G;
    const int z = it / per_z;
    int rem = it - z * per_z;
    const int e = rem / (tiles_per_expert * splits);
    rem -= e * tiles_per_expert * splits;
    const int tile = rem / splits, sp = rem - tile * splits;
    const int Mdim = (z == 0) ? d : f, Ndim = (z == 0) ? f : d;
    const int tiles_n = (Ndim + BN - 1) / BN;
    const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
    const int p0 = g.offsets[e], p1 = g.offsets[e + 1];
    const int nk_all = (p1 - p0 + BK - 1) / BK;
    const int per_split = (nk_all + splits - 1) / splits;
    const int kt0 = min(nk_all, sp * per_split), kt1 = min(nk_all, kt0 + per_split);
    // m0 >= Mdim: no such tile for this z (tiles_per_expert is the max over z)
    cand0[t] = make_int4(m0 < Mdim ? z : -1, e, m0, n0);
    cand1[t] = make_int4(p0 + kt0 * BK, min(p1, p0 + kt1 * BK), kt1 - kt0, tile | (sp << 16));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0, S = 0;
    for (int t = 0; t < n_cand; ++t) {
      if (cand0[t].x < 0 || cand1[t].z == 0) continue;
      sched.d0[n] = cand0[t];
      sched.d1[n] = cand1[t];
      S += cand1[t].z;
      ++n;
    }
    sched.n = n;
    sched.S = S;
  }
  // items with an empty K range: zero output
  for (int t = 0; t < n_cand; ++t) {
    const int4 c0 = cand0[t], c1 = cand1[t];
    if (c0.x < 0 || c1.z != 0) continue;
    const int z = c0.x, e = c0.y, m0 = c0.z, n0 = c0.w;
    const int Mdim = (z == 0) ? d : f, Ndim = (z == 0) ? f : d;
    if (splits > 1) {
      float* dst = partial +
                   ((static_cast<int64_t>(z) * E + e) * tiles_per_expert + (c1.w & 0xFFFF)) *
                       static_cast<int64_t>(splits) * (BM * BN) +
                   static_cast<int64_t>(c1.w >> 16) * (BM * BN);
      for (int v = threadIdx.x; v < BM * BN / 4; v += NT)
        reinterpret_cast<float4*>(dst)[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    } else if (g.out_f32) {
      float* dst = reinterpret_cast<float*>((z == 0) ? g.c0 : (z == 1 ? g.c1 : g.c2)) +
                   static_cast<int64_t>(e) * d * f;
      const int mv = min(BM, Mdim - m0), nv4 = min(BN, Ndim - n0) / 4;
      for (int v = threadIdx.x; v < BM * (BN / 4); v += NT) {
        const int r = v / (BN / 4), c = v % (BN / 4);
        if (r < mv && c < nv4)
          *reinterpret_cast<float4*>(dst + static_cast<int64_t>(m0 + r) * Ndim + n0 + c * 4) =
              make_float4(0.f, 0.f, 0.f, 0.f);
      }
    } else {
      bf16_t* dst = ((z == 0) ? g.c0 : (z == 1 ? g.c1 : g.c2)) + static_cast<int64_t>(e) * d * f;
      const int mv = min(BM, Mdim - m0), nv8 = min(BN, Ndim - n0) / 8;
      for (int v = threadIdx.x; v < BM * (BN / 8); v += NT) {
        const int r = v / (BN / 8), c = v % (BN / 8);
        if (r < mv && c < nv8)
          *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(m0 + r) * Ndim + n0 + c * 8) =
              make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  __syncthreads();
  const int n_items = sched.n;
  if (n_items == 0) return;

  AccT<BIG> acc;
  zero_acc<BIG>(acc);
  constexpr int NSETS = kWgradSets;
  MPart<BM, NT> pa[NSETS];
  MPart<BN, NT> pb[NSETS];
  uint32_t voff_a[MA], voff_b[MBn];
  int p_item = -1, p_z = 0, p_m0 = 0, p_n0 = 0, p_pb = 0, p_pe = 0;
  auto prep = [&](int item) {
    const int4 a = sched.d0[item], b = sched.d1[item];
    p_z = __builtin_amdgcn_readfirstlane(a.x);
    p_m0 = __builtin_amdgcn_readfirstlane(a.z);
    p_n0 = __builtin_amdgcn_readfirstlane(a.w);
    p_pb = __builtin_amdgcn_readfirstlane(b.x);
    p_pe = __builtin_amdgcn_readfirstlane(b.y);
    const int Mdim = (p_z == 0) ? d : f, Ndim = (p_z == 0) ? f : d;
#pragma unroll
    for (int i = 0; i < MA; ++i) {
      int jb, kq;
      mblock<NT>(i, &jb, &kq);
      voff_a[i] = (p_m0 + jb * 8 < Mdim) ? static_cast<uint32_t>((kq * 4 * Mdim + jb * 8) * 2)
                                         : kOutOfRange;
    }
#pragma unroll
    for (int i = 0; i < MBn; ++i) {
      int jb, kq;
      mblock<NT>(i, &jb, &kq);
      voff_b[i] = (p_n0 + jb * 8 < Ndim) ? static_cast<uint32_t>((kq * 4 * Ndim + jb * 8) * 2)
                                         : kOutOfRange;
    }
  };
  auto nk_of = [&](int item) { return sched.d1[item].z; };
  auto load = [&](int item, int kt, auto set_c) {
    constexpr int set = decltype(set_c)::value;
    const int Mdim = (p_z == 0) ? d : f, Ndim = (p_z == 0) ? f : d;
    const bf16_t* Asrc = (p_z == 0) ? g.a0 : (p_z == 1 ? g.a1 : g.aux0);
    const bf16_t* Bsrc = (p_z == 0) ? g.b0 : g.b1;
    const int p = p_pb + kt * BK;
    const auto ra = rsrc_at(Asrc + static_cast<int64_t>(p) * Mdim + p_m0,
                            ((p_pe - p) * Mdim - p_m0) * 2);
#pragma unroll
    for (int i = 0; i < MA; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) pa[set].v[i][r] = bload(ra, voff_a[i] + r * Mdim * 2);
    if (GATHER && p_z != 0) {
      // rows p + 4 kq + r of the expert are X rows x_rows[...]; past p_pe: zero
      int kq, jb;
      mblock<NT>(0, &jb, &kq);
      int32_t xr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) xr[r] = g.x_rows[min(p + 4 * kq + r, p_pe - 1)];
      const auto rb = rsrc_at(Bsrc + p_n0, g.x_bytes - p_n0 * 2);
#pragma unroll
      for (int i = 0; i < MBn; ++i) {
        mblock<NT>(i, &jb, &kq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t vo = (p + 4 * kq + r < p_pe && voff_b[i] != kOutOfRange)
                                  ? (static_cast<uint32_t>(xr[r]) * Ndim + jb * 8) * 2
                                  : kOutOfRange;
          pb[set].v[i][r] = bload(rb, vo);
        }
      }
    } else {
      const auto rb = rsrc_at(Bsrc + static_cast<int64_t>(p) * Ndim + p_n0,
                              ((p_pe - p) * Ndim - p_n0) * 2);
#pragma unroll
      for (int i = 0; i < MBn; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[set].v[i][r] = bload(rb, voff_b[i] + r * Ndim * 2);
    }
  };
  auto store = [&](auto set_c, bf16_t* As, bf16_t* Bs) {
    constexpr int set = decltype(set_c)::value;
    mstore_raw<BM, NT>(pa[set], As);
    mstore_raw<BN, NT>(pb[set], Bs);
  };
  auto epilogue = [&](int item, bf16_t* buf) {
    const int4 a = sched.d0[item], b = sched.d1[item];
    const int z = a.x, e = a.y, m0 = a.z, n0 = a.w;
    const int Mdim = (z == 0) ? d : f, Ndim = (z == 0) ? f : d;
    if (splits > 1) {
      float* dst = partial +
                   ((static_cast<int64_t>(z) * E + e) * tiles_per_expert + (b.w & 0xFFFF)) *
                       static_cast<int64_t>(splits) * (BM * BN) +
                   static_cast<int64_t>(b.w >> 16) * (BM * BN);
      for_each_quad<BIG>(acc, [&](int m, int n, float v0, float v1, float v2, float v3) {
        *reinterpret_cast<float4*>(dst + m * BN + n) = make_float4(v0, v1, v2, v3);
      });
      return;
    }
    if (g.out_f32) {   // fp32 weight gradients: straight from the accumulators
      float* dst = reinterpret_cast<float*>((z == 0) ? g.c0 : (z == 1 ? g.c1 : g.c2)) +
                   static_cast<int64_t>(e) * d * f;
      const int mv = min(BM, Mdim - m0), nv = min(BN, Ndim - n0);
      for_each_quad<BIG>(acc, [&](int m, int n, float v0, float v1, float v2, float v3) {
        if (m < mv && n < nv)
          *reinterpret_cast<float4*>(dst + static_cast<int64_t>(m0 + m) * Ndim + n0 + n) =
              make_float4(v0, v1, v2, v3);
      });
      return;
    }
    int key;
    asm volatile("v_mov_b32 %0, %1" : "=v"(key) : "v"(static_cast<int>(threadIdx.x & 15)));
    for_each_quad<BIG>(acc, [&](int m, int n, float v0, float v1, float v2, float v3) {
      *reinterpret_cast<uint2*>(buf + m * BN + (((n >> 3) ^ key) << 3) + (n & 4)) =
          pack4(v0, v1, v2, v3);
    });
    __syncthreads();
    bf16_t* dst = ((z == 0) ? g.c0 : (z == 1 ? g.c1 : g.c2)) + static_cast<int64_t>(e) * d * f;
    const int mv = min(BM, Mdim - m0), nv8 = min(BN, Ndim - n0) / 8;
    constexpr int CH = BN / 8;
#pragma unroll
    for (int it = 0; it < BM * CH / NT; ++it) {
      const int v = threadIdx.x + NT * it;
      const int r = v / CH, c = v % CH;
      if (r >= mv || c >= nv8) continue;
      *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(m0 + r) * Ndim + n0 + c * 8) =
          *reinterpret_cast<const uint4*>(buf + r * BN + ((c ^ (r & 15)) << 3));
    }
    __syncthreads();
  };
  auto prep_if = [&](int item) {
    if (item != p_item) {
      prep(item);
      p_item = item;
    }
  };
  run_stream<BIG, NSETS, (MA + MBn) * 4, (MA + MBn) * 8>(acc, lds, n_items, sched.S, nk_of,
                                                         prep_if, load, store, epilogue);
}

// Adds the split-K partial tiles in split order and rounds once to bf16 (or
// stores the fp32 sum when the weight gradients are fp32).
// One thread per 8 consecutive outputs of a tile row (small tiles only).
__global__ __launch_bounds__(kThreads) void wgrad_reduce_kernel(Args g, int32_t tiles_per_expert,
                                                                int32_t splits,
                                                                const float* partial) {
  constexpr int BM = Cfg<false>::BM, BN = Cfg<false>::BN;
  const int64_t chunk = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per_tile = BM * BN / 8;
  const int64_t tile_id = chunk / per_tile;
  if (tile_id >= 3LL * g.E * tiles_per_expert) return;
  const int within = static_cast<int>(chunk - tile_id * per_tile);
  const int r = within / (BN / 8), c = (within % (BN / 8)) * 8;
  const int z = static_cast<int>(tile_id / (static_cast<int64_t>(g.E) * tiles_per_expert));
  const int rem = static_cast<int>(tile_id - static_cast<int64_t>(z) * g.E * tiles_per_expert);
  const int e = rem / tiles_per_expert, t = rem % tiles_per_expert;
  const int d = g.d, f = g.f;
  const int Mdim = (z == 0) ? d : f;
  const int Ndim = (z == 0) ? f : d;
  const int tiles_n = (Ndim + BN - 1) / BN;
  const int m0 = (t / tiles_n) * BM, n0 = (t % tiles_n) * BN;
  if (m0 + r >= Mdim || n0 + c >= Ndim) return;
  const float* src = partial + tile_id * splits * static_cast<int64_t>(BM * BN) + r * BN + c;
  float v[8];
  {
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  for (int s = 1; s < splits; ++s) {
    const float* q = src + static_cast<int64_t>(s) * (BM * BN);
    const float4 a = *reinterpret_cast<const float4*>(q);
    const float4 b = *reinterpret_cast<const float4*>(q + 4);
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
    v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
  }
  const int64_t at = static_cast<int64_t>(e) * d * f + static_cast<int64_t>(m0 + r) * Ndim + n0 + c;
  bf16_t* const out = (z == 0) ? g.c0 : (z == 1 ? g.c1 : g.c2);
  if (g.out_f32) {
    float* dst = reinterpret_cast<float*>(out) + at;
    reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
    return;
  }
  *reinterpret_cast<uint4*>(out + at) =
      make_uint4(bf_pack(v[0], v[1]), bf_pack(v[2], v[3]), bf_pack(v[4], v[5]), bf_pack(v[6], v[7]));
}

template <bool BIG>
int wgrad_tiles_per_expert(const moe_dims& dm) {
  constexpr int BM = Cfg<BIG>::BM, BN = Cfg<BIG>::BN;
  const int tiles = ((dm.d + BM - 1) / BM) * ((dm.f + BN - 1) / BN);
  const int tiles_t = ((dm.f + BM - 1) / BM) * ((dm.d + BN - 1) / BN);
  return std::max(tiles, tiles_t);
}

unsigned pad8(int64_t n) { return static_cast<unsigned>((n + kXcd - 1) / kXcd * kXcd); }

// grid of the big weight-gradient kernel: ceil(3 E / 8) snake rounds of tpe
// tiles on each of the 8 XCDs
unsigned wgrad_snake_grid(int E, int tpe) {
  return static_cast<unsigned>((3LL * E + kXcd - 1) / kXcd * kXcd * tpe);
}

constexpr int kCUs = 256;

// Big tiles for long reductions (K >= 1024: the matrix cores, not the memory
// ramp, bound the tile) when they alone give at least two workgroups per CU
// (and, for UP, f splits into 128-column halves); otherwise the small tile.
bool use_big_rows(const moe_dims& dm, int n_big, int K) {
  const int64_t R = dm.T * dm.k;
  return K >= 1024 && (R / 256) * n_big >= 2 * kCUs && dm.f % 128 == 0;
}
bool use_big_wgrad(const moe_dims& dm) {
  return 3LL * dm.E * wgrad_tiles_per_expert<true>(dm) >= 2 * kCUs;
}

// Small tile: persistent grid of the workgroups resident at once (two per
// CU), fewer when there are fewer items, more when a workgroup would otherwise
// hold over kMaxItems of them.  Big tile: one workgroup per tile.
template <int MODE>
hipError_t launch_rows_small(const Args& base, int64_t R, int E, int n_tiles_n, hipStream_t s) {
  Args g = base;
  g.n_tiles_n = n_tiles_n;
  const int64_t row_tiles = (R + Cfg<false>::BM - 1) / Cfg<false>::BM + E;  // >= sum_e ceil(M_e/BM)
  const int64_t items = row_tiles * n_tiles_n;
  const int64_t slots = 2 * static_cast<int64_t>(kCUs);
  const int64_t grid = std::max(std::min(items, slots), (items + kMaxItems - 1) / kMaxItems);
  g.grid_pad = static_cast<int32_t>(pad8(grid));
  if constexpr (MODE == UP || MODE == DGRAD_DOWN) {
    if (g.gate_rows) {   // gate folded (gathered rows)
      hipLaunchKernelGGL((rows_kernel<MODE, false, true, true>), dim3(g.grid_pad),
                         dim3(Cfg<false>::THREADS), 0, s, g);
      return hipGetLastError();
    }
  }
  if constexpr (MODE == UP) {
    if (g.x_rows) {
      hipLaunchKernelGGL((rows_kernel<MODE, false, true>), dim3(g.grid_pad),
                         dim3(Cfg<false>::THREADS), 0, s, g);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((rows_kernel<MODE, false>), dim3(g.grid_pad), dim3(Cfg<false>::THREADS), 0,
                     s, g);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_rows_big(const Args& base, int64_t R, int E, int n_tiles_n, hipStream_t s) {
  // gate folded (UP, DGRAD_DOWN): the FOLD instances; a gathered dgrad
  // operand exists only with the gate folded
  const bool fold = base.gate_rows != nullptr;
  if (fold && !(MODE == UP || MODE == DGRAD_DOWN)) return hipErrorNotSupported;
  if (!fold && MODE == DGRAD_DOWN && base.x_rows) return hipErrorNotSupported;
  Args g = base;
  g.n_tiles_n = n_tiles_n;
  const int64_t row_tiles = (R + Cfg<true>::BM - 1) / Cfg<true>::BM + E;
  g.grid_pad = static_cast<int32_t>(pad8(row_tiles * n_tiles_n));
  if constexpr (MODE == UP || MODE == DOWN) {
    if constexpr (MODE == UP) {
      if (fold) {
        hipLaunchKernelGGL((dma_rows_kernel<MODE, true>), dim3(g.grid_pad), dim3(dma64::NT), 0,
                           s, g);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((dma_rows_kernel<MODE>), dim3(g.grid_pad), dim3(dma64::NT), 0, s, g);
  } else {
    if constexpr (MODE == DGRAD_DOWN) {
      if (fold) {
        hipLaunchKernelGGL((dgrad_dma_kernel<MODE, true>), dim3(g.grid_pad), dim3(dma64::NT), 0,
                           s, g);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((dgrad_dma_kernel<MODE>), dim3(g.grid_pad), dim3(dma64::NT), 0, s, g);
  }
  return hipGetLastError();
}

// n_cols: the N extent of the mode (UP: f, covered in halves of BN/2); K: its
// reduction length
template <int MODE>
hipError_t launch_rows(const Args& g, const moe_dims& dm, int n_cols, int K, hipStream_t s) {
  const int64_t R = dm.T * dm.k;
  const int n_big = (MODE == UP) ? n_cols / 128 : (n_cols + 255) / 256;
  if (use_big_rows(dm, n_big, K)) return launch_rows_big<MODE>(g, R, dm.E, n_big, s);
  const int n_small = (MODE == UP) ? n_cols / 64 : (n_cols + 127) / 128;
  return launch_rows_small<MODE>(g, R, dm.E, n_small, s);
}

Args base_args(const moe_dims& dm, const int32_t* offsets) {
  Args g{};
  g.offsets = offsets;
  g.E = dm.E;
  g.d = dm.d;
  g.f = dm.f;
  return g;
}

}  // namespace

hipError_t launch_up_bf16(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                          const int32_t* offsets, const void* w1, const void* w3, void* a,
                          void* b, void* h, hipStream_t s) {
  Args g = base_args(dm, offsets);
  g.a0 = static_cast<const bf16_t*>(x_perm);
  g.x_rows = x_rows;
  g.x_bytes = static_cast<int32_t>(dm.T * dm.d * 2);
  g.b0 = static_cast<const bf16_t*>(w1);
  g.b1 = static_cast<const bf16_t*>(w3);
  g.c0 = static_cast<bf16_t*>(a);
  g.c1 = static_cast<bf16_t*>(b);
  g.c2 = static_cast<bf16_t*>(h);
  return launch_rows<UP>(g, dm, dm.f, dm.d, s);
}

hipError_t launch_down_bf16(const moe_dims& dm, const void* h, const int32_t* offsets,
                            const void* w2, void* y, hipStream_t s) {
  Args g = base_args(dm, offsets);
  g.a0 = static_cast<const bf16_t*>(h);
  g.b0 = static_cast<const bf16_t*>(w2);
  g.c0 = static_cast<bf16_t*>(y);
  return launch_rows<DOWN>(g, dm, dm.d, dm.f, s);
}

hipError_t launch_dgrad_down_bf16(const moe_dims& dm, const void* dy_perm, const int32_t* offsets,
                                  const void* w2, const void* a, const void* b, void* da,
                                  void* db, hipStream_t s) {
  Args g = base_args(dm, offsets);
  g.a0 = static_cast<const bf16_t*>(dy_perm);
  g.b0 = static_cast<const bf16_t*>(w2);
  g.aux0 = static_cast<const bf16_t*>(a);
  g.aux1 = static_cast<const bf16_t*>(b);
  g.c0 = static_cast<bf16_t*>(da);
  g.c1 = static_cast<bf16_t*>(db);
  return launch_rows<DGRAD_DOWN>(g, dm, dm.f, dm.d, s);
}

hipError_t launch_dgrad_up_bf16(const moe_dims& dm, const void* da, const void* db,
                                const int32_t* offsets, const void* w1, const void* w3,
                                void* dx_perm, hipStream_t s) {
  Args g = base_args(dm, offsets);
  g.a0 = static_cast<const bf16_t*>(da);
  g.a1 = static_cast<const bf16_t*>(db);
  g.b0 = static_cast<const bf16_t*>(w1);
  g.b1 = static_cast<const bf16_t*>(w3);
  g.c0 = static_cast<bf16_t*>(dx_perm);
  return launch_rows<DGRAD_UP>(g, dm, dm.d, 2 * dm.f, s);
}

hipError_t launch_wgrad_bf16(const moe_dims& dm, const void* x_perm, const int32_t* x_rows,
                             const int32_t* offsets, const void* h, const void* dy_perm,
                             const void* da, const void* db, void* dw1, void* dw3, void* dw2,
                             bool out_f32, float* partial, hipStream_t s) {
  Args g = base_args(dm, offsets);
  g.out_f32 = out_f32 ? 1 : 0;
  g.x_rows = x_rows;
  g.x_bytes = static_cast<int32_t>(dm.T * dm.d * 2);
  g.a0 = static_cast<const bf16_t*>(dy_perm);   // z = 0: A = dy (m over d), B = h (n over f)
  g.b0 = static_cast<const bf16_t*>(h);
  g.a1 = static_cast<const bf16_t*>(da);        // z = 1: A = da (m over f), B = x (n over d)
  g.aux0 = static_cast<const bf16_t*>(db);      // z = 2: A = db (m over f), B = x (n over d)
  g.b1 = static_cast<const bf16_t*>(x_perm);
  g.c0 = static_cast<bf16_t*>(dw2);
  g.c1 = static_cast<bf16_t*>(dw1);
  g.c2 = static_cast<bf16_t*>(dw3);
  // fp32 weight gradients go through the persistent stream kernel (its
  // epilogue and the split-K reduction store fp32), never the one-pass
  // direct-to-LDS kernels, whose epilogues stage bf16 tiles
  if (!out_f32 && use_big_wgrad(dm)) {
    const int tpe = wgrad_tiles_per_expert<true>(dm);
    const unsigned grid = wgrad_snake_grid(dm.E, tpe);
    g.grid_pad = static_cast<int32_t>(grid);
    if (g.x_rows)
      hipLaunchKernelGGL((wgrad_dma_kernel<true>), dim3(grid), dim3(dmaw::NT), 0, s, g, tpe);
    else
      hipLaunchKernelGGL((wgrad_dma_kernel<false>), dim3(grid), dim3(dmaw::NT), 0, s, g, tpe);
    return hipGetLastError();
  }
  const int tpe = wgrad_tiles_per_expert<false>(dm);
  const int splits = wgrad_splits_bf16(dm, out_f32);
  if (splits == 1 && !out_f32) {
    const unsigned grid = pad8(static_cast<int64_t>(3) * dm.E * tpe);
    g.grid_pad = static_cast<int32_t>(grid);
    const bool big = grid <= static_cast<unsigned>(kCUs);
    if (g.x_rows) {
      if (big)
        hipLaunchKernelGGL((wgrad_dma_small_kernel<8, true>), dim3(grid), dim3(dmas::NT), 0, s,
                           g, tpe);
      else
        hipLaunchKernelGGL((wgrad_dma_small_kernel<4, true>), dim3(grid), dim3(dmas::NT), 0, s,
                           g, tpe);
    } else if (big) {
      hipLaunchKernelGGL((wgrad_dma_small_kernel<8, false>), dim3(grid), dim3(dmas::NT), 0, s, g,
                         tpe);
    } else {
      hipLaunchKernelGGL((wgrad_dma_small_kernel<4, false>), dim3(grid), dim3(dmas::NT), 0, s, g,
                         tpe);
    }
    return hipGetLastError();
  }
  const int64_t items = static_cast<int64_t>(3) * dm.E * tpe * splits;
  const int64_t grid = std::max(std::min(items, static_cast<int64_t>(2 * kCUs)),
                                (items + kMaxItems - 1) / kMaxItems);
  g.grid_pad = static_cast<int32_t>(pad8(grid));
  if (g.x_rows)
    hipLaunchKernelGGL((wgrad_stream_kernel<true>), dim3(g.grid_pad), dim3(Cfg<false>::THREADS),
                       0, s, g, tpe, splits, partial);
  else
    hipLaunchKernelGGL((wgrad_stream_kernel<false>), dim3(g.grid_pad), dim3(Cfg<false>::THREADS),
                       0, s, g, tpe, splits, partial);
  if (splits > 1) {
    const int64_t chunks = static_cast<int64_t>(3) * dm.E * tpe * (128 * 128 / 8);
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((chunks + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, s, g, tpe, splits, partial);
  }
  return hipGetLastError();
}

// The gate-folded path runs on the LDS-DMA kernels (small and big tiles) where
// the weight gradients take a one-pass kernel (not the split-K stream).
bool folded_bf16_ok(const moe_dims& dm) {
  return dm.act == MOE_BF16 && (use_big_wgrad(dm) || wgrad_splits_bf16(dm) == 1);
}

// dgate parts per row: one per column tile of DGRAD_DOWN (256 wide on the big
// tile, 128 on the small one)
int dgate_parts_bf16(const moe_dims& dm) {
  const int n_big = (dm.f + 255) / 256;
  if (use_big_rows(dm, n_big, dm.d)) return n_big;
  return (dm.f + Cfg<false>::BN - 1) / Cfg<false>::BN;
}

hipError_t launch_up_folded_bf16(const moe_dims& dm, const void* x, const int32_t* x_rows,
                                 const int32_t* offsets, const float* gate_rows, const void* w1,
                                 const void* w3, void* a, void* b, void* hg, hipStream_t s) {
  if (dm.T * dm.k == 0) return hipSuccess;   // no expert rows
  if (!folded_bf16_ok(dm) || !x_rows || !gate_rows) return hipErrorNotSupported;
  Args g = base_args(dm, offsets);
  g.a0 = static_cast<const bf16_t*>(x);
  g.x_rows = x_rows;
  g.x_bytes = static_cast<int32_t>(dm.T * dm.d * 2);
  g.b0 = static_cast<const bf16_t*>(w1);
  g.b1 = static_cast<const bf16_t*>(w3);
  g.c0 = static_cast<bf16_t*>(a);
  g.c1 = static_cast<bf16_t*>(b);
  g.c2 = static_cast<bf16_t*>(hg);
  g.gate_rows = gate_rows;
  return launch_rows<UP>(g, dm, dm.f, dm.d, s);
}

hipError_t launch_dgrad_down_folded_bf16(const moe_dims& dm, const void* dy,
                                         const int32_t* x_rows, const int32_t* offsets,
                                         const float* gate_rows, const void* w2, const void* a,
                                         const void* b, void* da, void* db, float* dgate_part,
                                         hipStream_t s) {
  if (dm.T * dm.k == 0) return hipSuccess;   // no expert rows
  if (!folded_bf16_ok(dm) || !x_rows || !gate_rows || !dgate_part) return hipErrorNotSupported;
  Args g = base_args(dm, offsets);
  g.a0 = static_cast<const bf16_t*>(dy);
  g.x_rows = x_rows;
  g.x_bytes = static_cast<int32_t>(dm.T * dm.d * 2);
  g.b0 = static_cast<const bf16_t*>(w2);
  g.aux0 = static_cast<const bf16_t*>(a);
  g.aux1 = static_cast<const bf16_t*>(b);
  g.c0 = static_cast<bf16_t*>(da);
  g.c1 = static_cast<bf16_t*>(db);
  g.gate_rows = gate_rows;
  g.dgate_part = dgate_part;
  return launch_rows<DGRAD_DOWN>(g, dm, dm.f, dm.d, s);
}

hipError_t launch_wgrad_folded_bf16(const moe_dims& dm, const void* x, const int32_t* x_rows,
                                    const int32_t* offsets, const void* hg, const void* dy,
                                    const void* da, const void* db, void* dw1, void* dw3,
                                    void* dw2, hipStream_t s) {
  // no expert rows: every weight gradient is zero, as the unfolded call writes it
  if (dm.T * dm.k == 0)
    return launch_wgrad_bf16(dm, x, x_rows, offsets, hg, dy, da, db, dw1, dw3, dw2, false, nullptr,
                             s);
  if (!folded_bf16_ok(dm) || !x_rows) return hipErrorNotSupported;
  Args g = base_args(dm, offsets);
  g.x_rows = x_rows;
  g.x_bytes = static_cast<int32_t>(dm.T * dm.d * 2);
  g.a0 = static_cast<const bf16_t*>(dy);   // z = 0: A = dy through the table, B = g h
  g.b0 = static_cast<const bf16_t*>(hg);
  g.a1 = static_cast<const bf16_t*>(da);
  g.aux0 = static_cast<const bf16_t*>(db);
  g.b1 = static_cast<const bf16_t*>(x);
  g.c0 = static_cast<bf16_t*>(dw2);
  g.c1 = static_cast<bf16_t*>(dw1);
  g.c2 = static_cast<bf16_t*>(dw3);
  if (use_big_wgrad(dm)) {
    const int tpe = wgrad_tiles_per_expert<true>(dm);
    const unsigned grid = wgrad_snake_grid(dm.E, tpe);
    g.grid_pad = static_cast<int32_t>(grid);
    hipLaunchKernelGGL((wgrad_dma_kernel<true, true>), dim3(grid), dim3(dmaw::NT), 0, s, g, tpe);
    return hipGetLastError();
  }
  const int tpe = wgrad_tiles_per_expert<false>(dm);
  const unsigned grid = pad8(static_cast<int64_t>(3) * dm.E * tpe);
  g.grid_pad = static_cast<int32_t>(grid);
  if (grid <= static_cast<unsigned>(kCUs))
    hipLaunchKernelGGL((wgrad_dma_small_kernel<8, true, true>), dim3(grid), dim3(dmas::NT), 0, s,
                       g, tpe);
  else
    hipLaunchKernelGGL((wgrad_dma_small_kernel<4, true, true>), dim3(grid), dim3(dmas::NT), 0, s,
                       g, tpe);
  return hipGetLastError();
}

// Split-K count for the (small-tile) weight gradients: none when the tiles
// alone give about two thirds of a workgroup per CU (the persistent kernel
// streams long K ranges well); otherwise enough splits for about 320 items,
// at most 8.  Big tiles (bf16 output only) never split.
int wgrad_splits_bf16(const moe_dims& dm, bool out_f32) {
  if (!out_f32 && use_big_wgrad(dm)) return 1;
  const int64_t base = static_cast<int64_t>(3) * dm.E * wgrad_tiles_per_expert<false>(dm);
  if (base >= kWgradNoSplitItems) return 1;
  const int64_t want = 2 * kWgradNoSplitItems;
  int s = static_cast<int>((want + base - 1) / base);
  return std::max(1, std::min(s, 8));
}

size_t wgrad_partial_bytes_bf16(const moe_dims& dm, bool out_f32) {
  const int s = wgrad_splits_bf16(dm, out_f32);
  if (s <= 1) return 0;
  return static_cast<size_t>(3) * dm.E * wgrad_tiles_per_expert<false>(dm) * s * (128 * 128) *
         sizeof(float);
}

}  // namespace moe

