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
// way and written in permuted row order, or in token-slot order for the
// matrix-core dWr), dWr partial sums (over contiguous parts of each expert's
// rows, which the permutation lists in ascending token order; or, for bf16 X
// with E <= 64 and d >= 1024, over token ranges on the matrix cores, reading X
// once), and a fixed-order reduction of the parts.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// dX rows:
//   dl[t,j] = g_j (dg_j - sum_i g_i dg_i)          (the fp32 sum in slot order)
//   dX[t]   = sum_j dx_perm[pos[t,j]] + sum_j dl[t,j] wr[idx[t,j]]
// summed in fp32 in slot order and rounded once.  Workgroup (column block,
// token range): the block's bc columns of every router row (E x bc fp32) are
// staged in LDS once, so the router rows come from LDS rather than from L2
// once per chunk and slot.  The token range goes in batches of kBatch tokens
// (kThreads, or half of it for k > 8): first thread i reads the slots of token i of the batch (gates,
// dgate or its column-tile parts, positions, ids: coalesced across the
// threads, each once per column block), forms dl, and puts (position, id, dl)
// of every slot in an LDS table; the workgroups of column block 0 also
// scatter dl into permuted row order for the dWr kernel (and, gate folded,
// write dgate).  Then each thread takes one 16-byte chunk of dX for
// kThreads / (bc / kPer) tokens at a time, with the slots from the table; K
// is the compile-time k (0: runtime k <= 16), and every row load of a token is
// issued before any is used (positions clamped, invalid slots masked), so a
// row costs one memory latency rather than one per slot.
// tokens per slot-table batch (the table takes 12 KM kBatch bytes of LDS)
constexpr int dx_batch(int km) { return km <= 8 ? kThreads : kThreads / 2; }

template <typename TA, int K, bool FOLD>
__global__ __launch_bounds__(kThreads) void router_dx_kernel(
    const uint4* __restrict__ dxp, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const float* __restrict__ dgate, const float* __restrict__ wr, uint4* __restrict__ dx,
    float* __restrict__ dl_perm, int64_t T, int32_t vpr, int32_t d, int32_t k, int32_t E,
    const float* __restrict__ dgate_part, int32_t nparts, float* __restrict__ dgate_out,
    int32_t bc, int32_t tok_per_wg, float* __restrict__ dl_tok) {
  // [E][bc] router block, then the batch's slot table [KM][kBatch] x 3
  extern __shared__ __attribute__((aligned(16))) float wl[];
  constexpr int kPer = Act<TA>::kPer16B;
  constexpr int KM = K > 0 ? K : 16;
  constexpr int kBatch = dx_batch(KM);
  const int kk = K > 0 ? K : k;
  const int col0 = blockIdx.x * bc;
  int32_t* const tab_p = reinterpret_cast<int32_t*>(wl + E * bc);
  int32_t* const tab_e = tab_p + KM * kBatch;
  float* const tab_dl = reinterpret_cast<float*>(tab_e + KM * kBatch);
  {
    const int q4 = bc / 4;
    for (int i = threadIdx.x; i < E * q4; i += kThreads) {
      const int e = i / q4, q = i - e * q4;
      *reinterpret_cast<float4*>(wl + e * bc + q * 4) =
          *reinterpret_cast<const float4*>(wr + static_cast<int64_t>(e) * d + col0 + q * 4);
    }
  }
  const int cpr = bc / kPer;                    // chunks of the block per row
  const int tpp = kThreads / cpr;               // tokens per pass
  const int cl = threadIdx.x % cpr;             // chunk within the block
  const int32_t c = col0 / kPer + cl;           // chunk within the row
  const bool first_block = blockIdx.x == 0;
  const int64_t t_beg = static_cast<int64_t>(blockIdx.y) * tok_per_wg;
  const int64_t t_end = min<int64_t>(T, t_beg + tok_per_wg);
  for (int64_t b0 = t_beg; b0 < t_end; b0 += kBatch) {
    __syncthreads();   // the router block is staged; the previous table is read
    {
      const int64_t t = b0 + threadIdx.x;
      if (static_cast<int>(threadIdx.x) < kBatch && t < t_end) {
        float g[KM], dg[KM];
        int32_t p[KM], e[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          const int64_t q = t * kk + min(j, kk - 1);
          g[j] = gate[q];
          dg[j] = FOLD ? 0.f : dgate[q];   // folded: from the parts below
          p[j] = pos[q];
          e[j] = idx[q];
        }
        if constexpr (FOLD) {
          // gate folded onto the rows: dg is the sum of the row's column-tile
          // parts in tile order (0 for a dropped slot); the first kPartsU
          // parts of every slot are loaded at once, the rest (wide f) in a loop
          constexpr int kPartsU = 4;
          float pv[KM][kPartsU];
#pragma unroll
          for (int j = 0; j < KM; ++j) {
            const float* pp = dgate_part + static_cast<int64_t>(max(p[j], 0)) * nparts;
#pragma unroll
            for (int q = 0; q < kPartsU; ++q) pv[j][q] = pp[min(q, nparts - 1)];
          }
#pragma unroll
          for (int j = 0; j < KM; ++j) {
            const float* pp = dgate_part + static_cast<int64_t>(max(p[j], 0)) * nparts;
            float sum = pv[j][0];
#pragma unroll
            for (int q = 1; q < kPartsU; ++q)
              if (q < nparts) sum += pv[j][q];
            for (int q = kPartsU; q < nparts; ++q) sum += pp[q];
            dg[j] = (p[j] >= 0) ? sum : 0.f;
          }
          if (first_block) {
#pragma unroll
            for (int j = 0; j < KM; ++j)
              if (j < kk) dgate_out[t * kk + j] = dg[j];
          }
        }
        float inner = 0.f;
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (j < kk) inner = fmaf(g[j], dg[j], inner);
        float dlv[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          const float dl = g[j] * (dg[j] - inner);
          const bool live = j < kk;
          dlv[j] = dl;
          if (first_block && live && p[j] >= 0) dl_perm[p[j]] = dl;
          tab_p[j * kBatch + threadIdx.x] = live ? p[j] : -1;
          tab_e[j * kBatch + threadIdx.x] = (live && e[j] >= 0 && e[j] < E) ? e[j] : -1;
          tab_dl[j * kBatch + threadIdx.x] = dl;
        }
        if (dl_tok && first_block) {   // dl in token-slot order, for the dWr kernel
#pragma unroll
          for (int j = 0; j < KM; ++j)
            if (j < kk) dl_tok[t * kk + j] = dlv[j];
        }
      }
    }
    __syncthreads();
    const int nb = static_cast<int>(min<int64_t>(kBatch, t_end - b0));
    for (int i = threadIdx.x / cpr; i < nb; i += tpp) {
      int32_t p[KM], e[KM];
      float dl[KM];
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        p[j] = tab_p[j * kBatch + i];
        e[j] = tab_e[j * kBatch + i];
        dl[j] = tab_dl[j * kBatch + i];
      }
      uint4 rows[KM];
#pragma unroll
      for (int j = 0; j < KM; ++j)
        rows[j] = dxp ? ld_nt16(dxp + static_cast<int64_t>(max(p[j], 0)) * vpr + c)
                      : make_uint4(0u, 0u, 0u, 0u);
      float acc[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) acc[q] = 0.f;
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (!dxp || p[j] < 0) continue;
        float r[kPer];
        unpack16(rows[j], r, TA{});
#pragma unroll
        for (int q = 0; q < kPer; ++q) acc[q] += r[q];
      }
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (e[j] < 0) continue;
        const float* wp = wl + e[j] * bc + cl * kPer;
#pragma unroll
        for (int q = 0; q < kPer; q += 4) {
          const float4 w4 = *reinterpret_cast<const float4*>(wp + q);
          acc[q] = fmaf(dl[j], w4.x, acc[q]);
          acc[q + 1] = fmaf(dl[j], w4.y, acc[q + 1]);
          acc[q + 2] = fmaf(dl[j], w4.z, acc[q + 2]);
          acc[q + 3] = fmaf(dl[j], w4.w, acc[q + 3]);
        }
      }
      st_nt16(dx + (b0 + i) * vpr + c, pack16(acc, TA{}));
    }
  }
}

// Router-row columns per dX workgroup: 128 up to 64 experts, 64 up to 128, 32
// beyond, so that the staged block (E x bc fp32: at most 32 KB) leaves room
// for several workgroups per CU, whose gathered row loads are what keeps HBM
// busy (each of them 256 bytes of a row at 128 columns: C5's dX 3 us faster
// than at 64).
constexpr int kDxCols = 64;

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

// dWr on the matrix cores (bf16 X, E <= 64), from the logit gradient in
// token-slot order (dl_tok [T][k] with the ids idx [T][k]):
//   partial[e][s][c] = sum over the tokens t of split s of dl[t][e] X[t][c],
// dl[t][e] the sum of dl_tok over the token's slots that chose e (zero for the
// rest; a repeated id adds in slot order).  The thread of (token, 8-expert
// piece) builds that piece of a chunk's dl rows in LDS, split exactly into
// three bf16 parts (hi + mid + lo = dl), so every bf16 x bf16 product is exact
// in fp32 and the three parts accumulate in fp32 (in chunk order, hi, mid, lo
// within a chunk).  Workgroup (128-column
// block, token split): the split's tokens go in chunks of 32 (the K of one
// v_mfma_f32_16x16x32_bf16); a chunk's X rows and the three parts of its dl
// rows sit in LDS token-major (rows padded by 16 bytes),
// and the fragments (8 consecutive tokens of one column or one expert) come
// from the gfx950 transposing LDS read: within each 16-lane group, lane s
// reads 8 bytes of row s / 4 at column 4 (s % 4), and lane j receives column
// j of the four rows.  Wavefront w owns columns 32 w ... 32 w + 31 and every
// expert block.  The next chunk's global loads are in registers while the
// current one runs (two LDS buffers, one barrier per chunk).
constexpr int kDwBN = 128;                 // columns per workgroup
constexpr int kDwChunk = 32;               // tokens per chunk
constexpr int kDwXs = kDwBN * 2 + 16;      // X tile row stride (bytes)
typedef short dw_v4s __attribute__((ext_vector_type(4)));
typedef short dw_v8s __attribute__((ext_vector_type(8)));
typedef __bf16 dw_bf16x8 __attribute__((ext_vector_type(8)));
typedef float dw_f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dw_v4s* dw_lds_v4s_t;

__device__ __forceinline__ dw_bf16x8 dw_tr_frag(const unsigned char* lds, uint32_t lo,
                                                uint32_t hi) {
  const dw_v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dw_lds_v4s_t)(lds + lo));
  const dw_v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dw_lds_v4s_t)(lds + hi));
  const dw_v8s both = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(dw_bf16x8, both);
}

template <int NT, int K>   // E <= 16 NT; K = k (0: runtime k <= 16)
__global__ __launch_bounds__(kThreads) void router_dwr_mfma_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ idx, const float* __restrict__ dl,
    float* __restrict__ partial, int64_t T, int32_t d, int32_t n_experts, int32_t k, int32_t S,
    int32_t L) {
  constexpr int KM = K > 0 ? K : 16;
  constexpr int kM = 16 * NT;                     // experts, zero-padded
  constexpr int kAs = kM * 2 + 16;                // dl-part tile row stride (bytes)
  constexpr int kXB = kDwChunk * kDwXs;
  constexpr int kAB = kDwChunk * kAs;
  constexpr int kBuf = kXB + 3 * kAB;
  constexpr int kXv = kDwChunk * kDwBN / 8 / kThreads;         // 16-byte X pieces per thread (2)
  constexpr int kPc = kM / 8;                                  // 8-expert pieces of a dl row
  constexpr int kAct = kDwChunk * kPc;                         // threads building dl rows
  const int kk = K > 0 ? K : k;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kBuf];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * kDwBN;
  const int sp = blockIdx.y;
  const int64_t t_lo = static_cast<int64_t>(sp) * L;
  const int64_t t_hi = min<int64_t>(T, t_lo + L);
  const int nch = static_cast<int>((t_hi - t_lo + kDwChunk - 1) / kDwChunk);

  uint4 xr[kXv];
  int32_t ir[KM];
  float vr[KM];
  auto load = [&](int ch) {   // rows past t_hi read as zeros, their ids as -1
    const int64_t tb = t_lo + static_cast<int64_t>(ch) * kDwChunk;
#pragma unroll
    for (int i = 0; i < kXv; ++i) {
      const int v = tid + i * kThreads;
      const int64_t t = tb + v / (kDwBN / 8);
      xr[i] = (t < t_hi) ? ld_nt16(reinterpret_cast<const uint4*>(x + t * d + n0 + (v % (kDwBN / 8)) * 8))
                         : make_uint4(0u, 0u, 0u, 0u);
    }
    const int64_t t = tb + tid / kPc;
    const bool ok = tid < kAct && t < t_hi;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      ir[j] = (ok && j < kk) ? idx[t * kk + j] : -1;
      vr[j] = (ok && j < kk) ? dl[t * kk + j] : 0.f;
    }
  };
  auto store = [&](unsigned char* buf) {
#pragma unroll
    for (int i = 0; i < kXv; ++i) {
      const int v = tid + i * kThreads;
      *reinterpret_cast<uint4*>(buf + (v / (kDwBN / 8)) * kDwXs + (v % (kDwBN / 8)) * 16) = xr[i];
    }
    if (tid < kAct) {
      // experts 8 q ... 8 q + 7 of the chunk's token row: the sum of the
      // slots that chose each (slot order), then its three bf16 parts
      const int row = tid / kPc, q = tid % kPc;
      float w[8];
#pragma unroll
      for (int z = 0; z < 8; ++z) {
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (ir[j] == 8 * q + z) v += vr[j];
        w[z] = v;
      }
      uint32_t h[4], m[4], l[4];
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2) {
        h[p2] = bf16x2_rne(w[2 * p2], w[2 * p2 + 1]);
        const float r0 = w[2 * p2] - __uint_as_float(h[p2] << 16);
        const float r1 = w[2 * p2 + 1] - __uint_as_float(h[p2] & 0xFFFF0000u);
        m[p2] = bf16x2_rne(r0, r1);
        l[p2] = bf16x2_rne(r0 - __uint_as_float(m[p2] << 16),
                           r1 - __uint_as_float(m[p2] & 0xFFFF0000u));
      }
      unsigned char* a = buf + kXB + row * kAs + q * 16;
      *reinterpret_cast<uint4*>(a) = make_uint4(h[0], h[1], h[2], h[3]);
      *reinterpret_cast<uint4*>(a + kAB) = make_uint4(m[0], m[1], m[2], m[3]);
      *reinterpret_cast<uint4*>(a + 2 * kAB) = make_uint4(l[0], l[1], l[2], l[3]);
    }
  };
  // transposing-read addresses within a buffer: rows 8 g + (c >> 2) (+ 4 for
  // the second half), column 4 (c & 3) of the fragment's 16
  const int r0 = 8 * g + (c >> 2);
  uint32_t bx[2], ba[NT];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) bx[nb] = r0 * kDwXs + (32 * wave + 16 * nb + 4 * (c & 3)) * 2;
#pragma unroll
  for (int mb = 0; mb < NT; ++mb) ba[mb] = kXB + r0 * kAs + (16 * mb + 4 * (c & 3)) * 2;

  dw_f32x4 acc[NT][2];
#pragma unroll
  for (int mb = 0; mb < NT; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = dw_f32x4{0.f, 0.f, 0.f, 0.f};

  load(0);
  store(lds);
  if (nch > 1) load(1);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const unsigned char* cur = lds + (ch & 1) * kBuf;
    if (ch + 1 < nch) {
      store(lds + ((ch + 1) & 1) * kBuf);   // the other buffer: read two barriers ago
      if (ch + 2 < nch) load(ch + 2);
    }
    dw_bf16x8 fb[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) fb[nb] = dw_tr_frag(cur, bx[nb], bx[nb] + 4 * kDwXs);
#pragma unroll
    for (int part = 0; part < 3; ++part) {
#pragma unroll
      for (int mb = 0; mb < NT; ++mb) {
        const uint32_t o = ba[mb] + part * kAB;
        const dw_bf16x8 fa = dw_tr_frag(cur, o, o + 4 * kAs);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[nb], acc[mb][nb], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // lane (g, c) of block (mb, nb): experts 16 mb + 4 g + q, column 32 w + 16 nb + c
#pragma unroll
  for (int mb = 0; mb < NT; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = 16 * mb + 4 * g + q;
        if (e < n_experts)
          partial[(static_cast<int64_t>(e) * S + sp) * d + n0 + 32 * wave + 16 * nb + c] =
              acc[mb][nb][q];
      }
}

// Adds the per-split partial sums of dWr.  Workgroup (column block of 64,
// expert): thread (split lane sl = t / 16, column group cg = t % 16) adds
// splits sl, sl + 16, ... in order (all loads issued first), then thread
// group sl = 0 adds the 16 lane sums in order: a fixed summation order, so
// the result is reproducible, and one memory latency per thread.
template <int kMaxPer>   // splits <= 16 kMaxPer
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

// ---------------------------------------------------------------- dense form
// With dropped assignments (capacity) or the auxiliary losses the logit
// gradient is no longer confined to the k chosen experts of a token that have
// a permuted row, so the dense form is used:
//   dl[t,e] = sum_{j : S_j(t) = e} g_j (dg_j - sum_i g_i dg_i)
//           + aux_scale p[t,e] (f[r,e] - sum_e' f[r,e'] p[t,e'])   (GShard balancing)
//           + z_scale lse_t p[t,e]                                  (ST-MoE z-loss)
// with p the full softmax, f = count / (n k) of the token's block r, and
//   dX[t] = sum_e dl[t,e] Wr[e] + sum_{j : pos >= 0} dx_perm[pos[t,j]],
//   dWr   = dl^T X.
// Dropped slots keep their gate term: the dropped expert's logit still sets
// the renormalised gates of the kept ones.

// One wavefront per token; lane l holds experts l, l + 64, ...  Wavefront
// sums and maxima are xor butterflies, which leave the same bits in every lane.
template <int EPL>
__global__ __launch_bounds__(kThreads) void router_dl_dense_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const float* __restrict__ dgate,
    const int32_t* __restrict__ count, int32_t n, float f_scale, float aux_scale, float z_scale,
    float* __restrict__ dl, float* __restrict__ dl_out, int64_t T, int32_t k, int32_t E) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;   // wavefront-uniform; no workgroup barrier below
  float l[EPL], p[EPL], dv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    l[i] = (e < E) ? logits[t * E + e] : -INFINITY;
    dv[i] = 0.f;
  }
  float m = l[0];
#pragma unroll
  for (int i = 1; i < EPL; ++i) m = fmaxf(m, l[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    p[i] = (lane + 64 * i < E) ? __expf(l[i] - m) : 0.f;
    s += p[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  const float inv = 1.0f / s;
#pragma unroll
  for (int i = 0; i < EPL; ++i) p[i] *= inv;
  if (aux_scale != 0.f) {
    const int32_t* cr = count + (t / n) * E;
    float f[EPL];
    float fp = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      f[i] = (e < E) ? static_cast<float>(cr[e]) * f_scale : 0.f;
      fp = fmaf(f[i], p[i], fp);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) fp += __shfl_xor(fp, off, 64);
#pragma unroll
    for (int i = 0; i < EPL; ++i) dv[i] = aux_scale * p[i] * (f[i] - fp);
  }
  if (z_scale != 0.f) {
    const float zl = z_scale * (m + __logf(s));
#pragma unroll
    for (int i = 0; i < EPL; ++i) dv[i] = fmaf(zl, p[i], dv[i]);
  }
  float inner = 0.f;
  for (int j = 0; j < k; ++j) inner = fmaf(gate[t * k + j], dgate[t * k + j], inner);
  for (int j = 0; j < k; ++j) {
    const int32_t e = idx[t * k + j];
    if (e < 0 || e >= E || (e & 63) != lane) continue;
    const float v = gate[t * k + j] * (dgate[t * k + j] - inner);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if ((e >> 6) == i) dv[i] += v;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e >= E) continue;
    dl[t * E + e] = dv[i];
    if (dl_out) dl_out[t * E + e] = dv[i];
  }
}

__device__ __forceinline__ void store4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16_t* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3]));
}

// dX rows of the dense form: a wavefront computes kDxTok tokens x 256 columns
// (4 per lane).  Per element: the kept dx_perm rows in slot order, then
// sum_e dl[t,e] Wr[e] (e ascending), in fp32, rounded once.  The rows of
// several tokens are loaded together (UT tokens x k slots in flight); the
// wavefront's kDxTok x E block of dl is staged in LDS as [e][token], so two
// broadcast reads give the eight tokens' weights of expert e; Wr rows come
// from L2, eight experts' loads issued before they are used.  Every address
// is clamped in bounds, so no load sits behind a branch.
// K is the compile-time k (0: runtime k <= 16).
constexpr int kDxTok = 8;
template <typename TA, int K>
__global__ __launch_bounds__(kThreads) void router_dx_dense_kernel(
    const TA* __restrict__ dxp, const int32_t* __restrict__ pos, const float* __restrict__ dl,
    const float* __restrict__ wr, TA* __restrict__ dx, int64_t T, int32_t d, int32_t k,
    int32_t E) {
  constexpr int KM = K > 0 ? K : 16;
  constexpr int kMaxRows = sizeof(TA) == 2 ? 32 : 8;          // row pieces in flight
  constexpr int UT0 = kMaxRows / KM >= 8 ? 8 : kMaxRows / KM >= 4 ? 4 : kMaxRows / KM >= 2 ? 2 : 1;
  constexpr int UT = UT0;                                      // tokens whose rows load together
  static_assert(kDxTok % UT == 0, "token groups must tile the wavefront's tokens");
  const int kk = K > 0 ? K : k;
  extern __shared__ float sdl[];   // [4 waves][E8][kDxTok], E8 = E rounded up to 8
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ncb = (d + 255) / 256;
  const int E8 = (E + 7) & ~7;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + w;
  const int64_t t0 = (wid / ncb) * kDxTok;
  const int cb = static_cast<int>(wid % ncb);
  float* my = sdl + static_cast<int64_t>(w) * E8 * kDxTok;
  for (int i = lane; i < kDxTok * E8; i += 64) {   // padding experts weigh 0
    const int tl = i / E8, e = i - tl * E8;
    my[e * kDxTok + tl] = (t0 + tl < T && e < E) ? dl[(t0 + tl) * E + e] : 0.f;
  }
  __syncthreads();
  if (t0 >= T) return;   // wavefront-uniform; no barrier below
  const int col = cb * 256 + lane * 4;
  const int colc = col < d ? col : 0;   // lanes past d compute on column 0 and store nothing
  float acc[kDxTok][4];
#pragma unroll
  for (int u = 0; u < kDxTok; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[u][i] = 0.f;
  if (dxp) {
#pragma unroll
    for (int u0 = 0; u0 < kDxTok; u0 += UT) {
      int32_t pp[UT][KM];
      float v[UT][KM][4];
#pragma unroll
      for (int u = 0; u < UT; ++u) {
        const int64_t t = min<int64_t>(t0 + u0 + u, T - 1);
#pragma unroll
        for (int j = 0; j < KM; ++j) pp[u][j] = pos[t * kk + min(j, kk - 1)];
      }
#pragma unroll
      for (int u = 0; u < UT; ++u)
#pragma unroll
        for (int j = 0; j < KM; ++j)
          load4(dxp + static_cast<int64_t>(max(pp[u][j], 0)) * d + colc, v[u][j]);
#pragma unroll
      for (int u = 0; u < UT; ++u)
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          const bool keep = j < kk && pp[u][j] >= 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[u0 + u][i] += keep ? v[u][j][i] : 0.f;
        }
      // one group's loads in flight at a time (bounds the registers they hold)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (int e0 = 0; e0 < E; e0 += 8) {
    float4 wv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      wv[u] = *reinterpret_cast<const float4*>(wr + static_cast<int64_t>(min(e0 + u, E - 1)) * d +
                                              colc);
#pragma unroll
    for (int u = 0; u < 8; ++u) {   // experts past E: a clamped Wr row times weight 0
      const float4* dq = reinterpret_cast<const float4*>(my + (e0 + u) * kDxTok);
#pragma unroll
      for (int q = 0; q < kDxTok / 4; ++q) {
        const float4 g = dq[q];
        const float gg[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          acc[4 * q + z][0] = fmaf(gg[z], wv[u].x, acc[4 * q + z][0]);
          acc[4 * q + z][1] = fmaf(gg[z], wv[u].y, acc[4 * q + z][1]);
          acc[4 * q + z][2] = fmaf(gg[z], wv[u].z, acc[4 * q + z][2]);
          acc[4 * q + z][3] = fmaf(gg[z], wv[u].w, acc[4 * q + z][3]);
        }
      }
    }
  }
  if (col >= d) return;
#pragma unroll
  for (int u = 0; u < kDxTok; ++u)
    if (t0 + u < T) store4(dx + (t0 + u) * d + col, acc[u]);
}

// dWr partial sums of the dense form: partial[e][sp][c] = sum over the
// tokens of split sp of dl[t,e] x[t,c].  Workgroup (256-column block, block of
// kDwEB experts, split sp): wavefront w takes tokens lo + w, lo + w + 4, ...
// in order, four at a time in flight; the four wavefronts are added in order
// through LDS, and router_dwr_reduce_kernel adds the splits in order.
constexpr int kDwEB = 16;
template <typename TA>
__global__ __launch_bounds__(kThreads) void router_dwr_dense_partial_kernel(
    const TA* __restrict__ x, const float* __restrict__ dl, float* __restrict__ partial,
    int64_t T, int32_t d, int32_t E, int32_t splits) {
  __shared__ float red[4][8][256];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int cb = blockIdx.x, e0 = blockIdx.y * kDwEB, sp = blockIdx.z;
  const int col = cb * 256 + lane * 4;
  const bool cok = col < d;
  const int64_t lo = (T * sp) / splits, hi = (T * (sp + 1)) / splits;
  float acc[kDwEB][4];
#pragma unroll
  for (int e = 0; e < kDwEB; ++e)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[e][i] = 0.f;
  constexpr int U = 4;
  const int colc = cok ? col : 0;   // lanes past d read column 0 and write nothing
  for (int64_t t = lo + w; t < hi; t += 4 * U) {
    float xv[U][4];
    float g[U][kDwEB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tc = min<int64_t>(t + 4 * u, hi - 1);
      load4(x + tc * d + colc, xv[u]);
      // kDwEB consecutive values of the token's row (the buffer is padded by
      // kDwEB floats, so the last row's tail stays in bounds; masked below)
      const float* row = dl + tc * E + e0;
#pragma unroll
      for (int e = 0; e < kDwEB; ++e) g[u][e] = row[e];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool tok = t + 4 * u < hi;
#pragma unroll
      for (int e = 0; e < kDwEB; ++e) {
        const float ge = (tok && e0 + e < E) ? g[u][e] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[e][i] = fmaf(ge, xv[u][i], acc[e][i]);
      }
    }
  }
#pragma unroll
  for (int ec = 0; ec < kDwEB; ec += 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][e][lane * 4 + i] = acc[ec + e][i];
    __syncthreads();
    for (int v = threadIdx.x; v < 8 * 256; v += kThreads) {
      const int e = v / 256, c = v % 256;
      const int ee = e0 + ec + e, cc = cb * 256 + c;
      if (ee < E && cc < d)
        partial[(static_cast<int64_t>(ee) * splits + sp) * d + cc] =
            ((red[0][e][c] + red[1][e][c]) + red[2][e][c]) + red[3][e][c];
    }
    __syncthreads();
  }
}

}  // namespace

// the router weight gradient on the matrix cores: bf16 X, E <= 64, d a
// multiple of 128 from 1024 (on narrower rows the per-expert kernel's k-fold
// reads of X cost less than this kernel's chunk loop and partial sums); dl
// rows of route_bwd_mfma_ld experts, token splits of route_bwd_mfma_len tokens
// (about 512 workgroups, and no more partial sums than X has bytes)
bool route_bwd_mfma_ok(const moe_dims& dm) {
  return dm.act == MOE_BF16 && dm.E <= 64 && dm.d % kDwBN == 0 && dm.d >= 1024 && dm.T > 0;
}
int route_bwd_mfma_ld(const moe_dims& dm) {
  const int nt = (dm.E + 15) / 16;
  return 16 * (nt <= 1 ? 1 : nt <= 2 ? 2 : 4);
}
int64_t route_bwd_mfma_len(const moe_dims& dm) {
  const int64_t ncb = std::max(dm.d / kDwBN, 1);
  int64_t s0 = std::max<int64_t>(1, (512 + ncb - 1) / ncb);
  s0 = std::min<int64_t>(s0, std::max<int64_t>(1, dm.T / (2 * dm.E)));
  int64_t len = (dm.T + s0 - 1) / s0;
  len = std::max<int64_t>(kDwChunk, (len + kDwChunk - 1) / kDwChunk * kDwChunk);
  // at most 256 splits (the reduction's limit)
  const int64_t min_len = (dm.T + 255) / 256;
  if (len < min_len) len = (min_len + kDwChunk - 1) / kDwChunk * kDwChunk;
  return len;
}
int route_bwd_mfma_splits(const moe_dims& dm) {
  return static_cast<int>((dm.T + route_bwd_mfma_len(dm) - 1) / route_bwd_mfma_len(dm));
}

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
                            float* ws_dl_sel, float* ws_partial, hipStream_t s,
                            const float* dgate_part, int32_t nparts, float* dgate_out) {
  // the matrix-core weight gradient reads dl in token-slot order (ws_dl_sel)
  const bool mfma = route_bwd_mfma_ok(dm);
  float* const dl_tok = mfma ? ws_dl_sel : nullptr;
  if (dm.T > 0) {
    const int elem = (dm.act == MOE_BF16) ? 2 : 4;
    const int32_t vpr = dm.d * elem / 16;
    // column blocks x token ranges
    int bc = dm.E <= 64 ? 2 * kDxCols : dm.E <= 128 ? kDxCols : kDxCols / 2;   // router block <= 32 KB
    while (dm.d % bc) bc >>= 1;   // a divisor of d (a multiple of 64)
    const int ncb = dm.d / bc;
    // token ranges for about two workgroups per CU, all resident at once (three
    // fit): each stages its router block once for several batches.  Measured
    // at C5: 129 us against 138 at three per CU, 142 at eight and 159 at one
    // (C3: 25 against 30 us at eight)
    constexpr int kCUs = 256;
    const int64_t want = std::max<int64_t>(1, (2 * kCUs + ncb - 1) / ncb);
    const int64_t tpw = std::max<int64_t>((dm.T + want - 1) / want, 1);
    const dim3 grid(ncb, static_cast<unsigned>((dm.T + tpw - 1) / tpw));
    // the router block, then the slot table (3 words per slot of a batch):
    // at most 32 KB + 24 KB
    const int km = (dm.k == 1 || dm.k == 2 || dm.k == 4 || dm.k == 6 || dm.k == 8) ? dm.k : 16;
    const size_t lds = (static_cast<size_t>(dm.E) * bc + 3 * static_cast<size_t>(km) * dx_batch(km)) *
                       sizeof(float);
    const uint4* dxp = static_cast<const uint4*>(dx_perm);
    uint4* dxo = static_cast<uint4*>(dx);
#define MOE_DX(TA, KC)                                                                        \
  if (dgate_part)                                                                             \
    hipLaunchKernelGGL((router_dx_kernel<TA, KC, true>), grid, dim3(kThreads), lds, s,        \
                       dxp, pos, idx, gate, dgate, wr, dxo, ws_dl_perm, dm.T, vpr, dm.d, dm.k, \
                       dm.E, dgate_part, nparts, dgate_out, bc, static_cast<int32_t>(tpw),     \
                       dl_tok);                                                                \
  else                                                                                        \
    hipLaunchKernelGGL((router_dx_kernel<TA, KC, false>), grid, dim3(kThreads), lds, s, dxp,  \
                       pos, idx, gate, dgate, wr, dxo, ws_dl_perm, dm.T, vpr, dm.d, dm.k,     \
                       dm.E, dgate_part, nparts, dgate_out, bc, static_cast<int32_t>(tpw),     \
                       dl_tok)
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
  if (mfma) {
    const int S = route_bwd_mfma_splits(dm);
    const int32_t L = static_cast<int32_t>(route_bwd_mfma_len(dm));
    const dim3 g1(dm.d / kDwBN, S);
    const bf16_t* xb = static_cast<const bf16_t*>(x);
#define MOE_DW(N, KC)                                                                         \
  hipLaunchKernelGGL((router_dwr_mfma_kernel<N, KC>), g1, dim3(kThreads), 0, s, xb, idx,       \
                     dl_tok, ws_partial, dm.T, dm.d, dm.E, dm.k, S, L)
#define MOE_DW_K(N)                                                  \
  switch (dm.k) {                                                    \
    case 1: MOE_DW(N, 1); break;                                     \
    case 2: MOE_DW(N, 2); break;                                     \
    case 4: MOE_DW(N, 4); break;                                     \
    case 6: MOE_DW(N, 6); break;                                     \
    case 8: MOE_DW(N, 8); break;                                     \
    default: MOE_DW(N, 0); break;                                    \
  }
    switch (route_bwd_mfma_ld(dm)) {
      case 16: MOE_DW_K(1) break;
      case 32: MOE_DW_K(2) break;
      default: MOE_DW_K(4) break;
    }
#undef MOE_DW_K
#undef MOE_DW
    hipLaunchKernelGGL(router_dwr_reduce_kernel<16>, dim3((dm.d + 63) / 64, dm.E), dim3(kThreads),
                       0, s, ws_partial, dwr, dm.E, dm.d, S);
    return hipGetLastError();
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
  hipLaunchKernelGGL(router_dwr_reduce_kernel<4>, dim3((dm.d + 63) / 64, dm.E), dim3(kThreads),
                     0, s, ws_partial, dwr, dm.E, dm.d, splits);
  return hipGetLastError();
}

// splits over tokens for the dense router weight gradient: about 2048
// workgroups, at most 256 splits, at least 64 tokens per split
int route_bwd_dense_splits(const moe_dims& dm) {
  const int64_t base = static_cast<int64_t>((dm.d + 255) / 256) * ((dm.E + kDwEB - 1) / kDwEB);
  int64_t s = (2048 + base - 1) / base;
  s = std::min<int64_t>(s, std::max<int64_t>(dm.T / 64, 1));
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(s, 256)));
}

hipError_t launch_route_bwd_dense(const moe_dims& dm, const void* x, const float* wr,
                                  const float* logits, const int32_t* idx, const float* gate,
                                  const float* dgate, const int32_t* pos, const void* dx_perm,
                                  int32_t G, const int32_t* count, float aux_coef, float z_coef,
                                  void* dx, float* dwr, float* dlogits, float* ws_dl,
                                  float* ws_partial, hipStream_t s) {
  if (dm.T > 0) {
    const int64_t n = dm.T / std::max(G, 1);
    const float f_scale = static_cast<float>(1.0 / (static_cast<double>(n) * dm.k));
    const float aux_scale =
        static_cast<float>(aux_coef * static_cast<double>(dm.E) / (static_cast<double>(G) * n));
    const float z_scale = static_cast<float>(z_coef * 2.0 / static_cast<double>(dm.T));
    const dim3 g1((dm.T + 3) / 4);
#define MOE_DL(EPL)                                                                            \
  hipLaunchKernelGGL((router_dl_dense_kernel<EPL>), g1, dim3(kThreads), 0, s, logits, idx, gate, \
                     dgate, count, static_cast<int32_t>(n), f_scale, aux_scale, z_scale, ws_dl,  \
                     dlogits, dm.T, dm.k, dm.E)
    if (dm.E <= 64) MOE_DL(1);
    else if (dm.E <= 128) MOE_DL(2);
    else MOE_DL(4);
#undef MOE_DL
    const int ncb = (dm.d + 255) / 256;
    const int64_t waves = ((dm.T + kDxTok - 1) / kDxTok) * ncb;
    const dim3 g2((waves + 3) / 4);
    const size_t lds = static_cast<size_t>(4) * ((dm.E + 7) & ~7) * kDxTok * sizeof(float);
#define MOE_DXD(TA, KC)                                                                       \
  hipLaunchKernelGGL((router_dx_dense_kernel<TA, KC>), g2, dim3(kThreads), lds, s,             \
                     static_cast<const TA*>(dx_perm), pos, ws_dl, wr, static_cast<TA*>(dx),  \
                     dm.T, dm.d, dm.k, dm.E)
#define MOE_DXD_K(TA)                  \
  switch (dm.k) {                      \
    case 1: MOE_DXD(TA, 1); break;     \
    case 2: MOE_DXD(TA, 2); break;     \
    case 4: MOE_DXD(TA, 4); break;     \
    case 6: MOE_DXD(TA, 6); break;     \
    case 8: MOE_DXD(TA, 8); break;     \
    default: MOE_DXD(TA, 0); break;    \
  }
    if (dm.act == MOE_BF16) {
      MOE_DXD_K(bf16_t)
    } else {
      MOE_DXD_K(float)
    }
#undef MOE_DXD_K
#undef MOE_DXD
  }
  const int splits = route_bwd_dense_splits(dm);
  const dim3 g3((dm.d + 255) / 256, (dm.E + kDwEB - 1) / kDwEB, splits);
  if (dm.act == MOE_BF16)
    hipLaunchKernelGGL(router_dwr_dense_partial_kernel<bf16_t>, g3, dim3(kThreads), 0, s,
                       static_cast<const bf16_t*>(x), ws_dl, ws_partial, dm.T, dm.d, dm.E, splits);
  else
    hipLaunchKernelGGL(router_dwr_dense_partial_kernel<float>, g3, dim3(kThreads), 0, s,
                       static_cast<const float*>(x), ws_dl, ws_partial, dm.T, dm.d, dm.E, splits);
  hipLaunchKernelGGL(router_dwr_reduce_kernel<16>, dim3((dm.d + 63) / 64, dm.E), dim3(kThreads),
                     0, s, ws_partial, dwr, dm.E, dm.d, splits);
  return hipGetLastError();
}

}  // namespace moe
