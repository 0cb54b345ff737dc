// Host side of libmoe: argument validation, workspace carving, kernel launch
// and error reporting behind the C ABI declared in moe.h.
//
// Nothing here allocates device memory or synchronises: every entry point
// validates its arguments, then enqueues kernels on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"

namespace {

thread_local char g_last_error[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

moe_status ok() {
  g_last_error[0] = '\0';
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A required pointer may be NULL only when the tensor it addresses is empty.
#define MOE_REQUIRE_PTR(p, n)                                                                \
  do {                                                                                       \
    if (!(p) && (n) > 0)                                                                     \
      return fail(MOE_ERR_INVALID_ARGUMENT, "%s: '%s' is NULL", __func__, #p);               \
    if (!aligned16(p))                                                                       \
      return fail(MOE_ERR_INVALID_ARGUMENT, "%s: '%s' is not 16-byte aligned", __func__, #p); \
  } while (0)

#define MOE_REQUIRE_PTR_FN(p, n, fn)                                                         \
  do {                                                                                       \
    if (!(p) && (n) > 0)                                                                     \
      return fail(MOE_ERR_INVALID_ARGUMENT, "%s: '%s' is NULL", fn, #p);                     \
    if (!aligned16(p))                                                                       \
      return fail(MOE_ERR_INVALID_ARGUMENT, "%s: '%s' is not 16-byte aligned", fn, #p);      \
  } while (0)

#define MOE_OPTIONAL_PTR_FN(p, fn)                                                           \
  do {                                                                                       \
    if ((p) && !aligned16(p))                                                                \
      return fail(MOE_ERR_INVALID_ARGUMENT, "%s: '%s' is not 16-byte aligned", fn, #p);      \
  } while (0)

#define MOE_OPTIONAL_PTR(p)                                                                  \
  do {                                                                                       \
    if ((p) && !aligned16(p))                                                                \
      return fail(MOE_ERR_INVALID_ARGUMENT, "%s: '%s' is not 16-byte aligned", __func__, #p); \
  } while (0)

moe_status check_dims(const moe_dims* dm, const char* fn) {
  if (!dm) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: dims is NULL", fn);
  if (dm->T < 0 || dm->d <= 0 || dm->E <= 0 || dm->f <= 0 || dm->k <= 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need T >= 0 and d, E, f, k > 0 (T=%lld d=%d E=%d f=%d k=%d)",
                fn, static_cast<long long>(dm->T), dm->d, dm->E, dm->f, dm->k);
  if (dm->E > 256) return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d > 256", fn, dm->E);
  if (dm->k > dm->E || dm->k > 16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: k=%d must be <= min(E, 16)", fn, dm->k);
  if (dm->d % 64 || dm->f % 64)
    return fail(MOE_ERR_UNSUPPORTED, "%s: d=%d and f=%d must be multiples of 64", fn, dm->d, dm->f);
  if (dm->T * static_cast<int64_t>(dm->k) >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: T*k must be < 2^31", fn);
  if (dm->act != MOE_F32 && dm->act != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: act=%d is neither MOE_F32 nor MOE_BF16", fn, dm->act);
  return MOE_OK;
}

size_t elem_size(const moe_dims& dm) { return dm.act == MOE_BF16 ? 2 : 4; }

// ---------------------------------------------------------------- workspace layout
// Each entry point carves the caller's workspace from offset 0; the required
// size is the maximum over entry points.
struct Carver {
  size_t off = 0;
  template <typename T>
  T* take(void* base, size_t count) {
    T* p = base ? reinterpret_cast<T*>(static_cast<char*>(base) + off) : nullptr;
    off += moe::align256(count * sizeof(T));
    return p;
  }
};

// Tokens per router workgroup: the matrix-core routers (64-token tiles for
// bf16, 16-token tiles for fp32) run when those tiles never straddle two
// balancing blocks.
int route_tile(int64_t T, int32_t G, int32_t act) {
  const int mt = (act == MOE_F32) ? moe::kRouteF32Tile : moe::kRouteMfmaTile;
  if (G <= 1 || (T / G) % mt == 0) return mt;
  if (G <= 1) return moe::kRouteTileMax;
  const int64_t per = T / G;
  int tile = moe::kRouteTileMax;
  while (tile > 1 && per % tile) tile >>= 1;
  return tile;
}

struct RouteWs {
  float* psum;
  int32_t* pcnt;
  int32_t* ptie;
  size_t bytes;
};
RouteWs route_ws(const moe_dims& dm, int tile, void* ws) {
  const int64_t n_tiles = (dm.T + tile - 1) / tile;
  Carver c;
  RouteWs r;
  const int64_t ep4 = (dm.E + 3) & ~3;   // partial rows padded to 16 bytes
  r.psum = c.take<float>(ws, n_tiles * ep4);
  r.pcnt = c.take<int32_t>(ws, n_tiles * ep4);
  r.ptie = c.take<int32_t>(ws, std::max<int64_t>(n_tiles, 1));
  r.bytes = c.off;
  return r;
}

struct PermWs {
  int32_t* hist;
  int32_t* base;
  size_t bytes;
};
PermWs perm_ws(int64_t T, int32_t keys, void* ws) {
  const int64_t nb = std::max<int64_t>((T + moe::kPermBlock - 1) / moe::kPermBlock, 1);
  Carver c;
  PermWs r;
  r.hist = c.take<int32_t>(ws, nb * keys);
  r.base = c.take<int32_t>(ws, nb * keys);
  r.bytes = c.off;
  return r;
}

// fp32 partial tiles of the split-K weight gradients
size_t wgrad_ws_bytes(const moe_dims& dm, bool wgrad_f32) {
  return dm.act == MOE_BF16 ? moe::wgrad_partial_bytes_bf16(dm, wgrad_f32) : 0;
}

// da, db and the weight-gradient partials; with `recompute` also a, b, h of
// the forward pass, which the call then recomputes from the expert input
struct BwdWs {
  void* da;
  void* db;
  float* partial;
  void* a;
  void* b;
  void* h;
  size_t bytes;
};
BwdWs bwd_ws(const moe_dims& dm, void* ws, bool recompute = false, bool wgrad_f32 = false) {
  const int64_t R = dm.T * dm.k;
  const size_t rf = R * dm.f * elem_size(dm);
  Carver c;
  BwdWs r{};
  r.da = c.take<char>(ws, rf);
  r.db = c.take<char>(ws, rf);
  r.partial = c.take<float>(ws, wgrad_ws_bytes(dm, wgrad_f32) / sizeof(float));
  if (recompute) {
    r.a = c.take<char>(ws, rf);
    r.b = c.take<char>(ws, rf);
    r.h = c.take<char>(ws, rf);
  }
  r.bytes = c.off;
  return r;
}

struct RouteBwdWs {
  float* dl_perm;
  float* dl_sel;
  float* partial;
  size_t bytes;
};
RouteBwdWs route_bwd_ws(const moe_dims& dm, void* ws) {
  const int64_t R = dm.T * dm.k;
  Carver c;
  RouteBwdWs r;
  r.dl_perm = c.take<float>(ws, std::max<int64_t>(R, 1));
  r.dl_sel = c.take<float>(ws, std::max<int64_t>(R, 1));
  const bool mfma = moe::route_bwd_mfma_ok(dm);
  const int64_t splits = mfma ? moe::route_bwd_mfma_splits(dm) : moe::route_bwd_splits(dm);
  r.partial = c.take<float>(ws, static_cast<int64_t>(dm.E) * splits * dm.d);
  r.bytes = c.off;
  return r;
}

struct RouteBwdDenseWs {
  float* dl;
  float* partial;
  size_t bytes;
};
RouteBwdDenseWs route_bwd_dense_ws(const moe_dims& dm, void* ws) {
  Carver c;
  RouteBwdDenseWs r;
  r.dl = c.take<float>(ws, dm.T * dm.E + 16);   // + the dWr kernel's read-ahead pad
  r.partial =
      c.take<float>(ws, static_cast<int64_t>(dm.E) * moe::route_bwd_dense_splits(dm) * dm.d);
  r.bytes = c.off;
  return r;
}

struct VariantWs {
  int32_t* hist;
  float* zpart;
  size_t bytes;
};
VariantWs variant_ws(const moe_dims& dm, int32_t G, void* ws) {
  Carver c;
  VariantWs r;
  const int32_t g = std::max(G, 1);
  r.hist = c.take<int32_t>(ws, static_cast<int64_t>(g) * moe::capacity_chunks(dm.T, g) * dm.k * dm.E);
  r.zpart = c.take<float>(ws, static_cast<int64_t>(g) * moe::zloss_chunks(dm.T, g));
  r.bytes = c.off;
  return r;
}

struct PlanWs {
  uint64_t* mask;
  int32_t* hist;
  int32_t* base;
  int32_t* stat;
  size_t bytes;
};
PlanWs plan_ws(int64_t T, int32_t G, void* ws) {
  const int64_t nb = std::max<int64_t>((T + moe::kPermBlock - 1) / moe::kPermBlock, 1);
  Carver c;
  PlanWs r;
  r.mask = c.take<uint64_t>(ws, std::max<int64_t>(T, 1));
  r.hist = c.take<int32_t>(ws, nb * G);
  r.base = c.take<int32_t>(ws, nb * G);
  r.stat = c.take<int32_t>(ws, nb * 3);
  r.bytes = c.off;
  return r;
}

size_t workspace_needed(const moe_dims& dm, int32_t n_groups) {
  const int32_t G = std::max(n_groups, 1);
  size_t need = route_ws(dm, 1, nullptr).bytes;  // tile 1 is the largest layout
  need = std::max(need, perm_ws(dm.T, dm.E, nullptr).bytes);
  need = std::max(need, bwd_ws(dm, nullptr, false, false).bytes);
  need = std::max(need, bwd_ws(dm, nullptr, false, true).bytes);
  need = std::max(need, route_bwd_ws(dm, nullptr).bytes);
  need = std::max(need, route_bwd_dense_ws(dm, nullptr).bytes);
  need = std::max(need, variant_ws(dm, G, nullptr).bytes);
  need = std::max(need, moe::align256(static_cast<size_t>(dm.E) * std::max(G, 64) * 4));
  need = std::max(need, plan_ws(dm.T, std::max(G, 64), nullptr).bytes);
  return need;
}

moe_status check_ws(void* ws, size_t have, size_t need, const char* fn) {
  if (need == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: workspace is not 16-byte aligned", fn);
  if (have < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, have, need);
  return MOE_OK;
}

moe_status check_placement_impl(int32_t E, int32_t G, const int32_t* placement, const char* fn) {
  if (!placement) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: placement is NULL", fn);
  if (E <= 0 || G <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need E, G > 0", fn);
  if (E % G) return fail(MOE_ERR_INVALID_PLACEMENT, "%s: G=%d does not divide E=%d", fn, G, E);
  std::vector<int32_t> per(G, 0);
  for (int32_t e = 0; e < E; ++e) {
    const int32_t g = placement[e];
    if (g < 0 || g >= G)
      return fail(MOE_ERR_INVALID_PLACEMENT, "%s: expert %d placed in group %d outside [0, %d)",
                  fn, e, g, G);
    per[g] += 1;
  }
  for (int32_t g = 0; g < G; ++g)
    if (per[g] != E / G)
      return fail(MOE_ERR_INVALID_PLACEMENT, "%s: group %d owns %d experts, expected %d", fn, g,
                  per[g], E / G);
  return MOE_OK;
}

// Gathered expert input: bf16 offsets into X are 32-bit.
moe_status check_gather(const moe_dims& dm, const void* x, const int32_t* src_token,
                        const char* fn) {
  if (!x && dm.T > 0) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: 'x' is NULL", fn);
  if (x && !aligned16(x)) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: 'x' is not 16-byte aligned", fn);
  if (!src_token && dm.T > 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: 'src_token' is NULL", fn);
  if (dm.act == MOE_BF16 && dm.T * dm.d * 2 >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: X must be under 2 GiB to be gathered", fn);
  return MOE_OK;
}

// wgrad_dtype: the type of dW1, dW3, dW2 (MOE_BF16 only for bf16 layers)
moe_status check_wgrad_dtype(const moe_dims& dm, int32_t wgrad_dtype, bool* f32, const char* fn) {
  if (wgrad_dtype != MOE_F32 && wgrad_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: wgrad_dtype=%d is neither MOE_F32 nor MOE_BF16", fn,
                wgrad_dtype);
  if (dm.act == MOE_F32 && wgrad_dtype != MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "%s: an fp32 layer keeps fp32 weight gradients", fn);
  *f32 = wgrad_dtype == MOE_F32;
  return MOE_OK;
}

// moe_grouped_swiglu_bwd and its gathered form (x_rows != NULL: xin is X)
moe_status swiglu_bwd_impl(const moe_dims* dims, const void* xin, const int32_t* x_rows,
                           bool gather, const int32_t* expert_offsets, const void* w1,
                           const void* w3, const void* w2, const void* a_save, const void* b_save,
                           const void* h_save, const void* dy_perm, void* dx_perm, void* dw1,
                           void* dw3, void* dw2, int32_t wgrad_dtype, void* workspace,
                           size_t workspace_bytes, void* stream, const char* fn) {
  moe_status st = check_dims(dims, fn);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  const int64_t R = dm.T * dm.k, W = int64_t(dm.E) * dm.f * dm.d;
  if (gather) {
    st = check_gather(dm, xin, x_rows, fn);
    if (st != MOE_OK) return st;
  } else {
    MOE_REQUIRE_PTR_FN(xin, R * dm.d, fn);
  }
  MOE_REQUIRE_PTR_FN(expert_offsets, dm.E + 1, fn);
  MOE_REQUIRE_PTR_FN(w1, W, fn);
  MOE_REQUIRE_PTR_FN(w3, W, fn);
  MOE_REQUIRE_PTR_FN(w2, W, fn);
  const int n_saved = (a_save != nullptr) + (b_save != nullptr) + (h_save != nullptr);
  if (n_saved != 0 && n_saved != 3)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: a_save, b_save and h_save are all given, or all "
                "NULL to recompute them", fn);
  const bool recompute = n_saved == 0;
  MOE_OPTIONAL_PTR_FN(a_save, fn);
  MOE_OPTIONAL_PTR_FN(b_save, fn);
  MOE_OPTIONAL_PTR_FN(h_save, fn);
  MOE_REQUIRE_PTR_FN(dy_perm, R * dm.d, fn);
  MOE_REQUIRE_PTR_FN(dx_perm, R * dm.d, fn);
  MOE_REQUIRE_PTR_FN(dw1, W, fn);
  MOE_REQUIRE_PTR_FN(dw3, W, fn);
  MOE_REQUIRE_PTR_FN(dw2, W, fn);
  bool f32 = false;
  st = check_wgrad_dtype(dm, wgrad_dtype, &f32, fn);
  if (st != MOE_OK) return st;
  st = check_ws(workspace, workspace_bytes, bwd_ws(dm, nullptr, recompute, f32).bytes, fn);
  if (st != MOE_OK) return st;
  const BwdWs w = bwd_ws(dm, workspace, recompute, f32);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (recompute) {
    st = hip_status(moe::launch_expert_up(dm, xin, x_rows, expert_offsets, w1, w3, w.a, w.b, w.h,
                                          s),
                    fn);
    if (st != MOE_OK) return st;
    a_save = w.a;
    b_save = w.b;
    h_save = w.h;
  }
  return hip_status(moe::launch_swiglu_bwd(dm, xin, x_rows, expert_offsets, w1, w3, w2, a_save,
                                           b_save, h_save, dy_perm, dx_perm, dw1, dw3, dw2, f32,
                                           w.da, w.db, w.partial, s),
                    fn);
}

// moe_expert_wgrad and its gathered form
moe_status expert_wgrad_impl(const moe_dims* dims, const void* xin, const int32_t* x_rows,
                             bool gather, const int32_t* expert_offsets, const void* h_save,
                             const void* dy_perm, const void* da, const void* db, void* dw1,
                             void* dw3, void* dw2, int32_t wgrad_dtype, void* workspace,
                             size_t workspace_bytes, void* stream, const char* fn) {
  moe_status st = check_dims(dims, fn);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  const int64_t R = dm.T * dm.k, W = int64_t(dm.E) * dm.f * dm.d;
  if (gather) {
    st = check_gather(dm, xin, x_rows, fn);
    if (st != MOE_OK) return st;
  } else {
    MOE_REQUIRE_PTR_FN(xin, R * dm.d, fn);
  }
  MOE_REQUIRE_PTR_FN(expert_offsets, dm.E + 1, fn);
  MOE_REQUIRE_PTR_FN(h_save, R * dm.f, fn);
  MOE_REQUIRE_PTR_FN(dy_perm, R * dm.d, fn);
  MOE_REQUIRE_PTR_FN(da, R * dm.f, fn);
  MOE_REQUIRE_PTR_FN(db, R * dm.f, fn);
  MOE_REQUIRE_PTR_FN(dw1, W, fn);
  MOE_REQUIRE_PTR_FN(dw3, W, fn);
  MOE_REQUIRE_PTR_FN(dw2, W, fn);
  bool f32 = false;
  st = check_wgrad_dtype(dm, wgrad_dtype, &f32, fn);
  if (st != MOE_OK) return st;
  st = check_ws(workspace, workspace_bytes, wgrad_ws_bytes(dm, f32), fn);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_expert_wgrad(dm, xin, x_rows, expert_offsets, h_save, dy_perm, da,
                                             db, dw1, dw3, dw2, f32,
                                             static_cast<float*>(workspace),
                                             static_cast<hipStream_t>(stream)),
                    fn);
}

}  // namespace

extern "C" {

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_INVALID_PLACEMENT: return "MOE_ERR_INVALID_PLACEMENT";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error; }

size_t moe_workspace_bytes(const moe_dims* dims, int32_t n_groups) {
  if (check_dims(dims, __func__) != MOE_OK) return 0;
  return workspace_needed(*dims, n_groups);
}

size_t moe_grouped_swiglu_bwd_workspace_bytes(const moe_dims* dims, int32_t recompute) {
  if (check_dims(dims, __func__) != MOE_OK) return 0;
  return std::max(bwd_ws(*dims, nullptr, recompute != 0, false).bytes,
                  bwd_ws(*dims, nullptr, recompute != 0, true).bytes);
}

int32_t moe_expert_wgrad_launches(const moe_dims* dims) {
  if (check_dims(dims, __func__) != MOE_OK) return 0;
  if (dims->act != MOE_BF16) return 1;
  return moe::wgrad_splits_bf16(*dims) > 1 ? 2 : 1;
}

namespace {
moe_status route_impl(const moe_dims* dims, const void* x, const float* w_router, float* logits,
                     int32_t* topk_idx, float* topk_gate, float* margin, float near_tie_eps,
                     int32_t* near_tie_count, int32_t n_groups, int32_t* group_count,
                     float* group_mean_prob, float* group_aux, void* workspace,
                     size_t workspace_bytes, void* stream, const char* fn) {
  moe_status st = check_dims(dims, fn);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR_FN(x, dm.T * dm.d, fn);
  MOE_REQUIRE_PTR_FN(w_router, int64_t(dm.E) * dm.d, fn);
  MOE_REQUIRE_PTR_FN(logits, dm.T * dm.E, fn);
  MOE_REQUIRE_PTR_FN(topk_idx, dm.T * dm.k, fn);
  MOE_REQUIRE_PTR_FN(topk_gate, dm.T * dm.k, fn);
  MOE_REQUIRE_PTR_FN(margin, dm.T, fn);
  MOE_REQUIRE_PTR_FN(near_tie_count, 1, fn);
  MOE_OPTIONAL_PTR_FN(group_count, fn);
  MOE_OPTIONAL_PTR_FN(group_mean_prob, fn);
  MOE_OPTIONAL_PTR_FN(group_aux, fn);
  if (n_groups < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: n_groups=%d must be >= 1", fn, n_groups);
  if (dm.T % n_groups)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: n_groups=%d does not divide T=%lld", fn,
                n_groups, static_cast<long long>(dm.T));
  if (!std::isfinite(near_tie_eps))
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: near_tie_eps is not finite", fn);
  const int tile = route_tile(dm.T, n_groups, dm.act);
  if ((dm.T + tile - 1) / tile * int64_t((dm.E + 3) & ~3) * 4 >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: T=%lld with %d balancing groups needs over 2 GiB of "
                "router partial sums", fn, static_cast<long long>(dm.T), n_groups);
  const RouteWs need = route_ws(dm, tile, nullptr);
  st = check_ws(workspace, workspace_bytes, need.bytes, fn);
  if (st != MOE_OK) return st;
  const RouteWs w = route_ws(dm, tile, workspace);
  return hip_status(moe::launch_route(dm, x, w_router, logits, topk_idx, topk_gate, margin,
                                      near_tie_eps, near_tie_count, n_groups, group_count,
                                      group_mean_prob, group_aux, tile, w.psum, w.pcnt, w.ptie,
                                      static_cast<hipStream_t>(stream)),
                    fn);
}
}  // namespace

moe_status moe_route(const moe_dims* dims, const void* x, const float* w_router, float* logits,
                     int32_t* topk_idx, float* topk_gate, float* margin, float near_tie_eps,
                     int32_t* near_tie_count, int32_t n_groups, int32_t* group_count,
                     float* group_mean_prob, float* group_aux, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return route_impl(dims, x, w_router, logits, topk_idx, topk_gate, margin, near_tie_eps,
                    near_tie_count, n_groups, group_count, group_mean_prob, group_aux, workspace,
                    workspace_bytes, stream, __func__);
}

// ---------------------------------------------------------------- allocation-free router
// moe_route with its scratch (the per-tile partial sums) in a
// file-scope device array instead of a caller workspace.  Each device holds
// its own copy of the array; host code never passes the array's name (a host
// stand-in, not a device address) but the address hipGetSymbolAddress gives
// for the current device, looked up once per device and kept.
namespace {
constexpr size_t kScratchBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_address(void** out, const char* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d is beyond the %d devices the static scratch "
                "table covers", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (!p) return fail(MOE_ERR_HIP, "%s: hipGetSymbolAddress returned NULL", fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

size_t moe_route_noalloc_max_bytes(void) { return kScratchBytes; }

moe_status moe_route_noalloc(const moe_dims* dims, const void* x, const float* w_router,
                             float* logits, int32_t* topk_idx, float* topk_gate, float* margin,
                             float near_tie_eps, int32_t* near_tie_count, int32_t n_groups,
                             int32_t* group_count, float* group_mean_prob, float* group_aux,
                             void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  if (n_groups >= 1 && dims->T % n_groups == 0) {
    const int tile = route_tile(dims->T, n_groups, dims->act);
    const size_t need = route_ws(*dims, tile, nullptr).bytes;
    if (need > kScratchBytes)
      return fail(MOE_ERR_UNSUPPORTED, "%s: these dims need %zu bytes of router scratch; the "
                  "library's static scratch holds %zu (use moe_route with a workspace)",
                  __func__, need, kScratchBytes);
  }
  void* ws = nullptr;
  st = scratch_address(&ws, __func__);
  if (st != MOE_OK) return st;
  return route_impl(dims, x, w_router, logits, topk_idx, topk_gate, margin, near_tie_eps,
                    near_tie_count, n_groups, group_count, group_mean_prob, group_aux, ws,
                    kScratchBytes, stream, __func__);
}

moe_status moe_permute(const moe_dims* dims, const int32_t* topk_idx, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* pos, int32_t* src_token, const void* x,
                       void* x_perm, void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(topk_idx, dm.T * dm.k);
  MOE_REQUIRE_PTR(expert_counts, dm.E);
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(pos, dm.T * dm.k);
  MOE_REQUIRE_PTR(src_token, dm.T * dm.k);
  if ((x == nullptr) != (x_perm == nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: pass both x and x_perm, or neither", __func__);
  MOE_OPTIONAL_PTR(x);
  MOE_OPTIONAL_PTR(x_perm);
  const PermWs need = perm_ws(dm.T, dm.E, nullptr);
  st = check_ws(workspace, workspace_bytes, need.bytes, __func__);
  if (st != MOE_OK) return st;
  const PermWs w = perm_ws(dm.T, dm.E, workspace);
  return hip_status(moe::launch_permute(dm, topk_idx, expert_counts, expert_offsets, pos,
                                        src_token, x, x_perm, w.hist, w.base,
                                        static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_grouped_swiglu_fwd(const moe_dims* dims, const void* x_perm,
                                  const int32_t* expert_offsets, const void* w1, const void* w3,
                                  const void* w2, void* a_save, void* b_save, void* h_save,
                                  void* y_perm, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(x_perm, dm.T * dm.k * dm.d);
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(w1, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(w3, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(w2, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(a_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(b_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(h_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(y_perm, dm.T * dm.k * dm.d);
  return hip_status(moe::launch_swiglu_fwd(dm, x_perm, nullptr, expert_offsets, w1, w3, w2, a_save,
                                           b_save, h_save, y_perm,
                                           static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_combine(const moe_dims* dims, const void* rows, const int32_t* pos,
                       const float* gate, void* out, void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(rows, dm.T * dm.k * dm.d);
  MOE_REQUIRE_PTR(pos, dm.T * dm.k);
  MOE_OPTIONAL_PTR(gate);
  MOE_REQUIRE_PTR(out, dm.T * dm.d);
  return hip_status(moe::launch_combine(*dims, rows, pos, gate, out,
                                        static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_combine_bwd(const moe_dims* dims, const void* dy, const void* y_perm,
                           const int32_t* pos, const float* gate, void* dy_perm, float* dgate,
                           void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(dy, dm.T * dm.d);
  MOE_REQUIRE_PTR(y_perm, dm.T * dm.k * dm.d);
  MOE_REQUIRE_PTR(pos, dm.T * dm.k);
  MOE_REQUIRE_PTR(gate, dm.T * dm.k);
  MOE_REQUIRE_PTR(dy_perm, dm.T * dm.k * dm.d);
  MOE_REQUIRE_PTR(dgate, dm.T * dm.k);
  return hip_status(moe::launch_combine_bwd(*dims, dy, y_perm, pos, gate, dy_perm, dgate,
                                            static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_grouped_swiglu_bwd(const moe_dims* dims, const void* x_perm,
                                  const int32_t* expert_offsets, const void* w1, const void* w3,
                                  const void* w2, const void* a_save, const void* b_save,
                                  const void* h_save, const void* dy_perm, void* dx_perm,
                                  void* dw1, void* dw3, void* dw2, int32_t wgrad_dtype,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return swiglu_bwd_impl(dims, x_perm, nullptr, false, expert_offsets, w1, w3, w2, a_save, b_save,
                         h_save, dy_perm, dx_perm, dw1, dw3, dw2, wgrad_dtype, workspace,
                         workspace_bytes, stream, __func__);
}

moe_status moe_expert_up(const moe_dims* dims, const void* x_perm,
                         const int32_t* expert_offsets, const void* w1, const void* w3,
                         void* a_save, void* b_save, void* h_save, void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(x_perm, dm.T * dm.k * dm.d);
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(w1, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(w3, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(a_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(b_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(h_save, dm.T * dm.k * dm.f);
  return hip_status(moe::launch_expert_up(dm, x_perm, nullptr, expert_offsets, w1, w3, a_save, b_save,
                                          h_save, static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_expert_down(const moe_dims* dims, const void* h_save,
                           const int32_t* expert_offsets, const void* w2, void* y_perm,
                           void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(h_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(w2, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(y_perm, dm.T * dm.k * dm.d);
  return hip_status(moe::launch_expert_down(dm, h_save, expert_offsets, w2, y_perm,
                                            static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_expert_dgrad_down(const moe_dims* dims, const void* dy_perm,
                                 const int32_t* expert_offsets, const void* w2,
                                 const void* a_save, const void* b_save, void* da, void* db,
                                 void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(dy_perm, dm.T * dm.k * dm.d);
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(w2, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(a_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(b_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(da, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(db, dm.T * dm.k * dm.f);
  return hip_status(moe::launch_expert_dgrad_down(dm, dy_perm, expert_offsets, w2, a_save, b_save,
                                                  da, db, static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_expert_dgrad_up(const moe_dims* dims, const void* da, const void* db,
                               const int32_t* expert_offsets, const void* w1, const void* w3,
                               void* dx_perm, void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(da, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(db, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(w1, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(w3, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(dx_perm, dm.T * dm.k * dm.d);
  return hip_status(moe::launch_expert_dgrad_up(dm, da, db, expert_offsets, w1, w3, dx_perm,
                                                static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_expert_wgrad(const moe_dims* dims, const void* x_perm,
                            const int32_t* expert_offsets, const void* h_save,
                            const void* dy_perm, const void* da, const void* db, void* dw1,
                            void* dw3, void* dw2, int32_t wgrad_dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return expert_wgrad_impl(dims, x_perm, nullptr, false, expert_offsets, h_save, dy_perm, da, db,
                           dw1, dw3, dw2, wgrad_dtype, workspace, workspace_bytes, stream,
                           __func__);
}

moe_status moe_route_bwd(const moe_dims* dims, const void* x, const float* w_router,
                         const int32_t* topk_idx, const float* topk_gate, const float* dgate,
                         const int32_t* expert_offsets, const int32_t* pos,
                         const int32_t* src_token, const void* dx_perm, void* dx,
                         float* dw_router, void* workspace, size_t workspace_bytes,
                         void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(x, dm.T * dm.d);
  MOE_REQUIRE_PTR(w_router, int64_t(dm.E) * dm.d);
  MOE_REQUIRE_PTR(topk_idx, dm.T * dm.k);
  MOE_REQUIRE_PTR(topk_gate, dm.T * dm.k);
  MOE_REQUIRE_PTR(dgate, dm.T * dm.k);
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(pos, dm.T * dm.k);
  MOE_REQUIRE_PTR(src_token, dm.T * dm.k);
  MOE_OPTIONAL_PTR(dx_perm);
  MOE_REQUIRE_PTR(dx, dm.T * dm.d);
  MOE_REQUIRE_PTR(dw_router, int64_t(dm.E) * dm.d);
  const RouteBwdWs need = route_bwd_ws(dm, nullptr);
  st = check_ws(workspace, workspace_bytes, need.bytes, __func__);
  if (st != MOE_OK) return st;
  const RouteBwdWs w = route_bwd_ws(dm, workspace);
  return hip_status(moe::launch_route_bwd(dm, x, w_router, topk_idx, topk_gate, dgate,
                                          expert_offsets, pos, src_token, dx_perm, dx, dw_router,
                                          w.dl_perm, w.dl_sel, w.partial,
                                          static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_coselect(int64_t T, int32_t k, int32_t E, const int32_t* topk_idx,
                        int32_t* coselect, void* stream) {
  if (T < 0 || k <= 0 || E <= 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need T >= 0 and k, E > 0", __func__);
  if (E > 256 || k > E || k > 16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: need E <= 256 and k <= min(E, 16)", __func__);
  if (T * k >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: T*k must be < 2^31", __func__);
  MOE_REQUIRE_PTR(topk_idx, T * k);
  MOE_REQUIRE_PTR(coselect, int64_t(E) * E);
  return hip_status(moe::launch_coselect(T, k, E, topk_idx, coselect,
                                         static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_check_placement(int32_t E, int32_t G, const int32_t* placement) {
  const moe_status st = check_placement_impl(E, G, placement, __func__);
  return st == MOE_OK ? ok() : st;
}

moe_status moe_dispatch_plan(int64_t T, int32_t k, int32_t E, int32_t G, const int32_t* topk_idx,
                             const int32_t* placement, int32_t* n_dest, int32_t* group_rows,
                             int32_t* group_offsets, int32_t* row_token, int32_t* assign_row,
                             int32_t* stats, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (T < 0 || k <= 0 || E <= 0 || G <= 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need T >= 0 and k, E, G > 0", __func__);
  if (E > 256 || k > E || k > 16 || G > 64)
    return fail(MOE_ERR_UNSUPPORTED, "%s: need E <= 256, k <= min(E, 16), G <= 64", __func__);
  if (T * k >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: T*k must be < 2^31", __func__);
  if (T % G)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: G=%d does not divide T=%lld", __func__, G,
                static_cast<long long>(T));
  moe_status st = check_placement_impl(E, G, placement, __func__);
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR(topk_idx, T * k);
  MOE_REQUIRE_PTR(n_dest, T);
  MOE_REQUIRE_PTR(group_rows, G);
  MOE_REQUIRE_PTR(group_offsets, G + 1);
  MOE_REQUIRE_PTR(row_token, T * k);
  MOE_REQUIRE_PTR(assign_row, T * k);
  MOE_REQUIRE_PTR(stats, 4);
  const PlanWs need = plan_ws(T, G, nullptr);
  st = check_ws(workspace, workspace_bytes, need.bytes, __func__);
  if (st != MOE_OK) return st;
  const PlanWs w = plan_ws(T, G, workspace);
  moe::PlacementArg pl{};
  for (int32_t e = 0; e < E; ++e) pl.group_of[e] = placement[e];
  return hip_status(moe::launch_dispatch_plan(T, k, E, G, topk_idx, pl, n_dest, group_rows,
                                              group_offsets, row_token, assign_row, stats, w.mask,
                                              w.hist, w.base, w.stat,
                                              static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_placement_greedy(int32_t E, int32_t G, const int64_t* coselect,
                                int32_t* placement) {
  if (!coselect || !placement)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: NULL argument", __func__);
  if (E <= 0 || G <= 0 || E > 256)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need 0 < E <= 256 and G > 0", __func__);
  if (E % G) return fail(MOE_ERR_INVALID_PLACEMENT, "%s: G=%d does not divide E=%d", __func__, G, E);
  const int32_t cap = E / G;
  std::vector<char> free_(E, 1);
  std::vector<int64_t> mass(E, 0);   // co-selection count to the still-unassigned experts
  for (int32_t e = 0; e < E; ++e)
    for (int32_t o = 0; o < E; ++o)
      if (o != e) mass[e] += coselect[static_cast<int64_t>(e) * E + o];
  auto take = [&](int32_t e) {
    free_[e] = 0;
    for (int32_t o = 0; o < E; ++o)
      if (free_[o]) mass[o] -= coselect[static_cast<int64_t>(o) * E + e];
  };
  std::vector<int64_t> link(E, 0);   // co-selection count to the current group's members
  for (int32_t g = 0; g < G; ++g) {
    int32_t seed = -1;
    for (int32_t e = 0; e < E; ++e)
      if (free_[e] && (seed < 0 || mass[e] > mass[seed])) seed = e;
    std::fill(link.begin(), link.end(), 0);
    int32_t members = 0;
    int32_t pick = seed;
    while (true) {
      placement[pick] = g;
      take(pick);
      ++members;
      for (int32_t o = 0; o < E; ++o) link[o] += coselect[static_cast<int64_t>(o) * E + pick];
      if (members == cap) break;
      pick = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (!free_[e]) continue;
        if (pick < 0 || link[e] > link[pick] || (link[e] == link[pick] && mass[e] > mass[pick]))
          pick = e;
      }
    }
  }
  return ok();
}


// ---------------------------------------------------------------- gathered expert input
// The expert input row p is X[src_token[p]] (the table moe_permute writes), so
// x_perm is never materialised (check_gather above holds the limits).

moe_status moe_expert_up_gather(const moe_dims* dims, const void* x, const int32_t* src_token,
                                const int32_t* expert_offsets, const void* w1, const void* w3,
                                void* a_save, void* b_save, void* h_save, void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  st = check_gather(dm, x, src_token, __func__);
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(w1, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(w3, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(a_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(b_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(h_save, dm.T * dm.k * dm.f);
  return hip_status(moe::launch_expert_up(dm, x, src_token, expert_offsets, w1, w3, a_save,
                                          b_save, h_save, static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_expert_wgrad_gather(const moe_dims* dims, const void* x,
                                   const int32_t* src_token, const int32_t* expert_offsets,
                                   const void* h_save, const void* dy_perm, const void* da,
                                   const void* db, void* dw1, void* dw3, void* dw2,
                                   int32_t wgrad_dtype, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return expert_wgrad_impl(dims, x, src_token, true, expert_offsets, h_save, dy_perm, da, db, dw1,
                           dw3, dw2, wgrad_dtype, workspace, workspace_bytes, stream, __func__);
}

moe_status moe_grouped_swiglu_fwd_gather(const moe_dims* dims, const void* x,
                                         const int32_t* src_token,
                                         const int32_t* expert_offsets, const void* w1,
                                         const void* w3, const void* w2, void* a_save,
                                         void* b_save, void* h_save, void* y_perm,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  st = check_gather(dm, x, src_token, __func__);
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(w1, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(w3, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(w2, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(a_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(b_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(h_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(y_perm, dm.T * dm.k * dm.d);
  return hip_status(moe::launch_swiglu_fwd(dm, x, src_token, expert_offsets, w1, w3, w2, a_save,
                                           b_save, h_save, y_perm,
                                           static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_grouped_swiglu_bwd_gather(const moe_dims* dims, const void* x,
                                         const int32_t* src_token,
                                         const int32_t* expert_offsets, const void* w1,
                                         const void* w3, const void* w2, const void* a_save,
                                         const void* b_save, const void* h_save,
                                         const void* dy_perm, void* dx_perm, void* dw1,
                                         void* dw3, void* dw2, int32_t wgrad_dtype,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  return swiglu_bwd_impl(dims, x, src_token, true, expert_offsets, w1, w3, w2, a_save, b_save,
                         h_save, dy_perm, dx_perm, dw1, dw3, dw2, wgrad_dtype, workspace,
                         workspace_bytes, stream, __func__);
}

// ---------------------------------------------------------------- EP dispatch on one device
moe_status moe_dispatch_pack(const moe_dims* dims, int32_t G, const void* x,
                             const int32_t* group_offsets, const int32_t* row_token, void* send,
                             void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  if (G <= 0 || G > 64)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need 1 <= G <= 64", __func__);
  MOE_REQUIRE_PTR(x, dm.T * dm.d);
  MOE_REQUIRE_PTR(group_offsets, G + 1);
  MOE_REQUIRE_PTR(row_token, dm.T * dm.k);
  MOE_REQUIRE_PTR(send, dm.T * dm.k * dm.d);
  return hip_status(moe::launch_ep_pack(dm, G, x, group_offsets, row_token, send,
                                        static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_dispatch_expand(const moe_dims* dims, const void* recv,
                               const int32_t* assign_row, const int32_t* pos, void* x_perm,
                               void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(recv, dm.T * dm.k * dm.d);
  MOE_REQUIRE_PTR(assign_row, dm.T * dm.k);
  MOE_REQUIRE_PTR(pos, dm.T * dm.k);
  MOE_REQUIRE_PTR(x_perm, dm.T * dm.k * dm.d);
  return hip_status(moe::launch_ep_expand(dm, recv, assign_row, pos, x_perm,
                                          static_cast<hipStream_t>(stream)),
                    __func__);
}

// ---------------------------------------------------------------- definitional variants
int32_t moe_expert_capacity(int64_t T, int32_t k, int32_t E, int32_t n_groups, double factor) {
  if (T < 0 || k <= 0 || E <= 0 || n_groups <= 0 || T % n_groups || !std::isfinite(factor) ||
      factor < 0.0)
    return -1;
  const int64_t n = T / n_groups;
  const double c = std::ceil(factor * static_cast<double>(n * k) / E);
  return c >= 2147483647.0 ? 2147483647 : static_cast<int32_t>(c);
}

static moe_status check_groups(const moe_dims& dm, int32_t n_groups, const char* fn) {
  if (n_groups < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: n_groups=%d must be >= 1", fn, n_groups);
  if (dm.T % n_groups)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: n_groups=%d does not divide T=%lld", fn, n_groups,
                static_cast<long long>(dm.T));
  return MOE_OK;
}

moe_status moe_capacity(const moe_dims* dims, int32_t n_groups, int32_t capacity,
                        const int32_t* topk_idx, int32_t* kept_idx, int32_t* group_dropped,
                        void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  st = check_groups(dm, n_groups, __func__);
  if (st != MOE_OK) return st;
  if (capacity < 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: capacity=%d must be >= 0", __func__, capacity);
  MOE_REQUIRE_PTR(topk_idx, dm.T * dm.k);
  MOE_REQUIRE_PTR(kept_idx, dm.T * dm.k);
  MOE_REQUIRE_PTR(group_dropped, n_groups);
  const VariantWs need = variant_ws(dm, n_groups, nullptr);
  st = check_ws(workspace, workspace_bytes, need.bytes, __func__);
  if (st != MOE_OK) return st;
  const VariantWs w = variant_ws(dm, n_groups, workspace);
  return hip_status(moe::launch_capacity(dm.T, dm.k, dm.E, n_groups, capacity, topk_idx, kept_idx,
                                         group_dropped, w.hist, static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_router_zloss(const moe_dims* dims, const float* logits, int32_t n_groups,
                            float* group_z, void* workspace, size_t workspace_bytes,
                            void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  st = check_groups(dm, n_groups, __func__);
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR(logits, dm.T * dm.E);
  MOE_REQUIRE_PTR(group_z, n_groups);
  const VariantWs need = variant_ws(dm, n_groups, nullptr);
  st = check_ws(workspace, workspace_bytes, need.bytes, __func__);
  if (st != MOE_OK) return st;
  const VariantWs w = variant_ws(dm, n_groups, workspace);
  return hip_status(moe::launch_router_z(dm.T, dm.E, n_groups, logits, group_z, w.zpart,
                                         static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_route_bwd_dense(const moe_dims* dims, const void* x, const float* w_router,
                               const float* logits, const int32_t* topk_idx,
                               const float* topk_gate, const float* dgate, const int32_t* pos,
                               const void* dx_perm, int32_t n_groups, const int32_t* group_count,
                               float aux_coef, float z_coef, void* dx, float* dw_router,
                               float* dlogits, void* workspace, size_t workspace_bytes,
                               void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  st = check_groups(dm, n_groups, __func__);
  if (st != MOE_OK) return st;
  if (!std::isfinite(aux_coef) || !std::isfinite(z_coef))
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: aux_coef and z_coef must be finite", __func__);
  MOE_REQUIRE_PTR(x, dm.T * dm.d);
  MOE_REQUIRE_PTR(w_router, int64_t(dm.E) * dm.d);
  MOE_REQUIRE_PTR(logits, dm.T * dm.E);
  MOE_REQUIRE_PTR(topk_idx, dm.T * dm.k);
  MOE_REQUIRE_PTR(topk_gate, dm.T * dm.k);
  MOE_REQUIRE_PTR(dgate, dm.T * dm.k);
  MOE_REQUIRE_PTR(pos, dm.T * dm.k);
  MOE_OPTIONAL_PTR(dx_perm);
  if (aux_coef != 0.f) {
    MOE_REQUIRE_PTR(group_count, int64_t(n_groups) * dm.E);
  } else {
    MOE_OPTIONAL_PTR(group_count);
  }
  MOE_REQUIRE_PTR(dx, dm.T * dm.d);
  MOE_REQUIRE_PTR(dw_router, int64_t(dm.E) * dm.d);
  MOE_OPTIONAL_PTR(dlogits);
  const RouteBwdDenseWs need = route_bwd_dense_ws(dm, nullptr);
  st = check_ws(workspace, workspace_bytes, need.bytes, __func__);
  if (st != MOE_OK) return st;
  const RouteBwdDenseWs w = route_bwd_dense_ws(dm, workspace);
  return hip_status(moe::launch_route_bwd_dense(dm, x, w_router, logits, topk_idx, topk_gate,
                                                dgate, pos, dx_perm, n_groups, group_count,
                                                aux_coef, z_coef, dx, dw_router, dlogits, w.dl,
                                                w.partial, static_cast<hipStream_t>(stream)),
                    __func__);
}

// ---------------------------------------------------------------- token-shuffle planning
static moe_status check_index_dims(int64_t T, int32_t k, int32_t E, const char* fn) {
  if (T < 0 || k <= 0 || E <= 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need T >= 0 and k, E > 0", fn);
  if (E > 256 || k > E || k > 16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: need E <= 256 and k <= min(E, 16)", fn);
  if (T * k >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: T*k must be < 2^31", fn);
  return MOE_OK;
}

moe_status moe_coselect_cross(int64_t T, int32_t k, int32_t E, const int32_t* topk_idx_cur,
                              const int32_t* topk_idx_next, int32_t* coselect, void* stream) {
  moe_status st = check_index_dims(T, k, E, __func__);
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR(topk_idx_cur, T * k);
  MOE_REQUIRE_PTR(topk_idx_next, T * k);
  MOE_REQUIRE_PTR(coselect, int64_t(E) * E);
  return hip_status(moe::launch_coselect_cross(T, k, E, topk_idx_cur, topk_idx_next, coselect,
                                               static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_shuffle_plan(int64_t T, int32_t k, int32_t E, int32_t G,
                            const int32_t* topk_idx_cur, const int32_t* predictor,
                            const int32_t* placement_next, const int32_t* topk_idx_next,
                            int32_t* owner, int32_t* group_tokens, int32_t* stats,
                            void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_index_dims(T, k, E, __func__);
  if (st != MOE_OK) return st;
  if (G < 1 || G > 64)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: need 1 <= G <= 64", __func__);
  if (T % G)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s: G=%d does not divide T=%lld", __func__, G,
                static_cast<long long>(T));
  if (static_cast<int64_t>(E) * G > 8192)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E*G=%d exceeds 8192", __func__, E * G);
  st = check_placement_impl(E, G, placement_next, __func__);
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR(topk_idx_cur, T * k);
  MOE_REQUIRE_PTR(predictor, int64_t(E) * E);
  MOE_OPTIONAL_PTR(topk_idx_next);
  MOE_REQUIRE_PTR(owner, T);
  MOE_REQUIRE_PTR(group_tokens, G);
  MOE_REQUIRE_PTR(stats, 2);
  st = check_ws(workspace, workspace_bytes, static_cast<size_t>(E) * G * 4, __func__);
  if (st != MOE_OK) return st;
  moe::PlacementArg pl{};
  for (int32_t e = 0; e < E; ++e) pl.group_of[e] = placement_next[e];
  return hip_status(moe::launch_shuffle_plan(T, k, E, G, topk_idx_cur, predictor, pl,
                                             topk_idx_next, owner, group_tokens, stats,
                                             static_cast<int32_t*>(workspace),
                                             static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_route_flips(int64_t T, int32_t k, int32_t E, const int32_t* topk_idx_a,
                           const int32_t* topk_idx_b, int32_t* flips, int32_t* n_flips,
                           void* stream) {
  moe_status st = check_index_dims(T, k, E, __func__);
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR(topk_idx_a, T * k);
  MOE_REQUIRE_PTR(topk_idx_b, T * k);
  MOE_REQUIRE_PTR(flips, T);
  MOE_REQUIRE_PTR(n_flips, 1);
  return hip_status(moe::launch_route_flips(T, k, E, topk_idx_a, topk_idx_b, flips, n_flips,
                                            static_cast<hipStream_t>(stream)),
                    __func__);
}

// ------------------------------------------------ gate folded into the expert rows

int32_t moe_gate_folded_supported(const moe_dims* dims) {
  if (check_dims(dims, __func__) != MOE_OK) return 0;
  return moe::folded_bf16_ok(*dims) ? 1 : 0;
}

int32_t moe_dgate_parts(const moe_dims* dims) {
  if (check_dims(dims, __func__) != MOE_OK) return 0;
  return moe::dgate_parts_bf16(*dims);
}

namespace {
moe_status check_folded(const moe_dims* dims, const char* fn) {
  moe_status st = check_dims(dims, fn);
  if (st != MOE_OK) return st;
  if (!moe::folded_bf16_ok(*dims))
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: the gate-folded path needs bf16 and dims whose weight gradients take a "
                "one-pass kernel (moe_gate_folded_supported)",
                fn);
  return MOE_OK;
}
}  // namespace

moe_status moe_permute_gates(const moe_dims* dims, const int32_t* topk_idx,
                             const float* topk_gate, int32_t* expert_counts,
                             int32_t* expert_offsets, int32_t* pos, int32_t* src_token,
                             float* gate_perm, void* workspace, size_t workspace_bytes,
                             void* stream) {
  moe_status st = check_dims(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(topk_idx, dm.T * dm.k);
  MOE_REQUIRE_PTR(topk_gate, dm.T * dm.k);
  MOE_REQUIRE_PTR(expert_counts, dm.E);
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(pos, dm.T * dm.k);
  MOE_REQUIRE_PTR(src_token, dm.T * dm.k);
  MOE_REQUIRE_PTR(gate_perm, dm.T * dm.k);
  const PermWs need = perm_ws(dm.T, dm.E, nullptr);
  st = check_ws(workspace, workspace_bytes, need.bytes, __func__);
  if (st != MOE_OK) return st;
  const PermWs w = perm_ws(dm.T, dm.E, workspace);
  return hip_status(moe::launch_permute(dm, topk_idx, expert_counts, expert_offsets, pos,
                                        src_token, nullptr, nullptr, w.hist, w.base,
                                        static_cast<hipStream_t>(stream), topk_gate, gate_perm),
                    __func__);
}

moe_status moe_expert_up_folded(const moe_dims* dims, const void* x, const int32_t* src_token,
                                const int32_t* expert_offsets, const float* gate_perm,
                                const void* w1, const void* w3, void* a_save, void* b_save,
                                void* hg_save, void* stream) {
  moe_status st = check_folded(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  st = check_gather(dm, x, src_token, __func__);
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(gate_perm, dm.T * dm.k);
  MOE_REQUIRE_PTR(w1, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(w3, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(a_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(b_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(hg_save, dm.T * dm.k * dm.f);
  return hip_status(moe::launch_up_folded_bf16(dm, x, src_token, expert_offsets, gate_perm, w1,
                                               w3, a_save, b_save, hg_save,
                                               static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_expert_dgrad_down_folded(const moe_dims* dims, const void* dy,
                                        const int32_t* src_token, const int32_t* expert_offsets,
                                        const float* gate_perm, const void* w2, const void* a_save,
                                        const void* b_save, void* da, void* db, float* dgate_part,
                                        void* stream) {
  moe_status st = check_folded(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  st = check_gather(dm, dy, src_token, __func__);
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(gate_perm, dm.T * dm.k);
  MOE_REQUIRE_PTR(w2, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(a_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(b_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(da, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(db, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(dgate_part, dm.T * dm.k * moe::dgate_parts_bf16(dm));
  return hip_status(moe::launch_dgrad_down_folded_bf16(dm, dy, src_token, expert_offsets,
                                                       gate_perm, w2, a_save, b_save, da, db,
                                                       dgate_part,
                                                       static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_dgate_from_parts(const moe_dims* dims, const float* dgate_part,
                                const int32_t* pos, float* dgate, void* stream) {
  moe_status st = check_folded(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(dgate_part, dm.T * dm.k * moe::dgate_parts_bf16(dm));
  MOE_REQUIRE_PTR(pos, dm.T * dm.k);
  MOE_REQUIRE_PTR(dgate, dm.T * dm.k);
  return hip_status(moe::launch_dgate_from_parts(dm, dgate_part, moe::dgate_parts_bf16(dm), pos,
                                                 dgate, static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_expert_wgrad_folded(const moe_dims* dims, const void* x, const void* dy,
                                   const int32_t* src_token, const int32_t* expert_offsets,
                                   const void* hg_save, const void* da, const void* db,
                                   void* dw1, void* dw3, void* dw2, void* stream) {
  moe_status st = check_folded(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  st = check_gather(dm, x, src_token, __func__);
  if (st != MOE_OK) return st;
  st = check_gather(dm, dy, src_token, __func__);
  if (st != MOE_OK) return st;
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(hg_save, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(da, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(db, dm.T * dm.k * dm.f);
  MOE_REQUIRE_PTR(dw1, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(dw3, int64_t(dm.E) * dm.f * dm.d);
  MOE_REQUIRE_PTR(dw2, int64_t(dm.E) * dm.f * dm.d);
  return hip_status(moe::launch_wgrad_folded_bf16(dm, x, src_token, expert_offsets, hg_save, dy,
                                                  da, db, dw1, dw3, dw2,
                                                  static_cast<hipStream_t>(stream)),
                    __func__);
}

moe_status moe_route_bwd_folded(const moe_dims* dims, const void* x, const float* w_router,
                                const int32_t* topk_idx, const float* topk_gate,
                                const float* dgate_part, const int32_t* expert_offsets,
                                const int32_t* pos, const int32_t* src_token,
                                const void* dx_perm, float* dgate, void* dx, float* dw_router,
                                void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_folded(dims, __func__);
  if (st != MOE_OK) return st;
  const moe_dims& dm = *dims;
  MOE_REQUIRE_PTR(x, dm.T * dm.d);
  MOE_REQUIRE_PTR(w_router, int64_t(dm.E) * dm.d);
  MOE_REQUIRE_PTR(topk_idx, dm.T * dm.k);
  MOE_REQUIRE_PTR(topk_gate, dm.T * dm.k);
  MOE_REQUIRE_PTR(dgate_part, dm.T * dm.k * moe::dgate_parts_bf16(dm));
  MOE_REQUIRE_PTR(expert_offsets, dm.E + 1);
  MOE_REQUIRE_PTR(pos, dm.T * dm.k);
  MOE_REQUIRE_PTR(src_token, dm.T * dm.k);
  MOE_OPTIONAL_PTR(dx_perm);
  MOE_REQUIRE_PTR(dgate, dm.T * dm.k);
  MOE_REQUIRE_PTR(dx, dm.T * dm.d);
  MOE_REQUIRE_PTR(dw_router, int64_t(dm.E) * dm.d);
  const RouteBwdWs need = route_bwd_ws(dm, nullptr);
  st = check_ws(workspace, workspace_bytes, need.bytes, __func__);
  if (st != MOE_OK) return st;
  const RouteBwdWs w = route_bwd_ws(dm, workspace);
  return hip_status(moe::launch_route_bwd(dm, x, w_router, topk_idx, topk_gate, nullptr,
                                          expert_offsets, pos, src_token, dx_perm, dx, dw_router,
                                          w.dl_perm, w.dl_sel, w.partial,
                                          static_cast<hipStream_t>(stream), dgate_part,
                                          moe::dgate_parts_bf16(dm), dgate),
                    __func__);
}

}  // extern "C"
