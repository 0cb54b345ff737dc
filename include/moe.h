/*
 * moe.h -- C ABI of libmoe.so: the hot path of one Mixture-of-Experts layer on
 * one GPU's share of tokens, for AMD Instinct MI355X (gfx950).
 *
 * The layer (router -> top-k gating -> permutation into expert-contiguous rows
 * -> SwiGLU experts -> gate-weighted combine, and its backward) follows:
 *   [COUPLING] "Expert Coupling in MoE Pretraining: Reducing All-to-All
 *              Overhead with Correlated Placement and Token Shuffling":
 *              Abstract (each token routed to k of E experts; dispatch and
 *              combine in the forward and backward passes; a dispatcher that
 *              sends each token to each GPU once), Fig. 5 (steps 3-5: dispatch,
 *              expert computation, combine), Table I (placement statistics),
 *              Table III (notation t, T, E, k, S(t), W[e,e']).
 *   [REVISIT]  "Revisiting MoE and Dense Speed-Accuracy Comparisons for LLM
 *              Training": Sec. 2.1 (SwiGLU, Top-K routing, load-balancing
 *              loss), Sec. 2.2 (GShard gating/dispatch/combine, outer batches),
 *              Sec. 3.6 (the second expert is simply the second best).
 *   [LAYOUT]   "MoE Pretraining: Parallelism Layout Changes the Model, Not
 *              Quality": Finding 3 (routing margin, near-ties), Two Kinds of
 *              Layout Effects (per-machine balancing statistics), Correctness
 *              Checks (bit-identical reruns).
 *   [LOADING]  "Why does expert-parallel loading matter so much in MoE
 *              training?": What to verify (each expert owned by exactly one
 *              shard, equal expert counts per shard).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked [host].  Tensors are dense,
 *    row-major and 16-byte aligned.  Shapes are given in brackets.
 *  - "act" tensors (X, W1, W3, W2, Y, dY, dX, x_perm, y_perm, a, b, h, the
 *    weight gradients) are fp32 when dims->act == MOE_F32 and bfloat16 when
 *    dims->act == MOE_BF16.  The router weight, logits, gates, margins and
 *    router gradients are always fp32.  Accumulation is always fp32.
 *  - Weights are stored [expert, out, in]: W1, W3 [E, f, d]; W2 [E, d, f];
 *    Wr [E, d].
 *  - The caller owns all memory: outputs and the workspace are allocated by
 *    the caller; the library allocates and frees nothing and never
 *    synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream).  Outputs are fully overwritten.
 *  - Every argument is validated on the host before anything is enqueued; on
 *    an error nothing is enqueued, outputs are untouched, and
 *    moe_last_error() describes the problem.  Faults inside kernels surface
 *    at the caller's next synchronisation.
 *  - Results are bitwise reproducible from run to run: no floating-point
 *    atomics, every reduction has a fixed order.
 *  - Supported envelope (else MOE_ERR_UNSUPPORTED): 1 <= k <= min(E, 16),
 *    E <= 256, d % 64 == 0, f % 64 == 0, T * k < 2^31, act in {F32, BF16}.
 *  - topk_idx inputs must hold expert ids in [0, E) with no repeats within a
 *    token (moe_route produces such tables).  Out-of-range ids are ignored by
 *    the index kernels rather than written out of bounds; moe_permute sorts a
 *    repeated id by the definition (each slot its own row, in slot order).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,  /* null pointer, negative size, G not dividing T */
  MOE_ERR_UNSUPPORTED = 2,       /* outside the supported envelope above */
  MOE_ERR_WORKSPACE = 3,         /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_INVALID_PLACEMENT = 4, /* placement is not a balanced partition */
  MOE_ERR_HIP = 5                /* a HIP launch failed */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef struct moe_dims {
  int64_t T;    /* tokens */
  int32_t d;    /* model width */
  int32_t E;    /* experts */
  int32_t f;    /* expert FFN width */
  int32_t k;    /* experts per token */
  int32_t act;  /* moe_dtype of the act tensors */
} moe_dims;

/* [host] Static string naming a status code. */
const char* moe_status_string(int32_t status);

/* [host] Detail of the last error returned on the calling thread ("" if none). */
const char* moe_last_error(void);

/* [host] Workspace bytes that every entry point below needs for these dims
 * (the maximum over the entry points; n_groups is the largest LB-statistics
 * or dispatch-plan group count the caller will use).  Returns 0 when the dims
 * are invalid. */
size_t moe_workspace_bytes(const moe_dims* dims, int32_t n_groups);

/* [host] Kernels that moe_expert_wgrad enqueues for these dims with
 * wgrad_dtype = act: 1 (one
 * kernel writes dW1, dW3, dW2), 2 (the expert rows are split into parts whose
 * fp32 partial tiles a second kernel adds in a fixed order), or 0 when the
 * dims are invalid.  For profilers and benchmarks that attribute time to
 * kernels. */
int32_t moe_expert_wgrad_launches(const moe_dims* dims);

/*
 * moe_route -- router logits, top-k gating, margins, near-ties and
 * per-block load-balancing statistics.
 *   [COUPLING] Abstract / Table III: S(t) = the k experts selected for token t;
 *   [REVISIT] Sec. 2.1 Top-K routing, Sec. 3.6 naive second expert;
 *   [LAYOUT] Finding 3: margin between the k-th and (k+1)-th scores;
 *   [LAYOUT] Two Kinds of Layout Effects and [REVISIT] Sec. 2.2 (outer
 *   batches): balancing statistics per contiguous block of tokens.
 *
 * x [T,d] act; w_router [E,d] fp32.
 * logits [T,E] fp32: l[t,e] = sum_i x[t,i] w_router[e,i] (no bias).
 * topk_idx [T,k] int32: experts by descending logit, lower id first on ties.
 * topk_gate [T,k] fp32: softmax over the k chosen logits.
 * margin [T] fp32: l_(k) - l_(k+1) (the k-th minus the (k+1)-th largest
 *   logit; +inf when k == E).
 * near_tie_count [1] int32: number of tokens with margin < near_tie_eps.
 * n_groups: G >= 1 dividing T (G = 1 for whole-batch statistics).
 * group_count [G,E] int32: assignments of block r's tokens to expert e.
 * group_mean_prob [G,E] fp32: mean over block r of the full softmax p[t,e].
 * group_aux [G] fp32: E * sum_e (count[r,e] / (T/G * k)) * mean_prob[r,e].
 * group_count, group_mean_prob and group_aux may each be NULL.
 */
moe_status moe_route(const moe_dims* dims, const void* x, const float* w_router,
                     float* logits, int32_t* topk_idx, float* topk_gate, float* margin,
                     float near_tie_eps, int32_t* near_tie_count, int32_t n_groups,
                     int32_t* group_count, float* group_mean_prob, float* group_aux,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_noalloc -- moe_route for callers that cannot allocate device
 * memory or hand over a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, outputs,
 * kernels and bits as moe_route, without workspace and workspace_bytes: the
 * scratch (per-tile partial sums of the balancing statistics, each written
 * before it is read, so nothing in it has to start at zero) lives in a static
 * device array of moe_route_noalloc_max_bytes() = 4 MiB that the library holds on every GPU
 * it runs on until the process ends.  Dims whose scratch exceeds it (about
 * 2000 64-token tiles at E = 256, 8000 at E = 64) return MOE_ERR_UNSUPPORTED
 * with nothing enqueued.  Every call on one GPU shares that GPU's array and
 * leaves its last contents there: calls that overlap on one GPU (different
 * streams without ordering between them) race and must not be issued.
 */
size_t moe_route_noalloc_max_bytes(void);   /* [host] */
moe_status moe_route_noalloc(const moe_dims* dims, const void* x, const float* w_router,
                             float* logits, int32_t* topk_idx, float* topk_gate, float* margin,
                             float near_tie_eps, int32_t* near_tie_count, int32_t n_groups,
                             int32_t* group_count, float* group_mean_prob, float* group_aux,
                             void* stream);

/*
 * moe_permute -- stable counting sort of the T*k (token, slot) assignments by
 * expert, and the row gather into expert-contiguous order.
 *   [COUPLING] Abstract and Fig. 5 step 3 (dispatch tokens to their experts);
 *   [REVISIT] Sec. 2.2 (GShard dispatch: a token's position inside its expert
 *   is the running count of earlier tokens that chose that expert).
 *
 * topk_idx [T,k] int32 in.  An id of -1 marks a dropped assignment (see
 *   moe_capacity): it gets pos -1 and no row.  A token whose row repeats an
 *   expert (outside the routing contract) gets one row per slot, the slots
 *   in order, exactly as for distinct ids.
 * expert_counts [E], expert_offsets [E+1] (exclusive scan; offsets[E] = the
 *   number of kept assignments, T*k when nothing is dropped).
 * pos [T,k]: row of assignment (t, j) in the permuted order; rows of one
 *   expert are in ascending token id.
 * src_token [T*k]: token of each permuted row (entries past offsets[E] are
 *   left unchanged).
 * x [T,d] act and x_perm [T*k,d] act: x_perm[pos[t,j]] = x[t].  Pass both
 *   NULL to build the plan only.
 */
moe_status moe_permute(const moe_dims* dims, const int32_t* topk_idx,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* pos,
                       int32_t* src_token, const void* x, void* x_perm,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_grouped_swiglu_fwd -- the E SwiGLU experts as one grouped GEMM pair.
 *   [REVISIT] Sec. 2.1 (SwiGLU activation); [LAYOUT] Methodology (SwiGLU
 *   experts); [COUPLING] Fig. 5 step 4 (expert computation).
 *
 * For each expert e over rows p in [expert_offsets[e], expert_offsets[e+1]):
 *   a[p] = x_perm[p] W1[e]^T,  b[p] = x_perm[p] W3[e]^T,
 *   h[p] = silu(a[p]) * b[p]   (silu(z) = z / (1 + exp(-z))),
 *   y_perm[p] = h[p] W2[e]^T.
 * x_perm [T*k,d] act; expert_offsets [E+1] int32 (from moe_permute);
 * w1, w3 [E,f,d] act; w2 [E,d,f] act.
 * a_save, b_save, h_save [T*k,f] act: saved for the backward (required).
 * y_perm [T*k,d] act.
 */
moe_status moe_grouped_swiglu_fwd(const moe_dims* dims, const void* x_perm,
                                  const int32_t* expert_offsets, const void* w1,
                                  const void* w3, const void* w2, void* a_save, void* b_save,
                                  void* h_save, void* y_perm, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * moe_combine -- gate-weighted sum of each token's k expert rows.
 *   [COUPLING] Abstract and Fig. 5 step 5 (combine the results);
 *   [REVISIT] Sec. 2.2 (GShard combine).
 *
 * out[t] = sum_{j<k} gate[t,j] * rows[pos[t,j]], accumulated in fp32 in slot
 * order j = 0..k-1, then stored as act; slots with pos -1 (dropped) add
 * nothing.  gate == NULL means unit weights
 * (the plain unpermute-and-sum used for the input gradient).
 * rows [T*k,d] act; pos [T,k]; gate [T,k] fp32 or NULL; out [T,d] act.
 */
moe_status moe_combine(const moe_dims* dims, const void* rows, const int32_t* pos,
                       const float* gate, void* out, void* stream);

/*
 * moe_combine_bwd -- adjoint of moe_combine with respect to rows and gates
 * ("routed gradients" in the backward pass, [COUPLING] Abstract).
 *
 * dy_perm[pos[t,j]] = gate[t,j] * dy[t]           (act)
 * dgate[t,j]        = <dy[t], y_perm[pos[t,j]]>   (fp32 dot over d)
 * A dropped slot (pos -1) writes no row and gets dgate 0.
 * dy [T,d] act; y_perm [T*k,d] act; pos [T,k]; gate [T,k] fp32;
 * dy_perm [T*k,d] act; dgate [T,k] fp32.
 */
moe_status moe_combine_bwd(const moe_dims* dims, const void* dy, const void* y_perm,
                           const int32_t* pos, const float* gate, void* dy_perm,
                           float* dgate, void* stream);

/*
 * moe_grouped_swiglu_bwd -- dgrad and wgrad grouped GEMMs of the experts.
 *
 * For each expert e over its rows p:
 *   dh = dy_perm W2[e];  da = dh * b * silu'(a);  db = dh * silu(a)
 *   dx_perm = da W1[e] + db W3[e]
 *   dW2[e] = dy_perm^T h;  dW1[e] = da^T x_perm;  dW3[e] = db^T x_perm
 * with silu'(z) = s (1 + z (1 - s)), s = 1 / (1 + exp(-z)).
 * Inputs: x_perm [T*k,d], a_save, b_save, h_save [T*k,f], dy_perm [T*k,d]
 * (act); expert_offsets [E+1]; w1, w3 [E,f,d]; w2 [E,d,f] (act).
 * a_save, b_save and h_save are either all given (as moe_grouped_swiglu_fwd
 * wrote them) or all NULL: the call then recomputes them from x_perm, W1 and
 * W3 with the forward kernel (activation recomputation), bit for bit what
 * the forward pass stores, in workspace of
 * moe_grouped_swiglu_bwd_workspace_bytes(dims, 1) bytes; a mix of NULL and
 * non-NULL returns MOE_ERR_INVALID_ARGUMENT.
 * Outputs: dx_perm [T*k,d] act; dw1, dw3 [E,f,d] and dw2 [E,d,f] of type
 * wgrad_dtype: MOE_BF16 (bf16 layers only) or MOE_F32.  Each weight gradient
 * is accumulated in fp32 over all rows of its expert in a fixed order and
 * rounded once to bf16, or stored as the fp32 sum.  An fp32 layer takes
 * MOE_F32 only (MOE_ERR_UNSUPPORTED otherwise).  Experts with no rows get
 * zeros.
 */
moe_status moe_grouped_swiglu_bwd(const moe_dims* dims, const void* x_perm,
                                  const int32_t* expert_offsets, const void* w1,
                                  const void* w3, const void* w2, const void* a_save,
                                  const void* b_save, const void* h_save, const void* dy_perm,
                                  void* dx_perm, void* dw1, void* dw3, void* dw2,
                                  int32_t wgrad_dtype, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* [host] Workspace bytes moe_grouped_swiglu_bwd(_gather) needs with saved
 * activations (recompute = 0: at most moe_workspace_bytes()) or recomputing
 * them (recompute = 1: three more [T*k,f] act buffers).  0 for invalid dims. */
size_t moe_grouped_swiglu_bwd_workspace_bytes(const moe_dims* dims, int32_t recompute);

/*
 * Kernel-level phases of the two calls above, for callers that schedule the
 * expert GEMMs themselves (e.g. to overlap them with other work or to time
 * them one by one).  moe_grouped_swiglu_fwd = moe_expert_up + moe_expert_down;
 * moe_grouped_swiglu_bwd = moe_expert_dgrad_down + moe_expert_dgrad_up +
 * moe_expert_wgrad, with da and db held in its workspace.  Each phase is one
 * GEMM kernel (moe_expert_wgrad adds an ordered split-K reduction kernel when
 * E x output tiles alone cannot fill the GPU).  Same layouts, formulas and
 * precision as the calls above; da, db [T*k,f] act are caller buffers here.
 *   moe_expert_up:         a, b, h from x_perm, W1, W3
 *   moe_expert_down:       y_perm = h W2^T
 *   moe_expert_dgrad_down: dh = dy_perm W2 (stored precision), da, db
 *   moe_expert_dgrad_up:   dx_perm = da W1 + db W3
 *   moe_expert_wgrad:      dW2 = dy_perm^T h, dW1 = da^T x_perm, dW3 = db^T x_perm
 *                          (wgrad_dtype as in moe_grouped_swiglu_bwd)
 * moe_expert_wgrad's workspace: at least moe_workspace_bytes() bytes.
 */
moe_status moe_expert_up(const moe_dims* dims, const void* x_perm,
                         const int32_t* expert_offsets, const void* w1, const void* w3,
                         void* a_save, void* b_save, void* h_save, void* stream);
moe_status moe_expert_down(const moe_dims* dims, const void* h_save,
                           const int32_t* expert_offsets, const void* w2, void* y_perm,
                           void* stream);
moe_status moe_expert_dgrad_down(const moe_dims* dims, const void* dy_perm,
                                 const int32_t* expert_offsets, const void* w2,
                                 const void* a_save, const void* b_save, void* da, void* db,
                                 void* stream);
moe_status moe_expert_dgrad_up(const moe_dims* dims, const void* da, const void* db,
                               const int32_t* expert_offsets, const void* w1, const void* w3,
                               void* dx_perm, void* stream);
moe_status moe_expert_wgrad(const moe_dims* dims, const void* x_perm,
                            const int32_t* expert_offsets, const void* h_save,
                            const void* dy_perm, const void* da, const void* db, void* dw1,
                            void* dw3, void* dw2, int32_t wgrad_dtype, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Gathered expert input ("Expert Coupling in MoE Pretraining", Fig. 5: the
 * dispatch gathers each token's rows for its experts).  The same products as
 * moe_grouped_swiglu_fwd/bwd, moe_expert_up and moe_expert_wgrad, with the
 * expert input row p read as x[src_token[p]] instead of x_perm[p], so
 * moe_permute can run as a plan only (x_perm = NULL) and the [T*k, d] copy
 * of X is never written or read.  Results are bitwise those of the x_perm
 * calls on x_perm[p] = x[src_token[p]].
 * x [T,d] act; src_token [T*k] int32 in [0, T), as moe_permute writes it for
 * the same routing (not checked on the device).  bf16: T*d*2 < 2^31 bytes,
 * else MOE_ERR_UNSUPPORTED.  Other arguments, workspace and errors as in the
 * calls they mirror.
 */
moe_status moe_grouped_swiglu_fwd_gather(const moe_dims* dims, const void* x,
                                         const int32_t* src_token,
                                         const int32_t* expert_offsets, const void* w1,
                                         const void* w3, const void* w2, void* a_save,
                                         void* b_save, void* h_save, void* y_perm,
                                         void* workspace, size_t workspace_bytes, void* stream);
moe_status moe_grouped_swiglu_bwd_gather(const moe_dims* dims, const void* x,
                                         const int32_t* src_token,
                                         const int32_t* expert_offsets, const void* w1,
                                         const void* w3, const void* w2, const void* a_save,
                                         const void* b_save, const void* h_save,
                                         const void* dy_perm, void* dx_perm, void* dw1,
                                         void* dw3, void* dw2, int32_t wgrad_dtype,
                                         void* workspace, size_t workspace_bytes, void* stream);
moe_status moe_expert_up_gather(const moe_dims* dims, const void* x, const int32_t* src_token,
                                const int32_t* expert_offsets, const void* w1, const void* w3,
                                void* a_save, void* b_save, void* h_save, void* stream);
moe_status moe_expert_wgrad_gather(const moe_dims* dims, const void* x,
                                   const int32_t* src_token, const int32_t* expert_offsets,
                                   const void* h_save, const void* dy_perm, const void* da,
                                   const void* db, void* dw1, void* dw3, void* dw2,
                                   int32_t wgrad_dtype, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Gate folded into the expert rows.  The combine is the gate-weighted sum
 * y[t] = sum_j g_j E_{S_j}(x_t) ("Revisiting MoE and Dense Speed-Accuracy
 * Comparisons", Sec. 2.1; "Expert Coupling in MoE Pretraining", Fig. 5 steps
 * 3-4).  Since E(x) = W2 h is linear in h, these calls move g_j onto the
 * expert row: the forward stores hg = g h (then moe_expert_down gives g E(x)
 * and moe_combine with topk_gate = NULL sums the rows), and the backward
 * reads dY [T,d] itself through src_token (no dy_perm):
 *   u = dY[src] W2 (per row, over f; rounded to act), dh = g u,
 *   da = dh b silu'(a), db = dh silu(a)            (as moe_expert_dgrad_down),
 *   dgate[t,j] = <dY[t], W2 h> = <u, silu(a) b>     (per row, summed over f),
 *   dW2 = sum_rows dY[src]^T hg, dW1 = da^T X[src], dW3 = db^T X[src].
 * dgate comes out as parts, one per column tile of f (128 wide, 256 where the
 * output-gradient GEMM takes the big tile), in dgate_part
 * [T*k, moe_dgate_parts(dims)] fp32; moe_dgate_from_parts adds them in tile
 * order into dgate [T,k] (0 for a dropped slot, pos < 0).  The results match
 * the unfolded calls up to rounding (one rounding of g h instead of one of
 * h and one of g dY).
 *
 * Supported for bf16 dims whose weight gradients take a one-pass kernel
 * (not the split-K form used when E x output tiles are few):
 * moe_gate_folded_supported(dims) == 1 (otherwise each call returns
 * MOE_ERR_UNSUPPORTED).  The expert input is always X [T,d] through
 * src_token; dY has the same shape and the same 2^31-byte bound.
 *   moe_permute_gates:   moe_permute (no row copy) plus gate_perm [T*k] fp32,
 *                        the gate of each expert row (its workspace);
 *   moe_expert_up_folded: a, b, hg [T*k,f] from X, W1, W3 and gate_perm;
 *   moe_expert_dgrad_down_folded: da, db [T*k,f] and dgate_part from dY,
 *                        W2, a, b, gate_perm;
 *   moe_dgate_from_parts: dgate [T,k] from dgate_part and pos;
 *   moe_expert_wgrad_folded: dW1, dW3, dW2 from X, dY, hg, da, db.
 * Rows past expert_offsets[E] (dropped slots) are never read or written.
 */
int32_t moe_gate_folded_supported(const moe_dims* dims);   /* [host] 1 or 0 */
int32_t moe_dgate_parts(const moe_dims* dims);             /* [host] dgate parts per row */
moe_status moe_permute_gates(const moe_dims* dims, const int32_t* topk_idx,
                             const float* topk_gate, int32_t* expert_counts,
                             int32_t* expert_offsets, int32_t* pos, int32_t* src_token,
                             float* gate_perm, void* workspace, size_t workspace_bytes,
                             void* stream);
moe_status moe_expert_up_folded(const moe_dims* dims, const void* x, const int32_t* src_token,
                                const int32_t* expert_offsets, const float* gate_perm,
                                const void* w1, const void* w3, void* a_save, void* b_save,
                                void* hg_save, void* stream);
moe_status moe_expert_dgrad_down_folded(const moe_dims* dims, const void* dy,
                                        const int32_t* src_token, const int32_t* expert_offsets,
                                        const float* gate_perm, const void* w2, const void* a_save,
                                        const void* b_save, void* da, void* db, float* dgate_part,
                                        void* stream);
moe_status moe_dgate_from_parts(const moe_dims* dims, const float* dgate_part,
                                const int32_t* pos, float* dgate, void* stream);
moe_status moe_expert_wgrad_folded(const moe_dims* dims, const void* x, const void* dy,
                                   const int32_t* src_token, const int32_t* expert_offsets,
                                   const void* hg_save, const void* da, const void* db,
                                   void* dw1, void* dw3, void* dw2, void* stream);
/* moe_route_bwd with the dgate parts in place of dgate: the same router
 * backward (every assignment must have a row), its dgate [T,k] fp32 written
 * as an output (the sum of each row's parts in tile order), so that
 * moe_dgate_from_parts is not needed.  Same workspace as moe_route_bwd. */
moe_status moe_route_bwd_folded(const moe_dims* dims, const void* x, const float* w_router,
                                const int32_t* topk_idx, const float* topk_gate,
                                const float* dgate_part, const int32_t* expert_offsets,
                                const int32_t* pos, const int32_t* src_token,
                                const void* dx_perm, float* dgate, void* dx, float* dw_router,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_bwd -- adjoint of the router (logits -> top-k -> renormalised
 * softmax), fused with the unpermute-and-sum of the expert input gradient.
 *
 * dl[t, S_j(t)] = g_j (dg_j - sum_i g_i dg_i), zero for unchosen experts;
 * dx[t]  = sum_j dx_perm[pos[t,j]] + sum_j dl[t,S_j(t)] w_router[S_j(t)]
 *          (fp32, rounded once to act; the first sum is skipped when
 *          dx_perm == NULL);
 * dw_router[e] = sum over the tokens t that chose e of dl[t, e] * x[t]
 *          (fp32; partial sums over fixed token ranges added in a fixed
 *          order, so the result is reproducible: over each expert's rows
 *          in ascending token order, or, for bf16 x with E <= 64 and d a
 *          multiple of 128 from 1024, over 32-token chunks on the matrix
 *          cores with dl split exactly into three bf16 parts).
 * x [T,d] act; w_router [E,d]; topk_idx, topk_gate, dgate [T,k];
 * expert_offsets [E+1], pos [T,k], src_token [T*k] from moe_permute;
 * dx_perm [T*k,d] act or NULL; dx [T,d] act; dw_router [E,d] fp32.
 * Every assignment must have a row (pos >= 0): with dropped assignments use
 * moe_route_bwd_dense, which also carries the auxiliary losses.
 */
moe_status moe_route_bwd(const moe_dims* dims, const void* x, const float* w_router,
                         const int32_t* topk_idx, const float* topk_gate, const float* dgate,
                         const int32_t* expert_offsets, const int32_t* pos,
                         const int32_t* src_token, const void* dx_perm, void* dx,
                         float* dw_router, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Definitional variants of the routing rules ([REVISIT] Sec. 2.1: Top-K
 * routing with an expert capacity, the GShard load-balancing loss and the
 * ST-MoE router z-loss; Sec. 4: capacity 1.25 for training and 2.0 for
 * evaluation; [LAYOUT] Two Kinds of Layout Effects: capacity and balancing
 * rules evaluated per machine, here per contiguous block of T/G tokens).
 *
 * moe_expert_capacity -- [host] places per expert in one block of
 *   n = T / n_groups tokens: ceil(factor * (n * k) / E) in double precision,
 *   the capacity factor times the block's mean load per expert.  -1 when the
 *   arguments are invalid (n_groups not dividing T, factor negative or not
 *   finite); saturates at INT32_MAX.
 *
 * moe_capacity -- per-block capacity with dropping.  Inside block r the
 *   assignments queue for their experts slot-major, as GShard places second
 *   choices after every first choice: slot 0 of each token in token order,
 *   then slot 1, and so on.  An assignment is kept when fewer than `capacity`
 *   assignments of its block are ahead of it in its expert's queue.
 *   topk_idx [T,k] int32 in (ids outside [0,E) are written -1 and not
 *   counted); kept_idx [T,k] int32 out: the expert id, or -1 when dropped
 *   (a buffer of its own: moe_route_bwd_dense needs the original table);
 *   group_dropped [G] int32 out: dropped assignments per block.  Gates are
 *   not renormalised after dropping.  Feed kept_idx to moe_permute; the
 *   combine and its backward skip dropped slots.  capacity >= 0; 1 <= G, G
 *   divides T.
 *
 * moe_router_zloss -- group_z [G] fp32: the mean over block r of lse_t^2,
 *   lse_t = log sum_e exp logits[t,e].  The z-loss is z_coef times the mean of
 *   group_z (= the mean over all tokens).  The balancing loss is aux_coef
 *   times the mean of moe_route's group_aux.
 *
 * moe_route_bwd_dense -- the router backward over the dense [T,E] logit
 *   gradient, for dropped assignments and the auxiliary losses:
 *     dl[t,e] = sum_{j : topk_idx[t,j] = e} g_j (dg_j - sum_i g_i dg_i)
 *             + aux_coef * E / (G n) * p[t,e] (f[r,e] - sum_e' f[r,e'] p[t,e'])
 *             + z_coef * 2 / T * lse_t * p[t,e]
 *   with p the full softmax of logits[t], f = group_count / (n k) of the
 *   token's block r (held constant), n = T / G;
 *     dx[t]  = sum_{j : pos[t,j] >= 0} dx_perm[pos[t,j]] + sum_e dl[t,e] w_router[e]
 *              (fp32, slots in order then e ascending, rounded once to act;
 *              the first sum is skipped when dx_perm == NULL),
 *     dw_router = dl^T x (fp32, tokens in a fixed order).
 *   topk_idx is the router's selection (before dropping): a dropped slot
 *   keeps its gate term, since its logit still sets the kept gates; moe_combine_bwd
 *   gives it dgate 0.  logits [T,E] fp32 from moe_route; group_count [G,E]
 *   from moe_route (required when aux_coef != 0); pos from moe_permute on the
 *   kept table; dlogits [T,E] fp32 out, or NULL.  With aux_coef = z_coef = 0
 *   and nothing dropped the result equals moe_route_bwd's up to summation
 *   order.
 * moe_capacity, moe_router_zloss and moe_route_bwd_dense take a workspace of
 * moe_workspace_bytes(dims, n_groups) bytes or more.
 */
int32_t moe_expert_capacity(int64_t T, int32_t k, int32_t E, int32_t n_groups, double factor);
moe_status moe_capacity(const moe_dims* dims, int32_t n_groups, int32_t capacity,
                        const int32_t* topk_idx, int32_t* kept_idx, int32_t* group_dropped,
                        void* workspace, size_t workspace_bytes, void* stream);
moe_status moe_router_zloss(const moe_dims* dims, const float* logits, int32_t n_groups,
                            float* group_z, void* workspace, size_t workspace_bytes,
                            void* stream);
moe_status moe_route_bwd_dense(const moe_dims* dims, const void* x, const float* w_router,
                               const float* logits, const int32_t* topk_idx,
                               const float* topk_gate, const float* dgate, const int32_t* pos,
                               const void* dx_perm, int32_t n_groups, const int32_t* group_count,
                               float aux_coef, float z_coef, void* dx, float* dw_router,
                               float* dlogits, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * moe_coselect -- co-selection counts ([COUPLING] Table III, Fig. 2):
 * W[e,e'] = number of tokens whose chosen set contains both e and e' (e != e'),
 * diagonal zero.  topk_idx [T,k]; coselect [E,E] int32.
 */
moe_status moe_coselect(int64_t T, int32_t k, int32_t E, const int32_t* topk_idx,
                        int32_t* coselect, void* stream);

/*
 * moe_dispatch_plan -- the deduplicated dispatch row map: each token is sent
 * to each group once ([COUPLING] Abstract; Table I statistics).
 *
 * placement [host] [E]: group of each expert.  It must be a balanced
 *   partition (every entry in [0,G), exactly E/G experts per group), else
 *   MOE_ERR_INVALID_PLACEMENT ([LOADING] What to verify).  1 <= G <= 64,
 *   G divides E and T.
 * D_t = the distinct groups of token t's experts.  One row per (g, t) with g
 * in D_t, rows ordered by (g, t).
 * n_dest [T] int32 = |D_t|; group_rows [G]; group_offsets [G+1];
 * row_token [T*k] (first group_offsets[G] entries used): token of each row;
 * assign_row [T,k]: the row that carries expert slot j of token t;
 * stats [4] int32: rows_total = sum |D_t|, rows_removed = T*k - rows_total,
 *   tokens_single_group = #{t : |D_t| = 1},
 *   rows_off_home = #{rows (g,t) : g != t / (T/G)}.
 */
moe_status moe_dispatch_plan(int64_t T, int32_t k, int32_t E, int32_t G,
                             const int32_t* topk_idx, const int32_t* placement,
                             int32_t* n_dest, int32_t* group_rows, int32_t* group_offsets,
                             int32_t* row_token, int32_t* assign_row, int32_t* stats,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Expert-parallel dispatch emulated on one device ([COUPLING] Abstract: each
 * token is sent to each GPU once; Fig. 5: dispatch, then every GPU runs its
 * experts on the rows it received).
 *
 * moe_dispatch_pack: send[r] = x[row_token[r]] for r < group_offsets[G] (a
 *   device value), with row_token and group_offsets from moe_dispatch_plan for
 *   the same routing.  Rows are group-contiguous in (group, token) order, so
 *   group g's slice [group_offsets[g], group_offsets[g+1]) is what GPU g
 *   would receive.  x [T,d] act; send [T*k,d] act (capacity; rows past the
 *   plan's total are left unchanged).  1 <= G <= 64.
 * moe_dispatch_expand: x_perm[pos[t,j]] = recv[assign_row[t,j]] for every
 *   (t, j): the receivers' expansion into expert-contiguous rows.  With recv
 *   the send buffer (every slice received in place) and pos from moe_permute,
 *   x_perm equals moe_permute's bit for bit.  recv [T*k,d] act; assign_row,
 *   pos [T,k] int32; x_perm [T*k,d] act.
 */
moe_status moe_dispatch_pack(const moe_dims* dims, int32_t G, const void* x,
                             const int32_t* group_offsets, const int32_t* row_token, void* send,
                             void* stream);
moe_status moe_dispatch_expand(const moe_dims* dims, const void* recv,
                               const int32_t* assign_row, const int32_t* pos, void* x_perm,
                               void* stream);

/*
 * Token-shuffle planning ([COUPLING] Abstract: the experts a token selects at
 * one layer predict those it selects at the next; Fig. 2(b); Fig. 5 step 1 and
 * Fig. 6: a planner predicts each token's owner GPU from its previous-layer
 * routes, and the reduce-scatter delivers the token there; Table I: local
 * next-layer experts when moved versus when staying home).
 *
 * moe_coselect_cross -- W[e1,e2] = number of tokens that select e1 in
 *   topk_idx_cur (layer l) and e2 in topk_idx_next (layer l+1); e1 == e2
 *   counts.  topk_idx_cur, topk_idx_next [T,k]; coselect [E,E] int32.
 *
 * moe_shuffle_plan -- owner[t] = argmax over groups g of
 *     sum_{e1 in S_cur(t)} sum_{e2 : placement_next[e2] = g} predictor[e1,e2]
 *   (64-bit sums, ties to the lowest g), with predictor the cross-layer counts
 *   of other batches (moe_coselect_cross).  group_tokens [G]: tokens per
 *   owner.  stats [2] int32: next-layer assignments whose expert sits on the
 *   token's owner group (moved) and on its home group t / (T/G) (stays), when
 *   topk_idx_next [T,k] is given; zeros when it is NULL.
 *   placement_next [host] [E]: a balanced partition of layer l+1's experts
 *   over G groups (else MOE_ERR_INVALID_PLACEMENT); 1 <= G <= 64, G divides
 *   T, E*G <= 8192 (else MOE_ERR_UNSUPPORTED).  Workspace: E*G*4 bytes
 *   (moe_workspace_bytes covers it).
 */
moe_status moe_coselect_cross(int64_t T, int32_t k, int32_t E, const int32_t* topk_idx_cur,
                              const int32_t* topk_idx_next, int32_t* coselect, void* stream);
moe_status moe_shuffle_plan(int64_t T, int32_t k, int32_t E, int32_t G,
                            const int32_t* topk_idx_cur, const int32_t* predictor,
                            const int32_t* placement_next, const int32_t* topk_idx_next,
                            int32_t* owner, int32_t* group_tokens, int32_t* stats,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_flips -- routing decisions that differ between two runs ([LAYOUT]
 * Finding 3: flipped decisions and their margins; Measurement Framework: a
 * 1-ULP change to one weight as a yardstick).  flips [T] int32: 1 when token
 * t's chosen expert set in topk_idx_a differs from that in topk_idx_b (slot
 * order ignored), else 0; n_flips [1] int32: their number.  topk_idx_a,
 * topk_idx_b [T,k] with ids in [0, E) (others are ignored).
 */
moe_status moe_route_flips(int64_t T, int32_t k, int32_t E, const int32_t* topk_idx_a,
                           const int32_t* topk_idx_b, int32_t* flips, int32_t* n_flips,
                           void* stream);

/*
 * moe_placement_greedy -- [host] correlated expert placement ([COUPLING]
 * Abstract and Fig. 3: experts that are often selected together go to the
 * same GPU).  Deterministic, integer arithmetic only.  Fills one group at a
 * time: seed = the unassigned expert with the largest co-selection mass to
 * the other unassigned experts (ties: lowest id); then repeatedly add the
 * unassigned expert with the largest co-selection count to the group's
 * members (ties: larger mass to the unassigned experts, then lowest id)
 * until the group holds E/G experts.
 * coselect [host] [E,E] int64 (symmetric); placement [host] [E] int32 out.
 */
moe_status moe_placement_greedy(int32_t E, int32_t G, const int64_t* coselect,
                                int32_t* placement);

/* [host] 0 when placement [host][E] is a balanced partition over G groups,
 * else MOE_ERR_INVALID_PLACEMENT (or MOE_ERR_INVALID_ARGUMENT). */
moe_status moe_check_placement(int32_t E, int32_t G, const int32_t* placement);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
