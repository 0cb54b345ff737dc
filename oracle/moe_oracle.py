"""CPU oracle for the MoE-layer hot path -- TEST INFRASTRUCTURE ONLY.

This module is the plain, slow, obviously correct statement of what the GPU
path computes.  Only the tests, the smoke check in the repository's graft
entry and the benchmark's CPU-baseline leg may import it; the product path
never does.  It shares no code with the HIP library.

Arithmetic is numpy float64 throughout.  Inputs arrive as float32 arrays whose
values are exactly representable (bf16-rounded where the workload stores bf16)
and are upcast without change.  Per-expert matrix products use numpy's matmul;
everything else is written out step by step in the order the pages describe.

Sources (page title -- place on the page):
  [LAYOUT] "MoE Pretraining: Parallelism Layout Changes the Model, Not Quality"
           -- Methodology (Models and Data table), Two Kinds of Layout Effects,
           Finding 3 (routing margin and near-ties), Practical Implications.
  [COUPLING] "Expert Coupling in MoE Pretraining: Reducing All-to-All Overhead
           with Correlated Placement and Token Shuffling" -- Abstract, Fig. 2,
           Table I, Fig. 3, Fig. 5, Table III (notation t, T, E, k, S(t), W).
  [REVISIT] "Revisiting MoE and Dense Speed-Accuracy Comparisons for LLM
           Training" -- Sec. 2.1 (SwiGLU, Top-K routing, load-balancing loss),
           Sec. 2.2 (GShard gating/dispatch/combine, outer batches), Sec. 3.6
           (naive second-expert routing).
  [LOADING] "Why does expert-parallel loading matter so much in MoE training?"
           -- What to verify before trusting an MoE checkpoint load.

Readings where the pages are silent or garbled (listed with reasons in the
design notes of the repository):
  * no router bias; logits l = X Wr^T with Wr stored [E, d];
  * top-k by descending logit, lower expert id first on exact ties;
  * gates: softmax renormalised over the k chosen logits;
  * margin: raw gap between the k-th and (k+1)-th largest logits, near-tie when
    it is below eps (default 1e-3); the normalised margin of [LAYOUT] Finding 3
    (gap / spread of the token's logits) is reported beside it;
  * SwiGLU: h = silu(x W1^T) * (x W3^T), y = h W2^T, weights [E, out, in];
  * dropless routing in the main path; the capacity variant (capacity_keep)
    gives each expert C = ceil(factor * (T/G) * k / E) places per block of T/G
    tokens, filled slot-major (all first choices in token order, then all
    second choices, ...); assignments past C are dropped (expert id -1, no
    row, no output), gates are not renormalised after dropping;
  * auxiliary losses: L_aux = mean over blocks of E * sum_e f_e P_e (f held
    constant), L_z = mean over tokens of logsumexp(l)^2, each times its
    coefficient;
  * LB statistics per contiguous token block: f = count / (block tokens * k),
    P = mean full-softmax probability, aux = E * sum_e f_e P_e;
  * dedup plan rows ordered by (group, token); all destinations count,
    including the token's home block.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


def _f64(a):
    return np.asarray(a, dtype=F64)


# ---------------------------------------------------------------------------
# Storage precision of activations.  The bf16 workloads store weights and
# activations in bfloat16 and accumulate in higher precision.  With
# act="bf16" every activation or activation-gradient tensor that a step of the
# layer produces (a, b, h, y_perm, y, dy_perm, dh, da, db, dx_perm, dx) and the
# expert weight gradients are rounded to bfloat16 when they are formed; all
# sums are still carried out in float64.  act="f64" stores nothing rounded.
# The router (logits, gates, its gradients) is fp32 in every workload and is
# never rounded here.
# ---------------------------------------------------------------------------

def to_bf16(v):
    """Round to the nearest bfloat16 value (8 significant bits), ties to even.
    Written from the definition: v = m * 2**e with 0.5 <= |m| < 1, so m * 2**8
    holds the 8 kept bits in its integer part."""
    v = _f64(v)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def storage(act):
    if act in ("f64", "f32", None):
        return lambda v: _f64(v)
    if act == "bf16":
        return to_bf16
    raise ValueError(act)


# ---------------------------------------------------------------------------
# Router: logits, top-k, gates, margins  ([COUPLING] Abstract: each token is
# routed to k of E experts; [REVISIT] Sec. 2.1 Top-K routing, Table 1 router
# weight "ME" with no bias; [REVISIT] Sec. 3.6 the second expert is simply the
# second best; [LAYOUT] Finding 3 margin and near-ties)
# ---------------------------------------------------------------------------

def router_logits(x, wr):
    """l[t, e] = sum_i x[t, i] * wr[e, i]."""
    return _f64(x) @ _f64(wr).T


def topk_select(logits, k):
    """Experts ordered by descending logit, lower id first on exact ties.

    Returns (idx [T,k] int32, margin [T] f64).  margin[t] is the gap between
    the k-th and the (k+1)-th largest logits (+inf when k == E).
    """
    logits = _f64(logits)
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    if k < E:
        kth = np.take_along_axis(logits, order[:, k - 1:k], axis=1)[:, 0]
        nxt = np.take_along_axis(logits, order[:, k:k + 1], axis=1)[:, 0]
        margin = kth - nxt
    else:
        margin = np.full(T, np.inf)
    return idx, margin


def chosen_gates(logits, idx):
    """Softmax over the chosen k logits only: g_j = exp(l_j) / sum_i exp(l_i)."""
    logits = _f64(logits)
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def full_softmax(logits):
    logits = _f64(logits)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def normalized_margin(logits, margin):
    """[LAYOUT] Finding 3: the margin divided by the spread of the token's scores."""
    logits = _f64(logits)
    spread = logits.max(axis=1) - logits.min(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(spread > 0, margin / spread, np.inf)


def route(x, wr, k, near_tie_eps=1e-3):
    """Router forward: logits, top-k, renormalised gates, margins, near-tie count."""
    logits = router_logits(x, wr)
    idx, margin = topk_select(logits, k)
    gates = chosen_gates(logits, idx)
    near = margin < near_tie_eps
    return {
        "logits": logits,
        "topk_idx": idx,
        "gates": gates,
        "margin": margin,
        "near_tie": near,
        "near_tie_count": int(near.sum()),
        "norm_margin": normalized_margin(logits, margin),
    }


def lb_stats(logits, idx, E, G):
    """Load-balancing statistics per contiguous block of T/G tokens.

    [LAYOUT] Key Insight and Two Kinds of Layout Effects: balancing statistics
    computed per machine; [REVISIT] Sec. 2.2: tokens split into O outer batches;
    [REVISIT] Sec. 2.1: GShard load-balancing loss.
    Returns count [G,E] int64, f [G,E], P [G,E], aux [G].
    """
    logits = _f64(logits)
    T, k = idx.shape
    if T % G:
        raise ValueError("G must divide T")
    n = T // G
    p = full_softmax(logits)
    count = np.zeros((G, E), dtype=np.int64)
    P = np.zeros((G, E))
    for r in range(G):
        for t in range(r * n, (r + 1) * n):
            for j in range(k):
                count[r, idx[t, j]] += 1
        P[r] = p[r * n:(r + 1) * n].mean(axis=0)
    f = count / float(n * k)
    aux = E * (f * P).sum(axis=1)
    return {"count": count, "f": f, "P": P, "aux": aux}


# ---------------------------------------------------------------------------
# Permutation into expert-contiguous rows ([COUPLING] Abstract and Fig. 5 step
# 3: dispatch tokens to their experts; [REVISIT] Sec. 2.2 GShard dispatch)
# ---------------------------------------------------------------------------

def permute_plan(idx, E):
    """Stable counting sort of the T*k (token, slot) assignments by expert.

    Inside one expert's segment the rows are in ascending token id.  An
    expert id of -1 marks a dropped assignment (capacity_keep): it gets no row
    and pos -1.
    Returns counts [E], offsets [E+1], pos [T,k] (row of assignment (t, j)),
    src [T*k] (token of each row; -1 past offsets[E]), all int64.
    """
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if idx[t, j] >= 0:
                counts[idx[t, j]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    pos = np.full((T, k), -1, dtype=np.int64)
    src = np.full(T * k, -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if e < 0:
                continue
            pos[t, j] = fill[e]
            src[fill[e]] = t
            fill[e] += 1
    return {"counts": counts, "offsets": offsets, "pos": pos, "src": src}


def gather_rows(x, src):
    """x_perm[p] = x[src[p]]."""
    return _f64(x)[np.asarray(src, dtype=np.int64)]


# ---------------------------------------------------------------------------
# SwiGLU experts ([REVISIT] Sec. 2.1: SwiGLU activation; [LAYOUT] Methodology:
# SwiGLU experts; [COUPLING] Fig. 5 step 4: expert computation)
# ---------------------------------------------------------------------------

def _sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def silu(a):
    return a * _sigmoid(a)


def swiglu_experts(x_perm, offsets, w1, w3, w2, act="f64", row_scale=None):
    """Per expert e over rows [offsets[e], offsets[e+1]):
    a = X W1[e]^T, b = X W3[e]^T, h = silu(a) * b, y = h W2[e]^T.
    (act="bf16": a, b, h and y are stored as bfloat16 values.)
    row_scale [R], when given, multiplies h row by row before it is stored
    (the gate folded onto the expert row: y then carries the gate)."""
    st = storage(act)
    x_perm = _f64(x_perm)
    w1, w3, w2 = _f64(w1), _f64(w3), _f64(w2)
    R = x_perm.shape[0]
    E, f, d = w1.shape
    a = np.zeros((R, f))
    b = np.zeros((R, f))
    h = np.zeros((R, f))
    y = np.zeros((R, d))
    for e in range(E):
        s = slice(int(offsets[e]), int(offsets[e + 1]))
        xe = x_perm[s]
        a[s] = st(xe @ w1[e].T)
        b[s] = st(xe @ w3[e].T)
        hs = silu(a[s]) * b[s]
        if row_scale is not None:
            hs = hs * _f64(row_scale)[s, None]
        h[s] = st(hs)
        y[s] = st(h[s] @ w2[e].T)
    return {"a": a, "b": b, "h": h, "y_perm": y}


def swiglu_experts_bwd(x_perm, offsets, w1, w3, w2, a, b, dy_perm, act="f64"):
    """Backward of swiglu_experts for the upstream gradient dy_perm [R, d].

    dh = dy W2[e]; da = dh * b * silu'(a); db = dh * silu(a);
    dx = da W1[e] + db W3[e]; dW2[e] = dy^T h; dW1[e] = da^T x; dW3[e] = db^T x,
    with silu'(a) = s (1 + a (1 - s)), s = sigmoid(a) and h = silu(a) * b.
    (act="bf16": dh, da, db, dx and the weight gradients are stored as bfloat16.)
    """
    st = storage(act)
    x_perm, dy_perm = _f64(x_perm), _f64(dy_perm)
    a, b = _f64(a), _f64(b)
    w1, w3, w2 = _f64(w1), _f64(w3), _f64(w2)
    E, f, d = w1.shape
    R = x_perm.shape[0]
    dx = np.zeros((R, d))
    dh = np.zeros((R, f))
    da = np.zeros((R, f))
    db = np.zeros((R, f))
    h = np.zeros((R, f))
    for e in range(E):
        s = slice(int(offsets[e]), int(offsets[e + 1]))
        sg = _sigmoid(a[s])
        act_s = a[s] * sg
        dact = sg * (1.0 + a[s] * (1.0 - sg))
        dh[s] = st(dy_perm[s] @ w2[e])
        da[s] = st(dh[s] * b[s] * dact)
        db[s] = st(dh[s] * act_s)
        dx[s] = st(da[s] @ w1[e] + db[s] @ w3[e])
        h[s] = st(act_s * b[s])
    wg = expert_weight_grads(x_perm, offsets, h, dy_perm, da, db, E, act)
    return {"dx_perm": dx, "dw1": wg["dw1"], "dw3": wg["dw3"], "dw2": wg["dw2"],
            "dh": dh, "da": da, "db": db}


def expert_weight_grads(x_perm, offsets, h, dy_perm, da, db, E, act="f64"):
    """The expert weight gradients as products over each expert's rows
    [offsets[e], offsets[e+1]): dW2[e] = dy^T h, dW1[e] = da^T x, dW3[e] =
    db^T x (zero for an expert without rows).  On absolute values of the
    operands it gives the sums of |terms| of every entry.
    (act="bf16": the weight gradients are stored as bfloat16.)"""
    st = storage(act)
    x_perm, h, dy_perm = _f64(x_perm), _f64(h), _f64(dy_perm)
    da, db = _f64(da), _f64(db)
    d, f = x_perm.shape[1], h.shape[1]
    dw1 = np.zeros((E, f, d))
    dw3 = np.zeros((E, f, d))
    dw2 = np.zeros((E, d, f))
    for e in range(E):
        s = slice(int(offsets[e]), int(offsets[e + 1]))
        dw2[e] = st(dy_perm[s].T @ h[s])
        dw1[e] = st(da[s].T @ x_perm[s])
        dw3[e] = st(db[s].T @ x_perm[s])
    return {"dw1": dw1, "dw3": dw3, "dw2": dw2}


def swiglu_experts_bwd_folded(x_perm, offsets, w1, w3, w2, a, b, hg, dy_rows, g_row,
                              act="f64"):
    """swiglu_experts_bwd with the gate folded onto the rows ([REVISIT] Sec. 2.1:
    the combine weights each expert output by its gate, and the expert output
    is linear in h, so the gate may sit on h).  For the upstream dY rows of
    each expert row (dy_rows = dY[src]) and the row gates g_row:
      u = dy_rows W2[e] (stored), dh = g u (not stored),
      da = dh * b * silu'(a), db = dh * silu(a), dx = da W1[e] + db W3[e],
      dgate_row = <u, silu(a) * b>  (= <dY, y_perm> of the unfolded layer),
      dW2[e] = dy_rows^T hg with hg = g h the forward's stored rows,
      dW1[e] = da^T x, dW3[e] = db^T x."""
    st = storage(act)
    x_perm, dy_rows = _f64(x_perm), _f64(dy_rows)
    a, b, hg, g_row = _f64(a), _f64(b), _f64(hg), _f64(g_row)
    w1, w3, w2 = _f64(w1), _f64(w3), _f64(w2)
    E, f, d = w1.shape
    R = x_perm.shape[0]
    dx = np.zeros((R, d))
    u = np.zeros((R, f))
    da = np.zeros((R, f))
    db = np.zeros((R, f))
    dgate_row = np.zeros(R)
    dw1 = np.zeros_like(w1)
    dw3 = np.zeros_like(w3)
    dw2 = np.zeros_like(w2)
    for e in range(E):
        s = slice(int(offsets[e]), int(offsets[e + 1]))
        sg = _sigmoid(a[s])
        act_s = a[s] * sg
        dact = sg * (1.0 + a[s] * (1.0 - sg))
        u[s] = st(dy_rows[s] @ w2[e])
        dh = g_row[s, None] * u[s]
        dgate_row[s] = (u[s] * act_s * b[s]).sum(axis=1)
        da[s] = st(dh * b[s] * dact)
        db[s] = st(dh * act_s)
        dx[s] = st(da[s] @ w1[e] + db[s] @ w3[e])
        dw2[e] = st(dy_rows[s].T @ hg[s])
        dw1[e] = st(da[s].T @ x_perm[s])
        dw3[e] = st(db[s].T @ x_perm[s])
    return {"dx_perm": dx, "dw1": dw1, "dw3": dw3, "dw2": dw2, "u": u, "da": da, "db": db,
            "dgate_row": dgate_row}


# ---------------------------------------------------------------------------
# Combine and its adjoint ([COUPLING] Abstract and Fig. 5 step 5: combine the
# results; [REVISIT] Sec. 2.2 GShard combine)
# ---------------------------------------------------------------------------

def combine(rows, pos, gates=None, act="f64"):
    """y[t] = sum_j g[t, j] * rows[pos[t, j]]  (unit weights when gates is None);
    slots with pos -1 (dropped) add nothing."""
    rows = _f64(rows)
    T, k = pos.shape
    y = np.zeros((T, rows.shape[1]))
    for j in range(k):
        w = 1.0 if gates is None else _f64(gates)[:, j:j + 1]
        p = np.asarray(pos[:, j], dtype=np.int64)
        live = (p >= 0)[:, None]
        y += np.where(live, w * rows[np.maximum(p, 0)], 0.0)
    return storage(act)(y)


def combine_bwd(dy, y_perm, pos, gates, act="f64"):
    """dy_perm[pos[t,j]] = g[t,j] dY[t];  dgate[t,j] = <dY[t], y_perm[pos[t,j]]>;
    a dropped slot (pos -1) has no row and dgate 0.
    (act="bf16": dy_perm is stored as bfloat16; dgate is a router quantity.)"""
    st = storage(act)
    dy, y_perm, gates = _f64(dy), _f64(y_perm), _f64(gates)
    T, k = pos.shape
    dy_perm = np.zeros((T * k, dy.shape[1]))
    dgate = np.zeros((T, k))
    for j in range(k):
        p = np.asarray(pos[:, j], dtype=np.int64)
        live = p >= 0
        dy_perm[p[live]] = st(gates[live, j:j + 1] * dy[live])
        dgate[live, j] = (dy[live] * y_perm[p[live]]).sum(axis=1)
    return dy_perm, dgate


# ---------------------------------------------------------------------------
# Router backward (adjoint of logits -> top-k -> renormalised softmax)
# ---------------------------------------------------------------------------

def route_bwd(x, wr, idx, gates, dgate, logits=None, count=None, aux_coef=0.0, z_coef=0.0):
    """dl[t, S_j] = g_j (dg_j - sum_i g_i dg_i), zero for unchosen experts;
    plus aux_coef * dL_aux/dl and z_coef * dL_z/dl when those are non-zero
    (logits [T,E] and, for L_aux, the block counts [G,E] of lb_stats);
    dX_router = dl Wr;  dWr = dl^T X."""
    x, wr, gates, dgate = _f64(x), _f64(wr), _f64(gates), _f64(dgate)
    T, k = idx.shape
    E = wr.shape[0]
    inner = (gates * dgate).sum(axis=1, keepdims=True)
    dsel = gates * (dgate - inner)
    dl = np.zeros((T, E))
    for j in range(k):
        dl[np.arange(T), idx[:, j]] += dsel[:, j]
    if aux_coef != 0.0:
        dl += aux_coef * aux_loss_grad(logits, count, k)
    if z_coef != 0.0:
        dl += z_coef * z_loss_grad(logits)
    return {"dlogits": dl, "dx_router": dl @ wr, "dwr": dl.T @ x}


# ---------------------------------------------------------------------------
# Definitional variants ([REVISIT] Sec. 2.1: Top-K routing with an expert
# capacity, the GShard load-balancing loss and the ST-MoE router z-loss;
# Sec. 4: a lower capacity for training than for evaluation; [LAYOUT] Two
# Kinds of Layout Effects: capacity and balancing computed per machine, here
# per contiguous block of T/G tokens)
# ---------------------------------------------------------------------------

def expert_capacity(T, k, E, G, factor):
    """Places per expert in one block of n = T/G tokens: ceil(factor * (n k) / E),
    the capacity factor times the block's mean load per expert."""
    n = T // G
    return int(math.ceil(factor * float(n * k) / E))


def capacity_keep(idx, E, G, C):
    """Per-block capacity with dropping.

    Inside block r (tokens r n .. r n + n - 1) the assignments queue for their
    experts slot-major, as GShard places second choices after all first
    choices: slot 0 of every token in token order, then slot 1, and so on.
    place[t, j] is the number of assignments ahead of (t, j) in its expert's
    queue; the assignment is kept when place < C, else dropped.
    Returns kept_idx [T,k] (expert id, or -1 when dropped), place [T,k] and
    dropped [G] (dropped assignments per block).
    """
    T, k = idx.shape
    n = T // G
    kept = np.array(idx, dtype=np.int64)
    place = np.zeros((T, k), dtype=np.int64)
    dropped = np.zeros(G, dtype=np.int64)
    for r in range(G):
        load = np.zeros(E, dtype=np.int64)
        for j in range(k):
            for t in range(r * n, (r + 1) * n):
                e = idx[t, j]
                place[t, j] = load[e]
                load[e] += 1
                if place[t, j] >= C:
                    kept[t, j] = -1
                    dropped[r] += 1
    return {"kept_idx": kept, "place": place, "dropped": dropped}


def _logsumexp(logits):
    logits = _f64(logits)
    m = logits.max(axis=1)
    return m + np.log(np.exp(logits - m[:, None]).sum(axis=1))


def aux_loss(logits, count, k):
    """L_aux = (1/G) sum_r E sum_e f[r,e] P[r,e] with f = count / (n k) (a
    constant) and P[r] the mean full softmax over block r: the mean of
    lb_stats' aux over the blocks."""
    logits = _f64(logits)
    G, E = count.shape
    n = logits.shape[0] // G
    p = full_softmax(logits)
    total = 0.0
    for r in range(G):
        f = count[r] / float(n * k)
        P = p[r * n:(r + 1) * n].mean(axis=0)
        total += E * (f * P).sum()
    return total / G


def aux_loss_grad(logits, count, k):
    """dL_aux/dl[t,i] = E / (G n) * p[t,i] (f[r,i] - sum_e f[r,e] p[t,e]),
    the softmax Jacobian applied to f, for t in block r."""
    logits = _f64(logits)
    G, E = count.shape
    T = logits.shape[0]
    n = T // G
    p = full_softmax(logits)
    dl = np.zeros((T, E))
    for r in range(G):
        f = count[r] / float(n * k)
        pr = p[r * n:(r + 1) * n]
        fp = (pr * f[None, :]).sum(axis=1, keepdims=True)
        dl[r * n:(r + 1) * n] = (E / float(G * n)) * pr * (f[None, :] - fp)
    return dl


def z_loss(logits):
    """L_z = (1/T) sum_t (log sum_e exp l[t,e])^2."""
    return float((_logsumexp(logits) ** 2).mean())


def z_loss_groups(logits, G):
    """Per block r: the mean over its tokens of logsumexp(l[t])^2."""
    z = _logsumexp(logits) ** 2
    return z.reshape(G, -1).mean(axis=1)


def z_loss_grad(logits):
    """dL_z/dl[t,i] = (2 / T) lse_t p[t,i]."""
    logits = _f64(logits)
    T = logits.shape[0]
    return (2.0 / T) * _logsumexp(logits)[:, None] * full_softmax(logits)


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

def layer_forward(x, wr, w1, w3, w2, k, near_tie_eps=1e-3, routing=None, act="f64",
                  capacity=None, lb_groups=1, fold_gate=False):
    """Router -> permute -> SwiGLU experts -> combine.

    routing, when given, is a (topk_idx, gates) pair that replaces the router's
    own decision (the logits, margins and near-ties are still reported).
    act: storage precision of the activations ("f64" or "bf16").
    capacity, when given, is the per-block expert capacity C of capacity_keep
    over lb_groups blocks; dropped assignments get no row and no output.
    fold_gate: the gate multiplies h of each expert row (h holds g h) and the
    combine adds the rows unweighted; the same layer in exact arithmetic, with
    the storage rounding at different points.
    """
    E = np.asarray(wr).shape[0]
    r = route(x, wr, k, near_tie_eps)
    if routing is not None:
        idx, gates = routing
        idx = np.asarray(idx, dtype=np.int32)
        gates = _f64(gates)
    else:
        idx, gates = r["topk_idx"], r["gates"]
    kept = idx
    cap = None
    if capacity is not None:
        cap = capacity_keep(idx, E, lb_groups, capacity)
        kept = cap["kept_idx"]
    plan = permute_plan(kept, E)
    x_perm = gather_rows(x, plan["src"])
    g_row = None
    if fold_gate:
        g_row = np.zeros(x_perm.shape[0])
        live = plan["pos"] >= 0
        g_row[plan["pos"][live]] = _f64(gates)[live]
    ex = swiglu_experts(x_perm, plan["offsets"], w1, w3, w2, act, row_scale=g_row)
    y = combine(ex["y_perm"], plan["pos"], None if fold_gate else gates, act)
    out = dict(r)
    out.update(plan)
    out.update(ex)
    out.update({"topk_idx": idx, "gates": gates, "x_perm": x_perm, "y": y, "act": act,
                "kept_idx": kept, "lb_groups": lb_groups, "fold_gate": fold_gate,
                "g_row": g_row})
    if cap is not None:
        out["dropped"] = cap["dropped"]
    return out


def layer_backward(x, wr, w1, w3, w2, fwd, dy, aux_coef=0.0, z_coef=0.0):
    """Backward of layer_forward for the upstream gradient dy [T, d], in the
    forward's storage precision, plus the gradients of aux_coef * L_aux (over
    the forward's lb_groups blocks) and z_coef * L_z when they are non-zero."""
    act = fwd.get("act", "f64")
    if fwd.get("fold_gate"):
        # the gate sits on the rows: dY is read through src, dgate comes from
        # the rows' <u, h> (a dropped slot has no row and dgate 0)
        dy_perm = None
        eb = swiglu_experts_bwd_folded(fwd["x_perm"], fwd["offsets"], w1, w3, w2, fwd["a"],
                                       fwd["b"], fwd["h"], gather_rows(dy, fwd["src"]),
                                       fwd["g_row"], act)
        pos = fwd["pos"]
        dgate = np.where(pos >= 0, eb["dgate_row"][np.maximum(pos, 0)], 0.0)
        eb["dh"] = eb["u"] * _f64(fwd["g_row"])[:, None]
    else:
        dy_perm, dgate = combine_bwd(dy, fwd["y_perm"], fwd["pos"], fwd["gates"], act)
        eb = swiglu_experts_bwd(fwd["x_perm"], fwd["offsets"], w1, w3, w2,
                                fwd["a"], fwd["b"], dy_perm, act)
    dx_exp = combine(eb["dx_perm"], fwd["pos"], None)
    count = None
    if aux_coef != 0.0:
        E = np.asarray(wr).shape[0]
        count = lb_stats(fwd["logits"], fwd["topk_idx"], E, fwd.get("lb_groups", 1))["count"]
    rb = route_bwd(x, wr, fwd["topk_idx"], fwd["gates"], dgate, fwd["logits"], count,
                   aux_coef, z_coef)
    return {
        "dy_perm": dy_perm, "dgate": dgate,
        "dx_perm": eb["dx_perm"], "dh": eb["dh"], "da": eb["da"], "db": eb["db"],
        "dw1": eb["dw1"], "dw3": eb["dw3"], "dw2": eb["dw2"],
        "dx_expert": dx_exp, "dlogits": rb["dlogits"],
        "dx": storage(act)(dx_exp + rb["dx_router"]), "dwr": rb["dwr"],
    }


# ---------------------------------------------------------------------------
# Forward error bounds of the layer's float outputs
#
# A GPU layer stores activations in a short format (bfloat16: 8 significant
# bits, unit roundoff u = 2**-8) and accumulates in fp32 (unit roundoff
# 2**-24).  Its outputs then differ from the exact layer above by rounding
# alone, and that difference has a classical bound (Higham, "Accuracy and
# Stability of Numerical Algorithms", Sec. 3.1: a computed dot product of n
# terms is within gamma_n * sum |terms| of the exact one, gamma_n = n u /
# (1 - n u)).  Carried through the layer to first order, every quantity q that
# the layer forms gets a bound B(q) from the EXACT operands only:
#   * a stored result adds u |q| (one rounding, wherever it happens);
#   * a sum or dot product adds gamma_n(fp32) * sum |terms|, and passes on
#     the bounds of its operands through |other operand|;
#   * an elementwise function f(a) passes on |f'(a)| B(a).
# The bound is written for the plain (unfolded) layer: quantities that a
# computation may store are the named tensors of layer_forward/backward (a,
# b, h, y_perm, y, dy_perm, dh, da, db, dx_perm, dx, dW); the router-side
# quantities (gates, dgate, dlogits, dWr) are fp32.  A computation that
# stores a rescaled tensor instead (g h in place of h, dY W2 in place of
# g dY W2) has the same relative rounding, so the same bound covers it.
# The check |gpu - exact| <= c B(q) is then independent of where a kernel
# rounds, and a slip such as a dropped term, a wrong index or a wrong sign
# is far outside it (an error of the size of the terms, not u times them).
# ---------------------------------------------------------------------------

U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24


def gamma(n, u=U_F32):
    """Higham's gamma_n = n u / (1 - n u)."""
    return n * u / (1.0 - n * u)


def _silu_derivs(a):
    s = _sigmoid(a)
    d1 = s * (1.0 + a * (1.0 - s))
    d2 = s * (1.0 - s) * (2.0 + a * (1.0 - 2.0 * s))
    return a * s, d1, d2


def layer_error_bounds(x, wr, w1, w3, w2, fwd, bwd=None, dy=None, u=U_BF16,
                       aux_coef=0.0, z_coef=0.0, ufn=8 * U_F32):
    """First-order componentwise error bounds B(q) around the exact layer.

    fwd, bwd come from layer_forward / layer_backward with act="f64" and no
    gate folding (capacity and the auxiliary losses are allowed: pass the same
    aux_coef and z_coef as to layer_backward).  u is the unit roundoff of the
    stored activations (2**-8 for bfloat16, 2**-24 when they are fp32); ufn is
    the relative error allowed for one evaluation of an exp-based function
    (sigmoid, silu) in fp32.  Returns bounds shaped like the outputs: a, b, h,
    y_perm, y and, with bwd, dy_perm, dgate, dh, da, db, dx_perm, dw1, dw3,
    dw2, dlogits, dwr, dx.  Bounds are carried in float32: they are
    magnitudes, and six significant digits are more than a tolerance needs."""
    if fwd.get("fold_gate") or fwd.get("act", "f64") != "f64":
        raise ValueError("bounds are taken around the exact, unfolded layer")
    F = np.float32

    def A(v):
        return np.abs(np.asarray(v)).astype(F)

    x, wr = _f64(x), _f64(wr)
    w1, w3, w2 = _f64(w1), _f64(w3), _f64(w2)
    E, f, d = w1.shape
    off, pos, gates = fwd["offsets"], fwd["pos"], _f64(fwd["gates"])
    T, k = pos.shape
    xp, a, b, h, yp = fwd["x_perm"], fwd["a"], fwd["b"], fwd["h"], fwd["y_perm"]
    u, uf = F(u), F(ufn)
    g_d, g_f = F(gamma(d)), F(gamma(f))
    act_a, d1, d2 = _silu_derivs(a)
    act_a, d1, d2 = A(act_a), A(d1), A(d2)
    aW1, aW3, aW2 = A(w1), A(w3), A(w2)
    Ba = np.zeros(a.shape, F)
    Bb = np.zeros(b.shape, F)
    for e in range(E):
        s = slice(int(off[e]), int(off[e + 1]))
        ax = A(xp[s])
        Ba[s] = u * A(a[s]) + g_d * (ax @ aW1[e].T)
        Bb[s] = u * A(b[s]) + g_d * (ax @ aW3[e].T)
    ab = A(b)
    Bh = (u + uf) * A(h) + d1 * ab * Ba + act_a * Bb
    Byp = np.zeros(yp.shape, F)
    ah = A(h)
    for e in range(E):
        s = slice(int(off[e]), int(off[e + 1]))
        Byp[s] = u * A(yp[s]) + (Bh[s] + g_f * ah[s]) @ aW2[e].T
    live = pos >= 0
    ayp = A(yp)
    By = u * A(fwd["y"])
    ay = np.zeros(By.shape, F)
    for j in range(k):
        p = np.maximum(pos[:, j], 0)
        w = np.where(live[:, j], gates[:, j], 0.0).astype(F)[:, None]
        By += w * Byp[p]
        ay += w * ayp[p]
    By += F(gamma(k + 1)) * ay
    out = {"a": Ba, "b": Bb, "h": Bh, "y_perm": Byp, "y": By}
    if bwd is None:
        return out

    ady = A(dy)
    dyp, dh, da, db = bwd["dy_perm"], bwd["dh"], bwd["da"], bwd["db"]
    dxp = bwd["dx_perm"]
    # dy_perm = g dY (one rounding; g itself is an fp32 value)
    adyp = A(dyp)
    Bdyp = (u + F(U_F32)) * adyp
    # dgate = <dY, y_perm> over d, in fp32
    Bdg = np.zeros((T, k), F)
    for j in range(k):
        p = np.maximum(pos[:, j], 0)
        v = (ady * (Byp[p] + g_d * ayp[p])).sum(axis=1)
        Bdg[:, j] = np.where(live[:, j], v, 0.0)
    adh = A(dh)
    Bdh = np.zeros(dh.shape, F)
    for e in range(E):
        s = slice(int(off[e]), int(off[e + 1]))
        Bdh[s] = u * adh[s] + (Bdyp[s] + g_d * adyp[s]) @ aW2[e]
    ada, adb = A(da), A(db)
    Bda = (u + uf) * ada + Bdh * ab * d1 + adh * Bb * d1 + adh * ab * d2 * Ba
    Bdb = (u + uf) * adb + Bdh * act_a + adh * d1 * Ba
    g2f = F(gamma(2 * f))
    Bdxp = np.zeros(dxp.shape, F)
    Bdw1 = np.zeros(w1.shape, F)
    Bdw3 = np.zeros(w3.shape, F)
    Bdw2 = np.zeros(w2.shape, F)
    for e in range(E):
        s = slice(int(off[e]), int(off[e + 1]))
        n = int(off[e + 1] - off[e])
        Bdxp[s] = (u * A(dxp[s]) + (Bda[s] + g2f * ada[s]) @ aW1[e]
                   + (Bdb[s] + g2f * adb[s]) @ aW3[e])
        gn = F(gamma(max(n, 1)))
        ax = A(xp[s])
        Bdw1[e] = u * A(bwd["dw1"][e]) + (Bda[s] + gn * ada[s]).T @ ax
        Bdw3[e] = u * A(bwd["dw3"][e]) + (Bdb[s] + gn * adb[s]).T @ ax
        Bdw2[e] = (u * A(bwd["dw2"][e]) + (Bdyp[s] + gn * adyp[s]).T @ ah[s]
                   + adyp[s].T @ Bh[s])
    # dl[t, S_j] = g_j (dg_j - sum_i g_i dg_i) in fp32, plus the fp32 loss terms
    adg = np.abs(_f64(bwd["dgate"]))
    inner_b = (gates * Bdg).sum(axis=1, keepdims=True)
    inner_a = (gates * adg).sum(axis=1, keepdims=True)
    Bsel = gates * (Bdg + inner_b) + 8 * U_F32 * gates * (adg + inner_a)
    Bdl = np.zeros((T, E))
    for j in range(k):
        Bdl[np.arange(T), fwd["topk_idx"][:, j]] += Bsel[:, j]
    if aux_coef != 0.0 or z_coef != 0.0:
        p = full_softmax(fwd["logits"])
        if aux_coef != 0.0:
            G = fwd.get("lb_groups", 1)
            count = lb_stats(fwd["logits"], fwd["topk_idx"], E, G)["count"]
            n = T // G
            fr = np.repeat(count / float(n * fwd["topk_idx"].shape[1]), n, axis=0)
            mag = (E / float(G * n)) * p * (fr + (fr * p).sum(axis=1, keepdims=True))
            Bdl += 16 * U_F32 * abs(aux_coef) * mag
        if z_coef != 0.0:
            Bdl += 16 * U_F32 * abs(z_coef) * (2.0 / T) * np.abs(_logsumexp(fwd["logits"]))[:, None] * p
    Bdl = Bdl.astype(F)
    adl = A(bwd["dlogits"])
    Bdwr = F(U_F32) * A(bwd["dwr"]) + (Bdl + F(gamma(T)) * adl).T @ A(x)
    # dx = sum_j dx_perm[pos_j] + dl Wr, summed in fp32 and rounded once
    adxp = A(dxp)
    Bdx = u * A(bwd["dx"])
    adx = np.zeros(Bdx.shape, F)
    for j in range(k):
        p = np.maximum(pos[:, j], 0)
        m = live[:, j][:, None]
        Bdx += np.where(m, Bdxp[p], F(0))
        adx += np.where(m, adxp[p], F(0))
    awr = A(wr)
    adx += adl @ awr
    Bdx += Bdl @ awr + F(gamma(k + E + 1)) * adx
    out.update({"dy_perm": Bdyp, "dgate": Bdg, "dh": Bdh, "da": Bda, "db": Bdb,
                "dx_perm": Bdxp, "dw1": Bdw1, "dw3": Bdw3, "dw2": Bdw2, "dlogits": Bdl,
                "dwr": Bdwr, "dx": Bdx})
    return out


# ---------------------------------------------------------------------------
# Index products for expert-parallel layouts ([COUPLING] Table III notation,
# Fig. 2 co-selection, Fig. 3 correlated placement, Abstract: a dispatcher that
# sends each token to each GPU once, Table I statistics)
# ---------------------------------------------------------------------------

def coselect(idx, E):
    """W[e, e'] = number of tokens that select both e and e' (diagonal zero)."""
    T, k = idx.shape
    W = np.zeros((E, E), dtype=np.int64)
    for t in range(T):
        for i in range(k):
            for j in range(k):
                if i != j:
                    W[idx[t, i], idx[t, j]] += 1
    return W


def coselect_cross(idx_cur, idx_next, E):
    """Cross-layer co-selection ([COUPLING] Abstract: the experts a token picks
    at one layer predict its picks at the next; Fig. 2(b)): W[e1, e2] = number
    of tokens that select e1 at layer l (idx_cur) and e2 at layer l+1
    (idx_next).  e1 == e2 counts too: the layers' experts are distinct."""
    T, k = idx_cur.shape
    W = np.zeros((E, E), dtype=np.int64)
    for t in range(T):
        for i in range(k):
            for j in range(idx_next.shape[1]):
                W[idx_cur[t, i], idx_next[t, j]] += 1
    return W


def shuffle_plan(idx_cur, W, placement_next, G):
    """Token-shuffle planner ([COUPLING] Fig. 5 step 1, Fig. 6, Table I "token
    moved"): each token goes to the group expected to hold most of its
    next-layer experts, predicted from its current experts through the
    cross-layer counts W (fit on other batches):
        owner(t) = argmax_g sum_{e1 in S_cur(t)} sum_{e2 : placement(e2) = g} W[e1, e2],
    ties to the lowest group id.  Returns owner [T] and the tokens per group."""
    T, k = idx_cur.shape
    E = W.shape[0]
    owner = np.zeros(T, dtype=np.int64)
    for t in range(T):
        best, best_g = None, 0
        for g in range(G):
            score = 0
            for i in range(k):
                for e2 in range(E):
                    if placement_next[e2] == g:
                        score += int(W[idx_cur[t, i], e2])
            if best is None or score > best:
                best, best_g = score, g
        owner[t] = best_g
    return {"owner": owner, "group_tokens": np.bincount(owner, minlength=G)}


def shuffle_local(owner, idx_next, placement_next, G):
    """Table I "local experts": next-layer assignments served on the token's
    own group, when it sits on the planned owner (moved) and when it stays on
    its home group t // (T/G).  Returns (moved, stays) assignment counts."""
    T, k = idx_next.shape
    n = T // G
    moved = stays = 0
    for t in range(T):
        for j in range(k):
            g = placement_next[idx_next[t, j]]
            moved += int(g == owner[t])
            stays += int(g == t // n)
    return moved, stays


def route_flips(idx_a, idx_b):
    """[LAYOUT] Finding 3 (routing decisions that change between two runs):
    flips[t] is True when token t's chosen expert set differs (slot order
    ignored)."""
    return np.array([set(map(int, a)) != set(map(int, b)) for a, b in zip(idx_a, idx_b)],
                    dtype=bool)


def nudge_ulps(w, e, i, m):
    """Router weight with element (e, i) moved m units in the last place of
    fp32 (toward +inf for m > 0): [LAYOUT] Measurement Framework, the 1-ULP
    change to a single weight (m = 1)."""
    w = np.array(w, dtype=np.float32, copy=True)
    v = w[e, i]
    step = np.float32(np.inf) if m > 0 else np.float32(-np.inf)
    for _ in range(abs(int(m))):
        v = np.nextafter(v, step)
    w[e, i] = v
    return w


def placement_contiguous(E, G):
    """Expert e lives in group floor(e / (E/G))."""
    if E % G:
        raise ValueError("G must divide E")
    return np.arange(E, dtype=np.int64) // (E // G)


def check_placement(placement, E, G):
    """[LOADING] What to verify: every expert owned by exactly one group, and
    equal expert counts per group.  Raises ValueError otherwise."""
    placement = np.asarray(placement)
    if placement.shape != (E,) or E % G:
        raise ValueError("placement must have E entries and G must divide E")
    if placement.min() < 0 or placement.max() >= G:
        raise ValueError("placement entries must lie in [0, G)")
    per = np.bincount(placement, minlength=G)
    if not np.all(per == E // G):
        raise ValueError("placement must put E/G experts in every group")


def placement_greedy(W, G):
    """Correlated placement: fill one group at a time with experts that are
    often selected together ([COUPLING] Abstract and Fig. 3).

    The pages do not print the fitting algorithm; this is a plain greedy
    reading, in integer arithmetic:
      1. seed the group with the unassigned expert of largest co-selection mass
         to the other unassigned experts (ties: lowest id);
      2. repeatedly add the unassigned expert with the largest co-selection
         count to the group's members (ties: larger mass to the unassigned
         experts, then lowest id) until the group holds E/G experts.
    """
    W = np.asarray(W, dtype=np.int64)
    E = W.shape[0]
    if E % G:
        raise ValueError("G must divide E")
    cap = E // G
    placement = np.full(E, -1, dtype=np.int64)
    unassigned = list(range(E))
    for g in range(G):
        def mass(e):
            return sum(int(W[e, o]) for o in unassigned if o != e)
        seed = unassigned[0]
        best = mass(seed)
        for e in unassigned[1:]:
            m = mass(e)
            if m > best:
                seed, best = e, m
        members = [seed]
        unassigned.remove(seed)
        while len(members) < cap:
            pick, key = None, None
            for e in unassigned:
                cand = (sum(int(W[e, m]) for m in members), mass(e))
                if key is None or cand > key:
                    pick, key = e, cand
            members.append(pick)
            unassigned.remove(pick)
        for e in members:
            placement[e] = g
    return placement


def dispatch_plan(idx, placement, G):
    """Deduplicated dispatch: each token is sent to each group once.

    D_t = the distinct groups of the token's chosen experts; one row per
    (g, t) with g in D_t, rows ordered by (g, t).  assign_row[t, j] is the row
    that carries expert slot j of token t.  Table I statistics of [COUPLING]:
    share of tokens whose experts share one group, distinct destinations per
    token, and rows removed as duplicates.  home(t) = t // (T/G).
    """
    idx = np.asarray(idx)
    placement = np.asarray(placement, dtype=np.int64)
    T, k = idx.shape
    n_dest = np.zeros(T, dtype=np.int64)
    dest = []
    for t in range(T):
        groups = sorted({int(placement[idx[t, j]]) for j in range(k)})
        dest.append(groups)
        n_dest[t] = len(groups)
    group_rows = np.zeros(G, dtype=np.int64)
    for t in range(T):
        for g in dest[t]:
            group_rows[g] += 1
    group_offsets = np.zeros(G + 1, dtype=np.int64)
    for g in range(G):
        group_offsets[g + 1] = group_offsets[g] + group_rows[g]
    fill = group_offsets[:-1].copy()
    row_of = {}
    row_token = np.zeros(int(group_offsets[G]), dtype=np.int64)
    for t in range(T):
        for g in dest[t]:
            row_of[(g, t)] = fill[g]
            row_token[fill[g]] = t
            fill[g] += 1
    assign_row = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            assign_row[t, j] = row_of[(int(placement[idx[t, j]]), t)]
    rows_total = int(group_offsets[G])
    per_home = T // G if T % G == 0 else None
    off_home = 0
    if per_home:
        for t in range(T):
            for g in dest[t]:
                if g != t // per_home:
                    off_home += 1
    return {
        "n_dest": n_dest, "group_rows": group_rows, "group_offsets": group_offsets,
        "row_token": row_token, "assign_row": assign_row,
        "rows_total": rows_total, "rows_removed": T * k - rows_total,
        "tokens_single_group": int((n_dest == 1).sum()), "rows_off_home": off_home,
        "same_group_share": float((n_dest == 1).mean()),
        "mean_destinations": rows_total / T,
        "dedup_fraction": (T * k - rows_total) / (T * k),
    }


# ---------------------------------------------------------------------------
# Expert-parallel dispatch emulated on one device ([COUPLING] Abstract: the
# dispatcher sends each token to each GPU once; Fig. 5 steps 3-4: dispatch,
# then the receiving GPU runs its experts on the rows it received)
# ---------------------------------------------------------------------------

def dispatch_pack(x, row_token, n_rows):
    """Send buffer of the deduplicated plan: row r (group-contiguous, ordered
    by (group, token)) is X[row_token[r]], for r < n_rows."""
    x = np.asarray(x)
    row_token = np.asarray(row_token, dtype=np.int64)
    send = np.zeros((n_rows,) + x.shape[1:], dtype=x.dtype)
    for r in range(n_rows):
        send[r] = x[row_token[r]]
    return send


def dispatch_expand(recv, assign_row, pos):
    """The receivers' re-expansion into expert-contiguous rows: the row of
    assignment (t, j), pos[t, j], is the received row assign_row[t, j]."""
    recv = np.asarray(recv)
    assign_row = np.asarray(assign_row, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    T, k = pos.shape
    out = np.zeros((T * k,) + recv.shape[1:], dtype=recv.dtype)
    for t in range(T):
        for j in range(k):
            out[pos[t, j]] = recv[assign_row[t, j]]
    return out

