"""CPU oracle for the MoE-LoRA expert layer: forward and backward.

TEST INFRASTRUCTURE. Only tests/, the smoke check and the bench's CPU-baseline
leg may import or run this module. The HIP library never does, and this module
imports nothing from it: the two share no code.

Sources (cited by page and section):
  [moe]  Unsloth, "Fine-tune MoE models 12x faster" (unsloth.ai docs, faster-moe
         page, Japanese). Sections: "What is torch._grouped_mm?" (the per-expert
         for-loop and the stacked gate_up_proj [E, 2I, H] parameter), "Faster
         LoRA MoE training" (split LoRA: same losses, gradients and outputs,
         only the order of the products changes), "Implementation details"
         (LoRA shapes, frozen router, memory and FLOP equations).
  [lora] aiflowlearn.net, "Getting to know Unsloth" tutorial, section on the
         LoRA fine-tuning principle: the fused LoRA_MLP docstring defining the
         SwiGLU MLP (gate projection e, f = e * sigmoid(e), up projection g,
         h = f * g, down projection of h).

What it computes is the plain definition, step by step, in the form of the
per-expert loop the [moe] page shows as the baseline:

  route    : per token, the k experts with the largest logits (ties to the
             lower index) and their combine weights (router mode below).
  permute  : (token, slot) pairs grouped by expert, stable in pair order.
  experts  : for each expert e with rows X_e (loop over experts, skip empty):
               u_gu = X_e A_gu[e]^T                         (split LoRA: X A first)
               h    = X_e W_gu[e]^T + s u_gu B_gu[e]^T      (never W + s B A)
               g, v = h[:, :I], h[:, I:]                    (gate, up: chunk(2, -1))
               a    = g sigmoid(g) v                        (SwiGLU)
               u_d  = a A_d[e]^T
               y    = a W_d[e]^T + s u_d B_d[e]^T
  combine  : Y[t] = sum_j w[t, j] y[pos(t, j)]  (slot order j = 0..k-1)
  backward : the chain rule through the same steps with W frozen; the router
             is frozen too, so the only router gradient is d logits.

Readings where the pages are silent (each listed with its reason in the design
notes): LoRA layout A [E, r, in], B [E, out, r] with one adapter over the whole
stacked gate_up_proj; scale s = lora_scale (default 1); gate = first I columns;
SwiGLU with no clamp or bias; router modes softmax_topk, softmax_topk_renorm,
topk_softmax, sigmoid_topk_renorm; ties to the lower expert index; no capacity
limit, no dropped pairs.

Precision: every function takes `dtype` (default float32: fp32 accumulation,
the baseline the layer is specified against); the pins run it in float64.
bf16 inputs arrive as float32 arrays holding bf16-exact values and no
intermediate is rounded.

Weights are accessed as W[e], so any object indexable by expert works (a stacked
array, or a loader that fetches one expert's slice at a time).
"""
from __future__ import annotations

import numpy as np

ROUTERS = ("softmax_topk", "softmax_topk_renorm", "topk_softmax", "sigmoid_topk_renorm")


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------- route
def route(logits, k, router, dtype=np.float32):
    """Top-k routing. logits [T, E] float32 -> (topk_ids [T, k] int32, topk_w [T, k]).

    Selection compares the float32 logits themselves (softmax and sigmoid are
    strictly increasing, so this is the same choice as ranking probabilities,
    without ties made by rounding). Order: logit descending, then expert index
    ascending. Weights, per router mode:
      softmax_topk        : p = softmax over all E, w_j = p[S_j]
      softmax_topk_renorm : w_j = p[S_j] / sum_j p[S_j]
      topk_softmax        : w = softmax over the k selected logits
      sigmoid_topk_renorm : w_j = sigmoid(l[S_j]) / sum_j sigmoid(l[S_j])
    The [moe] page's loop consumes an expert mask built from such a top-k
    ("What is torch._grouped_mm?"); the router itself is frozen
    ("Implementation details").
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    if router not in ROUTERS:
        raise ValueError(f"unknown router {router!r}")
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -logits), axis=-1)          # primary key last
    ids = order[:, :k].astype(np.int32)
    l = logits.astype(dtype)
    sel = np.take_along_axis(l, ids, axis=1)
    if router in ("softmax_topk", "softmax_topk_renorm"):
        m = l.max(axis=1, keepdims=True)
        ex = np.exp(l - m)
        p = ex / ex.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, ids, axis=1)
        if router == "softmax_topk_renorm":
            w = w / w.sum(axis=1, keepdims=True)
    elif router == "topk_softmax":
        ex = np.exp(sel - sel.max(axis=1, keepdims=True))
        w = ex / ex.sum(axis=1, keepdims=True)
    else:
        sg = _sigmoid(sel)
        w = sg / sg.sum(axis=1, keepdims=True)
    return ids, w.astype(dtype)


def route_backward(logits, topk_ids, d_topk_w, router, dtype=np.float32):
    """d logits [T, E] from d topk_w [T, k], with the selection held fixed.

    With c = sum_j dw_j w_j:
      softmax_topk        : dl_i = p_i (dw^_i - c) for every i, dw^ = dw scattered to S
      softmax_topk_renorm : dl_{S_j} = w_j (dw_j - c), zero elsewhere
      topk_softmax        : dl_{S_j} = w_j (dw_j - c), zero elsewhere
      sigmoid_topk_renorm : dl_{S_j} = sigmoid'(l_{S_j}) (dw_j - c) / sum sigmoid(l_S)
    (Jacobians of the weight definitions in `route`.)
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.asarray(topk_ids)
    dw = np.asarray(d_topk_w, dtype=dtype)
    _, w = route(logits, ids.shape[1], router, dtype)
    l = logits.astype(dtype)
    c = (dw * w).sum(axis=1, keepdims=True)
    dl = np.zeros((T, E), dtype=dtype)
    rows = np.arange(T)[:, None]
    if router == "softmax_topk":
        m = l.max(axis=1, keepdims=True)
        ex = np.exp(l - m)
        p = ex / ex.sum(axis=1, keepdims=True)
        dhat = np.zeros((T, E), dtype=dtype)
        dhat[rows, ids] = dw
        dl = p * (dhat - c)
    elif router in ("softmax_topk_renorm", "topk_softmax"):
        dl[rows, ids] = w * (dw - c)
    else:
        sel = np.take_along_axis(l, ids, axis=1)
        sg = _sigmoid(sel)
        dl[rows, ids] = sg * (1 - sg) * (dw - c) / sg.sum(axis=1, keepdims=True)
    return dl.astype(dtype)


# ------------------------------------------------------------------------- permute
def permute(topk_ids, E):
    """Group the N = T*k (token, slot) pairs by expert, stable in pair order.

    Pair p = t*k + j goes to expert topk_ids[t, j]. Returns
      counts [E]       rows per expert
      offsets [E+1]    exclusive prefix sum of counts
      sorted_pair [N]  sorted_pair[i] = the pair at position i
      inv_pos [N]      inv_pos[sorted_pair[i]] = i
    so expert e owns positions offsets[e] .. offsets[e+1]-1 (the [moe] page's
    token_idx for that expert, "What is torch._grouped_mm?").
    """
    ids = np.asarray(topk_ids).ravel().astype(np.int64)
    N = ids.size
    counts = np.bincount(ids, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_pair = np.argsort(ids, kind="stable").astype(np.int32)
    inv_pos = np.empty(N, dtype=np.int32)
    inv_pos[sorted_pair] = np.arange(N, dtype=np.int32)
    return counts, offsets, sorted_pair, inv_pos


def gather_rows(x, sorted_pair, k):
    """X_perm[i] = x[sorted_pair[i] // k]: the rows each expert sees, in order."""
    return np.asarray(x)[np.asarray(sorted_pair) // k]


# ------------------------------------------------------------------------- experts
def expert_forward(X_e, w_gu, a_gu, b_gu, w_d, a_d, b_d, s=1.0, dtype=np.float32):
    """One expert's split-LoRA SwiGLU MLP on its rows X_e [n, H].

    w_gu [2I, H], a_gu [r, H], b_gu [2I, r], w_d [H, I], a_d [r, I], b_d [H, r].
    Split LoRA ([moe], "Faster LoRA MoE training"): the input meets A first,
    then B; W + s B A is never formed. SwiGLU as in [lora]: gate first.
    Returns dict with h [n, 2I], u_gu [n, r] (= X A_gu^T, unscaled),
    a [n, I], u_d [n, r] (= a A_d^T, unscaled), y [n, H].
    """
    X = np.asarray(X_e, dtype=dtype)
    W1, A1, B1 = (np.asarray(t, dtype=dtype) for t in (w_gu, a_gu, b_gu))
    W2, A2, B2 = (np.asarray(t, dtype=dtype) for t in (w_d, a_d, b_d))
    s = dtype(s)
    I = W1.shape[0] // 2
    u_gu = X @ A1.T
    h = X @ W1.T + s * (u_gu @ B1.T)
    g, v = h[:, :I], h[:, I:]
    a = g * _sigmoid(g) * v
    u_d = a @ A2.T
    y = a @ W2.T + s * (u_d @ B2.T)
    return {"h": h, "u_gu": u_gu, "a": a, "u_d": u_d, "y": y}


def expert_backward(X_e, G_e, fwd, w_gu, a_gu, b_gu, w_d, a_d, b_d, s=1.0,
                    dtype=np.float32, base_grads=False):
    """Backward of `expert_forward` for upstream gradient G_e = dL/dy [n, H].

    With LoRA the base weights are frozen ([moe], "Implementation details":
    only the rank-r adapters are trained), so there is no dW. Returns dict with
    dx [n, H], da_gu [r, H], db_gu [2I, r], da_d [r, I], db_d [H, r], dh [n, 2I].
    base_grads=True adds the base-weight gradients of full fine-tuning (a mode
    the [moe] page's introduction lists beside LoRA): dw_gu [2I, H] = dh^T X and
    dw_d [H, I] = G^T a (the chain rule through X W^T; the LoRA scale does not
    enter).
    """
    X = np.asarray(X_e, dtype=dtype)
    G = np.asarray(G_e, dtype=dtype)
    W1, A1, B1 = (np.asarray(t, dtype=dtype) for t in (w_gu, a_gu, b_gu))
    W2, A2, B2 = (np.asarray(t, dtype=dtype) for t in (w_d, a_d, b_d))
    s = dtype(s)
    I = W1.shape[0] // 2
    h, u_gu, a, u_d = fwd["h"], fwd["u_gu"], fwd["a"], fwd["u_d"]
    # down projection: y = a W2^T + s (a A2^T) B2^T
    gb = G @ B2                                   # [n, r]
    da = G @ W2 + s * (gb @ A2)                   # dL/da [n, I]
    db_d = s * (G.T @ u_d)                        # [H, r]
    da_d = s * (gb.T @ a)                         # [r, I]
    # SwiGLU: a = g sigmoid(g) v
    g, v = h[:, :I], h[:, I:]
    sg = _sigmoid(g)
    dg = da * v * sg * (1 + g * (1 - sg))
    dv = da * g * sg
    dh = np.concatenate([dg, dv], axis=1)         # [n, 2I]
    # gate_up projection: h = X W1^T + s (X A1^T) B1^T
    dhb = dh @ B1                                 # [n, r]
    dx = dh @ W1 + s * (dhb @ A1)                 # [n, H]
    db_gu = s * (dh.T @ u_gu)                     # [2I, r]
    da_gu = s * (dhb.T @ X)                       # [r, H]
    out = {"dx": dx, "da_gu": da_gu, "db_gu": db_gu, "da_d": da_d, "db_d": db_d, "dh": dh}
    if base_grads:
        out["dw_gu"] = dh.T @ X                   # [2I, H]
        out["dw_d"] = G.T @ a                     # [H, I]
    return out


# ------------------------------------------------------------------------- combine
def combine(y_perm, inv_pos, topk_w, T, k, dtype=np.float32):
    """Y[t] = sum over slots j = 0..k-1 of w[t, j] * y_perm[inv_pos[t*k + j]].

    topk_w None means weights 1 (the plain sum used to bring dX back to tokens).
    """
    y_perm = np.asarray(y_perm, dtype=dtype)
    pos = np.asarray(inv_pos).reshape(T, k)
    Y = np.zeros((T, y_perm.shape[1]), dtype=dtype)
    for j in range(k):
        rows = y_perm[pos[:, j]]
        if topk_w is None:
            Y += rows
        else:
            Y += np.asarray(topk_w, dtype=dtype)[:, j:j + 1] * rows
    return Y


def combine_backward(dY, y_perm, inv_pos, topk_w, T, k, dtype=np.float32):
    """Backward of `combine`: G[pos] = w[t, j] dY[t], dw[t, j] = <dY[t], y_perm[pos]>."""
    dY = np.asarray(dY, dtype=dtype)
    y_perm = np.asarray(y_perm, dtype=dtype)
    w = np.asarray(topk_w, dtype=dtype)
    pos = np.asarray(inv_pos).reshape(T, k)
    G = np.zeros_like(y_perm)
    dw = np.zeros((T, k), dtype=dtype)
    for j in range(k):
        G[pos[:, j]] = w[:, j:j + 1] * dY
        dw[:, j] = np.einsum("th,th->t", dY, y_perm[pos[:, j]])
    return G, dw


# --------------------------------------------------------------------------- layer
def layer_forward(x, logits, weights, k, router, s=1.0, dtype=np.float32):
    """Whole forward. weights: dict with w_gu, a_gu, b_gu, w_d, a_d, b_d (indexable by e).

    Returns (Y [T, H], cache) with the cache holding what the backward needs.
    """
    x = np.asarray(x, dtype=dtype)
    T, H = x.shape
    E = np.asarray(logits).shape[1]
    ids, w = route(logits, k, router, dtype)
    counts, offsets, sorted_pair, inv_pos = permute(ids, E)
    N = T * k
    I = None
    y_perm = np.zeros((N, H), dtype=dtype)
    per_expert = {}
    for e in range(E):                      # the baseline per-expert loop
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        token_idx = sorted_pair[lo:hi] // k
        X_e = x[token_idx]
        we = {n: weights[n][e] for n in ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")}
        f = expert_forward(X_e, **we, s=s, dtype=dtype)
        I = f["a"].shape[1]
        y_perm[lo:hi] = f["y"]
        per_expert[e] = f
    Y = combine(y_perm, inv_pos, w, T, k, dtype)
    cache = dict(x=x, logits=np.asarray(logits, np.float32), ids=ids, w=w, counts=counts,
                 offsets=offsets, sorted_pair=sorted_pair, inv_pos=inv_pos,
                 y_perm=y_perm, per_expert=per_expert, k=k, router=router, s=s,
                 weights=weights, dtype=dtype, I=I)
    return Y, cache


def layer_backward(dY, cache, base_grads=False):
    """Whole backward. Returns dict with dx [T, H], dlogits [T, E], and the LoRA
    gradients da_gu [E, r, H], db_gu [E, 2I, r], da_d [E, r, I], db_d [E, H, r]
    (zeros for experts that received no rows); base_grads=True adds
    dw_gu [E, 2I, H] and dw_d [E, H, I] (full fine-tuning)."""
    dtype = cache["dtype"]
    x, k, s, wts = cache["x"], cache["k"], cache["s"], cache["weights"]
    T, H = x.shape
    E = cache["logits"].shape[1]
    G, dw = combine_backward(dY, cache["y_perm"], cache["inv_pos"], cache["w"], T, k, dtype)
    dlogits = route_backward(cache["logits"], cache["ids"], dw, cache["router"], dtype)
    a_gu0, b_gu0, a_d0, b_d0 = (np.asarray(wts[n][0]) for n in ("a_gu", "b_gu", "a_d", "b_d"))
    grads = {"da_gu": np.zeros((E,) + a_gu0.shape, dtype),
             "db_gu": np.zeros((E,) + b_gu0.shape, dtype),
             "da_d": np.zeros((E,) + a_d0.shape, dtype),
             "db_d": np.zeros((E,) + b_d0.shape, dtype)}
    if base_grads:
        w_gu0, w_d0 = (np.asarray(wts[n][0]) for n in ("w_gu", "w_d"))
        grads["dw_gu"] = np.zeros((E,) + w_gu0.shape, dtype)
        grads["dw_d"] = np.zeros((E,) + w_d0.shape, dtype)
    N = T * k
    dx_perm = np.zeros((N, H), dtype=dtype)
    offsets, sorted_pair = cache["offsets"], cache["sorted_pair"]
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        X_e = x[sorted_pair[lo:hi] // k]
        we = {n: wts[n][e] for n in ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")}
        b = expert_backward(X_e, G[lo:hi], cache["per_expert"][e], **we, s=s, dtype=dtype,
                            base_grads=base_grads)
        dx_perm[lo:hi] = b["dx"]
        for n in grads:
            grads[n][e] = b[n]
    dx = combine(dx_perm, cache["inv_pos"], None, T, k, dtype)
    out = {"dx": dx, "dlogits": dlogits, "dw": dw}
    out.update(grads)
    return out


def merge_lora(weights, s=1.0, dtype=np.float32):
    """Merged export: every expert's adapter folded into its base weight,
    W' = W + s B A for gate_up ([2I, H]) and down ([H, I]), as a model saved in
    merged 16-bit form carries them (winningdata.io hands-on page, section
    "4. Salvando o modelo"). Returns {"w_gu": [E, 2I, H], "w_d": [E, H, I]}."""
    out = {}
    for name, a, b in (("w_gu", "a_gu", "b_gu"), ("w_d", "a_d", "b_d")):
        W = np.asarray(weights[name], dtype)
        A, B = np.asarray(weights[a], dtype), np.asarray(weights[b], dtype)
        out[name] = np.stack([W[e] + dtype(s) * (B[e] @ A[e]) for e in range(W.shape[0])])
    return out


def merged_forward(x, logits, weights, k, router, s=1.0, dtype=np.float32):
    """The PEFT-merge order the [moe] page contrasts with ("Faster LoRA MoE
    training"): form W' = W + s B A for every expert, then run the plain MoE.

    Only for pinning the split order on tiny layers: it materialises E deltas.
    """
    x = np.asarray(x, dtype=dtype)
    T, H = x.shape
    E = np.asarray(logits).shape[1]
    ids, w = route(logits, k, router, dtype)
    counts, offsets, sorted_pair, inv_pos = permute(ids, E)
    y_perm = np.zeros((T * k, H), dtype=dtype)
    merged = merge_lora(weights, s, dtype)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        W1, W2 = merged["w_gu"][e], merged["w_d"][e]
        X_e = x[sorted_pair[lo:hi] // k]
        h = X_e @ W1.T
        I = W1.shape[0] // 2
        a = h[:, :I] * _sigmoid(h[:, :I]) * h[:, I:]
        y_perm[lo:hi] = a @ W2.T
    return combine(y_perm, inv_pos, w, T, k, dtype)


def layer_forward_backward(x, logits, dY, weights, k, router, s=1.0, dtype=np.float32,
                           base_grads=False):
    """Forward then backward; returns (Y, grads dict, cache)."""
    Y, cache = layer_forward(x, logits, weights, k, router, s, dtype)
    return Y, layer_backward(dY, cache, base_grads), cache


# ------------------------------------------------------- router projection, shared expert
def router_logits(x, w_r, dtype=np.float32):
    """logits [T, E] = x W_r^T: the router projection whose output the routing
    consumes ([moe], "What is torch._grouped_mm?": the expert mask comes from
    the router's scores; "Implementation details": the router is frozen)."""
    return np.asarray(x, dtype) @ np.asarray(w_r, dtype).T


def router_input_grad(dlogits, w_r, dtype=np.float32):
    """dL/dx contribution of the router projection: dlogits [T, E] W_r [E, H]
    (the router weight itself is frozen, so it gets no gradient)."""
    return np.asarray(dlogits, dtype) @ np.asarray(w_r, dtype)


def layer_with_router_and_shared(x, w_r, dY, weights, shared, k, router, s=1.0,
                                 dtype=np.float32, logits=None):
    """The layer as a model block sees it: logits from the router projection,
    the routed experts, plus an always-on shared expert (a dense LoRA SwiGLU
    MLP over every token, as in the DeepSeek-style MoE the [moe] page describes
    for GLM-4.7-Flash: routed experts plus one shared expert, section "GLM 4.7
    benchmark"). shared: dict of one expert's w_gu, a_gu, b_gu, w_d, a_d, b_d, or
    None. Returns (Y, grads) with grads: dx (routed + shared + router), dlogits,
    the routed LoRA gradients, and shared_* for the shared expert's LoRA
    gradients. The routing selects on float32 logits; `logits`, when given, are
    those float32 logits (a caller comparing against another implementation
    passes that implementation's rounding of x W_r^T, so that both take the
    same top-k decisions), else x W_r^T is formed here in float64 and rounded
    to float32."""
    if logits is None:
        logits = router_logits(x, w_r, np.float64).astype(np.float32)
    logits = np.asarray(logits, np.float32)
    Y, g, _ = layer_forward_backward(x, logits, dY, weights, k, router, s, dtype)
    g = dict(g)
    g["dx"] = g["dx"] + router_input_grad(g["dlogits"], w_r, dtype)
    g["logits"] = logits
    if shared is not None:
        X = np.asarray(x, dtype)
        f = expert_forward(X, **shared, s=s, dtype=dtype)
        b = expert_backward(X, np.asarray(dY, dtype), f, **shared, s=s, dtype=dtype)
        Y = Y + f["y"]
        g["dx"] = g["dx"] + b["dx"]
        for n in ("da_gu", "db_gu", "da_d", "db_d"):
            g["shared_" + n] = b[n]
    return Y, g
