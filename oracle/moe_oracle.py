"""Plain fp64 CPU oracle of the sparsely-gated Mixture-of-Experts layer forward.

TEST INFRASTRUCTURE ONLY.  This is the parity authority for the HIP path.
Only the tests, the smoke check and the bench's CPU-baseline leg may import
it; the product path never calls it and shares no code with it.

Every stored input (fp32, or bf16 held as uint16 bit patterns) is widened
exactly to fp64 and all arithmetic below runs in fp64.  Matrix products use
numpy's BLAS (dgemm) and erf comes from scipy; nothing is blocked, fused or
reordered beyond the definitions cited on each function.

Sources (web pages on Mixture-of-Experts):
  [LH]  "Mixture of Experts: Scaling Parameters Without Scaling Compute"
        (ai-lecture-hall), section "The MoE layer" (the three-step definition
        and the PyTorch listing) and section "The central problem: load
        balancing" (the aux loss and expert capacity).
  [LD]  "Mixture-of-Experts — making a model wider without using all of it for
        every token" (llmdaily, day 59), sections "Replace one MLP with many
        experts" and "Experts also have capacity limits".
  [AB]  "Mixture of experts: big models, small bills" (aiinbed), section
        "Experts and the router" and its "Run it" demo (stable descending sort).

Readings where the pages are silent or garbled (all listed in the design notes):
  * experts are numbered from 0;
  * the router has no bias unless a workload supplies an fp32 logit bias;
  * top-k ranks experts by logit, descending, equal logits -> lower index
    first; softmax is monotone, so this is the same order as by probability;
  * an optional per-expert selection bias is added to the logits for ranking
    only; the routing weights stay softmax(logits) of the chosen experts;
  * the router z-loss is the mean over tokens of the squared log-sum-exp of
    the logits (router bias included, selection bias not);
  * renormalisation divides the chosen probabilities by their sum;
  * y sums the weighted expert outputs (each expert's output bias included)
    in slot order; no residual is added inside the layer;
  * GELU is the exact erf form;
  * f_i counts the top-1 choice of every token before any capacity drop,
    P_i averages the full softmax over all tokens, aux = E * sum_i f_i P_i;
  * capacity keeps, per expert, the C lowest-index tokens that chose it (any
    k); a dropped assignment contributes 0 (a token with every slot dropped
    gets 0);
  * the reroute policy (optional) serves overflow at the token's next-best
    unused expert in rounds (see reroute());
  * rows of one expert's segment are ordered by token index;
  * a shared expert (optional) runs on every token, dropped ones included, and
    its output is added to y after the routed sum, with weight 1.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

MARGIN_MIN = 1e-3


# ----------------------------------------------------------------------------
# Input widening
# ----------------------------------------------------------------------------
def widen(a):
    """Exact fp64 value of a stored array (fp32, or uint16 bf16 bit patterns)."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {a.dtype}")


# ----------------------------------------------------------------------------
# Router: logits, softmax, top-k, weights   [LH "The MoE layer", steps 1-2]
# ----------------------------------------------------------------------------
def router_logits(x64, wr64, br64=None):
    """g = W_r x for every token (rows of x), plus the optional fp32 logit bias."""
    g = x64 @ wr64.T
    if br64 is not None:
        g = g + br64[None, :]
    return g


def softmax(g):
    """p = softmax(g) over the experts axis (max subtracted; same value)."""
    z = np.exp(g - g.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def topk_by_logit(g, k):
    """Indices of the k largest logits per row, in rank order.

    Ties go to the lower expert index: a stable sort of the negated logits keeps
    equal keys in index order, as the stable descending sort of [AB]'s demo does.
    Returns (idx int64 [T,k], margin [T]) where margin is the smallest gap
    between consecutive ranked logits among ranks 0..k (k+1 is the first
    unselected expert; with k == E there is no boundary gap).
    """
    order = np.argsort(-g, axis=-1, kind="stable")
    idx = order[:, :k]
    ranked = np.take_along_axis(g, order, axis=-1)
    last = min(k + 1, g.shape[-1])
    if last >= 2:
        gaps = ranked[:, :last - 1] - ranked[:, 1:last]
        margin = gaps.min(axis=-1)
    else:
        margin = np.full(g.shape[0], np.inf)
    return idx, margin


def selection_scores(g, b_select64=None):
    """Scores the experts are ranked by: the logits, plus a per-expert bias when
    one is given.  The bias only decides which experts are chosen; the routing
    weights still come from softmax(g).  [LH "The central problem: load
    balancing", auxiliary-loss-free balancing: per-expert bias terms]"""
    return g if b_select64 is None else g + b_select64[None, :]


def router_z_loss(g):
    """z = mean over tokens of (log sum_e exp g_te)^2, the squared log-partition
    of the router logits.  [LH "The central problem: load balancing", router
    z-loss: a penalty on large router logits]"""
    m = g.max(axis=-1, keepdims=True)
    lse = (m + np.log(np.exp(g - m).sum(axis=-1, keepdims=True)))[:, 0]
    return float(np.mean(lse * lse))


def routing_weights(p, idx, renormalize):
    """Probabilities of the chosen experts, renormalised over the k chosen if asked."""
    w = np.take_along_axis(p, idx, axis=-1)
    if renormalize:
        w = w / w.sum(axis=-1, keepdims=True)
    return w


# ----------------------------------------------------------------------------
# Capacity and dispatch layout   [LH "The central problem", expert capacity]
# ----------------------------------------------------------------------------
def capacity_keep(idx, n_experts, capacity):
    """Boolean keep mask [T,k] of the drop policy: per expert, the `capacity`
    lowest-index tokens that chose it (in any slot) are kept, the rest dropped.
    A token picks an expert at most once, so this is well defined for any k."""
    T, k = idx.shape
    keep = np.ones((T, k), dtype=bool)
    if capacity and capacity > 0:
        seen = np.zeros(n_experts, dtype=np.int64)
        for t in range(T):
            for s in range(k):
                e = idx[t, s]
                keep[t, s] = seen[e] < capacity
                seen[e] += 1
    return keep


def reroute(idx, scores, probs, capacity, renormalize):
    """The reroute policy for expert overflow.  [LD "Experts also have capacity
    limits": overflow may be routed elsewhere; LH "The central problem: load
    balancing": overflow tokens are dropped or rerouted]

    Rounds.  Round 0 requests every chosen (t, s) -> idx[t, s].  In each round
    the requests to an expert are accepted in token order while the expert has
    capacity left; a rejected assignment asks, in the next round, for its
    token's best-scored expert that the token has not yet used (a token's
    pending slots take these in slot order); an assignment with no expert left
    is dropped.  A served assignment's weight is the router probability of the
    expert that serves it over the same denominator as the original choices
    (their probability sum when renormalising, else 1).

    Returns (served [T,k] expert or -1 if dropped, weights [T,k], rounds,
    margin [T]): margin is the smallest gap between consecutive ranked scores
    among the ranks the token's decisions consulted (its ranks 0 .. last tried,
    and the boundary to the next one)."""
    T, k = idx.shape
    E = scores.shape[1]
    order = np.argsort(-scores, axis=1, kind="stable")        # ranking, ties -> lower index
    served = np.full((T, k), -1, dtype=np.int64)
    used = [set(int(e) for e in idx[t]) for t in range(T)]
    nxt = [k] * T                                             # next rank to try, per token
    request = idx.copy().astype(np.int64)                     # round 0: the router's choices
    pending = np.ones((T, k), dtype=bool)
    left = np.full(E, capacity, dtype=np.int64)
    rounds = 0
    while pending.any():
        rounds += 1
        for t in range(T):                                    # token order within an expert
            for s in range(k):
                if pending[t, s] and request[t, s] >= 0:
                    e = request[t, s]
                    if left[e] > 0:
                        left[e] -= 1
                        served[t, s] = e
                        pending[t, s] = False
        for t in range(T):                                    # next candidates, slot order
            for s in range(k):
                if not pending[t, s]:
                    continue
                cand = -1
                while nxt[t] < E:
                    e = int(order[t, nxt[t]])
                    nxt[t] += 1
                    if e not in used[t]:
                        cand = e
                        break
                if cand < 0:
                    pending[t, s] = False                     # nothing left: dropped
                else:
                    used[t].add(cand)
                    request[t, s] = cand
    denom = probs[np.arange(T)[:, None], idx].sum(axis=1, keepdims=True) if renormalize \
        else np.ones((T, 1))
    w = np.where(served >= 0, np.take_along_axis(probs, np.maximum(served, 0), axis=1) / denom, 0.0)
    ranked = np.take_along_axis(scores, order, axis=1)
    margin = np.full(T, np.inf)
    for t in range(T):
        last = min(nxt[t], E - 1)
        if last >= 1:
            margin[t] = float((ranked[t, :last] - ranked[t, 1:last + 1]).min())
    return served, w, rounds, margin


def dispatch_layout(idx, keep, n_experts):
    """Expert-major layout of the kept assignments.

    counts[e]  kept rows of expert e
    offsets    exclusive prefix sum of counts, offsets[E] = R
    dest[t,s]  row of assignment (t,s) in the expert-major buffers, -1 if dropped
    src[r]     assignment id t*k+s stored at row r (rows ordered by expert, then token)
    """
    T, k = idx.shape
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in range(n_experts):
        counts[e] = int(np.sum((idx == e) & keep))
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    dest = np.full((T, k), -1, dtype=np.int64)
    src = np.zeros(int(offsets[-1]), dtype=np.int64)
    fill = offsets[:-1].copy()
    for t in range(T):              # token order gives the row order inside each segment
        for s in range(k):
            if keep[t, s]:
                e = idx[t, s]
                dest[t, s] = fill[e]
                src[fill[e]] = t * k + s
                fill[e] += 1
    return counts, offsets, dest, src


# ----------------------------------------------------------------------------
# Expert FFN   [LH "The MoE layer" listing: Linear(d, d_ff) -> GELU -> Linear(d_ff, d)]
# ----------------------------------------------------------------------------
def gelu_erf(z):
    """Exact GELU: z * Phi(z) = z * (1 + erf(z / sqrt 2)) / 2."""
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def expert_ffn(rows64, w1e, b1e, w2e, b2e):
    """W2 GELU(W1 v + b1) + b2 for every row v (fp64 in, fp64 out)."""
    h = rows64 @ w1e.T
    if b1e is not None:
        h += b1e[None, :]
    h = gelu_erf(h)
    o = h @ w2e.T
    if b2e is not None:
        o += b2e[None, :]
    return o


# ----------------------------------------------------------------------------
# Aux loss   [LH "The central problem", Switch-style loss; listing's last lines]
# ----------------------------------------------------------------------------
def aux_loss(idx, p, n_experts):
    """aux = E * sum_i f_i * P_i.

    f_i: fraction of tokens whose top-1 choice is i (before capacity).
    P_i: mean over all tokens of the softmax probability of expert i.
    Returns (aux, f, P, top1_count).
    """
    T = idx.shape[0]
    top1_count = np.bincount(idx[:, 0], minlength=n_experts).astype(np.int64)
    f = top1_count / T
    P = p.mean(axis=0)
    return float(n_experts * np.sum(f * P)), f, P, top1_count


# ----------------------------------------------------------------------------
# The layer
# ----------------------------------------------------------------------------
def route(inputs, desc):
    """Router half of the layer for all tokens: everything but the expert FFNs."""
    x64 = widen(inputs["x"])
    g = router_logits(x64, widen(inputs["w_router"]), widen(inputs.get("b_router")))
    p = softmax(g)
    sc = selection_scores(g, widen(inputs.get("b_select")))
    idx, margin = topk_by_logit(sc, desc["top_k"])
    w = routing_weights(p, idx, desc["renormalize"])
    aux, f, P, top1 = aux_loss(idx, p, desc["n_experts"])
    C = desc.get("capacity", 0)
    if C and desc.get("capacity_policy", "drop") == "reroute":
        served, final_w, rounds, rr_margin = reroute(idx, sc, p, C, desc["renormalize"])
        margin = np.minimum(margin, rr_margin)
        keep = served >= 0
        final_idx = np.where(keep, served, idx)     # dropped slots keep the router's choice
        final_w = np.where(keep, final_w, w)
    else:
        keep = capacity_keep(idx, desc["n_experts"], C)
        final_idx, final_w, rounds = idx, w, 0
    counts, offsets, dest, src = dispatch_layout(final_idx, keep, desc["n_experts"])
    return {"logits": g, "probs": p, "scores": sc, "router_idx": idx, "router_w": w,
            "topk_idx": final_idx, "topk_w": final_w, "margin": margin, "reroute_rounds": rounds,
            "keep": keep, "counts": counts, "offsets": offsets, "dest": dest, "src": src,
            "aux": aux, "f": f, "P": P, "top1_count": top1, "z_loss": router_z_loss(g),
            "x64": x64}


def forward(inputs, desc, tokens=None, chunk_rows=4096, check_margin=True):
    """The whole layer forward: y [T,d] (or the rows `tokens` of it) and aux.

    `tokens` (sorted or not) restricts the expert FFN work to those tokens'
    rows; routing, capacity and aux always use all tokens, since capacity
    depends on token order.  y rows are sum_s w[t,s] * FFN_{idx[t,s]}(x_t) over
    kept slots, accumulated in slot order; 0 when every slot was dropped.
    """
    r = route(inputs, desc)
    if check_margin:
        bad = np.flatnonzero(r["margin"] <= MARGIN_MIN)
        if bad.size:
            raise ValueError(f"top-k logit margin <= {MARGIN_MIN} at tokens {bad[:8].tolist()}")
    T, k = r["topk_idx"].shape
    sel = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    y = np.zeros((sel.size, desc["d_model"]), dtype=np.float64)
    contrib = np.zeros((sel.size, k, desc["d_model"]), dtype=np.float64)
    x64 = r["x64"]
    for e in range(desc["n_experts"]):
        pos, slot = np.nonzero((r["topk_idx"][sel] == e) & r["keep"][sel])
        if pos.size == 0:
            continue                      # experts with no rows do no work
        w1e = widen(inputs["w1"][e])
        w2e = widen(inputs["w2"][e])
        b1e = widen(inputs["b1"][e]) if inputs.get("b1") is not None else None
        b2e = widen(inputs["b2"][e]) if inputs.get("b2") is not None else None
        for c0 in range(0, pos.size, chunk_rows):
            pp, ss = pos[c0:c0 + chunk_rows], slot[c0:c0 + chunk_rows]
            contrib[pp, ss] = expert_ffn(x64[sel[pp]], w1e, b1e, w2e, b2e)
    w = r["topk_w"][sel]
    for s in range(k):                    # slot order
        y += np.where(r["keep"][sel][:, s:s + 1], w[:, s:s + 1] * contrib[:, s], 0.0)
    shared = shared_expert(inputs, x64[sel])
    if shared is not None:                # added after the routed sum, to every token
        y += shared
    r["y"] = y
    r["tokens"] = sel
    return r


def shared_expert(inputs, x64_rows):
    """The always-active shared expert on the given token rows: the same
    Linear-GELU-Linear as a routed expert, with no routing weight.  [LH "Design
    variations": shared experts, always active]  Several shared experts equal
    one whose hidden layer is their hidden layers side by side, so one FFN of
    width d_ff_shared covers them."""
    if inputs.get("w1_shared") is None:
        return None
    return expert_ffn(x64_rows, widen(inputs["w1_shared"]), widen(inputs.get("b1_shared")),
                      widen(inputs["w2_shared"]), widen(inputs.get("b2_shared")))


def expert_outputs(inputs, desc, rows=None):
    """Per-row expert outputs o[r] = FFN_e(x_perm[r]) in the expert-major layout,
    and the post-GELU activations h[r]; optionally only for the given rows."""
    r = route(inputs, desc)
    R = int(r["offsets"][-1])
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    k = desc["top_k"]
    seg = np.searchsorted(r["offsets"], rows, side="right") - 1
    d, F = desc["d_model"], desc["d_ff"]
    o = np.zeros((rows.size, d))
    h = np.zeros((rows.size, F))
    for e in np.unique(seg):
        m = seg == e
        v = r["x64"][r["src"][rows[m]] // k]
        w1e, w2e = widen(inputs["w1"][e]), widen(inputs["w2"][e])
        hh = v @ w1e.T
        if inputs.get("b1") is not None:
            hh += widen(inputs["b1"][e])[None, :]
        hh = gelu_erf(hh)
        h[m] = hh
        oo = hh @ w2e.T
        if inputs.get("b2") is not None:
            oo += widen(inputs["b2"][e])[None, :]
        o[m] = oo
    return {"rows": rows, "expert": seg, "h": h, "o": o, "route": r}


def desc_of(spec):
    """The option set of a workload as a plain dict."""
    return {"tokens": spec.tokens, "d_model": spec.d_model, "d_ff": spec.d_ff,
            "n_experts": spec.n_experts, "top_k": spec.top_k,
            "renormalize": bool(spec.renormalize), "capacity": spec.capacity,
            "capacity_policy": getattr(spec, "capacity_policy", "drop")}
