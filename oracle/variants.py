"""Two independent formulations of the MoE layer forward used to pin the oracle.

TEST INFRASTRUCTURE ONLY (same rule as the oracle: tests, smoke and the
bench's CPU baseline leg only).

* ``dense_masked``: every expert runs on every token; a 0/1 mask built by rank
  counting (not by sorting) selects the k experts, and capacity is applied by
  counting earlier tokens.  This is the "compute all E experts densely, then
  mask" brute force.
* ``loops``: pure-Python scalar loops with ``math.exp``/``math.erf`` for tiny
  shapes; shares no numpy arithmetic with the oracle.

Neither calls the oracle module.  Both follow the same readings of the pages as
the oracle (see its header): lower index wins ties, slot-order combination,
exact-erf GELU, top-1 fractions before capacity for the aux loss, a selection
bias that only ranks, z-loss as the mean squared log-sum-exp of the logits, a
shared expert added to every token after the routed sum.
"""
from __future__ import annotations

import math

import numpy as np


def _wide(a):
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def dense_masked(inputs, desc):
    """y = sum_e mask[t,e] * weight[t,e] * FFN_e(x_t) with FFN_e computed for all (t, e)."""
    x = _wide(inputs["x"])
    T = x.shape[0]
    E, k = desc["n_experts"], desc["top_k"]
    g = x @ _wide(inputs["w_router"]).T
    if inputs.get("b_router") is not None:
        g = g + _wide(inputs["b_router"])[None, :]
    gmax = g.max(axis=1, keepdims=True)
    ex = np.exp(g - gmax)
    p = ex / ex.sum(axis=1, keepdims=True)
    lse = gmax[:, 0] + np.log(ex.sum(axis=1))
    z_loss = float(np.mean(lse ** 2))
    sc = g if inputs.get("b_select") is None else g + _wide(inputs["b_select"])[None, :]
    # rank[t,e] = #experts strictly better than e (higher score, or equal score and lower index)
    better = (sc[:, None, :] > sc[:, :, None]) | \
             ((sc[:, None, :] == sc[:, :, None]) & (np.arange(E)[None, None, :] < np.arange(E)[None, :, None]))
    rank = better.sum(axis=2)                              # [T,E]
    mask = rank < k
    wsel = np.where(mask, p, 0.0)
    if desc["renormalize"]:
        wsel = wsel / wsel.sum(axis=1, keepdims=True)
    top1 = np.argmin(rank, axis=1)                         # rank 0
    C = desc.get("capacity", 0)
    if C:
        if desc.get("capacity_policy", "drop") != "drop":
            raise NotImplementedError("dense_masked covers the drop policy only")
        # keep (t, e) if fewer than C earlier tokens also chose e
        earlier = np.cumsum(mask, axis=0) - mask
        mask &= earlier < C
    y = np.zeros((T, x.shape[1]))
    b1 = inputs.get("b1")
    b2 = inputs.get("b2")
    for e in range(E):
        h = x @ _wide(inputs["w1"][e]).T
        if b1 is not None:
            h = h + _wide(b1[e])[None, :]
        h = h * 0.5 * (1.0 + _erf_py(h / math.sqrt(2.0)))
        o = h @ _wide(inputs["w2"][e]).T
        if b2 is not None:
            o = o + _wide(b2[e])[None, :]
        y += np.where(mask[:, e:e + 1], wsel[:, e:e + 1] * o, 0.0)
    if inputs.get("w1_shared") is not None:
        hs = x @ _wide(inputs["w1_shared"]).T
        if inputs.get("b1_shared") is not None:
            hs = hs + _wide(inputs["b1_shared"])[None, :]
        hs = hs * 0.5 * (1.0 + _erf_py(hs / math.sqrt(2.0)))
        os_ = hs @ _wide(inputs["w2_shared"]).T
        if inputs.get("b2_shared") is not None:
            os_ = os_ + _wide(inputs["b2_shared"])[None, :]
        y = y + os_
    f = np.bincount(top1, minlength=E) / T
    P = p.mean(axis=0)
    aux = E * float(np.sum(f * P))
    return {"y": y, "aux": aux, "mask": mask, "rank": rank, "z_loss": z_loss}


def _erf_py(z):
    """math.erf elementwise (kept independent of the oracle's scipy erf)."""
    flat = z.ravel()
    out = np.fromiter((math.erf(v) for v in flat), dtype=np.float64, count=flat.size)
    return out.reshape(z.shape)


def loops(inputs, desc):
    """Pure-Python scalar forward for tiny shapes (T, d, d_ff, E of a few units)."""
    def wide_list(a):
        return _wide(a).tolist() if a is not None else None
    X = wide_list(inputs["x"])
    WR = wide_list(inputs["w_router"])
    BR = wide_list(inputs.get("b_router"))
    BS = wide_list(inputs.get("b_select"))
    W1S, W2S = wide_list(inputs.get("w1_shared")), wide_list(inputs.get("w2_shared"))
    B1S, B2S = wide_list(inputs.get("b1_shared")), wide_list(inputs.get("b2_shared"))
    W1, W2 = wide_list(inputs["w1"]), wide_list(inputs["w2"])
    B1, B2 = wide_list(inputs.get("b1")), wide_list(inputs.get("b2"))
    E, k, C = desc["n_experts"], desc["top_k"], desc.get("capacity", 0)
    d, F = desc["d_model"], desc["d_ff"]
    T = len(X)
    ys, top1s, probs_all, lses = [], [], [], []
    reroute_served = None
    if C and desc.get("capacity_policy", "drop") == "reroute":
        reroute_served = _loops_reroute(X, WR, BR, BS, E, k, C)
    taken = [0] * E
    for t in range(T):
        g = []
        for e in range(E):
            s = 0.0
            for j in range(d):
                s += WR[e][j] * X[t][j]
            if BR is not None:
                s += BR[e]
            g.append(s)
        m = max(g)
        ex = [math.exp(v - m) for v in g]
        tot = sum(ex)
        p = [v / tot for v in ex]
        probs_all.append(p)
        lses.append(m + math.log(tot))
        sc = [g[e] + (BS[e] if BS is not None else 0.0) for e in range(E)]
        chosen = []
        for _ in range(k):                      # repeated argmax, first (lowest) index wins ties
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or sc[e] > sc[best]:
                    best = e
            chosen.append(best)
        top1s.append(chosen[0])
        w = [p[e] for e in chosen]
        if desc["renormalize"]:
            sw = sum(w)
            w = [v / sw for v in w]
        y = [0.0] * d
        for s, e in enumerate(chosen):
            if reroute_served is not None:
                e = reroute_served[t][s]
                if e < 0:
                    continue
                w[s] = p[e] / (sum(p[c] for c in chosen) if desc["renormalize"] else 1.0)
            elif C:
                if taken[e] >= C:
                    taken[e] += 1
                    continue
                taken[e] += 1
            h = []
            for f in range(F):
                a = sum(W1[e][f][j] * X[t][j] for j in range(d)) + (B1[e][f] if B1 else 0.0)
                h.append(0.5 * a * (1.0 + math.erf(a / math.sqrt(2.0))))
            for i in range(d):
                o = sum(W2[e][i][f] * h[f] for f in range(F)) + (B2[e][i] if B2 else 0.0)
                y[i] += w[s] * o
        if W1S is not None:
            Fs = len(W1S)
            hs = []
            for f in range(Fs):
                a = sum(W1S[f][j] * X[t][j] for j in range(d)) + (B1S[f] if B1S else 0.0)
                hs.append(0.5 * a * (1.0 + math.erf(a / math.sqrt(2.0))))
            for i in range(d):
                y[i] += sum(W2S[i][f] * hs[f] for f in range(Fs)) + (B2S[i] if B2S else 0.0)
        ys.append(y)
    f_frac = [sum(1 for t in range(T) if top1s[t] == e) / T for e in range(E)]
    P = [sum(probs_all[t][e] for t in range(T)) / T for e in range(E)]
    aux = E * sum(f_frac[e] * P[e] for e in range(E))
    z_loss = sum(v * v for v in lses) / T
    return {"y": np.array(ys), "aux": aux, "top1": top1s, "z_loss": z_loss}


def _loops_reroute(X, WR, BR, BS, E, k, C):
    """Reroute rounds with scalar loops: each round serves requests per expert in
    token order while capacity lasts; rejected slots ask for their token's next
    best unused expert (by score, lower index on ties); none left -> dropped."""
    T = len(X)
    d = len(X[0])
    ranking = []
    for t in range(T):
        sc = []
        for e in range(E):
            v = sum(WR[e][j] * X[t][j] for j in range(d))
            if BR is not None:
                v += BR[e]
            if BS is not None:
                v += BS[e]
            sc.append(v)
        rk = []
        for _ in range(E):                       # repeated argmax, lower index first on ties
            best = None
            for e in range(E):
                if e in rk:
                    continue
                if best is None or sc[e] > sc[best]:
                    best = e
            rk.append(best)
        ranking.append(rk)
    served = [[-1] * k for _ in range(T)]
    req = [[ranking[t][s] for s in range(k)] for t in range(T)]
    used = [set(ranking[t][:k]) for t in range(T)]
    pos = [k] * T
    load = [0] * E
    pend = [[True] * k for _ in range(T)]
    while any(any(row) for row in pend):
        for t in range(T):
            for s in range(k):
                if pend[t][s] and load[req[t][s]] < C:
                    load[req[t][s]] += 1
                    served[t][s] = req[t][s]
                    pend[t][s] = False
        for t in range(T):
            for s in range(k):
                if not pend[t][s]:
                    continue
                while pos[t] < E and ranking[t][pos[t]] in used[t]:
                    pos[t] += 1
                if pos[t] >= E:
                    pend[t][s] = False
                else:
                    req[t][s] = ranking[t][pos[t]]
                    used[t].add(req[t][s])
                    pos[t] += 1
    return served
