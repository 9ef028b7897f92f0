"""fp64 CPU oracle of the MiTA (Mixture-of-Top-k Attention) forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP
library never calls it, and it shares no code with the HIP library: it is
plain numpy in float64, written to be read against the pages, not to be fast.

Sources (cited by page title and section; the pages print no formulas, the
extraction stripped them, so each step below also states the reading taken):

  [ZH]  "NeurIPS'26：注意力也是FFN？从快权重出发，重新理解高效注意力"
        (新智元 / 36氪), section "用少量地标查询，同时构造全局概括与细节专家"
        (landmark queries, routed experts, shared expert, the s=1 output),
        Figure 3 and Algorithm 1 (算法1).
  [EN]  "NeurIPS'26: Is Attention Also FFN? Rethinking Efficient Attention
        From the Fast Weight Perspective" (36Kr, English), section
        "Construct global generalization and detail experts at the same time
        with a small number of landmark queries" (same content as [ZH],
        cut off at the s=1 output).
  [ABS] "Mixture-of-Top-k Attention: Efficient Attention via Scalable Fast
        Weights", abstract (landmark queries gather top-k key-value pairs
        as routed experts; the N-width MLP is compressed into a shared
        expert).

Per (batch b, head h), with N = grid_h*grid_w tokens in row-major order
(n = y*grid_w + x), m = m_h*m_w landmarks in row-major order (i = r*m_w + c),
tau = 1/sqrt(d):

  1. pool    Q_L[i]  = mean of Q over the 2-D adaptive-average-pooling window
                       of landmark i (rows [floor(r*gh/mh), ceil((r+1)*gh/mh)),
                       columns likewise); windows may overlap.
  2. score   S       = tau * Q_L K^T                                 (m x N)
  3. top-k   idx_i   = the k keys with the largest S[i, :], ties to the lowest
                       key index; reported in ascending key order.
  4. shared  V_L     = softmax_row(S) V  over all N keys            (m x d)
  5. route   route_n = argmax_i q_n . Q_L[i], ties to the lowest i.
  6. group   counts / offsets / perm = stable counting sort of the queries
                       by route (Algorithm 1 groups queries by route).
  7. attend  out_n   = softmax(tau*[q_n Q_L^T, q_n K[idx_e]^T]) [V_L; V[idx_e]],
                       e = route_n: ONE softmax over the m + k concatenated
                       logits (the shared expert has keys Q_L, values V_L).

Two variants the pages name beside the s = 1 pass ([ZH], landmark-query
section, "在每个查询选择一个路由专家，即s=1的配置下", which gives the output for
one routed expert per query; and [ZH], long-sequence section, the ablation
against a route-only version with the same number of entries per query):

  s > 1      each query goes to its s best landmarks (q_n . Q_L[i] descending,
             ties to the lowest i) and takes ONE softmax over the m shared
             entries and the s*k entries of its experts, concatenated in rank
             order.  The pages do not say whether keys two experts share are
             merged; the plain reading taken here concatenates them, so such a
             key appears once per expert that holds it.
  route-only no shared expert: each query's softmax covers only its routed
             experts' entries (pass k = m + k_mita for the ablation's equal
             entry count).  Pooling, scores, top-k and routing are unchanged.

Every function is pinned by tests under ``tests/`` (brute force on tiny
inputs, library special cases, closed forms and invariants); none is
"parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np


def tau(d: int) -> float:
    """Score scale 1/sqrt(d) used in S, in V_L's softmax and in the output logits."""
    return 1.0 / math.sqrt(d)


# --------------------------------------------------------------------------
# step 1: landmark queries by 2-D adaptive average pooling   ([ZH]/[EN] landmark section)
# --------------------------------------------------------------------------
def pool_windows(g: int, mg: int):
    """Adaptive-average-pooling windows [start, end) along one grid axis."""
    return [((i * g) // mg, -((-(i + 1) * g) // mg)) for i in range(mg)]


def landmark_queries(Q: np.ndarray, grid_h: int, grid_w: int, m_h: int, m_w: int) -> np.ndarray:
    """Q [..., N, d] -> Q_L [..., m, d]; each landmark is its window's plain mean."""
    Q = np.asarray(Q, dtype=np.float64)
    d = Q.shape[-1]
    Qg = Q.reshape(Q.shape[:-2] + (grid_h, grid_w, d))
    out = np.empty(Q.shape[:-2] + (m_h * m_w, d))
    for r, (y0, y1) in enumerate(pool_windows(grid_h, m_h)):
        for c, (x0, x1) in enumerate(pool_windows(grid_w, m_w)):
            win = Qg[..., y0:y1, x0:x1, :]
            out[..., r * m_w + c, :] = win.sum(axis=(-3, -2)) / ((y1 - y0) * (x1 - x0))
    return out


# --------------------------------------------------------------------------
# step 2: landmark scores, one matrix shared by top-k and by the shared expert
# --------------------------------------------------------------------------
def landmark_scores(QL: np.ndarray, K: np.ndarray) -> np.ndarray:
    """S = tau * Q_L K^T  ([..., m, N])."""
    K = np.asarray(K, dtype=np.float64)
    return (QL @ np.swapaxes(K, -1, -2)) * tau(K.shape[-1])


# --------------------------------------------------------------------------
# step 3: each landmark's top-k keys form one routed expert
# --------------------------------------------------------------------------
def expert_topk(S: np.ndarray, k: int):
    """Top-k key ids per landmark row, ties broken toward the lowest key id.

    Returns (idx [..., m, k] ascending int64, gap [..., m]) where gap is
    s_(k) - s_(k+1), the margin between the last kept and the first dropped
    score in the (score desc, key asc) order; +inf when k == N.
    """
    N = S.shape[-1]
    if not 1 <= k <= N:
        raise ValueError("need 1 <= k <= N")
    order = np.argsort(-S, axis=-1, kind="stable")  # stable: equal scores keep key order
    idx = np.sort(order[..., :k], axis=-1)
    ranked = np.take_along_axis(S, order, axis=-1)
    gap = ranked[..., k - 1] - ranked[..., k] if k < N else np.full(S.shape[:-1], np.inf)
    return idx, gap


# --------------------------------------------------------------------------
# step 4: shared expert -- landmarks cross-attend the complete context
# --------------------------------------------------------------------------
def softmax_rows(x: np.ndarray) -> np.ndarray:
    z = x - x.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def shared_values(S: np.ndarray, V: np.ndarray) -> np.ndarray:
    """V_L = softmax_row(S) V over all N keys."""
    return softmax_rows(S) @ np.asarray(V, dtype=np.float64)


# --------------------------------------------------------------------------
# step 5: each query goes to the expert of its best-matching landmark
# --------------------------------------------------------------------------
def route_queries(Q: np.ndarray, QL: np.ndarray, s: int = 1):
    """Routes by q . Q_L, ties to the lowest landmark id.

    s = 1: route [..., N] = argmax_i q_n . Q_L[i] and rgap = tau*(R_(1) - R_(2)).
    s > 1: route [..., N, s], the s best landmarks best first (the stable order
    of (score descending, id ascending)), and rgap = tau*(R_(s) - R_(s+1)), the
    margin of the last landmark taken over the first one left out.
    rgap is +inf when no landmark is left out (s = m).
    """
    Q = np.asarray(Q, dtype=np.float64)
    R = Q @ np.swapaxes(QL, -1, -2)                  # [..., N, m]
    m = R.shape[-1]
    if not 1 <= s <= m:
        raise ValueError("need 1 <= s <= m")
    if s == 1:
        route = np.argmax(R, axis=-1)                 # first maximum = lowest id
        if m == 1:
            rgap = np.full(R.shape[:-1], np.inf)
        else:
            srt = np.sort(R, axis=-1)
            rgap = (srt[..., -1] - srt[..., -2]) * tau(Q.shape[-1])
        return route, rgap
    order = np.argsort(-R, axis=-1, kind="stable")   # stable: equal scores keep id order
    route = order[..., :s]
    ranked = np.take_along_axis(R, order, axis=-1)
    rgap = (ranked[..., s - 1] - ranked[..., s]) * tau(Q.shape[-1]) if s < m \
        else np.full(R.shape[:-1], np.inf)
    return route, rgap


# --------------------------------------------------------------------------
# step 6: group the queries by their route (Algorithm 1)
# --------------------------------------------------------------------------
def group_by_route(route: np.ndarray, m: int):
    """Stable counting sort of one head's queries: counts [m], offsets [m+1], perm [N].

    With s > 1 routes per query (route [N, s]) the sorted items are the
    (query, rank) pairs t = n*s + j, each under the expert route[n, j]: counts,
    offsets and perm are then over the N*s items.
    """
    route = np.asarray(route).reshape(-1)
    counts = np.bincount(route, minlength=m)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.argsort(route, kind="stable")
    return counts, offsets, perm


# --------------------------------------------------------------------------
# step 7: one softmax over shared + routed entries (s = 1)
# --------------------------------------------------------------------------
def attend_head(Q, K, V, QL, VL, idx, route, return_weights=False, shared=True):
    """Output of one (b, h): query n attends [Q_L; K[idx_e]] -> [V_L; V[idx_e]], e = route_n.

    route [N] (s = 1) or [N, s] (the query's experts in rank order): the
    query's entries are then [Q_L; K[idx_e1]; ...; K[idx_es]] with values
    [V_L; V[idx_e1]; ...], no key merged across experts.  shared=False drops
    the Q_L / V_L entries (the route-only variant).  The queries are visited
    group by group (all queries with the same experts), as Algorithm 1
    groups them by route; each query still gets its own single softmax over
    all of its (shared and routed) logits.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N, d = Q.shape
    m, k = idx.shape
    routes = np.asarray(route).reshape(N, -1)               # [N, s]
    s = routes.shape[1]
    t = tau(d)
    out = np.empty((N, d))
    E = (m if shared else 0) + s * k
    weights = np.empty((N, E)) if return_weights else None
    experts, which = np.unique(routes, axis=0, return_inverse=True)
    which = np.asarray(which).reshape(-1)
    for gi, ex in enumerate(experts):
        g = np.nonzero(which == gi)[0]
        keys = ([QL] if shared else []) + [K[idx[e]] for e in ex]
        vals = ([VL] if shared else []) + [V[idx[e]] for e in ex]
        keys = np.concatenate(keys, axis=0)                 # E x d
        vals = np.concatenate(vals, axis=0)
        w = softmax_rows(t * (Q[g] @ keys.T))               # |g| x E
        out[g] = w @ vals
        if return_weights:
            weights[g] = w
    return (out, weights) if return_weights else out


# --------------------------------------------------------------------------
# the whole pass
# --------------------------------------------------------------------------
def mita_head(Q, K, V, grid_h, grid_w, m_h, m_w, k, keep_scores=False, s=1, shared=True):
    """All steps for one (b, h); Q, K, V are [N, d].  s: experts per query;
    shared=False: the route-only variant (V_L is still returned, unused)."""
    QL = landmark_queries(Q, grid_h, grid_w, m_h, m_w)
    S = landmark_scores(QL, K)
    idx, gap = expert_topk(S, k)
    VL = shared_values(S, V)
    route, rgap = route_queries(Q, QL, s)
    counts, offsets, perm = group_by_route(route, QL.shape[0])
    out = attend_head(Q, K, V, QL, VL, idx, route, shared=shared)
    res = dict(QL=QL, idx=idx, gap=gap, VL=VL, route=route, rgap=rgap,
               counts=counts, offsets=offsets, perm=perm, out=out)
    if keep_scores:
        res["S"] = S
    return res


# --------------------------------------------------------------------------
# backward: gradients of <dOut, out> with respect to Q, K and V
# --------------------------------------------------------------------------
# The pages time training with this attention ([ZH], long-sequence section,
# Table 5 and the route-only ablation), so its gradients are part of the
# method; they do not describe them.  The plain reading: the top-k sets and
# the routes are discrete choices, constant under small changes of the
# inputs, so no gradient flows through them (as through any argmax or sort);
# everything else is differentiated exactly: the one softmax of step 7, the
# shared expert's values V_L = softmax(S) V (step 4), the scores S (step 2),
# and the pooling that makes Q_L (step 1), which feeds both the shared keys
# and S.
def softmax_backward(w, dw):
    """Gradient with respect to the logits z of a row softmax w = softmax(z), given
    dw = d(loss)/dw:  w * (dw - sum(w * dw))."""
    return w * (dw - np.sum(w * dw, axis=-1, keepdims=True))


def mita_head_backward(Q, K, V, dOut, grid_h, grid_w, m_h, m_w, k, s=1, shared=True,
                       idx=None, route=None):
    """(dQ, dK, dV) of one (b, h): the gradients of sum(dOut * out), with the top-k sets and
    routes of the forward pass held fixed.  Steps 7, 4, 2, 1 in reverse.  idx / route, when
    given, replace the forward's own choices (to compare with a pass that took the other
    side of a near-tie)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dOut = np.asarray(dOut, dtype=np.float64)
    N, d = Q.shape
    t = tau(d)
    f = mita_head(Q, K, V, grid_h, grid_w, m_h, m_w, k, keep_scores=True, s=s, shared=shared)
    QL, S, VL = f["QL"], f["S"], f["VL"]
    idx = f["idx"] if idx is None else np.asarray(idx)
    m = QL.shape[0]
    routes = np.asarray(f["route"] if route is None else route).reshape(N, -1)
    dQ, dK, dV = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
    dQL, dVL = np.zeros((m, d)), np.zeros((m, d))
    # step 7: out_n = softmax(tau * keys q_n) . vals over the query's entries
    experts, which = np.unique(routes, axis=0, return_inverse=True)
    which = np.asarray(which).reshape(-1)
    for gi, ex in enumerate(experts):
        g = np.nonzero(which == gi)[0]
        keys = np.concatenate(([QL] if shared else []) + [K[idx[e]] for e in ex], axis=0)
        vals = np.concatenate(([VL] if shared else []) + [V[idx[e]] for e in ex], axis=0)
        w = softmax_rows(t * (Q[g] @ keys.T))                  # |g| x E
        dz = t * softmax_backward(w, dOut[g] @ vals.T)        # d/d(q . key)
        dQ[g] += dz @ keys
        dkeys = dz.T @ Q[g]                                    # E x d
        dvals = w.T @ dOut[g]
        off = 0
        if shared:
            dQL += dkeys[:m]
            dVL += dvals[:m]
            off = m
        for j, e in enumerate(ex):
            rows = slice(off + j * k, off + (j + 1) * k)
            np.add.at(dK, idx[e], dkeys[rows])
            np.add.at(dV, idx[e], dvals[rows])
    # step 4: V_L = A V with A = softmax_row(S), S = tau Q_L K^T (step 2)
    if shared:
        A = softmax_rows(S)
        dS = softmax_backward(A, dVL @ V.T)                    # m x N
        dV += A.T @ dVL
        dQL += t * (dS @ K)
        dK += t * (dS.T @ QL)
    # step 1: Q_L[i] = mean of Q over window i
    Qg = dQ.reshape(grid_h, grid_w, d)
    for r, (y0, y1) in enumerate(pool_windows(grid_h, m_h)):
        for c, (x0, x1) in enumerate(pool_windows(grid_w, m_w)):
            Qg[y0:y1, x0:x1] += dQL[r * m_w + c] / ((y1 - y0) * (x1 - x0))
    return dQ, dK, dV


def mita_forward(Q, K, V, grid_h, grid_w, m_h, m_w, k, heads=None, s=1, shared=True):
    """The pass over [B, H, N, d] inputs, head by head.

    ``heads`` optionally restricts the work to a list of (b, h) pairs; the
    result then stacks those heads in the given order along one axis.
    """
    Q = np.asarray(Q)
    B, H, N, d = Q.shape
    if grid_h * grid_w != N:
        raise ValueError("grid does not match N")
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    per = [mita_head(Q[b, h], K[b, h], V[b, h], grid_h, grid_w, m_h, m_w, k, s=s, shared=shared)
           for b, h in pairs]
    res = {key: np.stack([p[key] for p in per]) for key in per[0]}
    if heads is None:
        res = {key: val.reshape((B, H) + val.shape[1:]) for key, val in res.items()}
    return res
