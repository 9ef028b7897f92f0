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
def route_queries(Q: np.ndarray, QL: np.ndarray):
    """route [..., N] (lowest landmark id on ties) and rgap = tau*(R_(1) - R_(2))."""
    Q = np.asarray(Q, dtype=np.float64)
    R = Q @ np.swapaxes(QL, -1, -2)                  # [..., N, m]
    route = np.argmax(R, axis=-1)                     # first maximum = lowest id
    m = R.shape[-1]
    if m == 1:
        rgap = np.full(R.shape[:-1], np.inf)
    else:
        srt = np.sort(R, axis=-1)
        rgap = (srt[..., -1] - srt[..., -2]) * tau(Q.shape[-1])
    return route, rgap


# --------------------------------------------------------------------------
# step 6: group the queries by their route (Algorithm 1)
# --------------------------------------------------------------------------
def group_by_route(route: np.ndarray, m: int):
    """Stable counting sort of one head's queries: counts [m], offsets [m+1], perm [N]."""
    route = np.asarray(route)
    counts = np.bincount(route, minlength=m)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.argsort(route, kind="stable")
    return counts, offsets, perm


# --------------------------------------------------------------------------
# step 7: one softmax over shared + routed entries (s = 1)
# --------------------------------------------------------------------------
def attend_head(Q, K, V, QL, VL, idx, route, return_weights=False):
    """Output of one (b, h): query n attends [Q_L; K[idx_e]] -> [V_L; V[idx_e]], e = route_n.

    The queries are visited expert group by expert group, as Algorithm 1
    does; each query still gets its own single softmax over m + k logits.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N, d = Q.shape
    m, k = idx.shape
    t = tau(d)
    out = np.empty((N, d))
    weights = np.empty((N, m + k)) if return_weights else None
    counts, offsets, perm = group_by_route(route, m)
    for e in range(m):
        g = perm[offsets[e]:offsets[e + 1]]
        if g.size == 0:
            continue
        keys = np.concatenate([QL, K[idx[e]]], axis=0)     # (m + k) x d
        vals = np.concatenate([VL, V[idx[e]]], axis=0)
        w = softmax_rows(t * (Q[g] @ keys.T))               # |g| x (m + k)
        out[g] = w @ vals
        if return_weights:
            weights[g] = w
    return (out, weights) if return_weights else out


# --------------------------------------------------------------------------
# the whole pass
# --------------------------------------------------------------------------
def mita_head(Q, K, V, grid_h, grid_w, m_h, m_w, k, keep_scores=False):
    """All steps for one (b, h); Q, K, V are [N, d]."""
    QL = landmark_queries(Q, grid_h, grid_w, m_h, m_w)
    S = landmark_scores(QL, K)
    idx, gap = expert_topk(S, k)
    VL = shared_values(S, V)
    route, rgap = route_queries(Q, QL)
    counts, offsets, perm = group_by_route(route, QL.shape[0])
    out = attend_head(Q, K, V, QL, VL, idx, route)
    res = dict(QL=QL, idx=idx, gap=gap, VL=VL, route=route, rgap=rgap,
               counts=counts, offsets=offsets, perm=perm, out=out)
    if keep_scores:
        res["S"] = S
    return res


def mita_forward(Q, K, V, grid_h, grid_w, m_h, m_w, k, heads=None):
    """The pass over [B, H, N, d] inputs, head by head.

    ``heads`` optionally restricts the work to a list of (b, h) pairs; the
    result then stacks those heads in the given order along one axis.
    """
    Q = np.asarray(Q)
    B, H, N, d = Q.shape
    if grid_h * grid_w != N:
        raise ValueError("grid does not match N")
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    per = [mita_head(Q[b, h], K[b, h], V[b, h], grid_h, grid_w, m_h, m_w, k) for b, h in pairs]
    res = {key: np.stack([p[key] for p in per]) for key in per[0]}
    if heads is None:
        res = {key: val.reshape((B, H) + val.shape[1:]) for key, val in res.items()}
    return res
