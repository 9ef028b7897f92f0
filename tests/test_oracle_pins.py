"""The oracle against its pins, and planted mistakes against the pins."""
import numpy as np
import pytest

import oracle.mita_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)


# ---- planted mistakes: each must be caught by at least one pin -------------
def _floor_windows(g, mg):
    return [((i * g) // mg, ((i + 1) * g) // mg) for i in range(mg)]


def _scores_no_tau(QL, K):
    return QL @ np.swapaxes(np.asarray(K, dtype=np.float64), -1, -2)


def _topk_high_ties(S, k):
    N = S.shape[-1]
    rev = S[..., ::-1]
    order = N - 1 - np.argsort(-rev, axis=-1, kind="stable")
    idx = np.sort(order[..., :k], axis=-1)
    ranked = np.take_along_axis(S, order, axis=-1)
    gap = ranked[..., k - 1] - ranked[..., k] if k < N else np.full(S.shape[:-1], np.inf)
    return idx, gap


def _shared_wrong_axis(S, V):
    z = np.exp(S - S.max(axis=-2, keepdims=True))
    return (z / z.sum(axis=-2, keepdims=True)) @ np.asarray(V, dtype=np.float64)


def _route_high_ties(Q, QL, s=1):
    R = np.asarray(Q, dtype=np.float64) @ np.swapaxes(QL, -1, -2)
    m = R.shape[-1]
    if s > 1:
        order = m - 1 - np.argsort(-R[..., ::-1], axis=-1, kind="stable")
        return order[..., :s], _ORIG["route_queries"](Q, QL, s)[1]
    route = m - 1 - np.argmax(R[..., ::-1], axis=-1)
    return route, _ORIG["route_queries"](Q, QL)[1]


def _route_argmin(Q, QL, s=1):
    R = np.asarray(Q, dtype=np.float64) @ np.swapaxes(QL, -1, -2)
    if s > 1:
        return np.argsort(R, axis=-1, kind="stable")[..., :s], _ORIG["route_queries"](Q, QL, s)[1]
    return np.argmin(R, axis=-1), _ORIG["route_queries"](Q, QL)[1]


def _group_reversed(route, m):
    route = np.asarray(route).reshape(-1)
    counts, offsets, _ = _ORIG["group_by_route"](route, m)
    n = np.arange(len(route))
    perm = np.lexsort((-n, route))
    return counts, offsets, perm


def _attend_variant(kind):
    """The attend step written per query for s = 1 with one planted mistake
    (or none, for "plain"); with s > 1 or without the shared expert it defers
    to the oracle, so that only the s = 1 pins see the mistake."""
    def attend(Q, K, V, QL, VL, idx, route, return_weights=False, shared=True):
        if np.asarray(route).ndim > 1 or not shared:
            return _ORIG["attend_head"](Q, K, V, QL, VL, idx, route, return_weights, shared)
        Q = np.asarray(Q, dtype=np.float64); K = np.asarray(K, dtype=np.float64)
        V = np.asarray(V, dtype=np.float64)
        N, d = Q.shape
        m, k = idx.shape
        t = 1.0 / np.sqrt(d) if kind != "no_tau" else 1.0
        out = np.empty((N, d)); W = np.empty((N, m + k))
        for n in range(N):
            e = 0 if kind == "wrong_expert" else route[n]
            ls = t * (QL @ Q[n]); lr = t * (K[idx[e]] @ Q[n])
            if kind == "two_softmaxes":
                ws = np.exp(ls - ls.max()); ws /= ws.sum()
                wr = np.exp(lr - lr.max()); wr /= wr.sum()
                w = np.concatenate([ws, wr]) / 2
            elif kind == "no_shared":
                wr = np.exp(lr - lr.max()); wr /= wr.sum()
                w = np.concatenate([np.zeros(m), wr])
            else:
                z = np.concatenate([ls, lr]); w = np.exp(z - z.max()); w /= w.sum()
            out[n] = w @ np.concatenate([VL, V[idx[e]]]); W[n] = w
        return (out, W) if return_weights else out
    return attend


def _forward_heads_swapped(Q, K, V, grid_h, grid_w, m_h, m_w, k, heads=None, **kw):
    """The batched wrapper with the (b, h) loop order swapped when stacking."""
    res = _ORIG["mita_forward"](Q, K, V, grid_h, grid_w, m_h, m_w, k, heads=heads, **kw)
    if heads is None:
        B, H = np.asarray(Q).shape[:2]
        return {key: val.reshape((B * H,) + val.shape[2:]).reshape((H, B) + val.shape[2:])
                .swapaxes(0, 1) for key, val in res.items()}
    return {key: val[::-1] for key, val in res.items()}


def _attend_multi(kind):
    """The attend step for s > 1 / route-only with one planted mistake; the s = 1 shared
    pass defers to the oracle."""
    def attend(Q, K, V, QL, VL, idx, route, return_weights=False, shared=True):
        route = np.asarray(route)
        if route.ndim == 1 and shared:
            return _ORIG["attend_head"](Q, K, V, QL, VL, idx, route, return_weights, shared)
        Q = np.asarray(Q, dtype=np.float64); K = np.asarray(K, dtype=np.float64)
        V = np.asarray(V, dtype=np.float64)
        N, d = Q.shape
        routes = route.reshape(N, -1)
        t = 1.0 / np.sqrt(d)
        out = np.empty((N, d))
        W = []
        for n in range(N):
            ex = routes[n][:1] if kind == "first_only" else routes[n]
            keys_id = np.concatenate([idx[e] for e in ex])
            if kind == "dedup":
                keys_id = np.unique(keys_id)
            with_shared = shared or kind == "keeps_shared"
            keys = np.concatenate(([QL] if with_shared else []) + [K[keys_id]])
            vals = np.concatenate(([VL] if with_shared else []) + [V[keys_id]])
            z = t * (keys @ Q[n]); w = np.exp(z - z.max()); w /= w.sum()
            out[n] = w @ vals
            W.append(w)
        return (out, np.array(W, dtype=object)) if return_weights else out
    return attend


def _backward_variant(kind):
    """The oracle's backward with one planted mistake."""
    def backward(Q, K, V, dOut, grid_h, grid_w, m_h, m_w, k, s=1, shared=True):
        Q = np.asarray(Q, dtype=np.float64); K = np.asarray(K, dtype=np.float64)
        V = np.asarray(V, dtype=np.float64); dOut = np.asarray(dOut, dtype=np.float64)
        N, d = Q.shape
        t = 1.0 / np.sqrt(d)
        f = O.mita_head(Q, K, V, grid_h, grid_w, m_h, m_w, k, keep_scores=True, s=s,
                        shared=shared)
        QL, S, idx, VL = f["QL"], f["S"], f["idx"], f["VL"]
        m = QL.shape[0]
        routes = np.asarray(f["route"]).reshape(N, -1)
        dQ, dK, dV = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
        dQL, dVL = np.zeros((m, d)), np.zeros((m, d))
        for n in range(N):
            keys = np.concatenate(([QL] if shared else []) + [K[idx[e]] for e in routes[n]])
            vals = np.concatenate(([VL] if shared else []) + [V[idx[e]] for e in routes[n]])
            z = t * (keys @ Q[n]); w = np.exp(z - z.max()); w /= w.sum()
            dw = vals @ dOut[n]
            dz = t * (w * dw if kind == "softmax_grad_not_centred" else w * (dw - w @ dw))
            dQ[n] += dz @ keys
            dkeys, dvals = np.outer(dz, Q[n]), np.outer(w, dOut[n])
            off = m if shared else 0
            if shared:
                dQL += dkeys[:m]; dVL += dvals[:m]
            for j, e in enumerate(routes[n]):
                np.add.at(dK, idx[e], dkeys[off + j * k:off + (j + 1) * k])
                np.add.at(dV, idx[e], dvals[off + j * k:off + (j + 1) * k])
        if shared and kind != "no_landmark_value_path":
            A = np.exp(S - S.max(1, keepdims=True)); A /= A.sum(1, keepdims=True)
            dA = dVL @ V.T
            dS = A * (dA - (A * dA).sum(1, keepdims=True))
            dV += A.T @ dVL
            dQL += (1.0 if kind == "scores_path_without_tau" else t) * (dS @ K)
            dK += t * (dS.T @ QL)
        if kind != "no_pooling_backward":
            Qg = dQ.reshape(grid_h, grid_w, d)
            for r, (y0, y1) in enumerate(O.pool_windows(grid_h, m_h)):
                for c, (x0, x1) in enumerate(O.pool_windows(grid_w, m_w)):
                    Qg[y0:y1, x0:x1] += dQL[r * m_w + c] / ((y1 - y0) * (x1 - x0))
        return dQ, dK, dV
    return backward


def test_backward_harness_is_faithful():
    """The mutant harness for the backward, unmutated, reproduces the oracle."""
    rng = np.random.default_rng(1)
    Q, K, V, G = (rng.standard_normal((30, 8)) for _ in range(4))
    for s, shared in [(1, True), (2, True), (1, False)]:
        a = O.mita_head_backward(Q, K, V, G, 5, 6, 2, 2, 6, s=s, shared=shared)
        b = _backward_variant("plain")(Q, K, V, G, 5, 6, 2, 2, 6, s=s, shared=shared)
        for x, y in zip(a, b):
            assert np.allclose(x, y, rtol=0, atol=1e-12)


_ORIG = {name: getattr(O, name) for name in
         ["pool_windows", "landmark_scores", "expert_topk", "shared_values", "route_queries",
          "group_by_route", "attend_head", "mita_forward"]}

MUTANTS = {
    "pool_floor_windows": ("pool_windows", _floor_windows),
    "scores_without_tau": ("landmark_scores", _scores_no_tau),
    "topk_ties_to_highest": ("expert_topk", _topk_high_ties),
    "topk_smallest": ("expert_topk", lambda S, k: _ORIG["expert_topk"](-S, k)),
    "shared_softmax_wrong_axis": ("shared_values", _shared_wrong_axis),
    "route_ties_to_highest": ("route_queries", _route_high_ties),
    "route_argmin": ("route_queries", _route_argmin),
    "group_unstable": ("group_by_route", _group_reversed),
    "attend_without_tau": ("attend_head", _attend_variant("no_tau")),
    "attend_two_softmaxes": ("attend_head", _attend_variant("two_softmaxes")),
    "attend_wrong_expert": ("attend_head", _attend_variant("wrong_expert")),
    "attend_no_shared": ("attend_head", _attend_variant("no_shared")),
    "forward_heads_swapped": ("mita_forward", _forward_heads_swapped),
    "multi_expert_dedup": ("attend_head", _attend_multi("dedup")),
    "multi_expert_first_only": ("attend_head", _attend_multi("first_only")),
    "route_only_keeps_shared": ("attend_head", _attend_multi("keeps_shared")),
    "backward_softmax_grad_not_centred": ("mita_head_backward",
                                          _backward_variant("softmax_grad_not_centred")),
    "backward_no_landmark_value_path": ("mita_head_backward",
                                        _backward_variant("no_landmark_value_path")),
    "backward_scores_path_without_tau": ("mita_head_backward",
                                         _backward_variant("scores_path_without_tau")),
    "backward_no_pooling_backward": ("mita_head_backward", _backward_variant("no_pooling_backward")),
    "route_top_s_unsorted": ("route_queries",
                             lambda Q, QL, s=1: (np.sort(_ORIG["route_queries"](Q, QL, s)[0], -1)
                                                 if s > 1 else _ORIG["route_queries"](Q, QL, s)[0],
                                                 _ORIG["route_queries"](Q, QL, s)[1])),
}


def test_reference_attend_variant_is_faithful():
    """The mutant harness itself: its unmutated variant reproduces the oracle."""
    rng = np.random.default_rng(0)
    Q, K, V = (rng.standard_normal((36, 8)) for _ in range(3))
    r = O.mita_head(Q, K, V, 6, 6, 2, 2, 5)
    got = _attend_variant("plain")(Q, K, V, r["QL"], r["VL"], r["idx"], r["route"])
    assert np.allclose(got, r["out"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(O)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
