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


def _route_high_ties(Q, QL):
    R = np.asarray(Q, dtype=np.float64) @ np.swapaxes(QL, -1, -2)
    m = R.shape[-1]
    route = m - 1 - np.argmax(R[..., ::-1], axis=-1)
    return route, _ORIG["route_queries"](Q, QL)[1]


def _route_argmin(Q, QL):
    R = np.asarray(Q, dtype=np.float64) @ np.swapaxes(QL, -1, -2)
    return np.argmin(R, axis=-1), _ORIG["route_queries"](Q, QL)[1]


def _group_reversed(route, m):
    counts, offsets, _ = _ORIG["group_by_route"](route, m)
    n = np.arange(len(route))
    perm = np.lexsort((-n, route))
    return counts, offsets, perm


def _attend_variant(kind):
    def attend(Q, K, V, QL, VL, idx, route, return_weights=False):
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


_ORIG = {name: getattr(O, name) for name in
         ["pool_windows", "landmark_scores", "expert_topk", "shared_values", "route_queries",
          "group_by_route", "attend_head"]}

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
