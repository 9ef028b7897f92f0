"""Comparison of the HIP path's results with the fp64 oracle, head by head.

Acceptance (floating point decides the discrete choices, so near-ties are
allowed to go either way):

* Top-k row i: when the oracle's boundary gap s_(k) - s_(k+1) is at least
  1e-3 the GPU set must equal the oracle set exactly.  Below that the row is
  a counted near-tie: the GPU set must still hold k distinct ids, and every
  id in the symmetric difference must score within 1e-3 of s_(k).
* Route n: must equal the oracle route unless tau*(R_(1) - R_(2)) < 1e-3;
  then the GPU route r' is accepted when tau*(R[n, route_n] - R[n, r']) < 1e-3.
  With s routes per query: the list (best first) must equal the oracle's
  unless some gap among its first s + 1 ranked landmarks is below 1e-3; then
  each GPU route must score within 1e-3 of the oracle's route of that rank.
* Q_L, V_L: against the oracle's values.
* out: against the oracle's output step re-run with the GPU's idx and route
  (identical to the plain oracle wherever the choices agree).
* counts / offsets / perm: bit-exact against the stable counting sort of
  the GPU's own route.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import oracle.mita_oracle as O

NEAR = 1e-3


@dataclass
class Report:
    heads: int = 0
    topk_rows: int = 0
    topk_near_ties: int = 0
    topk_deviations: int = 0
    routes: int = 0
    route_near_ties: int = 0
    route_deviations: int = 0
    max_err: dict = field(default_factory=lambda: {"ql": 0.0, "vl": 0.0, "out": 0.0})

    def bump(self, key, val):
        self.max_err[key] = max(self.max_err[key], float(val))


def check_topk_head(idx_gpu, S, k, rep: Report):
    m, N = S.shape
    idx_o, gap = O.expert_topk(S, k)
    for i in range(m):
        g = np.asarray(idx_gpu[i])
        rep.topk_rows += 1
        if np.array_equal(g, idx_o[i]):
            if gap[i] < NEAR:
                rep.topk_near_ties += 1
            continue
        assert gap[i] < NEAR, f"top-k row {i} differs with boundary gap {gap[i]:.3g}"
        rep.topk_near_ties += 1
        rep.topk_deviations += 1
        assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < N, f"row {i} invalid"
        assert np.all(np.diff(g) > 0), f"row {i} not ascending"
        kth = np.sort(S[i])[::-1][k - 1]
        diff = np.setxor1d(g, idx_o[i])
        assert np.all(np.abs(S[i, diff] - kth) < NEAR), f"row {i}: deviation beyond near-tie"


def check_route_head(route_gpu, Q, QL, rep: Report):
    route_o, rgap = O.route_queries(Q, QL)
    R = np.asarray(Q, np.float64) @ QL.T
    t = O.tau(Q.shape[-1])
    rep.routes += len(route_o)
    rep.route_near_ties += int(np.sum(rgap < NEAR))
    bad = np.nonzero(route_gpu != route_o)[0]
    for n in bad:
        rep.route_deviations += 1
        assert rgap[n] < NEAR, f"route of query {n} differs with gap {rgap[n]:.3g}"
        loss = t * (R[n, route_o[n]] - R[n, route_gpu[n]])
        assert loss < NEAR, f"route of query {n}: accepted only within a near-tie"


def check_routes_multi(route_gpu, Q, QL, s, rep: Report):
    """s > 1: each query's s routes, best first.  Where the oracle's ranking has no gap
    below 1e-3 among its first s + 1 landmarks the GPU list must equal it; otherwise (a
    counted near-tie) every GPU route must be distinct and score within 1e-3 of the
    oracle's route of the same rank."""
    route_o, _ = O.route_queries(Q, QL, s)
    R = np.asarray(Q, np.float64) @ QL.T
    t = O.tau(Q.shape[-1])
    m = R.shape[-1]
    srt = -np.sort(-R, axis=-1)[:, :min(s + 1, m)]
    near = np.any(np.diff(-srt, axis=-1) * t < NEAR, axis=-1) if srt.shape[1] > 1 else \
        np.zeros(len(R), bool)
    rep.routes += len(route_o)
    rep.route_near_ties += int(np.sum(near))
    g = np.asarray(route_gpu).reshape(len(R), s)
    for n in np.nonzero(np.any(g != route_o, axis=-1))[0]:
        rep.route_deviations += 1
        assert near[n], f"routes of query {n} differ without a near-tie"
        assert len(set(g[n].tolist())) == s and g[n].min() >= 0 and g[n].max() < m, n
        loss = t * np.abs(R[n, route_o[n]] - R[n, g[n]])
        assert np.all(loss < NEAR), f"routes of query {n}: accepted only within a near-tie"


def check_grouping_head(route_gpu, counts, offsets, perm, m):
    c, o, p = O.group_by_route(np.asarray(route_gpu, dtype=np.int64), m)
    assert np.array_equal(counts, c), "counts"
    assert np.array_equal(offsets, o), "offsets"
    assert np.array_equal(perm, p), "perm"


def check_head(gpu: dict, Qh, Kh, Vh, grid_h, grid_w, m_h, m_w, k, tol, rep: Report, s=1,
               shared=True):
    """gpu: this head's arrays (out, idx, route and optionally ql, vl, counts, offsets, perm).
    s: experts per query; shared=False: the route-only variant (no V_L to compare)."""
    ref = O.mita_head(Qh, Kh, Vh, grid_h, grid_w, m_h, m_w, k, keep_scores=True, s=s,
                      shared=shared)
    rep.heads += 1
    if "ql" in gpu:
        e = np.abs(gpu["ql"] - ref["QL"]).max()
        rep.bump("ql", e)
        assert e <= tol, f"Q_L error {e:.3g}"
    if "vl" in gpu and shared:
        e = np.abs(gpu["vl"] - ref["VL"]).max()
        rep.bump("vl", e)
        assert e <= tol, f"V_L error {e:.3g}"
    check_topk_head(gpu["idx"], ref["S"], k, rep)
    if s == 1:
        check_route_head(gpu["route"], Qh, ref["QL"], rep)
    else:
        check_routes_multi(gpu["route"], Qh, ref["QL"], s, rep)
    if "perm" in gpu:
        check_grouping_head(gpu["route"], gpu["counts"], gpu["offsets"], gpu["perm"], m_h * m_w)
    cond = O.attend_head(Qh, Kh, Vh, ref["QL"], ref["VL"], np.asarray(gpu["idx"]),
                         np.asarray(gpu["route"]), shared=shared)
    e = np.abs(gpu["out"] - cond).max()
    rep.bump("out", e)
    assert e <= tol, f"out error {e:.3g}"


def run_and_check(res: dict, Q, K, V, grid_h, grid_w, m_h, m_w, k, tol, heads=None, s=1,
                  shared=True) -> Report:
    """res: full-batch GPU results already copied to numpy ([B,H,...] arrays)."""
    B, H = Q.shape[:2]
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    rep = Report()
    for b, h in pairs:
        gpu = {key: val[b, h] for key, val in res.items() if val is not None}
        try:
            check_head(gpu, Q[b, h], K[b, h], V[b, h], grid_h, grid_w, m_h, m_w, k, tol, rep,
                       s=s, shared=shared)
        except AssertionError as e:
            raise AssertionError(f"head (b={b}, h={h}): {e}") from None
    return rep
