"""Pins of the fp64 oracle against things other than itself.

Each ``pin_*`` takes the oracle module and raises AssertionError when the
oracle disagrees with a brute-force count on a tiny input, a library routine
the step reduces to (torch's adaptive average pooling and scaled-dot-product
attention, evaluated in float64 on the CPU), a closed form, or an invariant.
``test_oracle_pins.py`` runs them against the oracle as written and against
copies with planted mistakes, each of which must trip at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa(q, k, v, mask=None):
    """torch's scaled-dot-product attention in float64 on the CPU (scale 1/sqrt(d))."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    m = None if mask is None else torch.from_numpy(mask)
    return F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m).numpy()


# ---------------------------------------------------------------- pooling
def pin_pool_identity(O):
    """m = N (one landmark per token) makes Q_L = Q exactly."""
    Q = _rng(1).standard_normal((2, 6 * 5, 8))
    QL = O.landmark_queries(Q, 6, 5, 6, 5)
    assert np.array_equal(QL, Q), "pooling to m=N must return Q"


def pin_pool_vs_torch(O):
    """2-D adaptive average pooling equals torch.nn.functional.adaptive_avg_pool2d."""
    for gh, gw, mh, mw in [(14, 14, 5, 5), (56, 56, 7, 7), (128, 128, 16, 16),
                           (9, 6, 4, 5), (7, 10, 3, 4), (5, 5, 1, 1)]:
        d = 4
        Q = _rng(gh * 1000 + gw).standard_normal((3, gh * gw, d))
        ref = F.adaptive_avg_pool2d(
            torch.from_numpy(Q).reshape(3, gh, gw, d).permute(0, 3, 1, 2), (mh, mw))
        ref = ref.permute(0, 2, 3, 1).reshape(3, mh * mw, d).numpy()
        got = O.landmark_queries(Q, gh, gw, mh, mw)
        assert np.allclose(got, ref, rtol=0, atol=1e-12), f"pool {gh}x{gw}->{mh}x{mw}"


# ---------------------------------------------------------------- top-k
def _brute_topk(row, k):
    """Keys whose (score desc, key asc) rank is below k, counted one pair at a time."""
    n = len(row)
    sel, rank_of = [], {}
    for j in range(n):
        r = 0
        for jj in range(n):
            if row[jj] > row[j] or (row[jj] == row[j] and jj < j):
                r += 1
        rank_of[r] = j
        if r < k:
            sel.append(j)
    gap = row[rank_of[k - 1]] - row[rank_of[k]] if k < n else math.inf
    return sorted(sel), gap


def pin_topk_bruteforce(O):
    """Top-k sets and boundary gaps equal pairwise rank counting, ties included."""
    rng = _rng(7)
    cases = [rng.standard_normal((5, 17)),
             np.round(rng.standard_normal((6, 23)) * 2) / 2,   # many exact ties
             np.zeros((2, 9)),                                  # all tied
             np.tile(np.arange(4.0), (3, 3))]                   # repeated pattern
    for S in cases:
        n = S.shape[1]
        for k in sorted({1, 2, n // 2, n - 1, n}):
            idx, gap = O.expert_topk(S, k)
            for i in range(S.shape[0]):
                sel, g = _brute_topk(list(S[i]), k)
                assert list(idx[i]) == sel, f"top-{k} set of row {i}"
                assert (g == gap[i]) or (math.isinf(g) and math.isinf(gap[i])), "gap"


def pin_topk_zero_queries(O):
    """Q = 0 makes every score 0, so every expert is keys 0..k-1 and every route is 0."""
    rng = _rng(3)
    Q = np.zeros((7 * 6, 8))
    K = rng.standard_normal((42, 8))
    V = rng.standard_normal((42, 8))
    r = O.mita_head(Q, K, V, 7, 6, 3, 2, 5)
    assert np.array_equal(r["idx"], np.tile(np.arange(5), (6, 1)))
    assert np.array_equal(r["route"], np.zeros(42, dtype=r["route"].dtype))


# ---------------------------------------------------------------- routing
def pin_route_bruteforce(O):
    """Integer-valued inputs make every dot product exact; ties go to the lowest landmark."""
    rng = _rng(11)
    Q = rng.integers(-2, 3, size=(40, 6)).astype(np.float64)
    QL = rng.integers(-2, 3, size=(7, 6)).astype(np.float64)
    QL[4] = QL[1]
    QL[6] = QL[2]
    route, rgap = O.route_queries(Q, QL)
    for n in range(40):
        best, arg, vals = -math.inf, -1, []
        for i in range(7):
            v = sum(float(Q[n, c]) * float(QL[i, c]) for c in range(6))
            vals.append(v)
            if v > best:
                best, arg = v, i
        assert route[n] == arg, f"route of query {n}"
        vals.sort()
        assert rgap[n] == (vals[-1] - vals[-2]) / math.sqrt(6)


def pin_route_self_landmarks(O):
    """With m = N the landmarks are the queries: route_n = argmax_j q_n . q_j (lowest j)."""
    rng = _rng(5)
    Q = rng.integers(-2, 3, size=(4 * 5, 3)).astype(np.float64)
    QL = O.landmark_queries(Q, 4, 5, 4, 5)
    route, _ = O.route_queries(Q, QL)
    for n in range(20):
        dots = [sum(Q[n, c] * Q[j, c] for c in range(3)) for j in range(20)]
        assert route[n] == dots.index(max(dots))


def pin_group_by_route(O):
    """Counting sort of queries by route equals Python's stable sort and a tally."""
    route = _rng(13).integers(0, 6, size=50)
    counts, offsets, perm = O.group_by_route(route, 7)
    assert list(perm) == sorted(range(50), key=lambda n: route[n])
    tally = [0] * 7
    for r in route:
        tally[r] += 1
    assert list(counts) == tally
    assert list(offsets) == [sum(tally[:i]) for i in range(8)]


# ---------------------------------------------------------------- shared expert
def pin_shared_vs_sdpa(O):
    """V_L is the landmarks' cross-attention over all keys: torch SDPA(Q_L, K, V)."""
    rng = _rng(17)
    Q, K, V = (rng.standard_normal((2, 3, 8 * 9, 16)) for _ in range(3))
    QL = O.landmark_queries(Q, 8, 9, 3, 4)
    VL = O.shared_values(O.landmark_scores(QL, K), V)
    assert np.allclose(VL, _sdpa(QL, K, V), rtol=0, atol=1e-12)


def pin_shared_self_attention(O):
    """With m = N, V_L is plain softmax(Q K^T / sqrt(d)) V (textbook full attention)."""
    rng = _rng(19)
    Q, K, V = (rng.standard_normal((5 * 4, 8)) for _ in range(3))
    QL = O.landmark_queries(Q, 5, 4, 5, 4)
    VL = O.shared_values(O.landmark_scores(QL, K), V)
    logits = Q @ K.T / math.sqrt(8)
    w = np.exp(logits - logits.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    assert np.allclose(VL, w @ V, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- output
def pin_weights_sum_to_one(O):
    """Each query spreads one softmax over exactly m + k entries, summing to 1."""
    rng = _rng(23)
    Q, K, V = (rng.standard_normal((6 * 7, 8)) for _ in range(3))
    QL = O.landmark_queries(Q, 6, 7, 2, 3)
    S = O.landmark_scores(QL, K)
    idx, _ = O.expert_topk(S, 9)
    route, _ = O.route_queries(Q, QL)
    out, w = O.attend_head(Q, K, V, QL, O.shared_values(S, V), idx, route, return_weights=True)
    assert w.shape == (42, 6 + 9)
    assert np.all(w >= 0) and np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)


def pin_constant_values(O):
    """V = c everywhere gives V_L = c and out = c."""
    rng = _rng(29)
    Q, K = (rng.standard_normal((5 * 5, 8)) for _ in range(2))
    V = np.full((25, 8), 0.75)
    r = O.mita_head(Q, K, V, 5, 5, 2, 2, 7)
    assert np.allclose(r["VL"], 0.75, rtol=0, atol=1e-13)
    assert np.allclose(r["out"], 0.75, rtol=0, atol=1e-13)


def pin_dense_when_k_is_n(O):
    """k = N makes every expert all keys: out = attention over [Q_L; K] with values [V_L; V]."""
    rng = _rng(31)
    Q, K, V = (rng.standard_normal((6 * 6, 16)) for _ in range(3))
    r = O.mita_head(Q, K, V, 6, 6, 2, 3, 36)
    ref = _sdpa(Q, np.concatenate([r["QL"], K]), np.concatenate([r["VL"], V]))
    assert np.allclose(r["out"], ref, rtol=0, atol=1e-12)


def pin_single_landmark_closed_form(O):
    """m = 1, k = N: Q_L = mean(Q), V_L = attn(mean(Q), K, V), out = attn(Q, [Q_L;K], [V_L;V])."""
    rng = _rng(37)
    Q, K, V = (rng.standard_normal((5 * 7, 8)) for _ in range(3))
    r = O.mita_head(Q, K, V, 5, 7, 1, 1, 35)
    ql = Q.mean(axis=0, keepdims=True)
    vl = _sdpa(ql, K, V)
    ref = _sdpa(Q, np.concatenate([ql, K]), np.concatenate([vl, V]))
    assert np.allclose(r["QL"], ql, rtol=0, atol=1e-14)
    assert np.allclose(r["VL"], vl, rtol=0, atol=1e-12)
    assert np.allclose(r["out"], ref, rtol=0, atol=1e-12)
    assert np.all(r["route"] == 0)


def pin_masked_attention(O):
    """General m, k: out equals dense attention over [Q_L; K] masked to Q_L and K[idx_route]."""
    rng = _rng(41)
    for gh, gw, mh, mw, k in [(8, 8, 3, 3, 6), (6, 9, 2, 4, 11), (7, 7, 7, 7, 1)]:
        N, m = gh * gw, mh * mw
        Q, K, V = (rng.standard_normal((N, 16)) for _ in range(3))
        r = O.mita_head(Q, K, V, gh, gw, mh, mw, k)
        mask = np.zeros((N, m + N), dtype=bool)
        mask[:, :m] = True
        for n in range(N):
            mask[n, m + r["idx"][r["route"][n]]] = True
        ref = _sdpa(Q, np.concatenate([r["QL"], K]), np.concatenate([r["VL"], V]), mask)
        assert np.allclose(r["out"], ref, rtol=0, atol=1e-12), (gh, gw, mh, mw, k)


def pin_key_permutation(O):
    """Permuting K and V rows jointly leaves out and V_L unchanged and relabels idx."""
    rng = _rng(43)
    Q, K, V = (rng.standard_normal((6 * 8, 16)) for _ in range(3))
    p = rng.permutation(48)
    a = O.mita_head(Q, K, V, 6, 8, 2, 2, 10)
    b = O.mita_head(Q, K[p], V[p], 6, 8, 2, 2, 10)
    assert np.allclose(a["out"], b["out"], rtol=0, atol=1e-12)
    assert np.allclose(a["VL"], b["VL"], rtol=0, atol=1e-12)
    assert np.array_equal(a["route"], b["route"])
    for i in range(4):
        assert sorted(p[b["idx"][i]]) == list(a["idx"][i])


# ---------------------------------------------------------------- the pages' own numbers
def pin_page_numbers(O):
    """Entries per query (m+k) and the DeiT-S FLOPs drop printed on the pages.

    The pages print 25+25 = 50 entries per query at m = k = 25 and 98 at
    m = k = 49; and 4.6 G -> 4.4 G FLOPs for DeiT-S (12 layers, 6 heads of
    width 64, 14x14 patches) when full attention becomes MiTA at m = k = 25.
    The FLOPs check counts the multiply-adds of the oracle's products (S,
    V_L, the query-landmark logits reused for routing, the routed logits,
    and the output's weighted sum) against full attention's 2 N^2 d.
    """
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    rng = _rng(47)
    for case in facts["entries_per_query"]:
        m_side = int(round(math.sqrt(case["m"])))
        g = 2 * m_side
        N = g * g
        Q, K, V = (rng.standard_normal((N, 8)) for _ in range(3))
        QL = O.landmark_queries(Q, g, g, m_side, m_side)
        S = O.landmark_scores(QL, K)
        idx, _ = O.expert_topk(S, case["k"])
        route, _ = O.route_queries(Q, QL)
        _, w = O.attend_head(Q, K, V, QL, O.shared_values(S, V), idx, route, return_weights=True)
        assert w.shape[1] == case["entries"]
    f = facts["deit_s_flops"]
    N, d, m, k = f["tokens"], f["head_dim"], f["m"], f["k"]
    per_head_full = 2 * N * N * d
    per_head_mita = (m * N * d) * 2 + (N * m * d) + (N * k * d) + N * (m + k) * d
    delta = f["layers"] * f["heads"] * (per_head_full - per_head_mita) / 1e9
    printed = f["full_gflops"] - f["mita_gflops"]
    assert abs(delta - printed) <= 0.1 + 1e-9, (delta, printed)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
