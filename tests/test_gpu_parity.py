"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances: max-abs 1e-4 on fp32 inputs, 1e-2 on bf16 inputs, for Q_L, V_L
and out; top-k sets and routes bit-exact outside counted near-ties (see
tests/parity.py).  Every case prints its name before touching the GPU.
"""
import sys

import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return torch


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def _to_dev(x, dtype):
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def run_gpu(Q, K, V, dtype, grid_h, grid_w, m_h, m_w, k, path="auto", extras=True, s=1,
            route_only=False):
    import efficient_attention_avg_amd as mita
    torch = _torch()
    q, kk, v = (_to_dev(x, dtype) for x in (Q, K, V))
    res = mita.mita_forward_ex(q, kk, v, grid_h, grid_w, m_h, m_w, k, idx=True, route=True,
                               extras=extras, path=path, s=s, route_only=route_only)
    torch.cuda.synchronize()
    return {key: val.cpu().numpy() for key, val in res.items() if val is not None}


SMALL = [
    # B, H, gh, gw, mh, mw, k, dtype, smooth
    (2, 3, 14, 14, 5, 5, 25, "bf16", True),
    (1, 2, 20, 24, 6, 5, 37, "bf16", True),
    (1, 1, 56, 56, 7, 7, 64, "bf16", True),
    (1, 2, 9, 7, 3, 2, 63, "f32", False),     # k = N
    (1, 1, 10, 10, 1, 1, 100, "bf16", True),  # m = 1, k = N
    (1, 1, 6, 6, 6, 6, 3, "f32", False),      # m = N
    (3, 1, 5, 5, 2, 2, 1, "bf16", True),      # k = 1
    (1, 1, 1, 1, 1, 1, 1, "f32", False),      # N = 1
    (1, 1, 33, 31, 4, 5, 200, "bf16", True),  # ragged everywhere
    (1, 2, 24, 24, 4, 4, 450, "bf16", True),  # k past the MFMA landmark kernel's LDS buffers
    (2, 2, 14, 14, 5, 5, 25, "f32", False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:7])) + "-" + c[7])
def test_small_shapes(case):
    B, H, gh, gw, mh, mw, k, dtype, smooth = case
    _say(f"small shape {case}")
    Q, K, V = synth.make_qkv(B, H, gh, gw, 64, workload_id=100 + gh * 7 + gw, smooth=smooth,
                             dtype=dtype)
    res = run_gpu(Q, K, V, dtype, gh, gw, mh, mw, k)
    rep = parity.run_and_check(res, Q, K, V, gh, gw, mh, mw, k, TOL[dtype])
    _say(f"ok {rep}")


def _random_shapes(n, seed):
    """Seeded random configurations across the implementation's ranges: grids up
    to 64 on a side, landmark grids up to 16x16, k from 1 to min(N, 300), both
    input types (fp32 at small sizes), smooth or plain inputs."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        gh, gw = (int(x) for x in rng.integers(1, 65, size=2))
        mh, mw = int(rng.integers(1, min(gh, 16) + 1)), int(rng.integers(1, min(gw, 16) + 1))
        N = gh * gw
        k = int(rng.integers(1, min(N, 300) + 1))
        dtype = "f32" if N <= 1024 and rng.random() < 0.3 else "bf16"
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        out.append((B, H, gh, gw, mh, mw, k, dtype, bool(rng.random() < 0.7)))
    return out


RANDOM = _random_shapes(16, 2024)


def _random_fused_shapes(n, seed):
    """Seeded random configurations inside the single-kernel schedule's range
    (N <= 208, m <= 32, k <= 32, bf16)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        gh, gw = (int(x) for x in rng.integers(1, 17, size=2))
        if gh * gw > 208:
            continue
        mh, mw = int(rng.integers(1, gh + 1)), int(rng.integers(1, gw + 1))
        if mh * mw > 32:
            continue
        k = int(rng.integers(1, min(gh * gw, 32) + 1))
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 4)), gh, gw, mh, mw, k))
    return out


RANDOM_FUSED = _random_fused_shapes(12, 77)


@pytest.mark.parametrize("case", RANDOM, ids=lambda c: "x".join(map(str, c[:7])) + "-" + c[7])
def test_random_shapes(case):
    B, H, gh, gw, mh, mw, k, dtype, smooth = case
    _say(f"random shape {case}")
    Q, K, V = synth.make_qkv(B, H, gh, gw, 64, workload_id=500 + gh * 67 + gw, smooth=smooth,
                             dtype=dtype)
    res = run_gpu(Q, K, V, dtype, gh, gw, mh, mw, k)
    rep = parity.run_and_check(res, Q, K, V, gh, gw, mh, mw, k, TOL[dtype])
    _say(f"ok {rep}")


FUSED = RANDOM_FUSED + [
    # B, H, gh, gw, mh, mw, k: shapes the single-kernel schedule accepts
    (2, 3, 14, 14, 5, 5, 25),   # DeiT shape
    (2, 2, 13, 16, 8, 4, 32),   # largest N, m and k it takes
    (1, 3, 4, 4, 1, 1, 16),     # m = 1, k = N
    (1, 1, 5, 5, 5, 5, 25),     # m = N = k
    (2, 1, 7, 9, 3, 3, 1),      # k = 1
    (1, 1, 1, 1, 1, 1, 1),      # N = 1
    (3, 2, 11, 6, 4, 3, 17),    # ragged tails everywhere
]


@pytest.mark.parametrize("path", ["fused", "staged"])
@pytest.mark.parametrize("case", FUSED, ids=lambda c: "x".join(map(str, c)))
def test_both_schedules(case, path):
    B, H, gh, gw, mh, mw, k = case
    _say(f"{path} schedule {case}")
    Q, K, V = synth.make_qkv(B, H, gh, gw, 64, workload_id=300 + gh * 5 + gw + k)
    res = run_gpu(Q, K, V, "bf16", gh, gw, mh, mw, k, path=path)
    rep = parity.run_and_check(res, Q, K, V, gh, gw, mh, mw, k, TOL["bf16"])
    _say(f"ok {rep}")


@pytest.mark.parametrize("path", ["fused", "staged"])
def test_exact_ties_take_lowest_index(path):
    """Small-integer inputs with one landmark per token make every score and
    route logit exact in fp32 and fp64, so exact ties are common and both
    choices must equal the oracle's lowest-index picks bit for bit."""
    import oracle.mita_oracle as O
    B, H, gh, gw, k = 2, 2, 4, 8, 7
    rng = np.random.default_rng(5)
    Q, K, V = (rng.integers(-2, 3, size=(B, H, gh * gw, 64)).astype(np.float32) for _ in range(3))
    _say(f"exact ties ({path})")
    res = run_gpu(Q, K, V, "bf16", gh, gw, gh, gw, k, path=path)
    ties = 0
    for b in range(B):
        for h in range(H):
            ref = O.mita_head(Q[b, h], K[b, h], V[b, h], gh, gw, gh, gw, k)
            ties += int(np.sum(ref["gap"] == 0)) + int(np.sum(ref["rgap"] == 0))
            assert np.array_equal(res["idx"][b, h], ref["idx"]), (b, h)
            assert np.array_equal(res["route"][b, h], ref["route"]), (b, h)
    assert ties > 10, "the case must actually contain exact ties"
    rep = parity.run_and_check(res, Q, K, V, gh, gw, gh, gw, k, TOL["bf16"])
    _say(f"ok ties={ties} {rep}")


def test_equal_scores_overflow_the_candidate_buffer():
    """Rows whose boundary histogram bin holds more keys than the landmark
    pass's candidate buffer (k + 256 entries).  Head 0 has Q = 0, so every
    score and every route logit is equal and the answer is keys 0..k-1 and
    landmark 0; head 1 has integer Q and sparse ternary K, so scores are exact
    multiples of 1/512 that repeat many times.  idx and route must equal the
    oracle's lowest-index picks bit for bit."""
    import oracle.mita_oracle as O
    B, H, gh, gw, mh, mw, k = 1, 2, 24, 32, 3, 4, 20
    N = gh * gw
    rng = np.random.default_rng(11)
    Q = rng.integers(-2, 3, size=(B, H, N, 64)).astype(np.float32)
    Q[0, 0] = 0.0
    K = (rng.integers(-1, 2, size=(B, H, N, 64)) * (rng.random((B, H, N, 64)) < 0.1)).astype(np.float32)
    V = synth.bf16_round(rng.standard_normal((B, H, N, 64)).astype(np.float32))
    _say("equal scores, buffer overflow")
    res = run_gpu(Q, K, V, "bf16", gh, gw, mh, mw, k)
    for h in range(H):
        ref = O.mita_head(Q[0, h], K[0, h], V[0, h], gh, gw, mh, mw, k)
        assert np.array_equal(res["idx"][0, h], ref["idx"]), h
        assert np.array_equal(res["route"][0, h], ref["route"]), h
    assert np.array_equal(res["idx"][0, 0], np.tile(np.arange(k), (mh * mw, 1)))
    rep = parity.run_and_check(res, Q, K, V, gh, gw, mh, mw, k, TOL["bf16"])
    _say(f"ok {rep}")


def test_equal_scores_across_key_chunks():
    """A grid past 4096 keys (5120: two key chunks of 2560, joined by the
    merge kernel) with k = 200, so the landmark pass runs its three-pass,
    eight-wave form.  Windows of 16 x 16 tokens keep Q_L = (integer sum) / 256
    exact, so every score and route logit is exact in fp32 and ties are
    decided by key id alone.  Head 0 has Q = 0: every score is equal, each
    chunk hands the merge its 200 lowest keys, and the 400 equal candidates
    overflow the merge's 256-entry boundary list (the rank-against-everything
    path); the answer is keys 0..199.  Head 1 has integer Q and sparse
    ternary K: scores repeat exactly, most rows tie at the boundary, and the
    winners span both chunks (the ranked list and its cut).  idx and route
    must equal the oracle's lowest-index picks bit for bit."""
    import oracle.mita_oracle as O
    B, H, gh, gw, mh, mw, k = 1, 2, 64, 80, 4, 5, 200
    N = gh * gw
    rng = np.random.default_rng(13)
    Q = rng.integers(-2, 3, size=(B, H, N, 64)).astype(np.float32)
    Q[0, 0] = 0.0
    K = (rng.integers(-1, 2, size=(B, H, N, 64)) * (rng.random((B, H, N, 64)) < 0.1)).astype(np.float32)
    V = synth.bf16_round(rng.standard_normal((B, H, N, 64)).astype(np.float32))
    _say("equal scores across key chunks")
    res = run_gpu(Q, K, V, "bf16", gh, gw, mh, mw, k)
    ties = 0
    for h in range(H):
        ref = O.mita_head(Q[0, h], K[0, h], V[0, h], gh, gw, mh, mw, k)
        ties += int(np.sum(ref["gap"] == 0))
        assert np.array_equal(res["idx"][0, h], ref["idx"]), h
        assert np.array_equal(res["route"][0, h], ref["route"]), h
    assert np.array_equal(res["idx"][0, 0], np.tile(np.arange(k), (mh * mw, 1)))
    assert ties > mh * mw + 8, "the case must tie at the boundary beyond head 0"
    rep = parity.run_and_check(res, Q, K, V, gh, gw, mh, mw, k, TOL["bf16"])
    _say(f"ok ties={ties} {rep}")


@pytest.mark.parametrize("name", ["tiny-fp32", "deit-t", "deit-s", "hires-3136", "ade-1024",
                                  "ade-1600"])
def test_workload_full(name):
    w = synth.workload(name)
    _say(f"workload {name} (all heads)")
    Q, K, V = synth.workload_inputs(name)
    res = run_gpu(Q, K, V, w["dtype"], w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"])
    rep = parity.run_and_check(res, Q, K, V, w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"],
                               TOL[w["dtype"]])
    _say(f"ok {name}: {rep}")


def test_workload_long_16k_all_heads():
    name = "long-16k"
    w = synth.workload(name)
    _say(f"workload {name} (full launch, all 32 heads)")
    Q, K, V = synth.workload_inputs(name)
    res = run_gpu(Q, K, V, w["dtype"], w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"])
    rep = parity.run_and_check(res, Q, K, V, w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"],
                               TOL[w["dtype"]])
    assert rep.heads == w["B"] * w["H"]
    _say(f"ok {name}: {rep}")


@pytest.mark.parametrize("name,heads", [("seq-64k", [(0, 0), (3, 1)]), ("seq-256k", [(0, 1)])],
                         ids=lambda v: v if isinstance(v, str) else "")
def test_workload_sequence_sampled_heads(name, heads):
    """The 1-D sequences at full size (the launch bench.py times); the oracle,
    ~1.5 s (64K) and ~13 s (256K) a head, checks the listed heads."""
    w = synth.workload(name)
    _say(f"workload {name} (full launch, heads {heads})")
    Q, K, V = synth.workload_inputs(name)
    res = run_gpu(Q, K, V, w["dtype"], w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"])
    rep = parity.run_and_check(res, Q, K, V, w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"],
                               TOL[w["dtype"]], heads=heads)
    _say(f"ok {name}: {rep}")


# Shapes the ABI accepts whose bf16 inputs leave the MFMA kernels' ranges for a
# step and take another kernel: scalar attention for m > 256, scalar routing
# for m > 512, per-landmark window pooling for grid_w > 256.
FALLBACKS = [
    # B, H, gh, gw, mh, mw, k
    (1, 1, 32, 32, 20, 20, 30),   # m = 400: scalar attention
    (1, 1, 32, 32, 32, 20, 24),   # m = 640: scalar routing and attention
    (1, 2, 2, 300, 2, 10, 20),    # grid_w = 300: window pooling
    (1, 1, 3, 320, 1, 300, 9),    # grid_w = 320, m = 300: window pooling, scalar attention
    (2, 1, 1, 5000, 1, 37, 50),   # a 1-D row: ragged windows, keys split over chunks
]


@pytest.mark.parametrize("case", FALLBACKS, ids=lambda c: "x".join(map(str, c)))
def test_scalar_fallback_steps(case):
    B, H, gh, gw, mh, mw, k = case
    _say(f"scalar fallback {case}")
    Q, K, V = synth.make_qkv(B, H, gh, gw, 64, workload_id=900 + gw + mh, dtype="bf16")
    res = run_gpu(Q, K, V, "bf16", gh, gw, mh, mw, k)
    rep = parity.run_and_check(res, Q, K, V, gh, gw, mh, mw, k, TOL["bf16"])
    _say(f"ok {rep}")


# The variants: s experts per query (one softmax over m + s*k entries) and
# route-only (no shared expert), on the matrix-core kernels and the scalar ones.
VARIANTS = [
    # B, H, gh, gw, mh, mw, k, s, route_only, dtype
    (2, 3, 14, 14, 5, 5, 25, 2, False, "bf16"),    # DeiT shape, two experts per query
    (1, 2, 56, 56, 7, 7, 64, 2, False, "bf16"),
    (1, 2, 56, 56, 7, 7, 64, 4, False, "bf16"),
    (1, 1, 12, 12, 4, 4, 20, 8, False, "bf16"),    # the largest s
    (1, 1, 10, 10, 3, 3, 100, 3, False, "bf16"),   # k = N: every key held s times
    (2, 3, 14, 14, 5, 5, 50, 1, True, "bf16"),     # route-only at the DeiT budget m + k
    (1, 2, 56, 56, 7, 7, 113, 1, True, "bf16"),    # route-only at the 3136 budget 49 + 64
    (1, 2, 20, 24, 6, 5, 37, 3, True, "bf16"),     # route-only, three experts
    (1, 2, 9, 7, 3, 2, 21, 2, False, "f32"),       # scalar kernels
    (1, 1, 8, 8, 4, 4, 64, 3, True, "f32"),        # scalar, route-only, k = N
    (1, 1, 32, 32, 20, 20, 30, 2, False, "bf16"),  # m = 400: scalar attention
    (1, 1, 32, 32, 32, 20, 24, 3, False, "bf16"),  # m = 640: scalar routing and attention
]


@pytest.mark.parametrize("case", VARIANTS,
                         ids=lambda c: "x".join(map(str, c[:7])) + f"-s{c[7]}" +
                         ("-ro" if c[8] else "") + "-" + c[9])
def test_variants(case):
    B, H, gh, gw, mh, mw, k, s, ro, dtype = case
    _say(f"variant {case}")
    Q, K, V = synth.make_qkv(B, H, gh, gw, 64, workload_id=1300 + gh * 7 + gw + s,
                             smooth=dtype == "bf16", dtype=dtype)
    res = run_gpu(Q, K, V, dtype, gh, gw, mh, mw, k, s=s, route_only=ro)
    assert res["route"].shape == ((B, H, gh * gw) if s == 1 else (B, H, gh * gw, s))
    rep = parity.run_and_check(res, Q, K, V, gh, gw, mh, mw, k, TOL[dtype], s=s, shared=not ro)
    _say(f"ok {rep}")


@pytest.mark.parametrize("name,s,ro,k", [("deit-s", 2, False, None), ("hires-3136", 2, False, None),
                                         ("deit-s", 1, True, 50), ("hires-3136", 1, True, 113)],
                         ids=lambda v: str(v))
def test_workload_variants(name, s, ro, k):
    """The full DeiT-S and 3136-token workloads with two experts per query, and
    route-only with the same number of entries per query as the plain pass."""
    w = synth.workload(name)
    k = w["k"] if k is None else k
    _say(f"workload {name} s={s} route_only={ro} k={k} (all heads)")
    Q, K, V = synth.workload_inputs(name)
    res = run_gpu(Q, K, V, w["dtype"], w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], k, s=s,
                  route_only=ro)
    rep = parity.run_and_check(res, Q, K, V, w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], k,
                               TOL[w["dtype"]], s=s, shared=not ro)
    _say(f"ok {name}: {rep}")


def test_expert_attention_with_one_workgroup_per_expert():
    """One head with m = 256 experts and a small k: the expert-attention kernel
    gives every expert its own workgroup, so the head's 256 expert counts (used
    to deal the experts) exceed one workgroup's expert table; every output row
    must still be written (the output starts as NaN) and match the oracle."""
    import efficient_attention_avg_amd as mita
    torch = _torch()
    B, H, gh, gw, mh, mw, k = 1, 1, 32, 32, 16, 16, 8
    _say(f"one workgroup per expert {(B, H, gh, gw, mh, mw, k)}")
    Q, K, V = synth.make_qkv(B, H, gh, gw, 64, workload_id=4242)
    q, kk, v = (_to_dev(x, "bf16") for x in (Q, K, V))
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    res = mita.mita_forward_ex(q, kk, v, gh, gw, mh, mw, k, out=out, idx=True, route=True,
                               extras=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    res = {key: val.cpu().numpy() for key, val in res.items() if val is not None}
    rep = parity.run_and_check(res, Q, K, V, gh, gw, mh, mw, k, TOL["bf16"])
    _say(f"ok {rep}")


def test_stage_entry_points():
    """Each step's own entry point against the oracle, fed the oracle's inputs where it needs them."""
    import efficient_attention_avg_amd as mita
    import oracle.mita_oracle as O
    torch = _torch()
    B, H, gh, gw, mh, mw, k = 2, 2, 21, 19, 4, 3, 30
    _say("stage entry points")
    Q, K, V = synth.make_qkv(B, H, gh, gw, 64, workload_id=777)
    q, kk, v = (_to_dev(x, "bf16") for x in (Q, K, V))
    ql = mita.mita_pool(q, gh, gw, mh, mw)
    ref_ql = O.landmark_queries(Q, gh, gw, mh, mw)
    assert np.abs(ql.cpu().numpy() - ref_ql).max() < 1e-5
    ql_in = torch.from_numpy(ref_ql.astype(np.float32)).cuda()
    idx, vl = mita.mita_landmark(ql_in, kk, v, k)
    route, counts, offsets, perm = mita.mita_route(q, ql_in)
    out = mita.mita_attend(q, kk, v, ql_in, vl, idx, route, offsets, perm)
    torch.cuda.synchronize()
    res = dict(out=out, idx=idx, route=route, vl=vl, counts=counts, offsets=offsets, perm=perm)
    res = {key: val.cpu().numpy() for key, val in res.items()}
    rep = parity.run_and_check(res, Q, K, V, gh, gw, mh, mw, k, 1e-2)
    _say(f"ok stages: {rep}")


def test_deterministic_and_fully_written():
    import efficient_attention_avg_amd as mita
    torch = _torch()
    w = synth.workload("deit-s")
    _say("determinism + NaN-poisoned outputs")
    Q, K, V = synth.workload_inputs("deit-s", B=8)
    q, kk, v = (_to_dev(x, "bf16") for x in (Q, K, V))
    args = (w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"])
    out1 = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    mita.mita_forward(q, kk, v, *args, out=out1)
    out2 = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((mita.mita_workspace_bytes(8, 6, 14, 14, 64, 5, 5, 25, mita.MITA_BF16),),
                    255, dtype=torch.uint8, device="cuda")
    mita.mita_forward(q, kk, v, *args, out=out2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out1).all()
    assert torch.equal(out1, out2)


@pytest.mark.parametrize("shape,path", [((3, 2, 14, 14, 5, 5, 25), "fused"),
                                        ((3, 2, 14, 14, 5, 5, 25), "staged"),
                                        ((2, 2, 13, 11, 4, 3, 40), "staged"),
                                        ((1, 3, 9, 7, 3, 2, 21), "fused")],
                         ids=lambda c: "x".join(map(str, c)) if isinstance(c, tuple) else c)
def test_output_stays_inside_its_buffer(shape, path):
    """The output is a view in the middle of a larger buffer filled with a
    sentinel: every element of the view is written (finite), and not one byte
    on either side changes.  (The output stores address the head's rows through
    a buffer descriptor and send lanes without a query past its range.)"""
    import efficient_attention_avg_amd as mita
    torch = _torch()
    B, H, gh, gw, mh, mw, k = shape
    N = gh * gw
    _say(f"output guard {shape} {path}")
    Q, K, V = synth.make_qkv(B, H, gh, gw, 64, workload_id=70)
    q, kk, v = (_to_dev(x, "bf16") for x in (Q, K, V))
    n = B * H * N * 64
    guard = 4096 + 12  # floats on each side: the view is 16-byte aligned, not line-aligned
    big = torch.full((guard + n + guard,), -12345.0, dtype=torch.float32, device="cuda")
    out = big[guard:guard + n].view(B, H, N, 64)
    mita.mita_forward_ex(q, kk, v, gh, gw, mh, mw, k, out=out, path=path)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert (out != -12345.0).all()
    assert (big[:guard] == -12345.0).all() and (big[guard + n:] == -12345.0).all()
    ref = mita.mita_forward_ex(q, kk, v, gh, gw, mh, mw, k, path=path)["out"]
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("name,path,overlap", [("deit-s", "auto", False), ("hires-3136", "auto", False),
                                               ("hires-3136", "auto", True)])
def test_kernel_timing_events(name, path, overlap):
    """The per-kernel events of mita_forward_ex bracket every kernel: each
    kernel's interval (from its start event) is positive, the kernels on the
    caller's stream tile the call, and routing ends before the call does."""
    torch = _torch()
    import efficient_attention_avg_amd as mita
    w = synth.workload(name)
    B = 8
    Q, K, V = synth.workload_inputs(name, B=B)
    q, k, v = (_to_dev(x, w["dtype"]) for x in (Q, K, V))
    code = mita.MITA_BF16 if w["dtype"] == "bf16" else mita.MITA_F32
    sched = mita.mita_kernel_schedule(B, w["H"], w["grid_h"], w["grid_w"], 64, w["m_h"],
                                      w["m_w"], w["k"], code, path=path, overlap=overlap)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(sched) + 1)]
    for e in ev:
        e.record()
    _say(f"timing events {name}: {sched}")
    mita.mita_forward_ex(q, k, v, w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"],
                         path=path, events=ev, overlap=overlap)
    torch.cuda.synchronize()
    dts = {nm: ev[st].elapsed_time(ev[i + 1]) for i, (nm, st) in enumerate(sched)}
    assert all(dt > 0 for dt in dts.values()), dts
    total = ev[0].elapsed_time(ev[-1])
    # the caller's stream: each of its kernels opens with the previous one's end
    names = [nm for nm, _ in sched]
    main = [i for i, (nm, st) in enumerate(sched) if not overlap or nm not in ("route", "group")]
    chain = sum(dts[sched[i][0]] for i in main)
    assert abs(chain - total) <= 1e-3 * max(total, 1e-3) + 1e-4, (dts, total)
    if "route" in names:  # the side stream joined before attention ended
        assert ev[names.index("group") + 1].elapsed_time(ev[-1]) > 0


def test_side_stream_matches_one_stream():
    """Routing and grouping on the side stream, forked and joined through
    events from mita_sync_event_create (a device-scope release, no system
    fence), give the same bits as the one-stream schedule, over calls queued
    back to back on changing inputs (a stale read across the streams would
    show as a difference)."""
    torch = _torch()
    import efficient_attention_avg_amd as mita
    w = synth.workload("hires-3136")
    B, H = 2, w["H"]
    args = (w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"])
    ins = [tuple(_to_dev(x, "bf16") for x in synth.make_qkv(B, H, w["grid_h"], w["grid_w"], 64,
                                                             workload_id=60 + i))
           for i in range(3)]
    _say("side stream against one stream, 3 inputs x 2 rounds")
    ref = [mita.mita_forward_ex(*qkv, *args, route=True)["out"] for qkv in ins]
    torch.cuda.synchronize()
    got = []
    for _ in range(2):
        for qkv in ins:
            got.append(mita.mita_forward_ex(*qkv, *args, route=True, overlap=True))
    torch.cuda.synchronize()
    for i, res in enumerate(got):
        assert torch.equal(res["out"], ref[i % 3]), i


def test_sync_event_is_created():
    torch = _torch()
    import ctypes
    import efficient_attention_avg_amd as mita
    torch.cuda.init()
    h = ctypes.c_void_p()
    assert mita.lib().mita_sync_event_create(ctypes.byref(h)) == mita.MITA_OK
    assert h.value


def test_constant_values_give_constant_output():
    import efficient_attention_avg_amd as mita
    torch = _torch()
    _say("constant V")
    Q, K, _ = synth.make_qkv(2, 2, 14, 14, 64, workload_id=31)
    V = np.full_like(Q, 0.625)
    q, kk, v = (_to_dev(x, "bf16") for x in (Q, K, V))
    out = mita.mita_forward(q, kk, v, 14, 14, 5, 5, 25)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().numpy() - 0.625).max() < 1e-5
