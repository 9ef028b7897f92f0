"""Parity of the GPU backward (mita_backward, through the C ABI) with the fp64
oracle's gradients.

The oracle's backward is run with the GPU forward's own top-k sets and routes
(so a near-tie taken the other way by the GPU compares like with like), on
the same bf16-rounded (or fp32) inputs and the same dOut.  Gradients are fp32
sums of fp32 products: the bound is max-abs error <= 1e-3 * max(1, max|ref|)
per tensor (a sum of a few thousand fp32 terms, each within 2^-24 relative,
stays far inside it; the test also prints the errors it saw)."""
import sys

import numpy as np
import pytest

import oracle.mita_oracle as O
import synth

pytestmark = pytest.mark.gpu

RTOL = 1e-3


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def _run(Q, K, V, G, dtype, gh, gw, mh, mw, k, s=1, route_only=False):
    import torch

    import efficient_attention_avg_amd as mita
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    conv = (lambda x: torch.from_numpy(x).cuda()) if dtype == "f32" else \
        (lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda())
    q, kk, v = conv(Q), conv(K), conv(V)
    g = torch.from_numpy(G).cuda()
    fwd = mita.mita_forward_ex(q, kk, v, gh, gw, mh, mw, k, idx=True, route=True, s=s,
                               route_only=route_only)
    dq, dk, dv = mita.mita_backward(q, kk, v, g, gh, gw, mh, mw, k, s=s, route_only=route_only)
    torch.cuda.synchronize()
    return (fwd["idx"].cpu().numpy(), fwd["route"].cpu().numpy(),
            dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())


def _check(Q, K, V, G, gh, gw, mh, mw, k, res, s=1, route_only=False, heads=None):
    idx, route, dq, dk, dv = res
    B, H = Q.shape[:2]
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    worst = [0.0, 0.0, 0.0]
    for b, h in pairs:
        ref = O.mita_head_backward(Q[b, h], K[b, h], V[b, h], G[b, h], gh, gw, mh, mw, k, s=s,
                                   shared=not route_only, idx=idx[b, h], route=route[b, h])
        for i, (got, want) in enumerate(zip((dq[b, h], dk[b, h], dv[b, h]), ref)):
            scale = max(1.0, float(np.abs(want).max()))
            err = float(np.abs(got - want).max()) / scale
            worst[i] = max(worst[i], err)
            assert err <= RTOL, f"head ({b},{h}) {'dQ dK dV'.split()[i]}: error {err:.3g} x {scale:.3g}"
    return worst


CASES = [
    # B, H, gh, gw, mh, mw, k, dtype, s, route_only
    (2, 3, 14, 14, 5, 5, 25, "bf16", 1, False),     # DeiT shape, overlapping windows
    (1, 2, 9, 7, 3, 2, 21, "f32", 1, False),
    (1, 2, 56, 56, 7, 7, 64, "bf16", 1, False),
    (1, 1, 10, 10, 1, 1, 100, "bf16", 1, False),    # m = 1, k = N
    (1, 2, 20, 24, 6, 5, 37, "bf16", 2, False),     # two experts per query
    (2, 2, 14, 14, 5, 5, 50, "bf16", 1, True),      # route-only
    (1, 1, 12, 12, 4, 4, 20, "f32", 3, True),       # route-only, three experts
    (1, 1, 1, 3000, 1, 30, 50, "bf16", 1, False),   # a 1-D row
    (1, 1, 32, 32, 20, 20, 30, "bf16", 1, False),   # m = 400
    (1, 2, 16, 16, 5, 5, 64, "f32", 1, False),      # fp32, two entry tiles per wave
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:7])) + f"-{c[7]}-s{c[8]}"
                         + ("-ro" if c[9] else ""))
def test_backward_matches_oracle(case):
    B, H, gh, gw, mh, mw, k, dtype, s, ro = case
    _say(f"backward {case}")
    Q, K, V = synth.make_qkv(B, H, gh, gw, 64, workload_id=2100 + gh + gw + k,
                             smooth=dtype == "bf16", dtype=dtype)
    G = np.random.default_rng(gh * gw + k).standard_normal(Q.shape).astype(np.float32)
    res = _run(Q, K, V, G, dtype, gh, gw, mh, mw, k, s=s, route_only=ro)
    worst = _check(Q, K, V, G, gh, gw, mh, mw, k, res, s=s, route_only=ro)
    _say(f"ok relative max errors dQ {worst[0]:.2e} dK {worst[1]:.2e} dV {worst[2]:.2e}")


@pytest.mark.parametrize("name,B,heads", [("deit-s", 8, None), ("hires-3136", 2, None),
                                          ("long-16k", 1, [(0, 0), (0, 5)]),
                                          ("deit-s", 256, [(0, 0), (17, 3), (128, 1), (255, 5)])])
def test_backward_workloads(name, B, heads):
    """The workloads' shapes (leading batch entries), every head or a sample.  The full
    DeiT-S batch is the case where one workgroup walks all of a head's experts (the
    small batches give each expert a workgroup of its own)."""
    w = synth.workload(name)
    _say(f"backward workload {name} B={B}")
    Q, K, V = synth.workload_inputs(name, B=B)
    G = np.random.default_rng(7).standard_normal(Q.shape).astype(np.float32)
    args = (w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"])
    res = _run(Q, K, V, G, w["dtype"], *args)
    worst = _check(Q, K, V, G, *args, res, heads=heads)
    _say(f"ok relative max errors dQ {worst[0]:.2e} dK {worst[1]:.2e} dV {worst[2]:.2e}")
