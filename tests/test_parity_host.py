"""The parity checker on the host: it accepts the oracle's own results (for the
plain pass and the variants) and rejects results with a planted mistake, so a
GPU parity test cannot pass on a checker that looks at nothing."""
import numpy as np
import pytest

import oracle.mita_oracle as O
import synth
from tests import parity


def _oracle_as_gpu(Q, K, V, gh, gw, mh, mw, k, s, shared):
    B, H = Q.shape[:2]
    res = O.mita_forward(Q, K, V, gh, gw, mh, mw, k, s=s, shared=shared)
    out = dict(out=res["out"], idx=res["idx"], route=res["route"], ql=res["QL"],
               counts=res["counts"], offsets=res["offsets"], perm=res["perm"])
    if shared:
        out["vl"] = res["VL"]
    return {key: np.asarray(val) for key, val in out.items()}


CASES = [(1, True), (3, True), (1, False), (2, False)]


@pytest.mark.parametrize("s,shared", CASES)
def test_checker_accepts_the_oracle(s, shared):
    Q, K, V = synth.make_qkv(1, 2, 9, 8, 64, workload_id=11, dtype="bf16")
    got = _oracle_as_gpu(Q, K, V, 9, 8, 3, 2, 7, s, shared)
    rep = parity.run_and_check(got, Q, K, V, 9, 8, 3, 2, 7, 1e-9, s=s, shared=shared)
    assert rep.heads == 2 and rep.topk_deviations == 0 and rep.route_deviations == 0


@pytest.mark.parametrize("s,shared", CASES)
def test_checker_rejects_a_wrong_route(s, shared):
    Q, K, V = synth.make_qkv(1, 1, 9, 8, 64, workload_id=12, dtype="bf16")
    got = _oracle_as_gpu(Q, K, V, 9, 8, 3, 2, 7, s, shared)
    R = Q[0, 0].astype(np.float64) @ got["ql"][0, 0].T
    rgap = np.sort(R, axis=-1)[:, -1] - np.sort(R, axis=-1)[:, -2]
    n = int(np.argmax(rgap))                       # a query far from any tie
    worst = int(np.argmin(R[n]))
    r = got["route"].reshape(1, 1, 72, -1)
    r[0, 0, n, 0] = worst                           # its best route replaced by its worst
    with pytest.raises(AssertionError):
        parity.run_and_check(got, Q, K, V, 9, 8, 3, 2, 7, 1e-2, s=s, shared=shared)


def test_checker_rejects_a_wrong_topk_set():
    Q, K, V = synth.make_qkv(1, 1, 9, 8, 64, workload_id=13, dtype="bf16")
    got = _oracle_as_gpu(Q, K, V, 9, 8, 3, 2, 7, 1, True)
    row = got["idx"][0, 0, 0]
    missing = next(j for j in range(72) if j not in row)
    got["idx"][0, 0, 0] = np.sort(np.concatenate([row[1:], [missing]]))
    with pytest.raises(AssertionError):
        parity.run_and_check(got, Q, K, V, 9, 8, 3, 2, 7, 1e-2)
