"""mita_forward_noalloc (the static-scratch variant of mita_forward) against
mita_forward with a caller workspace, through the C ABI: the same kernels run,
so out, idx and route must be identical bit for bit.  Calls come in a row on
one device, the second on a smaller input than the first, so the second
reads a scratch array that still holds the first call's intermediates."""
import sys

import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def test_noalloc_matches_forward_on_calls_in_a_row():
    import torch

    import efficient_attention_avg_amd as mita
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    shapes = [
        # B, H, gh, gw, mh, mw, k: staged (uses the scratch), then smaller staged
        # shapes -- one row of 8192 tokens, whose keys split into two chunks
        # (candidate lists and V_L partials in the scratch, joined by the
        # merge kernel), and a 40x40 grid -- then a fused one (needs no scratch)
        (2, 6, 56, 56, 7, 7, 64),
        (1, 2, 1, 8192, 1, 32, 64),
        (1, 3, 40, 40, 5, 5, 30),
        (4, 6, 14, 14, 5, 5, 25),
    ]
    for i, (B, H, gh, gw, mh, mw, k) in enumerate(shapes):
        _say(f"noalloc call {i}: {(B, H, gh, gw, mh, mw, k)}")
        Q, K, V = synth.make_qkv(B, H, gh, gw, 64, workload_id=880 + i)
        q, kk, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (Q, K, V))
        ref = mita.mita_forward_ex(q, kk, v, gh, gw, mh, mw, k, idx=True, route=True)
        got = mita.mita_forward_noalloc(q, kk, v, gh, gw, mh, mw, k, idx=True, route=True)
        torch.cuda.synchronize()
        assert torch.equal(got["out"], ref["out"]), i
        assert torch.equal(got["idx"], ref["idx"]), i
        assert torch.equal(got["route"], ref["route"]), i
        if i in (1, 2):
            res = {key: val.cpu().numpy() for key, val in got.items()}
            rep = parity.run_and_check(res, Q, K, V, gh, gw, mh, mw, k, 1e-2)
            _say(f"ok parity {rep}")
