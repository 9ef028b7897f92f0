"""The C-ABI library on the host: it loads, exports every declared symbol, and
rejects bad arguments before anything reaches the GPU (no launches here)."""
import ctypes
import os
import re

import pytest

import efficient_attention_avg_amd as mita

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "mita.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mita_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(mita.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = mita.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert L.mita_version().decode().startswith("mita-gfx950")
    assert L.mita_route_workspace_bytes(32, 6, 3136, 64, 49, mita.MITA_BF16) > 0
    assert L.mita_route_workspace_bytes(1, 1, 196, 64, 25, mita.MITA_F32) == 0


def test_sync_event_needs_a_pointer():
    # rejected before any runtime call, so this runs without a GPU
    assert mita.lib().mita_sync_event_create(None) == mita.MITA_ERR_INVALID_ARG


def test_status_strings():
    L = mita.lib()
    names = [L.mita_status_string(s).decode() for s in range(5)]
    assert names == ["MITA_OK", "MITA_ERR_INVALID_ARG", "MITA_ERR_UNSUPPORTED",
                     "MITA_ERR_WORKSPACE", "MITA_ERR_HIP"]


def test_workspace_bytes():
    ws = mita.mita_workspace_bytes
    L = mita.lib()
    # the fused schedule (DeiT shapes) needs no workspace; forcing the staged one does
    assert L.mita_workspace_bytes(256, 6, 14, 14, 64, 5, 5, 25, mita.MITA_BF16) == 0
    assert ws(256, 6, 14, 14, 64, 5, 5, 25, mita.MITA_BF16) == 0
    assert ws(256, 6, 14, 14, 64, 5, 5, 25, mita.MITA_BF16, path="staged") > 0
    assert ws(256, 6, 14, 14, 64, 5, 5, 25, mita.MITA_F32) > 0      # fp32: staged
    assert L.mita_workspace_bytes_ex(256, 6, 14, 14, 64, 5, 5, 25, mita.MITA_BF16, None) == 0
    assert ws(32, 6, 56, 56, 64, 7, 7, 64, mita.MITA_BF16) > 0
    assert ws(32, 6, 56, 56, 64, 7, 7, 64, mita.MITA_BF16, path="fused") == 0  # unsupported
    assert ws(1, 1, 14, 14, 64, 5, 5, 0, mita.MITA_F32) == 0       # k < 1
    assert ws(1, 1, 14, 14, 32, 5, 5, 25, mita.MITA_F32) == 0      # d != 64
    assert ws(1, 1, 14, 14, 64, 15, 5, 25, mita.MITA_F32) == 0     # m_h > grid_h


def test_kernel_names_follow_the_schedule():
    names = mita.mita_kernel_names
    assert names(256, 6, 14, 14, 64, 5, 5, 25, mita.MITA_BF16) == ["fused"]
    staged = ["pool", "route", "group", "landmark", "attend"]
    assert names(256, 6, 14, 14, 64, 5, 5, 25, mita.MITA_BF16, path="staged") == staged
    assert names(32, 6, 56, 56, 64, 7, 7, 64, mita.MITA_BF16) == staged
    assert names(1, 1, 14, 14, 64, 5, 5, 25, mita.MITA_F32) == staged
    # one stream: each kernel opens with the previous one's end; with a side stream
    # routing and grouping run beside the landmark pass, both opening at pooling's end
    assert mita.mita_kernel_schedule(32, 6, 56, 56, 64, 7, 7, 64, mita.MITA_BF16) == [
        ("pool", 0), ("route", 1), ("group", 2), ("landmark", 3), ("attend", 4)]
    assert mita.mita_kernel_schedule(32, 6, 56, 56, 64, 7, 7, 64, mita.MITA_BF16,
                                     overlap=True) == [
        ("pool", 0), ("route", 1), ("group", 2), ("landmark", 1), ("attend", 4)]
    assert mita.mita_kernel_schedule(256, 6, 14, 14, 64, 5, 5, 25, mita.MITA_BF16) == [("fused", 0)]
    with pytest.raises(mita.MitaError):
        names(32, 6, 56, 56, 64, 7, 7, 64, mita.MITA_BF16, path="fused")
    with pytest.raises(mita.MitaError):
        names(1, 1, 14, 14, 64, 5, 5, 0, mita.MITA_BF16)


def test_schedule_choice():
    sched = mita.mita_schedule
    assert sched(256, 6, 14, 14, 64, 5, 5, 25, mita.MITA_BF16) == "fused"
    assert sched(32, 6, 56, 56, 64, 7, 7, 64, mita.MITA_BF16) == "staged"
    assert sched(1, 1, 14, 14, 64, 5, 5, 25, mita.MITA_F32) == "staged"
    assert sched(1, 1, 13, 16, 64, 8, 4, 32, mita.MITA_BF16) == "fused"
    assert sched(1, 1, 13, 16, 64, 8, 4, 33, mita.MITA_BF16) == "staged"
    with pytest.raises(mita.MitaError):
        sched(1, 1, 14, 14, 64, 5, 5, 0, mita.MITA_BF16)


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every case fails validation first


def _fwd(B=1, H=1, gh=14, gw=14, d=64, mh=5, mw=5, k=25, dt=mita.MITA_BF16, q=FAKE, out=FAKE,
         ws=FAKE, nbytes=1 << 40, extras=None):
    L = mita.lib()
    return L.mita_forward_ex(q, FAKE, FAKE, B, H, gh, gw, d, mh, mw, k, dt, out, None, None,
                             extras, ws, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), mita.MITA_ERR_INVALID_ARG),
    (dict(H=-1), mita.MITA_ERR_INVALID_ARG),
    (dict(k=0), mita.MITA_ERR_INVALID_ARG),
    (dict(k=197), mita.MITA_ERR_INVALID_ARG),
    (dict(mh=15), mita.MITA_ERR_INVALID_ARG),
    (dict(mw=0), mita.MITA_ERR_INVALID_ARG),
    (dict(gh=0), mita.MITA_ERR_INVALID_ARG),
    (dict(dt=7), mita.MITA_ERR_INVALID_ARG),
    (dict(d=128), mita.MITA_ERR_UNSUPPORTED),
    (dict(q=None), mita.MITA_ERR_INVALID_ARG),
    (dict(out=None), mita.MITA_ERR_INVALID_ARG),
    # fp32 inputs take the staged schedule, which needs a workspace
    (dict(ws=None, dt=mita.MITA_F32), mita.MITA_ERR_INVALID_ARG),
    (dict(nbytes=16, dt=mita.MITA_F32), mita.MITA_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x10010), dt=mita.MITA_F32), mita.MITA_ERR_INVALID_ARG),  # misaligned
    (dict(q=ctypes.c_void_p(0x10004)), mita.MITA_ERR_INVALID_ARG),    # Q not 16-byte aligned
    (dict(out=ctypes.c_void_p(0x10008)), mita.MITA_ERR_INVALID_ARG),  # out not 16-byte aligned
    (dict(B=65536), mita.MITA_ERR_UNSUPPORTED),
])
def test_forward_rejects_before_launch(kw, status):
    assert _fwd(**kw) == status
    assert mita.lib().mita_last_error().decode() != ""


def test_forward_rejects_unknown_path():
    ex = mita._Extras(path=9)
    assert _fwd(extras=ctypes.byref(ex)) == mita.MITA_ERR_INVALID_ARG


def test_staged_schedule_needs_a_workspace():
    ex = mita._Extras(path=mita.PATHS["staged"])
    assert _fwd(ws=None, nbytes=0, extras=ctypes.byref(ex)) == mita.MITA_ERR_INVALID_ARG
    assert "workspace" in mita.lib().mita_last_error().decode()


@pytest.mark.parametrize("s,ro,status", [(0, 2, mita.MITA_ERR_INVALID_ARG),
                                         (-1, 0, mita.MITA_ERR_INVALID_ARG),
                                         (9, 0, mita.MITA_ERR_INVALID_ARG),
                                         (26, 0, mita.MITA_ERR_INVALID_ARG)])  # s > m = 25
def test_forward_rejects_bad_variant(s, ro, status):
    ex = mita._Extras(s=s, route_only=ro)
    assert _fwd(extras=ctypes.byref(ex)) == status
    assert mita.lib().mita_last_error().decode() != ""


def test_binding_checks_grid_against_tokens():
    import torch
    q = torch.zeros(1, 1, 196, 64, dtype=torch.bfloat16)
    # the grid check runs before the device check would (host tensors here)
    with pytest.raises(ValueError, match="grid"):
        mita._grid(q, 14, 15)
    mita._grid(q, 14, 14)


def test_stage_entry_points_validate():
    L = mita.lib()
    assert L.mita_pool(None, 1, 1, 14, 14, 64, 5, 5, 1, FAKE, None) == mita.MITA_ERR_INVALID_ARG
    assert L.mita_landmark(FAKE, FAKE, FAKE, 1, 1, 196, 64, 25, 26 * 0 + 197, 1, FAKE, FAKE, FAKE,
                           1 << 40, None) == mita.MITA_ERR_INVALID_ARG          # k > N
    # fp32 inputs take the scalar landmark kernel, which needs scratch
    assert L.mita_landmark(FAKE, FAKE, FAKE, 1, 1, 196, 64, 25, 25, mita.MITA_F32, FAKE, FAKE,
                           FAKE, 4, None) == mita.MITA_ERR_WORKSPACE
    assert L.mita_landmark_workspace_bytes(1, 1, 196, 64, 25, 25, mita.MITA_BF16) == 0
    # the bf16 MFMA landmark kernel keeps a k + 64 candidate buffer per row in LDS: up to
    # k = 400; beyond, the scalar kernel and its score-row scratch (m * N floats) take over
    assert L.mita_landmark_workspace_bytes(1, 1, 16384, 64, 256, 401, mita.MITA_BF16) >= \
        256 * 16384 * 4
    # keys split over several workgroups per row leave candidates for a merge: the
    # long grid needs scratch, a short one (one chunk) none
    assert 0 < L.mita_landmark_workspace_bytes(1, 1, 16384, 64, 256, 400, mita.MITA_BF16) < \
        256 * 16384 * 4
    assert L.mita_route(FAKE, FAKE, 1, 1, 196, 64, 25, 1, FAKE, FAKE, None, FAKE, FAKE, 1 << 40,
                        None) == mita.MITA_ERR_INVALID_ARG
    assert L.mita_route(FAKE, FAKE, 1, 1, 3136, 64, 49, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 8,
                        None) == mita.MITA_ERR_WORKSPACE
    assert L.mita_attend(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 196, 64, 25,
                         25, 1, None, None) == mita.MITA_ERR_INVALID_ARG


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 1, 196, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mita.mita_forward(q, q, q, 14, 14, 5, 5, 25)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    L = mita.lib()
    # 1024 heads of 3136 tokens need far more than the 32 MiB static scratch;
    # refused before any device call
    assert L.mita_forward_noalloc(FAKE, FAKE, FAKE, 128, 8, 56, 56, 64, 7, 7, 64, mita.MITA_BF16,
                                  FAKE, None, None, None) == mita.MITA_ERR_WORKSPACE
    assert "scratch" in L.mita_last_error().decode()
    assert L.mita_forward_noalloc(FAKE, FAKE, FAKE, 1, 1, 14, 14, 64, 5, 5, 0, mita.MITA_BF16,
                                  FAKE, None, None, None) == mita.MITA_ERR_INVALID_ARG
