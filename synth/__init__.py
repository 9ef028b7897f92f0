"""Seeded synthetic inputs for the MiTA forward pass.

This module only *draws* inputs: it holds none of the method's arithmetic
(no pooling, scoring, selection, routing or softmax).  Both the fp64 oracle
and the HIP path consume what it returns, so it is the one piece of code
they share.

Workloads stand in for the token grids of the pages' experiments:
DeiT-T / DeiT-S on 224x224 ImageNet images (14x14 patch grid), a
high-resolution 56x56 vision grid, a 128x128 long-sequence grid, the
segmentation grids of 1,024 and 1,600 tokens with m = k = 49, and
one-dimensional sequences of 64K and 256K tokens with m * k = N / 4 (page
"NeurIPS'26: attention is also an FFN?", sections on image classification,
semantic segmentation and long-sequence modelling, Figure 4).  A 1-D
sequence is a grid of one row, so pooling is 1-D adaptive average pooling
and the smooth component varies along the sequence only.  No dataset is
read: every tensor is synthetic.

Recipe (per tensor Q, K, V of shape [B, H, N, d], N = grid_h * grid_w,
token n = y * grid_w + x):
  * one numpy PCG64 stream per (workload, tensor), seeded with
    ``SeedSequence(0, spawn_key=(workload_id, tensor_id))``;
  * for each batch index b in order: noise ~ N(0, 1) of shape [H, N, d],
    then (when ``smooth``) f_y, f_x ~ U[-2, 2] and phi ~ U[0, 2*pi) of shape
    [H, d, 4], and the smooth term
        sum_{j<4} sin(2*pi*(f_y[j]*y/grid_h + f_x[j]*x/grid_w) + phi[j])
    (four sinusoids of amplitude 1 per channel) is added to the noise;
  * the fp64 sum is cast to fp32, then (bf16 workloads) rounded to bfloat16
    with round-to-nearest-even and kept as the fp32 value of that bfloat16.
"""
from __future__ import annotations

import numpy as np

TENSOR_IDS = {"Q": 0, "K": 1, "V": 2}

# The five workloads.  "id" seeds the generator; the tiny fp32 case has no
# smooth component.
WORKLOADS = [
    dict(id=0, name="tiny-fp32", B=1, H=1, grid_h=14, grid_w=14, d=64, m_h=5, m_w=5, k=25,
         dtype="f32", smooth=False),
    dict(id=1, name="deit-t", B=256, H=3, grid_h=14, grid_w=14, d=64, m_h=5, m_w=5, k=25,
         dtype="bf16", smooth=True),
    dict(id=2, name="deit-s", B=256, H=6, grid_h=14, grid_w=14, d=64, m_h=5, m_w=5, k=25,
         dtype="bf16", smooth=True),
    dict(id=3, name="hires-3136", B=32, H=6, grid_h=56, grid_w=56, d=64, m_h=7, m_w=7, k=64,
         dtype="bf16", smooth=True),
    dict(id=4, name="long-16k", B=4, H=8, grid_h=128, grid_w=128, d=64, m_h=16, m_w=16, k=256,
         dtype="bf16", smooth=True),
    # segmentation-sized grids (1,024 and 1,600 patch tokens, m = k = 49) and
    # one-dimensional long sequences (a single row of tokens; m * k = N / 4;
    # two heads of width 64, i.e. model width 128)
    dict(id=5, name="ade-1024", B=32, H=6, grid_h=32, grid_w=32, d=64, m_h=7, m_w=7, k=49,
         dtype="bf16", smooth=True),
    dict(id=6, name="ade-1600", B=32, H=6, grid_h=40, grid_w=40, d=64, m_h=7, m_w=7, k=49,
         dtype="bf16", smooth=True),
    dict(id=7, name="seq-64k", B=4, H=2, grid_h=1, grid_w=65536, d=64, m_h=1, m_w=128, k=128,
         dtype="bf16", smooth=True),
    dict(id=8, name="seq-256k", B=1, H=2, grid_h=1, grid_w=262144, d=64, m_h=1, m_w=256, k=256,
         dtype="bf16", smooth=True),
]


def workload(name_or_id) -> dict:
    for w in WORKLOADS:
        if w["id"] == name_or_id or w["name"] == name_or_id:
            return dict(w)
    raise KeyError(name_or_id)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round-to-nearest-even), returned as fp32.

    NaN is not produced by the generator, so no NaN special case is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The uint16 bit patterns of fp32 values that are exactly bfloat16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bfloat16-representable")
    return (u >> np.uint32(16)).astype(np.uint16)


def _smooth_term(rng, H, grid_h, grid_w, d):
    fy = rng.uniform(-2.0, 2.0, size=(H, d, 4))
    fx = rng.uniform(-2.0, 2.0, size=(H, d, 4))
    phi = rng.uniform(0.0, 2.0 * np.pi, size=(H, d, 4))
    y = np.repeat(np.arange(grid_h, dtype=np.float64), grid_w) / grid_h   # [N]
    x = np.tile(np.arange(grid_w, dtype=np.float64), grid_h) / grid_w     # [N]
    acc = np.zeros((H, d, grid_h * grid_w))
    for j in range(4):
        ph = 2.0 * np.pi * (fy[..., j, None] * y + fx[..., j, None] * x) + phi[..., j, None]
        acc += np.sin(ph)
    return acc.transpose(0, 2, 1)  # [H, N, d]


def make_tensor(B, H, grid_h, grid_w, d, *, workload_id, tensor, smooth=True, dtype="bf16"):
    """One seeded input tensor [B, H, N, d] as fp32 (bf16-exact when dtype='bf16')."""
    tid = TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)
    rng = np.random.default_rng(np.random.SeedSequence(0, spawn_key=(int(workload_id), tid)))
    N = grid_h * grid_w
    out = np.empty((B, H, N, d), dtype=np.float32)
    for b in range(B):
        x = rng.standard_normal((H, N, d))
        if smooth:
            x = x + _smooth_term(rng, H, grid_h, grid_w, d)
        out[b] = x.astype(np.float32)
    if dtype == "bf16":
        out = bf16_round(out)
    elif dtype != "f32":
        raise ValueError(dtype)
    return out


def make_qkv(B, H, grid_h, grid_w, d, *, workload_id, smooth=True, dtype="bf16"):
    """(Q, K, V) for one workload shape; see the module docstring for the recipe."""
    return tuple(make_tensor(B, H, grid_h, grid_w, d, workload_id=workload_id, tensor=t,
                             smooth=smooth, dtype=dtype) for t in ("Q", "K", "V"))


def workload_inputs(name_or_id, B=None, H=None):
    """Inputs of a named workload; B / H may be cut down for quick checks.

    A cut-down batch gives the leading batch entries of the full workload,
    since the stream is consumed batch entry by batch entry.  Cutting H
    changes the draws and is only for tests that do not compare against the
    full workload.
    """
    w = workload(name_or_id)
    B = w["B"] if B is None else B
    H = w["H"] if H is None else H
    return make_qkv(B, H, w["grid_h"], w["grid_w"], w["d"], workload_id=w["id"],
                    smooth=w["smooth"], dtype=w["dtype"])
